// Per-kernel event timing of the library's launches (see profile.hip).
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/starkv.h"

namespace skv {

// Brackets the launches made while it is alive with two events on stream s (when enabled).
class ProfScope {
 public:
  ProfScope(const char* name, hipStream_t s);
  ~ProfScope();
  ProfScope(const ProfScope&) = delete;
  ProfScope& operator=(const ProfScope&) = delete;

 private:
  const char* name_;
  hipStream_t s_;
  void* a_;
};

int profile_enable(int on);
int profile_read(starkv_kernel_time* out, int max_entries, int* n_entries, int reset);

}  // namespace skv
