// Per-kernel timing of the library's launches (see profile.hip).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "../../include/starkv.h"

namespace skv {

// Names one kernel launch.  While timing is enabled it holds two events that the launch made
// through launch_k() below fills with the kernel's own start and end timestamps; on destruction
// the pair is queued for starkv_profile_read.  Disabled: no events, a plain launch.
class ProfScope {
 public:
  explicit ProfScope(const char* name);
  ~ProfScope();
  ProfScope(const ProfScope&) = delete;
  ProfScope& operator=(const ProfScope&) = delete;
  hipEvent_t start() const { return a_; }
  hipEvent_t stop() const { return b_; }

 private:
  const char* name_;
  hipEvent_t a_, b_;
};

// Launch of a kernel taking one argument block by value.
template <typename A>
hipError_t launch_k(const ProfScope& ps, void (*kernel)(A), dim3 grid, dim3 block, hipStream_t s, A arg) {
  void* argv[] = {(void*)&arg};
  if (ps.start() && ps.stop())
    return hipExtLaunchKernel((const void*)kernel, grid, block, argv, 0, s, ps.start(), ps.stop(), 0);
  return hipLaunchKernel((const void*)kernel, grid, block, argv, 0, s);
}

int profile_enable(int on);
int profile_read(starkv_kernel_time* out, int max_entries, int* n_entries, int reset);

}  // namespace skv
