// Per-kernel timing: when enabled, each kernel launch of the library is made with
// hipExtLaunchKernel and two events that take the kernel's own start and end timestamps (the
// same interval a kernel trace reports).  Reading the totals synchronises on those events.
// Off by default.
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "profile.h"

namespace skv {

namespace {
struct Pending {
  const char* name;
  hipEvent_t a, b;
};
struct Total {
  std::string name;
  int launches = 0;
  double ms = 0.0;
};
std::mutex g_mu;
bool g_on = false;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_pool;
std::vector<Total> g_totals;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

ProfScope::ProfScope(const char* name) : name_(name), a_(nullptr), b_(nullptr) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on) return;
  a_ = take_event();
  b_ = take_event();
  if (!a_ || !b_) {
    if (a_) g_pool.push_back(a_);
    if (b_) g_pool.push_back(b_);
    a_ = b_ = nullptr;
  }
}

ProfScope::~ProfScope() {
  if (!a_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  g_pending.push_back(Pending{name_, a_, b_});
}

int profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_on = on != 0;
  return 0;
}

int profile_read(starkv_kernel_time* out, int max_entries, int* n_entries, int reset) {
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto& p : g_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.b) != hipSuccess || hipEventElapsedTime(&ms, p.a, p.b) != hipSuccess) return -6;
    Total* t = nullptr;
    for (auto& x : g_totals)
      if (x.name == p.name) t = &x;
    if (!t) {
      g_totals.push_back(Total{p.name, 0, 0.0});
      t = &g_totals.back();
    }
    t->launches += 1;
    t->ms += ms;
    g_pool.push_back(p.a);
    g_pool.push_back(p.b);
  }
  g_pending.clear();
  const int n = (int)g_totals.size();
  if (n_entries) *n_entries = n;
  for (int i = 0; i < n && i < max_entries && out; ++i) {
    memset(out[i].name, 0, sizeof(out[i].name));
    strncpy(out[i].name, g_totals[i].name.c_str(), sizeof(out[i].name) - 1);
    out[i].launches = g_totals[i].launches;
    out[i].total_ms = g_totals[i].ms;
  }
  if (reset) g_totals.clear();
  return 0;
}

}  // namespace skv
