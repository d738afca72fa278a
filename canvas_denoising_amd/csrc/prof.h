// Scoped per-kernel event timing (see prof.cpp).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace dg {

bool prof_on();

// Times the launches issued while it lives. With `dispatch_events`, the launch site passes start()
// and stop() to hipExtLaunchKernel (when active()): the events are then taken by the kernel's own
// dispatch, at its start and end, instead of by marker packets queued around it.
class ProfScope {
 public:
  ProfScope(const char* name, hipStream_t s, bool dispatch_events = false);
  ~ProfScope();
  ProfScope(const ProfScope&) = delete;
  ProfScope& operator=(const ProfScope&) = delete;
  bool active() const { return active_; }
  hipEvent_t start() const { return a_; }
  hipEvent_t stop() const { return b_; }

 private:
  const char* name_;
  hipStream_t stream_;
  hipEvent_t a_ = nullptr, b_ = nullptr;
  bool active_ = false;
  bool dispatch_ = false;
};

// Launch `kernel` on s; under an active dispatch-event ProfScope the dispatch itself takes the events.
template <typename K, typename... Args>
inline void launch_timed(const ProfScope& ps, K kernel, dim3 grid, dim3 block, hipStream_t s, Args... args) {
  if (ps.active())
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ps.start(), ps.stop(), 0, args...);
  else
    kernel<<<grid, block, 0, s>>>(args...);
}

}  // namespace dg
