// Scoped per-kernel event timing (see prof.cpp).
#pragma once

#include <hip/hip_runtime.h>

namespace dg {

bool prof_on();

// Times the launches issued while it lives: an event before and after them on their stream.
class ProfScope {
 public:
  ProfScope(const char* name, hipStream_t s);
  ~ProfScope();
  ProfScope(const ProfScope&) = delete;
  ProfScope& operator=(const ProfScope&) = delete;

 private:
  const char* name_;
  hipStream_t stream_;
  hipEvent_t a_ = nullptr, b_ = nullptr;
  bool active_ = false;
};

}  // namespace dg
