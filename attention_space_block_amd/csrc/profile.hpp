// Scoped HIP-event timer around one kernel launch (active only while
// kvm_profile_enable(1) is in effect).
#pragma once
#include <hip/hip_runtime.h>

namespace kvm {
class KernelTimer {
 public:
  KernelTimer(const char* name, hipStream_t s);
  ~KernelTimer();
  KernelTimer(const KernelTimer&) = delete;
  KernelTimer& operator=(const KernelTimer&) = delete;

 private:
  const char* name_;
  hipStream_t s_;
  void* a_ = nullptr;
  void* b_ = nullptr;
};
}  // namespace kvm
