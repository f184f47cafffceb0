// Memory-range validation of pointer arguments (HIP runtime queries only).

#include "common.hpp"

namespace kvm {

int check_range(const void* p, size_t bytes, RangeKind kind, const char* what) {
  if (bytes == 0) return KVM_OK;
  if (p == nullptr) {
    set_error("%s is NULL", what);
    return KVM_EINVAL;
  }
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();                   // leave no sticky error behind
    at.type = hipMemoryTypeUnregistered;
  }
  if (at.type == hipMemoryTypeUnregistered) {
    set_error("%s (%p) is not in memory allocated through HIP (device, managed or pinned host)",
              what, p);
    return KVM_EINVAL;
  }
  if (kind == RANGE_PINNED_HOST && at.type != hipMemoryTypeHost) {
    set_error("%s (%p) must be pinned host memory", what, p);
    return KVM_EINVAL;
  }
  if (at.type == hipMemoryTypeDevice) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || at.device != dev) {
      set_error("%s (%p) is device memory of GPU %d, not of the current GPU %d", what, p,
                at.device, dev);
      return KVM_EINVAL;
    }
  }
  // The extent check needs the allocation's range; memory the runtime knows
  // but cannot give a range for (virtual-memory mappings) is accepted as is.
  void* base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(reinterpret_cast<hipDeviceptr_t*>(&base), &size,
                            const_cast<void*>(p)) != hipSuccess) {
    (void)hipGetLastError();
    return KVM_OK;
  }
  const size_t off = (size_t)((const char*)p - (const char*)base);
  if (off > size || bytes > size - off) {
    set_error("%s: %zu bytes from %p run past the end of its allocation (%zu bytes left)", what,
              bytes, p, off > size ? (size_t)0 : size - off);
    return KVM_EINVAL;
  }
  return KVM_OK;
}

}  // namespace kvm


