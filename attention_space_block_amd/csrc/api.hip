// Entry points that are not tied to one kernel: version, errors, validation.
#include <stdarg.h>

#include "common.hpp"

namespace kvm {

static thread_local char g_err[512];

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

void clear_error() { g_err[0] = 0; }

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

int check_dims(const kvm_dims* d, int32_t dtype) {
  KVM_CHECK_ARG(d != nullptr, "dims is NULL");
  KVM_CHECK_ARG(dtype == KVM_F32 || dtype == KVM_BF16 || dtype == KVM_FP8_E4M3,
                "dtype %d invalid", dtype);
  KVM_CHECK_ARG(d->n_layers > 0 && d->n_kv_heads > 0 && d->n_q_heads > 0,
                "layers/heads must be positive");
  KVM_CHECK_ARG(d->n_q_heads % d->n_kv_heads == 0, "n_q_heads %% n_kv_heads != 0");
  if (d->head_dim != 64 && d->head_dim != 128) {
    set_error("head_dim %d unsupported (64, 128)", d->head_dim);
    return KVM_ENOTSUP;
  }
  if (d->block_tokens != 32) {
    set_error("block_tokens %d unsupported (32)", d->block_tokens);
    return KVM_ENOTSUP;
  }
  return KVM_OK;
}

}  // namespace kvm

extern "C" int kvm_version(void) { return 100; }

extern "C" const char* kvm_last_error(void) { return kvm::g_err; }
