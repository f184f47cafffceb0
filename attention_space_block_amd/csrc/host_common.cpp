// Error reporting and shared argument checks (host only).
#include <stdarg.h>

#include "host_common.hpp"

namespace kvm {

static thread_local char g_err[512];

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

void clear_error() { g_err[0] = 0; }

const char* last_error() { return g_err; }

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

extern "C" int kvm_version(void) { return 104; }

extern "C" const char* kvm_last_error(void) { return kvm::last_error(); }
