// Host-side helpers of libkvm shared by the HIP sources and the host-only
// sources (block pool, data-plane sequencing, host tier): error reporting,
// argument checks and the exception guard of every C entry point. Nothing
// here includes HIP, so the host-only sources also build with a plain C++
// compiler (and its sanitizers).
#pragma once

#include <stdint.h>
#include <stdio.h>

#include <new>
#include <stdexcept>
#include <system_error>

#include "kvm.h"

namespace kvm {

// ---- error reporting (thread-local last error) ---------------------------
void set_error(const char* fmt, ...);
void clear_error();

#define KVM_CHECK_ARG(cond, ...)        \
  do {                                  \
    if (!(cond)) {                      \
      ::kvm::set_error(__VA_ARGS__);    \
      return KVM_EINVAL;                \
    }                                   \
  } while (0)

#define KVM_TRY(expr)             \
  do {                            \
    const int rc_ = (expr);       \
    if (rc_) return rc_;          \
  } while (0)

// Runs the body of a C entry point: no C++ exception leaves the library. Host
// allocation failures (std::bad_alloc) and resource exhaustion reported as
// std::system_error (thread creation) become KVM_ENOMEM; anything else
// KVM_EINTERNAL. The message goes to kvm_last_error().
template <class F>
int guarded(F&& body) noexcept {
  try {
    return body();
  } catch (const std::bad_alloc&) {
    set_error("host memory allocation failed");
    return KVM_ENOMEM;
  } catch (const std::system_error& e) {
    set_error("host resource unavailable: %s", e.what());
    return KVM_ENOMEM;
  } catch (const std::exception& e) {
    set_error("unexpected host exception: %s", e.what());
    return KVM_EINTERNAL;
  } catch (...) {
    set_error("unexpected host exception");
    return KVM_EINTERNAL;
  }
}

inline int dtype_bytes(int32_t dtype) {
  return dtype == KVM_F32 ? 4 : dtype == KVM_FP8_E4M3 ? 1 : 2;
}
// dtype of the Mean-K index rows for K of `dtype` (bf16 for FP8 K)
inline int32_t index_dtype(int32_t dtype) { return dtype == KVM_FP8_E4M3 ? KVM_BF16 : dtype; }

// Validate dims shared by every entry point.
int check_dims(const kvm_dims* d, int32_t dtype);

}  // namespace kvm
