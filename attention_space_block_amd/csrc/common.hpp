// Shared host/device helpers of libkvm (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "host_common.hpp"

namespace kvm {

#define KVM_HIP(call)                                                              \
  do {                                                                             \
    hipError_t e_ = (call);                                                        \
    if (e_ != hipSuccess) {                                                        \
      ::kvm::set_error("%s failed: %s (%s:%d)", #call, hipGetErrorString(e_),      \
                       __FILE__, __LINE__);                                        \
      return KVM_EHIP;                                                             \
    }                                                                              \
  } while (0)

// Memory-range check of a pointer argument (host calls only, no device work):
// the bytes [p, p + bytes) must lie in one allocation made through HIP that
// the current device can reach (device, managed or pinned host memory), so a
// pageable, freed or short buffer is reported as KVM_EINVAL instead of
// faulting in a kernel or a copy. RANGE_PINNED_HOST additionally requires
// pinned host memory (DMA sources, the host-tiled index). Device memory of
// another GPU is rejected. Allocators that carve tensors out of larger
// segments are checked against the segment; memory the runtime reports but
// cannot give a range for (virtual-memory mappings) skips the extent check.
enum RangeKind { RANGE_DEVICE = 0, RANGE_PINNED_HOST = 1 };
int check_range(const void* p, size_t bytes, RangeKind kind, const char* what);

#define KVM_CHECK_RANGE(p, bytes, kind, what)                         \
  do {                                                                \
    const int rc_ = ::kvm::check_range((p), (bytes), (kind), (what)); \
    if (rc_) return rc_;                                              \
  } while (0)

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Launcher of the de-RoPE Mean-K kernel (build_index.hip); arguments checked
// by the caller. table: device [>= pos0 + 32*n_blocks][d/2] (cos, sin).
int launch_build_rope(int32_t dtype, int32_t d, int32_t layout, const void* k_rope,
                      int64_t stride, int64_t n_blocks, int32_t nlg, int64_t pos0,
                      const void* table, int64_t first_block, int64_t cap, void* index,
                      hipStream_t s);

// ---- device helpers -------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Round-to-nearest-even float -> bf16 bits (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Round-to-nearest-even double -> bf16 bits, directly (no float detour), for
// normal-range finite values: keep 8 significant bits of the double.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  // bf16 keeps sign, 8 exponent bits (rebiased) and 7 mantissa bits. Round the
  // 52-bit double mantissa to 7 bits, ties to even, then rebias.
  uint64_t sign = u >> 63;
  int64_t exp = (int64_t)((u >> 52) & 0x7ff);
  uint64_t man = u & 0xfffffffffffffull;
  if (exp == 0) return (uint16_t)(sign << 15);  // zero (subnormal doubles -> 0)
  uint64_t keep = man >> 45;                     // 7 bits
  uint64_t rest = man & ((1ull << 45) - 1);
  uint64_t half = 1ull << 44;
  if (rest > half || (rest == half && (keep & 1))) keep += 1;
  if (keep == 128) { keep = 0; exp += 1; }
  int64_t e8 = exp - 1023 + 127;
  if (e8 <= 0) return (uint16_t)(sign << 15);    // below bf16 normal range
  if (e8 >= 255) return (uint16_t)((sign << 15) | 0x7f80u);
  return (uint16_t)((sign << 15) | ((uint64_t)e8 << 7) | keep);
}

// FP8 E4M3 (OCP E4M3FN) <-> fp32 with the gfx950 conversion instructions:
// decoding is exact; encoding rounds to nearest, ties to even, after a clamp
// to +-448 (so out-of-range values saturate instead of becoming NaN).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* x) {
  const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  x[0] = lo.x;
  x[1] = lo.y;
  x[2] = hi.x;
  x[3] = hi.y;
}
__device__ __forceinline__ uint32_t f32x4_to_fp8(const float* x) {
  const float a0 = __builtin_amdgcn_fmed3f(x[0], -448.0f, 448.0f);
  const float a1 = __builtin_amdgcn_fmed3f(x[1], -448.0f, 448.0f);
  const float a2 = __builtin_amdgcn_fmed3f(x[2], -448.0f, 448.0f);
  const float a3 = __builtin_amdgcn_fmed3f(x[3], -448.0f, 448.0f);
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, r, true);
  return (uint32_t)r;
}

// exp2 as the single hardware instruction (v_exp_f32). Results below the fp32
// normal range may flush to zero, which is harmless for softmax terms that are
// at least 2^126 times smaller than the row maximum.
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Streaming (non-temporal) 16-byte loads and stores.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_nt(void* p, const uint4& v) {
  u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}

// Plain (cached) 16-byte loads and stores: measured faster than the
// non-temporal forms for read-modify-write streams on gfx950.
__device__ __forceinline__ uint4 ld_plain(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st_plain(void* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }
// XCD-aware remap of a linear workgroup id: hardware dispatches workgroup i to
// XCD (i % 8). Returns a logical id such that each XCD receives one contiguous
// range of logical ids (so neighbouring logical work shares one L2).
// Requires total % 8 == 0.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t bid, uint32_t total) {
  return (bid & 7u) * (total >> 3) + (bid >> 3);
}

}  // namespace kvm
