// Conversion of bf16 or fp32 values to FP8 E4M3 (OCP E4M3FN) bytes: nearest,
// ties to even, saturating at +-448 (the largest finite value), the sign kept
// on zero. It forms the FP8 index and queries of the FP8 scoring ablation (the
// pages' engine runs an FP8 KV cache, KVMem Sec. 6.1).
#include "common.hpp"

namespace kvm {

template <typename T>
__device__ __forceinline__ float elem_f32(const T* p, int64_t i);
template <>
__device__ __forceinline__ float elem_f32<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}
template <>
__device__ __forceinline__ float elem_f32<float>(const float* p, int64_t i) {
  return p[i];
}

// Each thread converts 4 consecutive elements with one packed conversion.
template <typename T>
__global__ __launch_bounds__(256) void quantize_e4m3_kernel(const T* __restrict__ src, int64_t n,
                                                            uint8_t* __restrict__ dst) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  float x[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) x[j] = i + j < n ? elem_f32<T>(src, i + j) : 0.0f;
  const uint32_t w = f32x4_to_fp8(x);
  if (i + 4 <= n) {
    *reinterpret_cast<uint32_t*>(dst + i) = w;
  } else {
    for (int j = 0; i + j < n; ++j) dst[i + j] = (uint8_t)(w >> (8 * j));
  }
}

}  // namespace kvm

static int kvm_quantize_e4m3_body(const void* src, int32_t src_dtype, int64_t n, void* dst,
                                 void* stream) {
  using namespace kvm;
  clear_error();
  KVM_CHECK_ARG(src && dst, "null pointer");
  KVM_CHECK_ARG(src_dtype == KVM_F32 || src_dtype == KVM_BF16, "src_dtype must be F32 or BF16");
  KVM_CHECK_ARG(n >= 1 && n < (1LL << 40), "n out of range");
  KVM_CHECK_ARG((uintptr_t)dst % 4 == 0, "dst must be 4-byte aligned");
  KVM_CHECK_ARG((uintptr_t)src % (src_dtype == KVM_F32 ? 4 : 2) == 0, "src misaligned");
  KVM_CHECK_RANGE(src, (size_t)n * (src_dtype == KVM_F32 ? 4 : 2), RANGE_DEVICE, "src");
  KVM_CHECK_RANGE(dst, (size_t)n, RANGE_DEVICE, "dst");
  const int64_t groups = (n + 3) / 4;
  const dim3 grid((uint32_t)((groups + 255) / 256));
  hipStream_t s = as_stream(stream);
  if (src_dtype == KVM_F32)
    quantize_e4m3_kernel<float><<<grid, dim3(256), 0, s>>>(reinterpret_cast<const float*>(src), n,
                                                           reinterpret_cast<uint8_t*>(dst));
  else
    quantize_e4m3_kernel<uint16_t><<<grid, dim3(256), 0, s>>>(
        reinterpret_cast<const uint16_t*>(src), n, reinterpret_cast<uint8_t*>(dst));
  KVM_HIP(hipGetLastError());
  return KVM_OK;
}

extern "C" int kvm_quantize_e4m3(const void* src, int32_t src_dtype, int64_t n, void* dst,
                                 void* stream) {
  return kvm::guarded([&] {
    return kvm_quantize_e4m3_body(src, src_dtype, n, dst, stream);
  });
}
