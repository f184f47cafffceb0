// Mean-K index build / append (KVMem Sec. 4.3 Mean-K; Sec. 5 incremental
// indexing of completed blocks while their K is on the GPU).
//
// One wavefront reduces the B = 32 rows of one (block, layer, KV head): each
// lane streams 16-byte pieces of the rows (fully coalesced: the 32 rows of a
// (block, l, g) are one contiguous span), accumulates in float64 (the sum of
// 32 bf16 or typical fp32 values is exact there), and the partial sums are
// folded across the lanes that share a column with xor-shuffles. The mean is
// rounded once to the index dtype, so it is the correctly rounded block mean.
// HBM-bound: per (block, l, g) it reads B*d*e bytes and writes d*e bytes.
#include "common.hpp"
#include "profile.hpp"

namespace kvm {

template <typename T, int D>
struct BuildShape {
  static constexpr int VEC = 16 / sizeof(T);       // elements per 16-byte load
  static constexpr int LPR = D / VEC;              // lanes per row
  static constexpr int RPI = 64 / LPR;             // rows per wave-wide load
  static constexpr int ITERS = 32 / RPI;           // loads per lane (B = 32)
};

template <typename T>
__device__ __forceinline__ void widen(const uint4& v, double* out);

template <>
__device__ __forceinline__ void widen<uint16_t>(const uint4& v, double* out) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = (double)__uint_as_float(w[i] << 16);
    out[2 * i + 1] = (double)__uint_as_float(w[i] & 0xffff0000u);
  }
}

template <>
__device__ __forceinline__ void widen<float>(const uint4& v, double* out) {
  out[0] = (double)__uint_as_float(v.x);
  out[1] = (double)__uint_as_float(v.y);
  out[2] = (double)__uint_as_float(v.z);
  out[3] = (double)__uint_as_float(v.w);
}

template <typename T, int D>
__global__ __launch_bounds__(256) void build_index_kernel(const char* __restrict__ k_raw,
                                                          int64_t block_stride, int64_t n_blocks,
                                                          int32_t nlg, int64_t first_block,
                                                          int64_t cap, T* __restrict__ index) {
  using S = BuildShape<T, D>;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (i, lg) pair
  if (row >= n_blocks * nlg) return;
  const int64_t i = row / nlg;
  const int32_t lg = (int32_t)(row % nlg);
  const char* src = k_raw + i * block_stride + (int64_t)lg * 32 * D * sizeof(T);
  const int col = lane % S::LPR;
  const int r0 = lane / S::LPR;
  double acc[S::VEC];
#pragma unroll
  for (int e = 0; e < S::VEC; ++e) acc[e] = 0.0;
#pragma unroll
  for (int it = 0; it < S::ITERS; ++it) {
    const int r = r0 + it * S::RPI;
    const uint4 v = ld_nt(src + ((int64_t)r * D + col * S::VEC) * sizeof(T));
    double w[S::VEC];
    widen<T>(v, w);
#pragma unroll
    for (int e = 0; e < S::VEC; ++e) acc[e] += w[e];
  }
#pragma unroll
  for (int off = S::LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int e = 0; e < S::VEC; ++e) acc[e] += __shfl_xor(acc[e], off);
  }
  if (r0 == 0) {
    T* dst = index + ((int64_t)lg * cap + first_block + i) * D + col * S::VEC;
    uint4 out;
    if constexpr (sizeof(T) == 2) {
      uint32_t w[4];
#pragma unroll
      for (int p = 0; p < 4; ++p)
        w[p] = (uint32_t)f64_to_bf16(acc[2 * p] * (1.0 / 32.0)) |
               ((uint32_t)f64_to_bf16(acc[2 * p + 1] * (1.0 / 32.0)) << 16);
      out = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      out = make_uint4(__float_as_uint((float)(acc[0] * (1.0 / 32.0))),
                       __float_as_uint((float)(acc[1] * (1.0 / 32.0))),
                       __float_as_uint((float)(acc[2] * (1.0 / 32.0))),
                       __float_as_uint((float)(acc[3] * (1.0 / 32.0))));
    }
    *reinterpret_cast<uint4*>(dst) = out;
  }
}

template <typename T, int D>
static void launch_build(const void* k_raw, int64_t stride, int64_t n, int32_t nlg, int64_t first,
                         int64_t cap, void* index, hipStream_t s) {
  const int64_t rows = n * nlg;
  const int64_t grid = (rows + 3) / 4;
  KernelTimer tm("build_index", s);
  build_index_kernel<T, D><<<dim3((uint32_t)grid), dim3(256), 0, s>>>(
      reinterpret_cast<const char*>(k_raw), stride, n, nlg, first, cap,
      reinterpret_cast<T*>(index));
}

}  // namespace kvm

extern "C" int kvm_build_index(const kvm_dims* dims, int32_t dtype, const void* k_raw,
                               int64_t k_block_stride, int64_t first_block, int64_t n_blocks,
                               void* index, int64_t index_cap_blocks, void* stream) {
  using namespace kvm;
  clear_error();
  int rc = check_dims(dims, dtype);
  if (rc) return rc;
  KVM_CHECK_ARG(n_blocks >= 0 && first_block >= 0, "negative block range");
  if (n_blocks == 0) return KVM_OK;
  KVM_CHECK_ARG(k_raw && index, "null pointer");
  const int64_t blk = (int64_t)dims->n_layers * dims->n_kv_heads * 32 * dims->head_dim *
                      dtype_bytes(dtype);
  KVM_CHECK_ARG(k_block_stride >= blk, "k_block_stride %lld < block bytes %lld",
                (long long)k_block_stride, (long long)blk);
  KVM_CHECK_ARG(k_block_stride % 16 == 0 && ((uintptr_t)k_raw % 16) == 0 &&
                    ((uintptr_t)index % 16) == 0,
                "k_raw, index and stride must be 16-byte aligned");
  KVM_CHECK_ARG(first_block + n_blocks <= index_cap_blocks, "rows beyond index capacity");
  KVM_CHECK_ARG((n_blocks * dims->n_layers * dims->n_kv_heads + 3) / 4 < 0x7fffffffLL,
                "grid too large");
  const int32_t nlg = dims->n_layers * dims->n_kv_heads;
  hipStream_t s = as_stream(stream);
  if (dtype == KVM_BF16) {
    if (dims->head_dim == 128)
      launch_build<uint16_t, 128>(k_raw, k_block_stride, n_blocks, nlg, first_block,
                                  index_cap_blocks, index, s);
    else
      launch_build<uint16_t, 64>(k_raw, k_block_stride, n_blocks, nlg, first_block,
                                 index_cap_blocks, index, s);
  } else {
    if (dims->head_dim == 128)
      launch_build<float, 128>(k_raw, k_block_stride, n_blocks, nlg, first_block,
                               index_cap_blocks, index, s);
    else
      launch_build<float, 64>(k_raw, k_block_stride, n_blocks, nlg, first_block,
                              index_cap_blocks, index, s);
  }
  KVM_HIP(hipGetLastError());
  return KVM_OK;
}
