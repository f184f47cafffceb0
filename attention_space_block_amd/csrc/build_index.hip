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

// One 16-byte piece of P means (sum * 1/32), rounded once into T.
template <typename T>
__device__ __forceinline__ uint4 store_mean(const double* acc);
template <>
__device__ __forceinline__ uint4 store_mean<uint16_t>(const double* acc) {
  uint32_t w[4];
#pragma unroll
  for (int p = 0; p < 4; ++p)
    w[p] = (uint32_t)f64_to_bf16(acc[2 * p] * (1.0 / 32.0)) |
           ((uint32_t)f64_to_bf16(acc[2 * p + 1] * (1.0 / 32.0)) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}
template <>
__device__ __forceinline__ uint4 store_mean<float>(const double* acc) {
  return make_uint4(__float_as_uint((float)(acc[0] * (1.0 / 32.0))),
                    __float_as_uint((float)(acc[1] * (1.0 / 32.0))),
                    __float_as_uint((float)(acc[2] * (1.0 / 32.0))),
                    __float_as_uint((float)(acc[3] * (1.0 / 32.0))));
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

// ---------------------------------------------------------------------------
// Mean-K from K that already carries RoPE (KVMem Sec. 5: RoPE is removed from
// the K of completed blocks during prefill, then Mean-K is formed while that K
// is still on the GPU). Token j of block i sits at original position
// pos0 + 32*i + j; every (a, b) pair is turned back by that position's angle
// with the (cos, sin) of the context's fp32 table, in float64, and the block
// mean is rounded once. A wave takes `upw` (l, g) units of one block: its rows
// keep the same token indices across units, so their (cos, sin) pairs are
// loaded once per wave. Each lane owns two 16-byte pieces of a row (the two
// halves of its rotation pairs: adjacent pieces for interleaved pairs, pieces
// d/2 apart for the half-split layout).
template <typename T, int D, int LAYOUT>
__global__ __launch_bounds__(256) void build_index_rope_kernel(
    const char* __restrict__ k_rope, int64_t block_stride, int64_t n_blocks, int32_t nlg,
    int32_t upw, int64_t pos0, const float2* __restrict__ table, int64_t first_block,
    int64_t cap, T* __restrict__ index) {
  constexpr int P = 16 / sizeof(T);           // elements per piece
  constexpr int TPR = D / (2 * P);            // lanes per row
  constexpr int RPI = 64 / TPR;               // rows per wave-wide pass
  constexpr int ITERS = 32 / RPI;             // rows per lane
  constexpr int HALF = D / 2;
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t waves_per_block = nlg / upw;
  const int64_t i = wave / waves_per_block;
  if (i >= n_blocks) return;
  const int32_t lg0 = (int32_t)(wave % waves_per_block) * upw;
  const int trow = lane / TPR, tcol = lane % TPR;
  const int t0 = LAYOUT == 0 ? tcol * 2 * P : tcol * P;      // first element of piece 0
  const int off1 = LAYOUT == 0 ? P : HALF;                     // piece 1 offset
  const int tp = LAYOUT == 0 ? t0 / 2 : t0;                    // first pair index
  // (cos, sin) of the lane's P pairs for each of its ITERS rows
  float2 cs[ITERS][P];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const float2* row = table + (pos0 + 32 * i + trow + it * RPI) * HALF + tp;
#pragma unroll
    for (int q = 0; q < P; ++q) cs[it][q] = row[q];
  }
  const char* blk = k_rope + i * block_stride;
  for (int32_t u = 0; u < upw; ++u) {
    const int32_t lg = lg0 + u;
    const char* src = blk + (int64_t)lg * 32 * D * sizeof(T);
    uint4 v0[ITERS], v1[ITERS];
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const char* r = src + ((int64_t)(trow + it * RPI) * D + t0) * sizeof(T);
      v0[it] = ld_nt(r);
      v1[it] = ld_nt(r + off1 * sizeof(T));
    }
    double acc0[P], acc1[P];
#pragma unroll
    for (int e = 0; e < P; ++e) acc0[e] = acc1[e] = 0.0;
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      double x0[P], x1[P];
      widen<T>(v0[it], x0);
      widen<T>(v1[it], x1);
#pragma unroll
      for (int q = 0; q < P; ++q) {
        // pair q of the lane: interleaved (x0[2q], x0[2q+1]) for q < P/2, then
        // (x1[2(q-P/2)], ...); half-split (x0[q], x1[q])
        double a, b;
        if (LAYOUT == 0) {
          a = q < P / 2 ? x0[2 * q] : x1[2 * (q - P / 2)];
          b = q < P / 2 ? x0[2 * q + 1] : x1[2 * (q - P / 2) + 1];
        } else {
          a = x0[q];
          b = x1[q];
        }
        const double c = (double)cs[it][q].x, sn = (double)cs[it][q].y;
        const double ra = a * c + b * sn;      // R_{-p}
        const double rb = b * c - a * sn;
        if (LAYOUT == 0) {
          if (q < P / 2) {
            acc0[2 * q] += ra;
            acc0[2 * q + 1] += rb;
          } else {
            acc1[2 * (q - P / 2)] += ra;
            acc1[2 * (q - P / 2) + 1] += rb;
          }
        } else {
          acc0[q] += ra;
          acc1[q] += rb;
        }
      }
    }
#pragma unroll
    for (int off = TPR; off < 64; off <<= 1) {
#pragma unroll
      for (int e = 0; e < P; ++e) {
        acc0[e] += __shfl_xor(acc0[e], off);
        acc1[e] += __shfl_xor(acc1[e], off);
      }
    }
    if (trow == 0) {
      T* dst = index + ((int64_t)lg * cap + first_block + i) * D;
      *reinterpret_cast<uint4*>(dst + t0) = store_mean<T>(acc0);
      *reinterpret_cast<uint4*>(dst + t0 + off1) = store_mean<T>(acc1);
    }
  }
}

int launch_build_rope(int32_t dtype, int32_t d, int32_t layout, const void* k_rope,
                      int64_t stride, int64_t n_blocks, int32_t nlg, int64_t pos0,
                      const void* table, int64_t first_block, int64_t cap, void* index,
                      hipStream_t s) {
  int32_t upw = 1;
  while (upw < 8 && nlg % (upw * 2) == 0) upw *= 2;
  const int64_t waves = n_blocks * (nlg / upw);
  const int64_t grid = (waves + 3) / 4;
  if (grid >= 0x7fffffffLL) {
    set_error("grid too large");
    return KVM_EINVAL;
  }
  const float2* tb = reinterpret_cast<const float2*>(table);
  const char* src = reinterpret_cast<const char*>(k_rope);
  KernelTimer tm("build_index_rope", s);
#define KVM_BR(T, D, LAY)                                                                   \
  build_index_rope_kernel<T, D, LAY><<<dim3((uint32_t)grid), dim3(256), 0, s>>>(            \
      src, stride, n_blocks, nlg, upw, pos0, tb, first_block, cap, reinterpret_cast<T*>(index))
  if (dtype == KVM_BF16) {
    if (d == 128) { if (layout == 0) KVM_BR(uint16_t, 128, 0); else KVM_BR(uint16_t, 128, 1); }
    else { if (layout == 0) KVM_BR(uint16_t, 64, 0); else KVM_BR(uint16_t, 64, 1); }
  } else {
    if (d == 128) { if (layout == 0) KVM_BR(float, 128, 0); else KVM_BR(float, 128, 1); }
    else { if (layout == 0) KVM_BR(float, 64, 0); else KVM_BR(float, 64, 1); }
  }
#undef KVM_BR
  KVM_HIP(hipGetLastError());
  return KVM_OK;
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
