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
__device__ __forceinline__ void widen<uint8_t>(const uint4& v, double* out) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float x[4];
    fp8x4_to_f32(w[i], x);
#pragma unroll
    for (int e = 0; e < 4; ++e) out[4 * i + e] = (double)x[e];
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

// Index element type for K of element type T: bf16 for FP8 K.
template <typename T>
struct IndexOf {
  using type = T;
};
template <>
struct IndexOf<uint8_t> {
  using type = uint16_t;
};

// Store the P = 16 / sizeof(T) means of a lane's piece as index elements.
template <typename T>
__device__ __forceinline__ void store_means(const double* acc, typename IndexOf<T>::type* dst) {
  constexpr int P = 16 / sizeof(T);
  using TI = typename IndexOf<T>::type;
  constexpr int PER = 16 / sizeof(TI);          // index elements per 16-byte store
#pragma unroll
  for (int c = 0; c < P / PER; ++c)
    *reinterpret_cast<uint4*>(dst + c * PER) = store_mean<TI>(acc + c * PER);
}

// Wavefronts (one (block, l, g) unit each) per workgroup of the plain builds:
// 2048 blocks of the 1M-token workspace took 1.49 ms with 2, 1.50 with 1 and
// 1.53 with 4.
static constexpr int BUILD_WPG = 2;

template <typename T, int D>
__global__ __launch_bounds__(64 * BUILD_WPG) void build_index_kernel(const char* __restrict__ k_raw,
                                                          int64_t block_stride, int64_t n_blocks,
                                                          int32_t nlg, int64_t first_block,
                                                          int64_t cap, T* __restrict__ index) {
  using S = BuildShape<T, D>;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * BUILD_WPG + (threadIdx.x >> 6);  // (i, lg) pair
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

// FP8 E4M3 raw K: every value is a multiple of 2^-9 below 448 in magnitude,
// so any partial sum of a column's 32 values (|sum| < 2^14) is exact in fp32;
// the mean (sum / 32, exact) is rounded once to bf16. One wavefront per
// (block, l, g); lanes decode 16 values per 16-byte load with the hardware
// conversion and fold across the lanes sharing a column with xor-shuffles.
template <int D>
__global__ __launch_bounds__(64 * BUILD_WPG) void build_index_fp8_kernel(const char* __restrict__ k_raw,
                                                              int64_t block_stride,
                                                              int64_t n_blocks, int32_t nlg,
                                                              int64_t first_block, int64_t cap,
                                                              uint16_t* __restrict__ index) {
  constexpr int VEC = 16;                        // fp8 values per 16-byte load
  constexpr int LPR = D / VEC;                   // lanes per row
  constexpr int RPI = 64 / LPR;                  // rows per wave-wide load
  constexpr int ITERS = 32 / RPI;                // loads per lane (B = 32)
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * BUILD_WPG + (threadIdx.x >> 6);  // (i, lg) pair
  if (row >= n_blocks * nlg) return;
  const int64_t i = row / nlg;
  const int32_t lg = (int32_t)(row % nlg);
  const char* src = k_raw + i * block_stride + (int64_t)lg * 32 * D;
  const int col = lane % LPR;
  const int r0 = lane / LPR;
  uint4 v[ITERS];
#pragma unroll
  for (int it = 0; it < ITERS; ++it)
    v[it] = ld_nt(src + (int64_t)(r0 + it * RPI) * D + col * VEC);
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.0f;
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const uint32_t w[4] = {v[it].x, v[it].y, v[it].z, v[it].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float x[4];
      fp8x4_to_f32(w[q], x);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[4 * q + e] += x[e];
    }
  }
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] += __shfl_xor(acc[e], off);
  }
  if (r0 == 0) {
    uint16_t* dst = index + ((int64_t)lg * cap + first_block + i) * D + col * VEC;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      uint32_t w[4];
#pragma unroll
      for (int p = 0; p < 4; ++p)
        w[p] = (uint32_t)f32_to_bf16(acc[8 * c + 2 * p] * (1.0f / 32.0f)) |
               ((uint32_t)f32_to_bf16(acc[8 * c + 2 * p + 1] * (1.0f / 32.0f)) << 16);
      *reinterpret_cast<uint4*>(dst + 8 * c) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

template <int D>
static void launch_build_fp8(const void* k_raw, int64_t stride, int64_t n, int32_t nlg,
                             int64_t first, int64_t cap, void* index, hipStream_t s) {
  const int64_t grid = (n * nlg + BUILD_WPG - 1) / BUILD_WPG;
  KernelTimer tm("build_index", s);
  build_index_fp8_kernel<D><<<dim3((uint32_t)grid), dim3(64 * BUILD_WPG), 0, s>>>(
      reinterpret_cast<const char*>(k_raw), stride, n, nlg, first, cap,
      reinterpret_cast<uint16_t*>(index));
}

template <typename T, int D>
static void launch_build(const void* k_raw, int64_t stride, int64_t n, int32_t nlg, int64_t first,
                         int64_t cap, void* index, hipStream_t s) {
  const int64_t rows = n * nlg;
  const int64_t grid = (rows + BUILD_WPG - 1) / BUILD_WPG;
  KernelTimer tm("build_index", s);
  build_index_kernel<T, D><<<dim3((uint32_t)grid), dim3(64 * BUILD_WPG), 0, s>>>(
      reinterpret_cast<const char*>(k_raw), stride, n, nlg, first, cap,
      reinterpret_cast<T*>(index));
}

// ---------------------------------------------------------------------------
// Mean-K from K that already carries RoPE (KVMem Sec. 5: RoPE is removed from
// the K of completed blocks during prefill, then Mean-K is formed while that K
// is still on the GPU). Token j of block i sits at original position
// pos0 + 32*i + j; every (a, b) pair is turned back by that position's angle
// with the (cos, sin) of the context's fp32 table, in float64, and the block
// mean is rounded once.
// A workgroup covers 4*UPW (l, g) units of one block and first widens the
// block's 32 rows of (cos, sin) into LDS; a wave covers UPW units; within a unit,
// lane c owns the 16-byte pieces at elements c*P and d/2 + c*P of every row
// (so each load instruction reads contiguous runs) and walks all 32 rows
// itself, so the block sum needs no cross-lane reduction; the units of a wave
// share each row's (cos, sin). Half-split pairs (t, t + d/2) span the two
// pieces; interleaved pairs (2t, 2t+1) lie inside each piece.
template <typename T, int D, int LAYOUT>
__global__ __launch_bounds__(256) void build_index_rope_kernel(
    const char* __restrict__ k_rope, int64_t block_stride, int64_t n_blocks, int32_t nlg,
    int32_t wg_per_block, int64_t pos0, const float2* __restrict__ table, int64_t first_block,
    int64_t cap, typename IndexOf<T>::type* __restrict__ index) {
  constexpr int P = 16 / sizeof(T);           // elements per piece
  constexpr int TPU = D / (2 * P);            // lanes per unit
  constexpr int UPW = 64 / TPU;               // units per wave
  constexpr int HALF = D / 2;
  constexpr int PAD = HALF + HALF / P;        // one spare entry every P pairs (banks)
  constexpr int RB = 8;                       // rows whose loads are in flight together
  // (cos, sin) of the block's 32 positions, widened to float64 once per workgroup
  __shared__ double2 tab[32 * PAD];
  const int64_t i = blockIdx.x / wg_per_block;
  if (i >= n_blocks) return;                  // uniform over the workgroup
  const float2* tsrc = table + (pos0 + 32 * i) * HALF;
  for (int e = threadIdx.x; e < 32 * HALF; e += 256) {
    const int r = e / HALF, t = e % HALF;
    const float2 v = tsrc[e];
    tab[r * PAD + t + t / P] = make_double2((double)v.x, (double)v.y);
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int32_t lg = (int32_t)(blockIdx.x % wg_per_block) * 4 * UPW +
                     (threadIdx.x >> 6) * UPW + lane / TPU;
  const bool active = lg < nlg;
  const int tcol = lane % TPU;
  const int t0 = tcol * P;                                     // first element of piece 0
  const int off1 = HALF;                                       // piece 1 offset
  const char* src = k_rope + i * block_stride +
                    ((int64_t)(active ? lg : 0) * 32 * D + t0) * sizeof(T);
  double acc0[P], acc1[P];
#pragma unroll
  for (int e = 0; e < P; ++e) acc0[e] = acc1[e] = 0.0;
#pragma unroll 1
  for (int r0 = 0; r0 < 32; r0 += RB) {
    uint4 v0[RB], v1[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const char* rp = src + (int64_t)(r0 + r) * D * sizeof(T);
      v0[r] = ld_nt(rp);
      v1[r] = ld_nt(rp + off1 * sizeof(T));
    }
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const double2* cs = tab + (r0 + r) * PAD;
      double x0[P], x1[P];
      widen<T>(v0[r], x0);
      widen<T>(v1[r], x1);
#pragma unroll
      for (int q = 0; q < P; ++q) {
        // pair q: interleaved (x0[2q], x0[2q+1]) = pair t0/2 + q for q < P/2,
        // then the same in x1 = pair (t0 + d/2)/2 + q - P/2; half-split
        // (x0[q], x1[q]) = pair t0 + q. R_{-p}: (a c + b s, b c - a s).
        const int t = LAYOUT == 0 ? (q < P / 2 ? t0 / 2 + q : HALF / 2 + t0 / 2 + q - P / 2)
                                  : t0 + q;
        const double2 w = cs[t + t / P];
        const double c = w.x, sn = w.y;
        if (LAYOUT == 0) {
          double* acc = q < P / 2 ? acc0 : acc1;
          const double* x = q < P / 2 ? x0 : x1;
          const int e = 2 * (q % (P / 2));
          acc[e] = fma(x[e + 1], sn, fma(x[e], c, acc[e]));
          acc[e + 1] = fma(-x[e], sn, fma(x[e + 1], c, acc[e + 1]));
        } else {
          acc0[q] = fma(x1[q], sn, fma(x0[q], c, acc0[q]));
          acc1[q] = fma(-x0[q], sn, fma(x1[q], c, acc1[q]));
        }
      }
    }
  }
  if (active) {
    typename IndexOf<T>::type* dst = index + ((int64_t)lg * cap + first_block + i) * D;
    store_means<T>(acc0, dst + t0);
    store_means<T>(acc1, dst + t0 + off1);
  }
}

int launch_build_rope(int32_t dtype, int32_t d, int32_t layout, const void* k_rope,
                      int64_t stride, int64_t n_blocks, int32_t nlg, int64_t pos0,
                      const void* table, int64_t first_block, int64_t cap, void* index,
                      hipStream_t s) {
  // units per wave: 64 / (lanes per unit), lanes per unit = d / (2 * elements per piece);
  // a workgroup (4 waves) covers 4 * upw units of one block
  const int32_t upw = 64 / (d / (2 * (16 / dtype_bytes(dtype))));
  const int32_t wg_per_block = (nlg + 4 * upw - 1) / (4 * upw);
  const int64_t grid = n_blocks * wg_per_block;
  if (grid >= 0x7fffffffLL) {
    set_error("grid too large");
    return KVM_EINVAL;
  }
  const float2* tb = reinterpret_cast<const float2*>(table);
  const char* src = reinterpret_cast<const char*>(k_rope);
  KernelTimer tm("build_index_rope", s);
#define KVM_BR(T, D, LAY)                                                                   \
  build_index_rope_kernel<T, D, LAY><<<dim3((uint32_t)grid), dim3(256), 0, s>>>(            \
      src, stride, n_blocks, nlg, wg_per_block, pos0, tb, first_block, cap,                \
      reinterpret_cast<typename IndexOf<T>::type*>(index))
  if (dtype == KVM_FP8_E4M3) {
    if (d == 128) { if (layout == 0) KVM_BR(uint8_t, 128, 0); else KVM_BR(uint8_t, 128, 1); }
    else { if (layout == 0) KVM_BR(uint8_t, 64, 0); else KVM_BR(uint8_t, 64, 1); }
  } else if (dtype == KVM_BF16) {
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

static int kvm_build_index_body(const kvm_dims* dims, int32_t dtype, const void* k_raw,
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
  KVM_CHECK_ARG((n_blocks * dims->n_layers * dims->n_kv_heads + BUILD_WPG - 1) / BUILD_WPG <
                    0x7fffffffLL,
                "grid too large");
  const int32_t nlg = dims->n_layers * dims->n_kv_heads;
  KVM_CHECK_RANGE(k_raw, (size_t)((n_blocks - 1) * k_block_stride + blk), RANGE_DEVICE, "k_raw");
  KVM_CHECK_RANGE(index,
                  (size_t)nlg * index_cap_blocks * dims->head_dim *
                      dtype_bytes(index_dtype(dtype)),
                  RANGE_DEVICE, "index");
  hipStream_t s = as_stream(stream);
  if (dtype == KVM_FP8_E4M3) {
    if (dims->head_dim == 128)
      launch_build_fp8<128>(k_raw, k_block_stride, n_blocks, nlg, first_block, index_cap_blocks,
                            index, s);
    else
      launch_build_fp8<64>(k_raw, k_block_stride, n_blocks, nlg, first_block, index_cap_blocks,
                           index, s);
  } else if (dtype == KVM_BF16) {
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

extern "C" int kvm_build_index(const kvm_dims* dims, int32_t dtype, const void* k_raw,
                               int64_t k_block_stride, int64_t first_block, int64_t n_blocks,
                               void* index, int64_t index_cap_blocks, void* stream) {
  return kvm::guarded([&] {
    return kvm_build_index_body(dims, dtype, k_raw, k_block_stride, first_block, n_blocks, index,
                                index_cap_blocks, stream);
  });
}
