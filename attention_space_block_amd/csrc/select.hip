// Default selector (KVMem Sec. 4.3): keep the sink blocks [0, n_sink) and the
// recent blocks [N - n_recent, N), fill the remaining budget with the blocks of
// largest relevance R_b (exact ties to the lower block id) and return the
// selection in chronological (ascending) order with compact base positions
// i * B (Sec. 4.4, Sec. 5).
//
// One 1024-thread workgroup does the whole selection: N is at most a few
// hundred thousand blocks (a 10M-token workspace has 312,500), i.e. about a
// megabyte of scores that stays in L2, so a single CU finishes in tens of
// microseconds while scoring takes milliseconds.
//  1. Validate (every score finite and >= 0; -0.0 counts as 0).
//  2. Radix select on the fp32 bit pattern (non-negative floats order like
//     their bits): four 8-bit digit passes with LDS histograms find the exact
//     key T of the k-th largest candidate and how many candidates equal to T
//     must be taken.
//  3. Ordered compaction: each thread owns a contiguous index range; two
//     wavefront-shuffle scans (ties, then selected counts) give every thread
//     its tie rank and its output offset, so ties go to the lowest ids and the
//     output is ascending without a sort.
#include "common.hpp"
#include "profile.hpp"

namespace kvm {

__device__ __forceinline__ uint32_t score_key(float f) {
  return f == 0.0f ? 0u : __float_as_uint(f);
}

// Exclusive scan of one uint32 per thread over the 1024-thread workgroup.
// Returns the exclusive prefix; *total receives the sum over all threads.
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wave_tot, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wave_tot[wave] = x;
  __syncthreads();
  if (wave == 0) {
    uint32_t t = lane < 16 ? wave_tot[lane] : 0u;
    uint32_t s = t;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      uint32_t y = __shfl_up(s, off);
      if (lane >= off) s += y;
    }
    if (lane < 16) wave_tot[16 + lane] = s - t;  // exclusive wave offsets
    if (lane == 15) wave_tot[32] = s;
  }
  __syncthreads();
  const uint32_t res = wave_tot[16 + wave] + x - v;
  *total = wave_tot[32];
  __syncthreads();
  return res;
}

__global__ __launch_bounds__(1024) void select_kernel(const float* __restrict__ scores,
                                                      int64_t N, int32_t n_sink, int32_t n_recent,
                                                      int32_t budget, int32_t B,
                                                      int32_t* __restrict__ sel,
                                                      int32_t* __restrict__ n_sel,
                                                      int32_t* __restrict__ base_pos) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wave_tot[40];
  __shared__ uint32_t s_prefix, s_krem;
  const int tid = threadIdx.x;

  int bad = 0;
  for (int64_t i = tid; i < N; i += 1024) {
    const float f = scores[i];
    if (!(f >= 0.0f) || f == __builtin_inff()) bad = 1;
  }
  if (__syncthreads_or(bad)) {
    if (tid == 0) *n_sel = KVM_ERANGE;
    return;
  }
  if (N <= budget) {
    for (int64_t i = tid; i < N; i += 1024) {
      sel[i] = (int32_t)i;
      base_pos[i] = (int32_t)i * B;
    }
    if (tid == 0) *n_sel = (int32_t)N;
    return;
  }

  const int64_t c0 = n_sink, c1 = N - n_recent;
  const uint32_t k = (uint32_t)(budget - n_sink - n_recent);
  if (tid == 0) {
    s_prefix = 0u;
    s_krem = k;
  }
  __syncthreads();
  if (k > 0) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += 1024) hist[i] = 0u;
      __syncthreads();
      const uint32_t prefix = s_prefix;
      for (int64_t c = c0 + tid; c < c1; c += 1024) {
        const uint32_t key = score_key(scores[c]);
        const bool match = shift == 24 || ((key >> (shift + 8)) == (prefix >> (shift + 8)));
        if (match) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        uint32_t cum = 0, krem = s_krem;
        for (int dg = 255; dg >= 0; --dg) {
          if (cum + hist[dg] >= krem) {
            s_prefix = prefix | ((uint32_t)dg << shift);
            s_krem = krem - cum;
            break;
          }
          cum += hist[dg];
        }
      }
      __syncthreads();
    }
  }
  // T: key of the k-th largest candidate; take the first `krem` candidates
  // (lowest ids) whose key equals T. With k == 0 nothing is taken.
  const uint32_t T = k > 0 ? s_prefix : 0xffffffffu;
  const uint32_t krem = k > 0 ? s_krem : 0u;

  const int64_t per = (N + 1023) / 1024;
  const int64_t lo = (int64_t)tid * per;
  const int64_t hi = lo + per < N ? lo + per : N;
  uint32_t n_above = 0, n_tie = 0;
  for (int64_t i = lo; i < hi; ++i) {
    if (i < c0 || i >= c1) {
      ++n_above;
    } else {
      const uint32_t key = score_key(scores[i]);
      if (k > 0 && key > T) ++n_above;
      else if (k > 0 && key == T) ++n_tie;
    }
  }
  uint32_t tie_total;
  const uint32_t tie_base = block_exclusive_scan(n_tie, wave_tot, &tie_total);
  uint32_t take_ties = 0;
  if (krem > tie_base) take_ties = (krem - tie_base) < n_tie ? (krem - tie_base) : n_tie;
  uint32_t out_total;
  const uint32_t out_base = block_exclusive_scan(n_above + take_ties, wave_tot, &out_total);
  uint32_t o = out_base, t_seen = 0;
  for (int64_t i = lo; i < hi; ++i) {
    bool take;
    if (i < c0 || i >= c1) {
      take = true;
    } else {
      const uint32_t key = score_key(scores[i]);
      if (k > 0 && key > T) take = true;
      else if (k > 0 && key == T) take = (t_seen++ < take_ties);
      else take = false;
    }
    if (take) {
      sel[o] = (int32_t)i;
      base_pos[o] = (int32_t)o * B;
      ++o;
    }
  }
  if (tid == 0) *n_sel = (int32_t)out_total;
}

}  // namespace kvm

extern "C" size_t kvm_select_ws_bytes(int64_t n_blocks) {
  (void)n_blocks;
  return 0;
}

extern "C" int kvm_select(const float* scores, int64_t n_blocks, int32_t n_sink, int32_t n_recent,
                          int32_t budget_blocks, int32_t block_tokens, int32_t* sel,
                          int32_t* n_sel, int32_t* base_pos, void* ws, size_t ws_bytes,
                          void* stream) {
  using namespace kvm;
  (void)ws;
  (void)ws_bytes;
  clear_error();
  KVM_CHECK_ARG(scores && sel && n_sel && base_pos, "null pointer");
  KVM_CHECK_ARG(n_blocks >= 1 && n_blocks < 0x7fffffffLL, "n_blocks out of range");
  KVM_CHECK_ARG(n_sink >= 0 && n_recent >= 0 && budget_blocks >= 1 && block_tokens >= 1,
                "negative sizes");
  if ((int64_t)n_sink + n_recent > budget_blocks) {
    set_error("budget %d < sink %d + recent %d", budget_blocks, n_sink, n_recent);
    return KVM_ERANGE;
  }
  KVM_CHECK_ARG((int64_t)budget_blocks * block_tokens < 0x7fffffffLL, "positions overflow int32");
  KernelTimer tm("select", as_stream(stream));
  select_kernel<<<1, 1024, 0, as_stream(stream)>>>(scores, n_blocks, n_sink, n_recent,
                                                   budget_blocks, block_tokens, sel, n_sel,
                                                   base_pos);
  KVM_HIP(hipGetLastError());
  return KVM_OK;
}
