// Default selector (KVMem Sec. 4.3): keep the sink blocks [0, n_sink) and the
// recent blocks [N - n_recent, N), fill the remaining budget with the blocks of
// largest relevance R_b (exact ties to the lower block id) and return the
// selection in chronological (ascending) order with compact base positions
// i * B (Sec. 4.4, Sec. 5).
//
// Non-negative floats order like their bit patterns (-0.0 counts as 0), so
// the k-th largest candidate is found by an exact radix select on the fp32
// bits, 8 bits per round, spread over many workgroups (a 10M-token workspace
// has 312,500 blocks; one workgroup spends most of its time in LDS atomics on
// the few histogram bins that hold almost every key):
//  1. sel_init resets the control words and the four round histograms.
//  2. Four rounds of sel_hist: each workgroup first fixes the digits of the
//     earlier rounds from their 256-bin histograms (a workgroup scan per
//     round: the digit holding the krem-th largest key), then builds the
//     LDS histogram of the current digit over its chunk of candidates that
//     match them (per-thread run-length counting and one wave-aggregated add
//     for the most common pending digit) and adds it to the round's global
//     histogram. After four rounds T is the key of the k-th largest candidate
//     and krem the number of candidates equal to T that are taken (the
//     lowest ids).
//  3. sel_count fixes the last digit the same way, validates every score
//     (finite, >= 0) and counts per chunk the kept blocks (sink, recent,
//     keys > T) and the ties (keys == T).
//  4. sel_write: each chunk's output offset is (kept before it) + min(ties
//     before it, krem); inside the chunk every thread owns 16 consecutive
//     blocks and two workgroup scans give its tie rank and its offset, so the
//     output is ascending without a sort.
// With n_blocks <= budget every block is selected (select_all_kernel).
#include <algorithm>
#include <mutex>

#include "common.hpp"
#include "profile.hpp"

namespace kvm {

namespace {

constexpr int SEL_THREADS = 256;
constexpr int SEL_PER = 16;                          // blocks per thread
constexpr int SEL_CHUNK = SEL_THREADS * SEL_PER;     // blocks per workgroup
constexpr int CTL_WORDS = 64;                        // control area (words)
enum { CTL_BAD = 0, CTL_PREFIX = 1, CTL_KREM = 2 };
constexpr int HIST_WORDS = 4 * 256;                  // one 256-bin histogram per round

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

struct SelWs {
  uint32_t* ctl;    // [CTL_WORDS]
  uint32_t* hist;   // [4][256]: digit histogram of each round
  uint32_t* cnt;    // [nwg][2]: kept, ties
};

int64_t sel_nwg(int64_t n) { return (n + SEL_CHUNK - 1) / SEL_CHUNK; }

size_t sel_ws_bytes(int64_t n) {
  const int64_t nwg = sel_nwg(n);
  return align256(CTL_WORDS * 4) + align256(HIST_WORDS * 4) + align256((size_t)nwg * 8);
}

SelWs sel_ws(void* ws) {
  char* p = reinterpret_cast<char*>(ws);
  SelWs w;
  w.ctl = reinterpret_cast<uint32_t*>(p);
  w.hist = reinterpret_cast<uint32_t*>(p + align256(CTL_WORDS * 4));
  w.cnt = reinterpret_cast<uint32_t*>(p + align256(CTL_WORDS * 4) + align256(HIST_WORDS * 4));
  return w;
}

}  // namespace

__device__ __forceinline__ uint32_t score_key(float f) {
  return f == 0.0f ? 0u : __float_as_uint(f);
}

__device__ __forceinline__ bool score_bad(float f) {
  return !(f >= 0.0f) || f == __builtin_inff();
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Exclusive scan of one uint32 per thread over a workgroup of NT threads
// (NT / 64 <= 16 waves). Returns the exclusive prefix; *total receives the sum.
template <int NT>
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wave_tot, uint32_t* total) {
  constexpr int NW = NT / 64;
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
    uint32_t t = lane < NW ? wave_tot[lane] : 0u;
    uint32_t s = t;
#pragma unroll
    for (int off = 1; off < NW; off <<= 1) {
      uint32_t y = __shfl_up(s, off);
      if (lane >= off) s += y;
    }
    if (lane < NW) wave_tot[16 + lane] = s - t;  // exclusive wave offsets
    if (lane == NW - 1) wave_tot[32] = s;
  }
  __syncthreads();
  const uint32_t res = wave_tot[16 + wave] + x - v;
  *total = wave_tot[32];
  __syncthreads();
  return res;
}

__global__ __launch_bounds__(256) void sel_init(uint32_t* ctl, uint32_t* hist) {
  for (int i = threadIdx.x; i < HIST_WORDS; i += 256) hist[i] = 0u;
  if (threadIdx.x == 0) ctl[CTL_BAD] = 0u;
}

// The digits of rounds [0, rounds) from their histograms: in round r the digit
// dg at shift 24 - 8r is the largest whose keys, with all larger digits, reach
// krem; krem becomes the rank of the target inside digit dg. Every thread of a
// 256-thread workgroup gets the result (one bin per thread, descending scan).
__device__ void fix_digits(const uint32_t* __restrict__ hist, int rounds, uint32_t k,
                           uint32_t* wave_tot, uint32_t* s_fix, uint32_t& prefix,
                           uint32_t& krem) {
  const int t = threadIdx.x;
  prefix = 0u;
  krem = k;
  for (int r = 0; r < rounds; ++r) {
    const int shift = 24 - 8 * r;
    const uint32_t v = hist[r * 256 + (255 - t)];   // thread t holds digit 255 - t
    uint32_t total;
    const uint32_t ex = block_exclusive_scan<256>(v, wave_tot, &total);   // keys above it
    if (t == 0) {
      s_fix[0] = 0u;
      s_fix[1] = 0u;
    }
    __syncthreads();
    if (ex < krem && krem <= ex + v) {              // exactly one thread for consistent counts
      s_fix[0] = (uint32_t)(255 - t);
      s_fix[1] = ex;
    }
    __syncthreads();
    prefix |= s_fix[0] << shift;
    krem -= s_fix[1];
    __syncthreads();
  }
}

// Round `round`: histogram of digit (key >> shift) & 255, shift = 24 - 8*round,
// over this chunk's candidates whose higher digits equal the ones fixed by the
// earlier rounds, added to hist[round].
__global__ __launch_bounds__(SEL_THREADS) void sel_hist(const float* __restrict__ scores,
                                                        int64_t c0, int64_t c1, int round,
                                                        uint32_t k, uint32_t* __restrict__ hist) {
  __shared__ uint32_t h[256];
  __shared__ uint32_t wave_tot[40], s_fix[2];
  const int t = threadIdx.x, lane = t & 63;
  const int shift = 24 - 8 * round;
  uint32_t prefix, krem;
  fix_digits(hist, round, k, wave_tot, s_fix, prefix, krem);
  h[t] = 0u;
  const uint32_t hi = shift < 24 ? prefix >> (shift + 8) : 0u;
  const int64_t base = (int64_t)blockIdx.x * SEL_CHUNK;
  uint32_t key[SEL_PER];
  bool in[SEL_PER];
#pragma unroll
  for (int j = 0; j < SEL_PER; ++j) {   // all loads first (coalesced across lanes)
    const int64_t i = base + j * SEL_THREADS + t;
    in[j] = i >= c0 && i < c1;
    key[j] = in[j] ? score_key(scores[i]) : 0u;
  }
  __syncthreads();
  uint32_t cur = 0u, cnt = 0u;
#pragma unroll
  for (int j = 0; j < SEL_PER; ++j) {
    const bool match = in[j] && (shift == 24 || (key[j] >> (shift + 8)) == hi);
    if (!match) continue;
    const uint32_t d = (key[j] >> shift) & 255u;
    if (cnt > 0 && d != cur) atomicAdd(&h[cur], cnt), cnt = 0u;
    cur = d;
    ++cnt;
  }
  // The wave's most common pending digit is usually the first lane's: add it
  // once for all lanes that hold it, the rest directly.
  bool act = cnt > 0;
  const uint64_t m = __ballot(act);
  if (m != 0) {
    const int leader = __ffsll((unsigned long long)m) - 1;
    const uint32_t ld = __shfl(cur, leader);
    const bool same = act && cur == ld;
    const uint32_t tot = wave_sum(same ? cnt : 0u);
    if (lane == leader) atomicAdd(&h[ld], tot);
    if (same) act = false;
  }
  if (act) atomicAdd(&h[cur], cnt);
  __syncthreads();
  if (h[t] != 0u) atomicAdd(&hist[round * 256 + t], h[t]);
}

// Per chunk: validation of every score, kept blocks and ties.
__global__ __launch_bounds__(SEL_THREADS) void sel_count(const float* __restrict__ scores,
                                                         int64_t N, int64_t c0, int64_t c1,
                                                         uint32_t k,
                                                         const uint32_t* __restrict__ hist,
                                                         uint32_t* __restrict__ ctl,
                                                         uint32_t* __restrict__ cnt) {
  __shared__ uint32_t red[2][SEL_THREADS / 64];
  __shared__ uint32_t wave_tot[40], s_fix[2];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const bool has_k = k > 0;
  uint32_t T = 0xffffffffu, krem = 0u;
  if (has_k) fix_digits(hist, 4, k, wave_tot, s_fix, T, krem);   // uniform branch
  if (blockIdx.x == 0 && t == 0) {             // for sel_write
    ctl[CTL_PREFIX] = T;
    ctl[CTL_KREM] = krem;
  }
  const int64_t base = (int64_t)blockIdx.x * SEL_CHUNK;
  uint32_t kept = 0u, tie = 0u;
  bool bad = false;
#pragma unroll
  for (int j = 0; j < SEL_PER; ++j) {
    const int64_t i = base + j * SEL_THREADS + t;
    if (i >= N) continue;
    const float f = scores[i];
    bad |= score_bad(f);
    if (i < c0 || i >= c1) {
      ++kept;
    } else if (has_k) {
      const uint32_t key = score_key(f);
      kept += key > T;
      tie += key == T;
    }
  }
  if (__ballot(bad) != 0 && lane == 0) atomicOr(&ctl[CTL_BAD], 1u);
  kept = wave_sum(kept);
  tie = wave_sum(tie);
  if (lane == 0) {
    red[0][wave] = kept;
    red[1][wave] = tie;
  }
  __syncthreads();
  if (t == 0) {
    uint32_t a = 0u, b = 0u;
#pragma unroll
    for (int w = 0; w < SEL_THREADS / 64; ++w) {
      a += red[0][w];
      b += red[1][w];
    }
    cnt[2 * blockIdx.x] = a;
    cnt[2 * blockIdx.x + 1] = b;
  }
}

__global__ __launch_bounds__(SEL_THREADS) void sel_write(
    const float* __restrict__ scores, int64_t N, int64_t c0, int64_t c1, int has_k,
    const uint32_t* __restrict__ ctl, const uint32_t* __restrict__ cnt, int32_t B,
    int32_t budget, int32_t* __restrict__ sel, int32_t* __restrict__ n_sel, int32_t* __restrict__ base_pos) {
  __shared__ uint32_t wave_tot[40];
  __shared__ uint32_t s_before[2];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  if (ctl[CTL_BAD] != 0u) {
    if (blockIdx.x == 0 && t == 0) *n_sel = KVM_ERANGE;
    return;
  }
  const uint32_t T = has_k ? ctl[CTL_PREFIX] : 0xffffffffu;
  const uint32_t krem = has_k ? ctl[CTL_KREM] : 0u;
  if (wave == 0) {   // kept blocks and ties in the chunks before this one
    uint32_t a = 0u, b = 0u;
    for (int64_t w = lane; w < blockIdx.x; w += 64) {
      a += cnt[2 * w];
      b += cnt[2 * w + 1];
    }
    a = wave_sum(a);
    b = wave_sum(b);
    if (lane == 0) {
      s_before[0] = a;
      s_before[1] = b;
    }
  }
  __syncthreads();
  const uint32_t kept_before = s_before[0], tie_before = s_before[1];
  const uint32_t wg_ties = cnt[2 * blockIdx.x + 1];
  const uint32_t wg_take = krem > tie_before ? (krem - tie_before < wg_ties ? krem - tie_before
                                                                             : wg_ties)
                                             : 0u;
  const uint32_t out0 = kept_before + (tie_before < krem ? tie_before : krem);

  const int64_t lo = (int64_t)blockIdx.x * SEL_CHUNK + (int64_t)t * SEL_PER;
  uint32_t key[SEL_PER];
#pragma unroll
  for (int j = 0; j < SEL_PER; ++j) key[j] = lo + j < N ? score_key(scores[lo + j]) : 0u;
  auto kind = [&](int j) -> int {   // 0 none, 1 kept, 2 tie
    const int64_t i = lo + j;
    if (i >= N) return 0;
    if (i < c0 || i >= c1) return 1;
    if (!has_k) return 0;
    return key[j] > T ? 1 : (key[j] == T ? 2 : 0);
  };
  uint32_t n_kept = 0u, n_tie = 0u;
#pragma unroll
  for (int j = 0; j < SEL_PER; ++j) {
    const int k = kind(j);
    n_kept += k == 1;
    n_tie += k == 2;
  }
  uint32_t tie_total;
  const uint32_t tie_base = block_exclusive_scan<SEL_THREADS>(n_tie, wave_tot, &tie_total);
  uint32_t take = 0u;
  if (wg_take > tie_base) take = wg_take - tie_base < n_tie ? wg_take - tie_base : n_tie;
  uint32_t out_total;
  const uint32_t out_base = block_exclusive_scan<SEL_THREADS>(n_kept + take, wave_tot, &out_total);
  uint32_t o = out0 + out_base, seen = 0u;
#pragma unroll
  for (int j = 0; j < SEL_PER; ++j) {
    const int k = kind(j);
    const bool w = k == 1 || (k == 2 && seen++ < take);
    if (w && o < (uint32_t)budget) {   // always true for consistent counts
      sel[o] = (int32_t)(lo + j);
      base_pos[o] = (int32_t)o * B;
      ++o;
    }
  }
  if (blockIdx.x == gridDim.x - 1 && t == 0) *n_sel = (int32_t)(out0 + out_total);
}

// n_blocks <= budget: every block, after validation.
__global__ __launch_bounds__(1024) void select_all_kernel(const float* __restrict__ scores,
                                                          int64_t N, int32_t B,
                                                          int32_t* __restrict__ sel,
                                                          int32_t* __restrict__ n_sel,
                                                          int32_t* __restrict__ base_pos) {
  const int tid = threadIdx.x;
  int bad = 0;
  for (int64_t i = tid; i < N; i += 1024) bad |= score_bad(scores[i]);
  if (__syncthreads_or(bad)) {
    if (tid == 0) *n_sel = KVM_ERANGE;
    return;
  }
  for (int64_t i = tid; i < N; i += 1024) {
    sel[i] = (int32_t)i;
    base_pos[i] = (int32_t)i * B;
  }
  if (tid == 0) *n_sel = (int32_t)N;
}

}  // namespace kvm

extern "C" size_t kvm_select_ws_bytes(int64_t n_blocks) {
  return kvm::sel_ws_bytes(n_blocks > 0 ? n_blocks : 1);
}


namespace kvm {
namespace {

// Argument checks shared by both entry points (no device work).
int select_check(const float* scores, int64_t n_blocks, int32_t n_sink, int32_t n_recent,
                 int32_t budget_blocks, int32_t block_tokens, int32_t* sel, int32_t* n_sel,
                 int32_t* base_pos) {
  KVM_CHECK_ARG(scores && sel && n_sel && base_pos, "null pointer");
  KVM_CHECK_ARG(n_blocks >= 1 && n_blocks < 0x7fffffffLL, "n_blocks out of range");
  KVM_CHECK_ARG(n_sink >= 0 && n_recent >= 0 && budget_blocks >= 1 && block_tokens >= 1,
                "negative sizes");
  if ((int64_t)n_sink + n_recent > budget_blocks) {
    set_error("budget %d < sink %d + recent %d", budget_blocks, n_sink, n_recent);
    return KVM_ERANGE;
  }
  KVM_CHECK_ARG((int64_t)budget_blocks * block_tokens < 0x7fffffffLL, "positions overflow int32");
  const size_t out_bytes = (size_t)std::min<int64_t>(budget_blocks, n_blocks) * sizeof(int32_t);
  KVM_CHECK_RANGE(scores, (size_t)n_blocks * sizeof(float), RANGE_DEVICE, "scores");
  KVM_CHECK_RANGE(sel, out_bytes, RANGE_DEVICE, "sel");
  KVM_CHECK_RANGE(base_pos, out_bytes, RANGE_DEVICE, "base_pos");
  KVM_CHECK_RANGE(n_sel, sizeof(int32_t), RANGE_DEVICE, "n_sel");
  return KVM_OK;
}

// The launches of one selection; `ws` holds at least sel_ws_bytes(n_blocks)
// bytes of device memory (unused when n_blocks <= budget_blocks). sel_init
// clears the control words and histograms, so `ws` needs no clearing.
int select_launch(const float* scores, int64_t n_blocks, int32_t n_sink, int32_t n_recent,
                  int32_t budget_blocks, int32_t block_tokens, int32_t* sel, int32_t* n_sel,
                  int32_t* base_pos, void* ws, hipStream_t s, bool timed) {
  if (n_blocks <= budget_blocks) {
    KernelTimer tm(timed ? "select" : nullptr, s);
    select_all_kernel<<<1, 1024, 0, s>>>(scores, n_blocks, block_tokens, sel, n_sel, base_pos);
    KVM_HIP(hipGetLastError());
    return KVM_OK;
  }
  KernelTimer tm(timed ? "select" : nullptr, s);
  const SelWs w = sel_ws(ws);
  const int64_t nwg = sel_nwg(n_blocks);
  const int64_t c0 = n_sink, c1 = n_blocks - n_recent;
  const uint32_t k = (uint32_t)(budget_blocks - n_sink - n_recent);
  sel_init<<<1, 256, 0, s>>>(w.ctl, w.hist);
  if (k > 0) {
    for (int round = 0; round < 4; ++round)
      sel_hist<<<dim3((uint32_t)nwg), dim3(SEL_THREADS), 0, s>>>(scores, c0, c1, round, k,
                                                                 w.hist);
  }
  sel_count<<<dim3((uint32_t)nwg), dim3(SEL_THREADS), 0, s>>>(scores, n_blocks, c0, c1, k,
                                                              w.hist, w.ctl, w.cnt);
  sel_write<<<dim3((uint32_t)nwg), dim3(SEL_THREADS), 0, s>>>(scores, n_blocks, c0, c1, k > 0,
                                                              w.ctl, w.cnt, block_tokens,
                                                              budget_blocks, sel, n_sel, base_pos);
  KVM_HIP(hipGetLastError());
  return KVM_OK;
}

// Workspace of kvm_select_noalloc: one array per GPU, held until the process
// ends. Host code must use the address hipGetSymbolAddress returns for the
// current device (select_scratch), never the array's name.
static __device__ __align__(256) unsigned char scratch[KVM_SELECT_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch[MAX_DEVICES] = {};

// Device address of `scratch` on the current GPU (looked up once per GPU).
int select_scratch(void** out) {
  int dev = -1;
  KVM_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= MAX_DEVICES) {
    set_error("device %d outside the scratch table (%d devices)", dev, MAX_DEVICES);
    return KVM_ENOTSUP;
  }
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    KVM_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) {
      set_error("hipGetSymbolAddress returned no address for the select scratch");
      return KVM_EHIP;
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return KVM_OK;
}

}  // namespace
}  // namespace kvm

extern "C" int kvm_select(const float* scores, int64_t n_blocks, int32_t n_sink, int32_t n_recent,
                          int32_t budget_blocks, int32_t block_tokens, int32_t* sel,
                          int32_t* n_sel, int32_t* base_pos, void* ws, size_t ws_bytes,
                          void* stream) {
  using namespace kvm;
  return guarded([&]() -> int {
    clear_error();
    int rc = select_check(scores, n_blocks, n_sink, n_recent, budget_blocks, block_tokens, sel,
                          n_sel, base_pos);
    if (rc) return rc;
    if (n_blocks > budget_blocks) {
      const size_t need = sel_ws_bytes(n_blocks);
      if (!ws || ws_bytes < need) {
        set_error("select workspace %zu < %zu bytes", ws_bytes, need);
        return KVM_ENOMEM;
      }
      KVM_CHECK_ARG((uintptr_t)ws % 256 == 0, "ws must be 256-byte aligned");
      KVM_CHECK_RANGE(ws, need, RANGE_DEVICE, "ws");
    }
    return select_launch(scores, n_blocks, n_sink, n_recent, budget_blocks, block_tokens, sel,
                         n_sel, base_pos, ws, as_stream(stream), true);
  });
}

extern "C" int kvm_select_noalloc(const float* scores, int64_t n_blocks, int32_t n_sink,
                                  int32_t n_recent, int32_t budget_blocks, int32_t block_tokens,
                                  int32_t* sel, int32_t* n_sel, int32_t* base_pos, void* stream) {
  using namespace kvm;
  return guarded([&]() -> int {
    clear_error();
    if (n_blocks > KVM_SELECT_NOALLOC_MAX_BLOCKS) {
      set_error("n_blocks %lld exceeds the %lld blocks the built-in select scratch covers",
                (long long)n_blocks, (long long)KVM_SELECT_NOALLOC_MAX_BLOCKS);
      return KVM_ENOMEM;
    }
    int rc = select_check(scores, n_blocks, n_sink, n_recent, budget_blocks, block_tokens, sel,
                          n_sel, base_pos);
    if (rc) return rc;
    void* ws = nullptr;
    if (n_blocks > budget_blocks) {
      rc = select_scratch(&ws);
      if (rc) return rc;
    }
    return select_launch(scores, n_blocks, n_sink, n_recent, budget_blocks, block_tokens, sel,
                         n_sel, base_pos, ws, as_stream(stream), false);
  });
}
