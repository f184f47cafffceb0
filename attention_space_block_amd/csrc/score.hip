// Block relevance, KVMem Sec. 4.3 Eq. (10), with the tiled/global-softmax
// organisation of Sec. 5:
//   R_b = 1/(L*Hq) sum_{l,h,m} softmax_b( q[l,h,m] . kbar[l,g(h),b] / sqrt(d) ).
// All exponentials are exp2 of x = (q . kbar) * log2(e)/sqrt(d); LSE values
// are kept in the log2 domain.
//
// Two organisations, chosen by the row count TG = T*G of one (layer, KV head):
//
// MFMA path (bf16, TG >= 64): per (l, g) the scores are the dense product
// Q_g[TG x d] * Kbar^T[d x N] on v_mfma_f32_32x32x16_bf16. The per-row softmax
// needs each row's log-sum-exp before any block's share is known, so:
//   pass 1: rows stationary in registers (B operand), Mean-K tiles streamed
//           through double-buffered LDS (A operand) with direct global->LDS
//           copies (global_load_lds_dwordx4: no staging registers, no LDS
//           store instructions; 16-byte pieces XOR-swizzled per row so the
//           operand reads are bank-conflict free); the 32x32 result puts one
//           query row in each lane (16 blocks per lane), so the running
//           shift / sum-exp is lane-local: 16 exps against the current shift,
//           the shift refreshed (tile max, one rescale) only when a tile sum
//           outgrows it; tile sums folded in fp32, the running sum in fp64.
//   pass 2: blocks stationary (B operand), query tiles and their LSE streamed
//           through LDS (A operand); now one block per lane, so the column sum
//           over query rows is lane-local again. Partial R per (l, g) go to a
//           workspace and a fixed-order fp64 reduction makes R deterministic.
// Workgroup ids are remapped so that each XCD works on whole (l, g) pairs and
// the shared operand of a pair stays in that XCD's L2.
//
// Stored-score path (any dtype, small TG, and the host-tiled index): pass 1
// computes every score once on the VALU and stores it (fp32); a stats pass
// forms per-chunk (max, sum-exp) partials from the stored scores, a combine
// kernel the LSE in fp64; pass 2 reads the stored scores back and sums
// exp2(x - LSE) per block in fp64. HBM-bound: one pass over the index plus a
// write and two reads of TG*N*L*Hkv floats. The host-tiled form streams 64 MiB-class tiles H2D through two
// staging buffers on a side stream, double-buffered with events.
#include <math.h>

#include <algorithm>
#include <memory>
#include <mutex>
#include <type_traits>

#include "common.hpp"
#include "profile.hpp"

namespace kvm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) {
  return __builtin_bit_cast(bf16x8, u);
}

static constexpr float LOG2E = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// MFMA passes. Element type E: uint16_t = bf16 operands on
// v_mfma_f32_32x32x16_bf16 (k-steps of 16: 8 per 128-wide row, 4 per 64-wide
// row), uint8_t = FP8 E4M3 operands on v_mfma_scale_f32_32x32x64_f8f6f4 with
// unit scales (2 k-steps of 64, d = 128). Both take A as 32 rows (lane l: row l % 32) and B as 32 columns
// (lane l: column l % 32), the two lane halves holding disjoint k pieces of
// the same row; both operands use the same k pieces per lane, so the product
// is the full dot product. The 32x32 fp32 result layout is the same for both.
// A stage holds 128 rows in LDS, stored as 16-byte pieces XOR-swizzled by row
// so the operand reads are free of bank conflicts: 256-byte rows by row % 16,
// 128-byte rows (bf16 d = 64, FP8 d = 128) by (row / 2) % 8, so that 16 lanes
// reading one piece of 16 consecutive rows hit 16 distinct 16-byte bank groups.
typedef int i32x8 __attribute__((ext_vector_type(8)));

template <typename E, int DD>
struct MfmaShape {
  static constexpr int D = DD;                       // head dim: 128, or 64 for bf16
  static constexpr bool FP8 = sizeof(E) == 1;
  static_assert(D == 128 || (!FP8 && D == 64), "MFMA passes: d = 128, or bf16 with d = 64");
  static constexpr int ROW_B = D * (int)sizeof(E);   // bytes per row: 256 or 128
  static constexpr int PIECES = ROW_B / 16;          // 16-byte pieces per row
  static constexpr int KS = FP8 ? D / 64 : D / 16;   // MFMA k-steps
  static constexpr int PPK = FP8 ? 2 : 1;            // pieces per lane per k-step
  static constexpr int TILE = 128;                   // rows staged per stage
  static constexpr int SUB = TILE / 32;              // 32-row subtiles per stage
  static constexpr int TILE_B = TILE * ROW_B;        // bytes per stage buffer
  static constexpr int LOADS = TILE_B / (256 * 16);  // 16-byte copies per thread per stage
  static constexpr int RPC = 64 / PIECES;            // rows per 1 KiB wave copy
  using Op = typename std::conditional<FP8, i32x8, bf16x8>::type;
  // LDS slot of piece p of stage row r (an involution in p)
  static __device__ __forceinline__ int slot(int r, int p) {
    return ROW_B == 128 ? (p ^ ((r >> 1) & 7)) : (p ^ (r & 15));
  }
  // lane (half) piece j of k-step ks
  static __device__ __forceinline__ int piece(int ks, int half, int j) {
    return (ks * 2 + half) * PPK + j;
  }
  static __device__ __forceinline__ Op make_op(const uint4 (&u)[PPK]) {
    if constexpr (FP8) {
      i32x8 r;
      r[0] = (int)u[0].x; r[1] = (int)u[0].y; r[2] = (int)u[0].z; r[3] = (int)u[0].w;
      r[4] = (int)u[1].x; r[5] = (int)u[1].y; r[6] = (int)u[1].z; r[7] = (int)u[1].w;
      return r;
    } else {
      return as_bf16x8(u[0]);
    }
  }
  static __device__ __forceinline__ f32x16 mma(const Op& a, const Op& b, const f32x16& c) {
    if constexpr (FP8)
      return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
    else
      return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // an operand row from global memory: the lane's pieces of k-step ks (zero
  // when !ok, without a load)
  static __device__ __forceinline__ Op load_op(const char* row, bool ok, int half, int ks) {
    uint4 u[PPK];
#pragma unroll
    for (int j = 0; j < PPK; ++j)
      u[j] = ok ? *reinterpret_cast<const uint4*>(row + piece(ks, half, j) * 16)
                : make_uint4(0, 0, 0, 0);
    return make_op(u);
  }
  // a stationary operand row: the lane's pieces of every k-step
  static __device__ __forceinline__ void load_row(const char* row, bool ok, int half,
                                                  Op (&op)[KS]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) op[ks] = load_op(row, ok, half, ks);
  }
};

struct Pass1Args {
  const void* q;            // [L][Hq][T][D]
  const void* index;        // [L][Hkv][cap][D]
  int64_t cap;
  int32_t n_blocks;
  int32_t T, Hq, Hkv, G, TG;
  int32_t row_chunks;       // ceil(TG / 256)
  int32_t nsplit;
  int32_t split_blocks;     // blocks per split (multiple of 64)
  float scale;              // log2(e)/sqrt(d)
  float2* part;             // [nlg][nsplit][TGp] (max, sum)
  int32_t TGp;              // row_chunks * 256
  int32_t nlg;
  uint32_t total_wg;        // padded to a multiple of 8
};

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

// One wave-wide direct global->LDS copy: lane L's 16 bytes land at dst + 16*L.
__device__ __forceinline__ void dma16(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)src, (lds_void_t*)lds_dst, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)src, (lds_void_t*)lds_dst, 4, 0, 0);
}
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// 32 rows of a staged LDS tile (A operand: lane (half, col) reads its pieces
// of row col at tile + aoff[ks][j]) times the wave's two stationary B tiles,
// with the first level of two exp-sum trees of the previous subtile
// (branch-free VALU work, independent of these MFMAs) woven into the MFMA
// sequence: a wave issues those exps while its own matrix ops run instead of
// waiting for them. Scheduling fences fix the order: each of the 2*KS MFMA
// slots carries its share of the 16 pairs (c, v), v < 8: t[c][v] =
// exp2(fma(p[c][v])) + exp2(fma(p[c][v + 8])), shift sh(c, v). The operand
// reads run ahead of the MFMAs; `extra` issues further LDS reads after the
// first k-step. `tile` is a compile-time LDS address, so every read is a
// register plus an immediate.
template <typename S, typename Shift, typename Extra>
__device__ __forceinline__ void mfma_subtile_woven(f32x16 (&acc)[2], const char* tile,
                                                   const uint32_t (&aoff)[S::KS][S::PPK],
                                                   const typename S::Op (&bop)[2][S::KS],
                                                   const f32x16 (&p)[2], float scale, Shift&& sh,
                                                   float (&t)[2][8], Extra&& extra) {
  constexpr int KS = S::KS;
  constexpr int PPS = 16 / (2 * KS);   // pairs per MFMA slot
  constexpr int AHEAD = KS > 1 ? 2 : 1;
  auto ld = [&](int ks) {
    uint4 u[S::PPK];
#pragma unroll
    for (int j = 0; j < S::PPK; ++j) u[j] = *reinterpret_cast<const uint4*>(tile + aoff[ks][j]);
    return S::make_op(u);
  };
  auto pairs = [&](int slot) {
#pragma unroll
    for (int q = 0; q < PPS; ++q) {
      const int pr = slot * PPS + q, c = pr >> 3, v = pr & 7;
      t[c][v] = hw_exp2(fmaf(p[c][v], scale, -sh(c, v))) +
                hw_exp2(fmaf(p[c][v + 8], scale, -sh(c, v + 8)));
      asm volatile("" ::"v"(t[c][v]));   // keep the pair in its slot (no sinking)
    }
  };
  typename S::Op av[KS];
#pragma unroll
  for (int ks = 0; ks < AHEAD; ++ks) av[ks] = ld(ks);
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[c][v] = 0.0f;
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    acc[0] = S::mma(av[ks], bop[0][ks], acc[0]);
    __builtin_amdgcn_sched_barrier(0);
    pairs(2 * ks);
    if (ks + AHEAD < KS) av[ks + AHEAD] = ld(ks + AHEAD);
    if (ks == 0) extra();
    __builtin_amdgcn_sched_barrier(0);
    acc[1] = S::mma(av[ks], bop[1][ks], acc[1]);
    __builtin_amdgcn_sched_barrier(0);
    pairs(2 * ks + 1);
    __builtin_amdgcn_sched_barrier(0);
  }
  // With few MFMAs per block (FP8, bf16 at d = 64) the compiler would otherwise
  // sink them below the caller's branches, away from the exps they run under.
  if constexpr (S::KS <= 4) asm volatile("" : "+v"(acc[0]), "+v"(acc[1]));
}

// Per-lane byte offsets of the A-operand pieces inside a 32-row subtile:
// lane (half, col) reads pieces piece(ks, half, j) of row col.
template <typename S>
__device__ __forceinline__ void operand_offsets(uint32_t (&aoff)[S::KS][S::PPK], int half,
                                                int col) {
#pragma unroll
  for (int ks = 0; ks < S::KS; ++ks)
#pragma unroll
    for (int j = 0; j < S::PPK; ++j)
      aoff[ks][j] = (uint32_t)(col * S::ROW_B + S::slot(col, S::piece(ks, half, j)) * 16);
}

// Runs stage(it, BUF) for it in [0, n) with the stage buffer BUF = it & 1 as a
// compile-time constant.
template <typename F>
__device__ __forceinline__ void for_stages(int n, F&& stage) {
  for (int it = 0; it < n; it += 2) {
    stage(it, std::integral_constant<int, 0>{});
    if (it + 1 < n) stage(it + 1, std::integral_constant<int, 1>{});
  }
}

// Remaining levels (w = 4, 2, 1) of the exp-sum tree whose first level
// mfma_subtile_woven formed; the same order as exp_sum16.
__device__ __forceinline__ float tree8(float (&t)[8]) {
#pragma unroll
  for (int w = 4; w >= 1; w >>= 1)
#pragma unroll
    for (int v = 0; v < w; ++v) t[v] += t[v + w];
  return t[0];
}

// Sum of exp2(acc[v] * scale - m) over a lane's 16 values, fixed tree order.
__device__ __forceinline__ float exp_sum16(const f32x16& acc, float scale, float m) {
  float e[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) e[v] = hw_exp2(fmaf(acc[v], scale, -m));
#pragma unroll
  for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
    for (int v = 0; v < w; ++v) e[v] += e[v + w];
  return e[0];
}

// Online (shift, sum-exp) state of one lane's query row. The exps are taken
// against a running shift m_run (log2 units) that is refreshed lazily: scores
// are summed against the current shift, and only when a sum is not at most
// LAZY_MAX (some score more than 64 log2-units above the shift, no shift yet
// (-inf), or an inf/NaN) are the same scores taken again exactly: tile max, new
// shift, rescale of the running sum. Any shift gives the same log-sum-exp; a
// sum that passes the test holds no term above 2^64, so no fp32 exp or partial
// sum can overflow, and the fp64 running sum keeps every term. A lane that has
// seen only -inf keeps m = -inf and s = 0.
static constexpr float LAZY_MAX = 18446744073709551616.0f;   // 2^64

// The exact path for 16 new scores (raw dot products; x = acc * scale).
__device__ __forceinline__ void lse_exact(const f32x16& acc, float scale, float& m_run,
                                          double& s_run) {
  float mx = acc[0];
#pragma unroll
  for (int v = 1; v < 16; ++v) mx = fmaxf(mx, acc[v]);
  const float m_new = fmaxf(m_run, mx * scale);
  const float m_use = m_new == -INFINITY ? 0.0f : m_new;
  const float resc = hw_exp2(m_run - m_use);
  s_run = s_run * (double)resc + (double)exp_sum16(acc, scale, m_use);
  m_run = m_new;
}

// One lazy update with 16 new scores.
__device__ __forceinline__ void lse_update(const f32x16& acc, float scale, float& m_run,
                                           double& s_run) {
  const float tsum = exp_sum16(acc, scale, m_run);
  if (tsum <= LAZY_MAX) s_run += (double)tsum;
  else lse_exact(acc, scale, m_run, s_run);
}

__device__ __forceinline__ void mask_rows(f32x16 (&acc)[2], int half, int32_t nvalid) {
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int i = 8 * (v >> 2) + 4 * half + (v & 3);
      if (i >= nvalid) acc[c][v] = -INFINITY;
    }
}

template <typename E, int DD>
__global__ __launch_bounds__(256, 2) void score_pass1_mfma(Pass1Args a) {
  using S = MfmaShape<E, DD>;
  constexpr int D = S::D;
  __shared__ __attribute__((aligned(16))) char lds[2][S::TILE_B];
  const uint32_t lid = xcd_remap(blockIdx.x, a.total_wg);
  const int32_t per_lg = a.row_chunks * a.nsplit;
  const int32_t L_lg = (int32_t)(lid / per_lg);  // (l, g) flattened = l*Hkv + g
  if (L_lg >= a.nlg) return;                     // grid padding
  const int32_t rem = (int32_t)(lid % per_lg);
  const int32_t split = rem / a.row_chunks;
  const int32_t rchunk = rem % a.row_chunks;
  const int l = L_lg / a.Hkv, g = L_lg % a.Hkv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, col = lane & 31;

  // B operand: two 32-row tiles of this wave's query rows (stationary).
  typename S::Op bq[2][S::KS];
  const int row_base = rchunk * 256 + wave * 64;
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int rho = row_base + ct * 32 + col;
    const bool ok = rho < a.TG;
    const int hh = g * a.G + (ok ? rho / a.T : 0);
    const int m = ok ? rho % a.T : 0;
    const char* qp = reinterpret_cast<const char*>(a.q) +
                     (((int64_t)l * a.Hq + hh) * a.T + m) * S::ROW_B;
    S::load_row(qp, ok, half, bq[ct]);
  }

  const int32_t b_begin = split * a.split_blocks;
  int32_t b_end = b_begin + a.split_blocks;
  if (b_end > a.n_blocks) b_end = a.n_blocks;
  const int32_t ntiles = b_end > b_begin ? (b_end - b_begin + S::TILE - 1) / S::TILE : 0;
  const char* kb = reinterpret_cast<const char*>(a.index) + (int64_t)L_lg * a.cap * S::ROW_B;

  float m_run[2] = {-INFINITY, -INFINITY};
  double s_run[2] = {0.0, 0.0};

  // Direct global->LDS stage copy. Copy i of a wave fills the 1 KiB at slot
  // (i*4 + wave)*64: 16-byte slot s of stage row r receives piece
  // S::slot(r, s) (the swizzle is an involution), so the operand reads hit
  // distinct banks. A lane copies stage rows 4*RPC*i + dma_row, piece
  // dma_piece (the swizzle does not depend on i): the global address is a
  // uniform stage base plus one 32-bit lane offset. In a stage that runs past
  // b_end the rows past it re-read the last valid row (finite values, masked
  // to -inf later).
  const int dma_row = S::RPC * wave + lane / S::PIECES;
  const int dma_piece = S::slot(dma_row, lane % S::PIECES);
  const uint32_t dma_off = (uint32_t)(dma_row * S::ROW_B + dma_piece * 16);
  auto dma_stage = [&](int tile, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    const int32_t t0 = b_begin + tile * S::TILE;
    const char* base = kb + (int64_t)t0 * S::ROW_B;
    if (t0 + S::TILE <= b_end) {
#pragma unroll
      for (int i = 0; i < S::LOADS; ++i)
        dma16(base + i * 4096 + dma_off, &lds[BUF][(i * 4 + wave) * 1024]);
    } else {
#pragma unroll
      for (int i = 0; i < S::LOADS; ++i) {
        const int32_t r = t0 + 4 * S::RPC * i + dma_row;
        const int32_t b = r < b_end ? r : b_end - 1;
        dma16(kb + (int64_t)b * S::ROW_B + dma_piece * 16, &lds[BUF][(i * 4 + wave) * 1024]);
      }
    }
  };
  uint32_t aoff[S::KS][S::PPK];
  operand_offsets<S>(aoff, half, col);

  // Exact recomputation of subtiles [j0, j1) (j0 >= 0): their scores again,
  // with the index rows read from global memory straight into the A operand
  // (the stage buffers may already hold later rows), then the exact update.
  auto replay = [&](int j0, int j1) {
    for (int j = j0; j < j1; ++j) {
      const int32_t r0 = b_begin + 32 * j;
      const int32_t b = r0 + col;
      const bool ok = b < b_end;
      const char* row = kb + (int64_t)(ok ? b : 0) * S::ROW_B;
      f32x16 acc[2];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[c][v] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < S::KS; ++ks) {
        const typename S::Op av = S::load_op(row, ok, half, ks);
        acc[0] = S::mma(av, bq[0][ks], acc[0]);
        acc[1] = S::mma(av, bq[1][ks], acc[1]);
      }
      if (b_end - r0 < 32) mask_rows(acc, half, b_end - r0);
      lse_exact(acc[0], a.scale, m_run[0], s_run[0]);
      lse_exact(acc[1], a.scale, m_run[1], s_run[1]);
    }
  };

  // Software pipeline over 32-block subtiles: while the MFMAs of subtile j
  // run, the wave takes the exps of subtile j-1 (its scores sit in the other
  // accumulator set). ab[j & 1] holds subtile j; before the first subtile the
  // other set holds -inf scores. A stage holds SUB (even) subtiles; the next
  // stage's global loads are in flight while they are multiplied and reduced.
  // The exps a stage takes (subtiles 4it-1 .. 4it+2) are summed in fp32
  // against the shift the stage started with, without a branch; at the end of
  // the stage the sums enter the fp64 running sums, unless some lane's sum
  // fails the lazy test (always so in the first stage, where there is no shift
  // yet): then the wave takes those subtiles again on the exact path.
  static_assert(S::SUB == 4, "a stage's exps cover subtiles 4it-1 .. 4it+2");
  f32x16 ab[2][2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) ab[1][c][v] = -INFINITY;
  if (ntiles > 0) dma_stage(0, std::integral_constant<int, 0>{});
  wait_dma();
  __syncthreads();
  for_stages(ntiles, [&](int it, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    const int32_t t0 = b_begin + it * S::TILE;
    if (it + 1 < ntiles) dma_stage(it + 1, std::integral_constant<int, BUF ^ 1>{});
    float g_sum[2] = {0.0f, 0.0f};
    const float m0 = m_run[0], m1 = m_run[1];
#pragma unroll
    for (int sub = 0; sub < S::SUB; ++sub) {
      f32x16 (&cur)[2] = ab[sub & 1];
      f32x16 (&prv)[2] = ab[(sub & 1) ^ 1];
      float t[2][8];
      mfma_subtile_woven<S>(cur, &lds[BUF][sub * 32 * S::ROW_B], aoff, bq, prv, a.scale,
                            [&](int c, int) { return c ? m1 : m0; }, t, [] {});
      g_sum[0] += tree8(t[0]);
      g_sum[1] += tree8(t[1]);
      asm volatile("" : "+v"(g_sum[0]), "+v"(g_sum[1]));   // sum each subtile here
      const int32_t nvalid = b_end - (t0 + 32 * sub);
      if (nvalid < 32) mask_rows(cur, half, nvalid);   // uniform: only a split's last stage
    }
    const bool good = g_sum[0] <= LAZY_MAX && g_sum[1] <= LAZY_MAX;
    if (__builtin_amdgcn_ballot_w64(!good) == 0) {
      s_run[0] += (double)g_sum[0];
      s_run[1] += (double)g_sum[1];
    } else {
      replay(it > 0 ? 4 * it - 1 : 0, 4 * it + 3);
    }
    wait_dma();
    __syncthreads();
  });
  lse_update(ab[1][0], a.scale, m_run[0], s_run[0]);   // the last subtile
  lse_update(ab[1][1], a.scale, m_run[1], s_run[1]);
  // Merge the two lane halves (same query row, disjoint blocks).
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const float mo = __shfl_xor(m_run[ct], 32);
    const double so = __shfl_xor(s_run[ct], 32);
    const float mm = fmaxf(m_run[ct], mo);
    double s = 0.0;
    if (mm != -INFINITY)
      s = s_run[ct] * (double)hw_exp2(m_run[ct] - mm) + so * (double)hw_exp2(mo - mm);
    if (half == 0) {
      const int rho = row_base + ct * 32 + col;
      a.part[((int64_t)L_lg * a.nsplit + split) * a.TGp + rho] = make_float2(mm, (float)s);
    }
  }
}

// LSE (log2 domain) per (l, g, row) from split partials, fp64.
__global__ void score_lse_combine(const float2* __restrict__ part, int32_t nlg, int32_t nsplit,
                                  int32_t TGp, int32_t TG, float* __restrict__ lse) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)nlg * TGp) return;
  const int64_t lg = i / TGp;
  const int32_t r = (int32_t)(i % TGp);
  if (r >= TG) {
    lse[i] = INFINITY;  // padded rows contribute exp2(-inf) = 0
    return;
  }
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part[(lg * nsplit + s) * TGp + r].x);
  double sum = 0.0;
  for (int s = 0; s < nsplit; ++s) {
    const float2 p = part[(lg * nsplit + s) * TGp + r];
    if (p.x != -INFINITY) sum += (double)p.y * exp2((double)p.x - (double)M);
  }
  lse[i] = (float)((double)M + log2(sum));
}

// ---------------------------------------------------------------------------
// MFMA pass 2: column sums of exp2(x - lse) per (l, g) over all query rows.
struct Pass2Args {
  const void* q;
  const void* index;
  int64_t cap;
  int32_t n_blocks;
  int32_t T, Hq, Hkv, G, TG, TGp;
  int32_t block_chunks;     // ceil(N / 256)
  float scale;
  const float* lse;         // [nlg][TGp]
  float* rp;                // [nlg][N]
  int32_t nlg;
  uint32_t total_wg;
};

// Column sum over one subtile's 16 rows of a lane: sum of exp2(acc*scale - lse),
// fixed tree order.
__device__ __forceinline__ float exp_sum16_rows(const f32x16& acc, const float (&ls)[16],
                                                float scale) {
  float e[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) e[v] = hw_exp2(fmaf(acc[v], scale, -ls[v]));
#pragma unroll
  for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
    for (int v = 0; v < w; ++v) e[v] += e[v + w];
  return e[0];
}

template <typename E, int DD>
__global__ __launch_bounds__(256, 2) void score_pass2_mfma(Pass2Args a) {
  using S = MfmaShape<E, DD>;
  __shared__ __attribute__((aligned(16))) char lds[2][S::TILE_B];
  __shared__ __attribute__((aligned(16))) float lse_s[2][S::TILE];
  const uint32_t lid = xcd_remap(blockIdx.x, a.total_wg);
  const int32_t lg = (int32_t)(lid / a.block_chunks);
  if (lg >= a.nlg) return;                       // grid padding
  const int32_t bchunk = (int32_t)(lid % a.block_chunks);
  const int l = lg / a.Hkv, g = lg % a.Hkv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, col = lane & 31;

  // B operand: this wave's two 32-block tiles (stationary).
  typename S::Op bk[2][S::KS];
  const int32_t blk_base = bchunk * 256 + wave * 64;
  const char* kb = reinterpret_cast<const char*>(a.index) + (int64_t)lg * a.cap * S::ROW_B;
#pragma unroll
  for (int bt = 0; bt < 2; ++bt) {
    const int32_t b = blk_base + bt * 32 + col;
    const bool ok = b < a.n_blocks;
    S::load_row(kb + (int64_t)(ok ? b : 0) * S::ROW_B, ok, half, bk[bt]);
  }
  const float* lse_lg = a.lse + (int64_t)lg * a.TGp;
  const int32_t ntiles = (a.TG + S::TILE - 1) / S::TILE;
  // Query rows of (l, g) are contiguous: heads g*G .. g*G+G-1, tokens 0..T-1.
  const char* qg = reinterpret_cast<const char*>(a.q) +
                   ((int64_t)l * a.Hq + (int64_t)g * a.G) * a.T * S::ROW_B;
  // Stage copies as in pass 1 (same slot layout), plus the stage's LSE values
  // (waves 0 and 1, 64 each; rows past TG read the +inf padding of the LSE
  // array, whose rows TG..TGp-1 exist because TGp is a multiple of 256).
  const int dma_row = S::RPC * wave + lane / S::PIECES;
  const int dma_piece = S::slot(dma_row, lane % S::PIECES);
  const uint32_t dma_off = (uint32_t)(dma_row * S::ROW_B + dma_piece * 16);
  auto dma_stage = [&](int tile, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    const int32_t r0 = tile * S::TILE;
    const char* base = qg + (int64_t)r0 * S::ROW_B;
    if (r0 + S::TILE <= a.TG) {
#pragma unroll
      for (int i = 0; i < S::LOADS; ++i)
        dma16(base + i * 4096 + dma_off, &lds[BUF][(i * 4 + wave) * 1024]);
    } else {
#pragma unroll
      for (int i = 0; i < S::LOADS; ++i) {
        const int32_t r = r0 + 4 * S::RPC * i + dma_row;
        const int32_t rho = r < a.TG ? r : a.TG - 1;   // padded rows: lse = +inf
        dma16(qg + (int64_t)rho * S::ROW_B + dma_piece * 16, &lds[BUF][(i * 4 + wave) * 1024]);
      }
    }
    if (wave < 2) dma4(lse_lg + r0 + wave * 64 + lane, &lse_s[BUF][wave * 64]);
  };
  uint32_t aoff[S::KS][S::PPK];
  operand_offsets<S>(aoff, half, col);
  // LSE of the 16 rows a lane holds in a subtile: rows 8*q4 + 4*half + 0..3.
  auto load_lse = [&](float (&ls)[16], const float* sub_lse) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 v4 = *reinterpret_cast<const float4*>(sub_lse + 8 * q4 + 4 * half);
      ls[4 * q4 + 0] = v4.x;
      ls[4 * q4 + 1] = v4.y;
      ls[4 * q4 + 2] = v4.z;
      ls[4 * q4 + 3] = v4.w;
    }
  };
  // Software pipeline as in pass 1: the exps and column sums of subtile j-1
  // run under the MFMAs of subtile j. Each subtile's LSE values are read from
  // LDS in the block that multiplies it (before the barrier that frees its
  // buffer) and kept in registers for the next block. The dummy subtile
  // before the first (-inf scores, LSE 0) adds exactly 0.
  static_assert(S::SUB % 2 == 0, "subtile slots alternate within a stage");
  double colsum[2] = {0.0, 0.0};
  f32x16 ab[2][2];
  float lsb[2][16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    ab[1][0][v] = -INFINITY;
    ab[1][1][v] = -INFINITY;
    lsb[1][v] = 0.0f;
  }
  dma_stage(0, std::integral_constant<int, 0>{});
  wait_dma();
  __syncthreads();
  for_stages(ntiles, [&](int it, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    if (it + 1 < ntiles) dma_stage(it + 1, std::integral_constant<int, BUF ^ 1>{});
#pragma unroll
    for (int sub = 0; sub < S::SUB; ++sub) {
      const int j = sub & 1;
      float t[2][8];
      const float (&lp)[16] = lsb[j ^ 1];
      mfma_subtile_woven<S>(ab[j], &lds[BUF][sub * 32 * S::ROW_B], aoff, bk, ab[j ^ 1], a.scale,
                            [&](int, int v) { return lp[v]; }, t,
                            [&] { load_lse(lsb[j], &lse_s[BUF][sub * 32]); });
      colsum[0] += (double)tree8(t[0]);
      colsum[1] += (double)tree8(t[1]);
    }
    wait_dma();
    __syncthreads();
  });
  colsum[0] += (double)exp_sum16_rows(ab[1][0], lsb[1], a.scale);   // the last subtile
  colsum[1] += (double)exp_sum16_rows(ab[1][1], lsb[1], a.scale);
#pragma unroll
  for (int bt = 0; bt < 2; ++bt) {
    const double tot = colsum[bt] + __shfl_xor(colsum[bt], 32);
    const int32_t b = blk_base + bt * 32 + col;
    if (half == 0 && b < a.n_blocks) a.rp[(int64_t)lg * a.n_blocks + b] = (float)tot;
  }
}

// R[b] = (sum over (l, g) of rp[lg][b], fp64) / (L*Hq). A workgroup takes 64
// blocks; its four waves sum the (l, g) rows lg = w, w + 4, ... of them and the
// four partial sums are added in wave order, so the result is deterministic.
__global__ __launch_bounds__(256) void score_reduce(const float* __restrict__ rp, int32_t nlg,
                                                   int32_t n_blocks, double inv_lh,
                                                   float* __restrict__ scores) {
  __shared__ double part[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int32_t b = blockIdx.x * 64 + lane;
  double s = 0.0;
  if (b < n_blocks) {
#pragma unroll 8
    for (int32_t lg = w; lg < nlg; lg += 4) s += (double)rp[(int64_t)lg * n_blocks + b];
  }
  part[w][lane] = s;
  __syncthreads();
  if (w == 0 && b < n_blocks)
    scores[b] = (float)((((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane]) *
                        inv_lh);
}

// ---------------------------------------------------------------------------
// Stored-score path. Pass 1: thread per block; the query rows of the (l, g)
// sit in LDS as fp32; each thread keeps its Mean-K row in registers.
template <typename T, int D>
__device__ __forceinline__ void load_row(const T* p, float* x);
template <>
__device__ __forceinline__ void load_row<uint16_t, 128>(const uint16_t* p, float* x) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint4 v = reinterpret_cast<const uint4*>(p)[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
      x[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  }
}
template <>
__device__ __forceinline__ void load_row<uint16_t, 64>(const uint16_t* p, float* x) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint4 v = reinterpret_cast<const uint4*>(p)[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
      x[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  }
}
template <>
__device__ __forceinline__ void load_row<float, 128>(const float* p, float* x) {
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float4 v = reinterpret_cast<const float4*>(p)[i];
    x[4 * i] = v.x; x[4 * i + 1] = v.y; x[4 * i + 2] = v.z; x[4 * i + 3] = v.w;
  }
}
template <>
__device__ __forceinline__ void load_row<float, 64>(const float* p, float* x) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float4 v = reinterpret_cast<const float4*>(p)[i];
    x[4 * i] = v.x; x[4 * i + 1] = v.y; x[4 * i + 2] = v.z; x[4 * i + 3] = v.w;
  }
}

template <typename T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t v) { return bf16_to_f32(v); }
template <>
__device__ __forceinline__ float to_f32<float>(float v) { return v; }

struct StoredArgs {
  const void* q;            // [L][Hq][T][D]
  const void* index;        // rows of this launch: index + lg*lg_stride + (b - b_first)*D
  int64_t lg_stride;        // elements between (l, g) row sets of `index`
  int32_t b_first;          // first block of this launch (multiple of 256)
  int32_t nb;               // blocks in this launch
  int32_t n_blocks;         // N (layout of S)
  int32_t T, Hq, Hkv, G, TG, nlg;
  int32_t chunks_total;     // (max, sum) partials per row: ceil(N / chunk)
  int32_t chunk;            // blocks per partial (bf16: rows per pass-1 workgroup)
  float scale;
  float* S;                 // [nlg][N][TG]
  float2* part;             // [nlg][chunks_total][TG]
};

template <typename T, int D>
__global__ __launch_bounds__(256) void score_stored_pass1(StoredArgs a) {
  extern __shared__ float smem[];       // q rows [TG][D]
  float* qs = smem;
  const int32_t chunks_here = (a.nb + 255) / 256;
  const int32_t lg = blockIdx.x / chunks_here;
  const int32_t ch = blockIdx.x % chunks_here;
  const int l = lg / a.Hkv, g = lg % a.Hkv;
  const T* q = reinterpret_cast<const T*>(a.q);
  for (int e = threadIdx.x; e < a.TG * D; e += 256) {
    const int rho = e / D, t = e % D;
    const int hh = g * a.G + rho / a.T, m = rho % a.T;
    qs[e] = to_f32<T>(q[(((int64_t)l * a.Hq + hh) * a.T + m) * D + t]);
  }
  __syncthreads();
  const int32_t bl = ch * 256 + threadIdx.x;       // block within this launch
  const bool valid = bl < a.nb;
  const int32_t b = a.b_first + bl;
  if (!valid) return;                          // no barrier follows
  float k[D];
  load_row<T, D>(reinterpret_cast<const T*>(a.index) + (int64_t)lg * a.lg_stride +
                     (int64_t)bl * D, k);
  float* srow = a.S + ((int64_t)lg * a.n_blocks + b) * a.TG;
  for (int rho = 0; rho < a.TG; ++rho) {
    const float* qr = qs + rho * D;
    float acc = 0.0f;
#pragma unroll
    for (int t = 0; t < D; ++t) acc = fmaf(qr[t], k[t], acc);
    srow[rho] = acc * a.scale;
  }
}

// Stored-score pass 1 on the matrix cores (bf16, or FP8 at d = 128): the scores
// of one (l, g) are the product Kbar[N x d] * Q_g^T[d x TG], taken in 16-row
// tiles (StoredOps below): A = 16 index rows (lane l holds row l % 16 and its
// k pieces, read straight from global memory), B = the TG query rows padded to
// 16-column tiles (stationary in registers). Each lane's 4 results are rows
// 4*(l/16) .. +3 of the tile at query row l % 16. The VALU only scales and
// stores, so the pass streams the index at memory speed. A workgroup takes
// `chunk` (512) rows of one (l, g); each wave keeps 4 tiles of loads in
// flight. Each lane also keeps an online (shift, sum-exp) of its query row, so
// the workgroup writes the chunk's partials for the LSE itself.
// Merge two (shift, sum-exp) pairs of the same row.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;                 // both empty
  s = s * hw_exp2(m - M) + s2 * hw_exp2(m2 - M);
  m = M;
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Operand traits of the stored pass 1: bf16 on v_mfma_f32_16x16x32_bf16 (k-steps
// of 32; lane l holds elements 32*ks + 8*(l/16) .. +8 of its row), FP8 E4M3 on
// v_mfma_scale_f32_16x16x128_f8f6f4 with unit scales (d = 128 in one step; lane
// l holds bytes 32*(l/16) .. +32 of its row). Both operands use the same k
// assignment, so the product is the full dot product; the 16x16 fp32 result
// layout is the same for both.
template <typename E, int D>
struct StoredOps {
  static constexpr int KS = D / 32;
  using Op = bf16x8_t;
  static __device__ __forceinline__ Op load(const char* row, int kg, int ks) {
    return __builtin_bit_cast(bf16x8_t,
                              *reinterpret_cast<const uint4*>(row + (32 * ks + 8 * kg) * 2));
  }
  static __device__ __forceinline__ Op zero() { return __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0)); }
  static __device__ __forceinline__ f32x4_t mma(const Op& a, const Op& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct StoredOps<uint8_t, 128> {
  static constexpr int KS = 1;
  using Op = i32x8;
  static __device__ __forceinline__ Op load(const char* row, int kg, int) {
    const uint4 u0 = *reinterpret_cast<const uint4*>(row + 32 * kg);
    const uint4 u1 = *reinterpret_cast<const uint4*>(row + 32 * kg + 16);
    i32x8 r;
    r[0] = (int)u0.x; r[1] = (int)u0.y; r[2] = (int)u0.z; r[3] = (int)u0.w;
    r[4] = (int)u1.x; r[5] = (int)u1.y; r[6] = (int)u1.z; r[7] = (int)u1.w;
    return r;
  }
  static __device__ __forceinline__ Op zero() { return i32x8{0, 0, 0, 0, 0, 0, 0, 0}; }
  static __device__ __forceinline__ f32x4_t mma(const Op& a, const Op& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
};

// STAGE (T*G <= 32): each wavefront collects the scores of its 64 rows in LDS
// and writes them as one contiguous span with consecutive lanes on consecutive
// words, instead of scattered per-tile stores of T*G words per row.
template <typename E, int D, bool STAGE>
__global__ __launch_bounds__(256) void score_stored_pass1_mfma(StoredArgs a) {
  using O = StoredOps<E, D>;
  constexpr int KS = O::KS;
  constexpr int ROW_B = D * (int)sizeof(E);
  constexpr int TU = 4;                        // 16-row tiles in flight per wave
  constexpr int MAXCT = 4;                     // TG < 64: at most 4 column tiles
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __shared__ float2 red[4][64];
  const int32_t chunks_here = (a.nb + a.chunk - 1) / a.chunk;
  const int32_t lg = blockIdx.x / chunks_here;
  const int32_t ch = blockIdx.x % chunks_here;
  const int32_t r_begin = ch * a.chunk;
  const int32_t r_end = r_begin + a.chunk < a.nb ? r_begin + a.chunk : a.nb;
  const int l = lg / a.Hkv, g = lg % a.Hkv;
  const int r16 = lane & 15, kg = lane >> 4;
  const int nct = (a.TG + 15) / 16;
  // B: query row rho = 16*ct + r16, the lane's k pieces
  typename O::Op bq[MAXCT][KS];
  const char* q = reinterpret_cast<const char*>(a.q);
#pragma unroll
  for (int ct = 0; ct < MAXCT; ++ct) {
    const int rho = 16 * ct + r16;
    const bool ok = rho < a.TG;
    const int hh = g * a.G + (ok ? rho / a.T : 0), m = ok ? rho % a.T : 0;
    const char* qp = q + (((int64_t)l * a.Hq + hh) * a.T + m) * ROW_B;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bq[ct][ks] = ok ? O::load(qp, kg, ks) : O::zero();
  }
  const char* base = reinterpret_cast<const char*>(a.index) + (int64_t)lg * a.lg_stride * sizeof(E);
  float* Sl = a.S + ((int64_t)lg * a.n_blocks + a.b_first) * a.TG;
  extern __shared__ __attribute__((aligned(16))) float stg_all[];   // STAGE: [4 waves][16*TU rows][TG]
  float* stg = stg_all + wave * (16 * TU) * a.TG;
  // online (shift, sum-exp) of the lane's query rows over its scores
  float m_run[MAXCT], s_run[MAXCT];
#pragma unroll
  for (int ct = 0; ct < MAXCT; ++ct) {
    m_run[ct] = -INFINITY;
    s_run[ct] = 0.0f;
  }
  for (int32_t r0 = r_begin + wave * 16 * TU; r0 < r_end; r0 += 4 * 16 * TU) {
    typename O::Op av[TU][KS];
#pragma unroll
    for (int t = 0; t < TU; ++t) {
      int32_t row = r0 + 16 * t + r16;
      row = row < r_end ? row : r_end - 1;     // rows past the end re-read the last one
      const char* rp = base + (int64_t)row * ROW_B;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) av[t][ks] = O::load(rp, kg, ks);
    }
#pragma unroll
    for (int t = 0; t < TU; ++t) {
      const int32_t t0 = r0 + 16 * t;
      if (t0 >= r_end) break;                  // uniform over the wave
#pragma unroll
      for (int ct = 0; ct < MAXCT; ++ct) {
        if (ct >= nct) break;                  // uniform
        f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          acc = O::mma(av[t][ks], bq[ct][ks], acc);
        const int rho = 16 * ct + r16;
        if (rho < a.TG) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int32_t row = t0 + 4 * kg + v;
            if (row < r_end) {
              const float x = acc[v] * a.scale;
              if (STAGE) stg[(row - r0) * a.TG + rho] = x;
              else Sl[(int64_t)row * a.TG + rho] = x;
              if (x > m_run[ct]) {
                s_run[ct] = s_run[ct] * hw_exp2(m_run[ct] - x) + 1.0f;
                m_run[ct] = x;
              } else {
                s_run[ct] += hw_exp2(x - m_run[ct]);
              }
            }
          }
        }
      }
    }
    if (STAGE) {
      // the wave's own LDS rows: its writes are visible to its reads once the
      // LDS counter drains, and the next group's writes follow these reads
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int32_t nrows = r_end - r0 < 16 * TU ? r_end - r0 : 16 * TU;
      const int n = nrows * a.TG;
      float* dst = Sl + (int64_t)r0 * a.TG;
      // 16-byte stores where the span starts 16-byte aligned (uniform: N*T*G
      // a multiple of 4; every wave's LDS rows start 16-byte aligned), else
      // 4-byte ones: 8.59-8.66 ms against 8.66-8.71 at 10M tokens
      if (((uintptr_t)dst & 15) == 0) {
        const int n4 = n >> 2;
        for (int i = lane; i < n4; i += 64)
          reinterpret_cast<float4*>(dst)[i] = reinterpret_cast<const float4*>(stg)[i];
        for (int i = 4 * n4 + lane; i < n; i += 64) dst[i] = stg[i];
      } else {
        for (int i = lane; i < n; i += 64) dst[i] = stg[i];
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
  // merge the four lanes of each query row (xor 16, 32), then the waves in order
  const int32_t gchunk = a.b_first / a.chunk + ch;
#pragma unroll
  for (int ct = 0; ct < MAXCT; ++ct) {
    if (ct >= nct) break;
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      const float m2 = __shfl_xor(m_run[ct], off), s2 = __shfl_xor(s_run[ct], off);
      lse_merge(m_run[ct], s_run[ct], m2, s2);
    }
    if (kg == 0) red[wave][16 * ct + r16] = make_float2(m_run[ct], s_run[ct]);
  }
  __syncthreads();
  if ((int)threadIdx.x < a.TG) {
    const int r = threadIdx.x;
    float mm = red[0][r].x, ss = red[0][r].y;
    for (int w = 1; w < 4; ++w) lse_merge(mm, ss, red[w][r].x, red[w][r].y);
    a.part[((int64_t)lg * a.chunks_total + gchunk) * a.TG + r] = make_float2(mm, ss);
  }
}

// (max, sum-exp) partials of the stored scores per (l, g, chunk of blocks, row),
// in a pass of their own so pass 1 streams the index without reductions. Rows
// are taken 8 at a time: each thread walks its blocks once per group with an
// online (shift, sum) per row (one exp per score; the shift moves up when a
// larger score arrives), then the pairs are merged in a fixed order (xor
// shuffles, then the four waves in order), so the partials are deterministic.

__global__ __launch_bounds__(256) void score_stored_stats(const float* __restrict__ S,
                                                          int32_t n_blocks, int32_t TG,
                                                          int32_t chunk, int32_t chunks_total,
                                                          float2* __restrict__ part) {
  constexpr int RG = 8;                        // rows per group
  __shared__ float2 red[4][RG];
  const int32_t lg = blockIdx.x / chunks_total, ch = blockIdx.x % chunks_total;
  const int32_t b0 = ch * chunk;
  const int32_t b1 = b0 + chunk < n_blocks ? b0 + chunk : n_blocks;
  const float* Sl = S + (int64_t)lg * n_blocks * TG;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int r0 = 0; r0 < TG; r0 += RG) {
    const int nr = TG - r0 < RG ? TG - r0 : RG;
    float m[RG], sm[RG];
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      m[r] = -INFINITY;
      sm[r] = 0.0f;
    }
    for (int32_t b = b0 + (int32_t)threadIdx.x; b < b1; b += 256) {
      const float* row = Sl + (int64_t)b * TG + r0;
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        if (r < nr) {
          const float x = row[r];
          if (x > m[r]) {
            sm[r] = sm[r] * hw_exp2(m[r] - x) + 1.0f;
            m[r] = x;
          } else {
            sm[r] += hw_exp2(x - m[r]);
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RG; ++r) {
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float m2 = __shfl_xor(m[r], off), s2 = __shfl_xor(sm[r], off);
        lse_merge(m[r], sm[r], m2, s2);
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < RG; ++r) red[wave][r] = make_float2(m[r], sm[r]);
    }
    __syncthreads();
    if ((int)threadIdx.x < nr) {
      const int r = threadIdx.x;
      float mm = red[0][r].x, ss = red[0][r].y;
      for (int w = 1; w < 4; ++w) lse_merge(mm, ss, red[w][r].x, red[w][r].y);
      part[((int64_t)lg * chunks_total + ch) * TG + r0 + r] = make_float2(mm, ss);
    }
    __syncthreads();
  }
}

// LSE (log2 domain) per (l, g, row) of the stored-score path from its chunk
// partials: one wavefront per row; lanes stride over the chunks, then xor
// trees (max in fp32, the rescaled sum in fp64), a fixed order throughout.
__global__ __launch_bounds__(64) void score_stored_lse(const float2* __restrict__ part,
                                                       int32_t nlg, int32_t chunks, int32_t TG,
                                                       float* __restrict__ lse) {
  const int64_t i = blockIdx.x;                // (lg, r)
  if (i >= (int64_t)nlg * TG) return;          // uniform
  const int64_t lg = i / TG;
  const int32_t r = (int32_t)(i % TG);
  const int lane = threadIdx.x;
  const float2* p = part + lg * chunks * TG + r;
  float M = -INFINITY;
  for (int c = lane; c < chunks; c += 64) M = fmaxf(M, p[(int64_t)c * TG].x);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  double sum = 0.0;
  for (int c = lane; c < chunks; c += 64) {
    const float2 v = p[(int64_t)c * TG];
    if (v.x != -INFINITY) sum += (double)v.y * exp2((double)v.x - (double)M);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane == 0) lse[i] = (float)((double)M + log2(sum));
}

// Pass 2 of the stored-score path: thread b sums exp2(S - LSE) over the TG
// scores of each (l, g) in row order in fp32, and those sums over (l, g) in
// order in fp64. TGC > 0 fixes the row count at compile time (decode-sized
// query rows), so the loads of several (l, g) are in flight at once; the
// arithmetic is the same either way.
template <int TGC>
__global__ __launch_bounds__(256) void score_stored_pass2(const float* __restrict__ S,
                                                          const float* __restrict__ lse,
                                                          int32_t nlg, int32_t TG_rt,
                                                          int32_t n_blocks, double inv_lh,
                                                          float* __restrict__ scores) {
  const int TG = TGC > 0 ? TGC : TG_rt;
  extern __shared__ float lse_s[];  // [nlg*TG]
  for (int i = threadIdx.x; i < nlg * TG; i += 256) lse_s[i] = lse[i];
  __syncthreads();
  const int32_t b = blockIdx.x * 256 + threadIdx.x;
  if (b >= n_blocks) return;
  const float* col = S + (int64_t)b * TG;
  const int64_t lg_stride = (int64_t)n_blocks * TG;
  double s = 0.0;
#pragma unroll 4
  for (int32_t lg = 0; lg < nlg; ++lg) {
    const float* row = col + lg * lg_stride;
    const float* ls = lse_s + lg * TG;
    float t = 0.0f;
    for (int r = 0; r < TG; ++r) t += hw_exp2(row[r] - ls[r]);
    s += (double)t;
  }
  scores[b] = (float)(s * inv_lh);
}

// ---------------------------------------------------------------------------
// Host side

struct Plan {
  bool mfma;
  int32_t TG, TGp, nsplit, split_blocks, row_chunks, block_chunks, chunks, chunk;
  size_t off_part, off_lse, off_rp, off_S, off_stage, bytes;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// blocks per (max, sum-exp) partial of the stored-score path
static constexpr int32_t STATS_CHUNK = 2048;

// The bf16 and FP8 stored-score pass 1 runs on the matrix cores for up to 64
// query rows (4 column tiles); wider cases and fp32 take the VALU kernel and
// the separate stats pass.
static bool stored_on_mfma(int32_t dtype, int32_t TG) {
  return (dtype == KVM_BF16 || dtype == KVM_FP8_E4M3) && TG <= 64;
}

// FP8 scores run only on the matrix cores with d = 128: the two-pass kernels
// (T*G >= 64, index in HBM) or the stored pass 1 (T*G <= 64, either location).
static bool fp8_supported(const Plan& p, int32_t D) {
  return p.mfma || (p.TG <= 64 && D == 128);
}

static Plan make_plan(const kvm_dims* d, int32_t dtype, int32_t T, int64_t N, int32_t loc,
                      int64_t tile_blocks) {
  Plan p{};
  const int32_t G = d->n_q_heads / d->n_kv_heads;
  const int32_t nlg = d->n_layers * d->n_kv_heads;
  p.TG = T * G;
  p.mfma = ((dtype == KVM_BF16 && (d->head_dim == 128 || d->head_dim == 64)) ||
            (dtype == KVM_FP8_E4M3 && d->head_dim == 128)) &&
           p.TG >= 64 && loc == KVM_INDEX_DEVICE;
  size_t off = 0;
  if (p.mfma) {
    p.row_chunks = (p.TG + 255) / 256;
    p.TGp = p.row_chunks * 256;
    // enough workgroups to fill 256 CUs several times over
    int32_t ns = 1;
    while ((int64_t)nlg * p.row_chunks * ns < 2048 && (int64_t)ns * 128 * 2 <= N) ns *= 2;
    p.nsplit = ns;
    p.split_blocks = (int32_t)(((N + ns - 1) / ns + 127) / 128 * 128);
    p.block_chunks = (int32_t)((N + 255) / 256);
    p.off_part = off;
    off = align256(off + (size_t)nlg * ns * p.TGp * sizeof(float2));
    p.off_lse = off;
    off = align256(off + (size_t)nlg * p.TGp * sizeof(float));
    p.off_rp = off;
    off = align256(off + (size_t)nlg * N * sizeof(float));
  } else {
    // (max, sum) partial granularity: bf16 pass 1 forms them per workgroup of
    // 512 rows (host tiles are multiples of 512, so the resident and the
    // host-tiled index give the same partials and bit-identical scores); the
    // other cases use the stats pass over the whole score array
    if (stored_on_mfma(dtype, p.TG)) {
      p.chunk = 512;
    } else {
      p.chunk = STATS_CHUNK;
    }
    p.chunks = (int32_t)((N + p.chunk - 1) / p.chunk);
    p.off_S = off;
    off = align256(off + (size_t)nlg * N * p.TG * sizeof(float));
    p.off_part = off;
    off = align256(off + (size_t)nlg * p.chunks * p.TG * sizeof(float2));
    p.off_lse = off;
    off = align256(off + (size_t)nlg * p.TG * sizeof(float));
    if (loc == KVM_INDEX_HOST_TILED) {
      p.off_stage = off;
      off = align256(off + 2 * (size_t)nlg * tile_blocks * d->head_dim * dtype_bytes(dtype));
    }
  }
  p.bytes = off;
  return p;
}

// Side stream and events of one host-tiled scoring call. Sets are kept per
// GPU and handed out one per call in progress (taken at the start of a call,
// returned once its work is queued: later calls queue behind it on the same
// side stream), so their number is bounded by the calls that overlap.
struct TiledRes {
  hipStream_t side = nullptr;
  hipEvent_t h2d[2] = {nullptr, nullptr};
  hipEvent_t used[2] = {nullptr, nullptr};
  int device = -1;
};
static std::mutex g_tiled_mu;
static std::vector<TiledRes*> g_tiled_free;

static int tiled_take(TiledRes** out) {
  int dev;
  KVM_HIP(hipGetDevice(&dev));
  {
    std::lock_guard<std::mutex> g(g_tiled_mu);
    for (size_t i = 0; i < g_tiled_free.size(); ++i)
      if (g_tiled_free[i]->device == dev) {
        *out = g_tiled_free[i];
        g_tiled_free.erase(g_tiled_free.begin() + (ptrdiff_t)i);
        return KVM_OK;
      }
  }
  std::unique_ptr<TiledRes> r(new TiledRes());
  auto undo = [&r] {
    for (int i = 0; i < 2; ++i) {
      if (r->h2d[i]) (void)hipEventDestroy(r->h2d[i]);
      if (r->used[i]) (void)hipEventDestroy(r->used[i]);
    }
    if (r->side) (void)hipStreamDestroy(r->side);
  };
  hipError_t e = hipStreamCreateWithFlags(&r->side, hipStreamNonBlocking);
  for (int i = 0; i < 2 && e == hipSuccess; ++i) {
    e = hipEventCreateWithFlags(&r->h2d[i], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&r->used[i], hipEventDisableTiming);
  }
  if (e != hipSuccess) {
    undo();
    set_error("host-tiled scoring resources: %s", hipGetErrorString(e));
    return KVM_EHIP;
  }
  r->device = dev;
  *out = r.release();
  return KVM_OK;
}

static void tiled_give_back(TiledRes* r) {
  std::lock_guard<std::mutex> g(g_tiled_mu);
  g_tiled_free.push_back(r);
}

template <typename T, int D>
static void launch_stored_pass1(const StoredArgs& a, hipStream_t s) {
  const int32_t chunks_here = (a.nb + 255) / 256;
  const size_t shm = ((size_t)a.TG * D + 8) * sizeof(float);
  KernelTimer tm("score_stored_pass1", s);
  score_stored_pass1<T, D><<<dim3((uint32_t)((int64_t)a.nlg * chunks_here)), dim3(256), shm, s>>>(a);
}

static void stored_pass1(int32_t dtype, int32_t D, const StoredArgs& a, hipStream_t s) {
  if (stored_on_mfma(dtype, a.TG)) {
    const int32_t chunks_here = (a.nb + a.chunk - 1) / a.chunk;
    const dim3 grid((uint32_t)((int64_t)a.nlg * chunks_here));
    KernelTimer tm("score_stored_pass1", s);
    const bool stage = a.TG <= 32;
    const size_t shm = stage ? (size_t)4 * 64 * a.TG * sizeof(float) : 0;
#define KVM_SP1(E, DD)                                                                     \
  do {                                                                                     \
    if (stage) score_stored_pass1_mfma<E, DD, true><<<grid, dim3(256), shm, s>>>(a);      \
    else score_stored_pass1_mfma<E, DD, false><<<grid, dim3(256), 0, s>>>(a);             \
  } while (0)
    if (dtype == KVM_FP8_E4M3) KVM_SP1(uint8_t, 128);
    else if (D == 128) KVM_SP1(uint16_t, 128);
    else KVM_SP1(uint16_t, 64);
#undef KVM_SP1
  } else if (dtype == KVM_BF16) {
    if (D == 128) launch_stored_pass1<uint16_t, 128>(a, s);
    else launch_stored_pass1<uint16_t, 64>(a, s);
  } else {
    if (D == 128) launch_stored_pass1<float, 128>(a, s);
    else launch_stored_pass1<float, 64>(a, s);
  }
}

}  // namespace kvm

static size_t kvm_score_ws_bytes_body(const kvm_dims* dims, int32_t dtype, int32_t n_q_tokens,
                                     int64_t n_blocks, int32_t index_loc, int64_t tile_blocks) {
  using namespace kvm;
  if (check_dims(dims, dtype) || n_q_tokens < 1 || n_blocks < 1) return 0;
  const Plan p = make_plan(dims, dtype, n_q_tokens, n_blocks, index_loc, tile_blocks);
  if (dtype == KVM_FP8_E4M3 && !fp8_supported(p, dims->head_dim)) return 0;
  return p.bytes;
}

extern "C" size_t kvm_score_ws_bytes(const kvm_dims* dims, int32_t dtype, int32_t n_q_tokens,
                                     int64_t n_blocks, int32_t index_loc, int64_t tile_blocks) {
  try {
    return kvm_score_ws_bytes_body(dims, dtype, n_q_tokens, n_blocks, index_loc, tile_blocks);
  } catch (...) {
    return 0;
  }
}

static int kvm_score_blocks_body(const kvm_dims* dims, int32_t dtype, const void* q,
                                int32_t n_q_tokens, const void* index, int64_t index_cap_blocks,
                                int64_t n_blocks, int32_t index_loc, int64_t tile_blocks,
                                float* scores, void* ws, size_t ws_bytes, void* stream) {
  using namespace kvm;
  clear_error();
  int rc = check_dims(dims, dtype);
  if (rc) return rc;
  KVM_CHECK_ARG(q && index && scores, "null pointer");
  KVM_CHECK_ARG(n_q_tokens >= 1 && n_blocks >= 1 && n_blocks < (1LL << 30),
                "n_q_tokens / n_blocks out of range");
  KVM_CHECK_ARG(index_loc == KVM_INDEX_DEVICE || index_loc == KVM_INDEX_HOST_TILED,
                "index_loc");
  const int32_t D = dims->head_dim;
  const int32_t G = dims->n_q_heads / dims->n_kv_heads;
  const int32_t nlg = dims->n_layers * dims->n_kv_heads;
  const int32_t TG = n_q_tokens * G;
  if (index_loc == KVM_INDEX_DEVICE)
    KVM_CHECK_ARG(n_blocks <= index_cap_blocks, "n_blocks > index_cap_blocks");
  if (index_loc == KVM_INDEX_HOST_TILED) {
    KVM_CHECK_ARG(tile_blocks >= 512 && tile_blocks % 512 == 0,
                  "tile_blocks must be a positive multiple of 512");
  }
  const Plan p = make_plan(dims, dtype, n_q_tokens, n_blocks, index_loc, tile_blocks);
  if (dtype == KVM_FP8_E4M3 && !fp8_supported(p, D)) {
    set_error("FP8 scores need d = 128 and either T*G <= 64 or an index in HBM");
    return KVM_ENOTSUP;
  }
  if (!p.mfma) {
    const size_t shm = ((size_t)TG * D + 8) * sizeof(float);
    const size_t shm2 = (size_t)nlg * TG * sizeof(float);
    if (shm > 64 * 1024 || shm2 > 64 * 1024) {
      set_error("T*G = %d (L*Hkv = %d) too large for the stored-score path", TG, nlg);
      return KVM_ENOTSUP;
    }
  }
  if (ws_bytes < p.bytes || !ws) {
    set_error("workspace %zu < %zu bytes", ws_bytes, p.bytes);
    return KVM_ENOMEM;
  }
  KVM_CHECK_ARG(((uintptr_t)q | (uintptr_t)index | (uintptr_t)ws) % 16 == 0,
                "q, index and ws must be 16-byte aligned");
  const size_t eb = (size_t)dtype_bytes(dtype);
  KVM_CHECK_RANGE(q, (size_t)dims->n_layers * dims->n_q_heads * n_q_tokens * D * eb,
                  RANGE_DEVICE, "q");
  if (index_loc == KVM_INDEX_DEVICE) {
    KVM_CHECK_RANGE(index, (size_t)nlg * index_cap_blocks * D * eb, RANGE_DEVICE, "index");
  } else {
    const size_t ntile = (size_t)((n_blocks + tile_blocks - 1) / tile_blocks);
    KVM_CHECK_RANGE(index, ntile * nlg * tile_blocks * D * eb, RANGE_PINNED_HOST,
                    "host-tiled index");
  }
  KVM_CHECK_RANGE(scores, (size_t)n_blocks * sizeof(float), RANGE_DEVICE, "scores");
  KVM_CHECK_RANGE(ws, p.bytes, RANGE_DEVICE, "ws");
  hipStream_t s = as_stream(stream);
  char* w = reinterpret_cast<char*>(ws);
  const float scale = LOG2E / sqrtf((float)D);
  const double inv_lh = 1.0 / ((double)dims->n_layers * dims->n_q_heads);
  if (p.mfma) {
    Pass1Args a1{};
    a1.q = q;
    a1.index = index;
    a1.cap = index_cap_blocks;
    a1.n_blocks = (int32_t)n_blocks;
    a1.T = n_q_tokens;
    a1.Hq = dims->n_q_heads;
    a1.Hkv = dims->n_kv_heads;
    a1.G = G;
    a1.TG = TG;
    a1.row_chunks = p.row_chunks;
    a1.nsplit = p.nsplit;
    a1.split_blocks = p.split_blocks;
    a1.scale = scale;
    a1.part = reinterpret_cast<float2*>(w + p.off_part);
    a1.TGp = p.TGp;
    a1.nlg = nlg;
    const int64_t wg1 = (int64_t)nlg * p.row_chunks * p.nsplit;
    a1.total_wg = (uint32_t)((wg1 + 7) / 8 * 8);
    { KernelTimer tm("score_pass1_mfma", s);
    if (dtype == KVM_FP8_E4M3)
      score_pass1_mfma<uint8_t, 128><<<dim3(a1.total_wg), dim3(256), 0, s>>>(a1);
    else if (D == 128)
      score_pass1_mfma<uint16_t, 128><<<dim3(a1.total_wg), dim3(256), 0, s>>>(a1);
    else
      score_pass1_mfma<uint16_t, 64><<<dim3(a1.total_wg), dim3(256), 0, s>>>(a1); }
    KVM_HIP(hipGetLastError());
    const int64_t nl = (int64_t)nlg * p.TGp;
    { KernelTimer tm("score_lse_combine", s);
    score_lse_combine<<<dim3((uint32_t)((nl + 255) / 256)), dim3(256), 0, s>>>(
        a1.part, nlg, p.nsplit, p.TGp, TG, reinterpret_cast<float*>(w + p.off_lse)); }
    KVM_HIP(hipGetLastError());
    Pass2Args a2{};
    a2.q = a1.q;
    a2.index = a1.index;
    a2.cap = index_cap_blocks;
    a2.n_blocks = (int32_t)n_blocks;
    a2.T = n_q_tokens;
    a2.Hq = dims->n_q_heads;
    a2.Hkv = dims->n_kv_heads;
    a2.G = G;
    a2.TG = TG;
    a2.TGp = p.TGp;
    a2.block_chunks = p.block_chunks;
    a2.scale = scale;
    a2.lse = reinterpret_cast<const float*>(w + p.off_lse);
    a2.rp = reinterpret_cast<float*>(w + p.off_rp);
    a2.nlg = nlg;
    const int64_t wg2 = (int64_t)nlg * p.block_chunks;
    a2.total_wg = (uint32_t)((wg2 + 7) / 8 * 8);
    { KernelTimer tm("score_pass2_mfma", s);
    if (dtype == KVM_FP8_E4M3)
      score_pass2_mfma<uint8_t, 128><<<dim3(a2.total_wg), dim3(256), 0, s>>>(a2);
    else if (D == 128)
      score_pass2_mfma<uint16_t, 128><<<dim3(a2.total_wg), dim3(256), 0, s>>>(a2);
    else
      score_pass2_mfma<uint16_t, 64><<<dim3(a2.total_wg), dim3(256), 0, s>>>(a2); }
    KVM_HIP(hipGetLastError());
    { KernelTimer tm("score_reduce", s);
    score_reduce<<<dim3((uint32_t)((n_blocks + 63) / 64)), dim3(256), 0, s>>>(
        a2.rp, nlg, (int32_t)n_blocks, inv_lh, scores); }
    KVM_HIP(hipGetLastError());
    return KVM_OK;
  }
  // Stored-score path.
  StoredArgs a{};
  a.q = q;
  a.n_blocks = (int32_t)n_blocks;
  a.T = n_q_tokens;
  a.Hq = dims->n_q_heads;
  a.Hkv = dims->n_kv_heads;
  a.G = G;
  a.TG = TG;
  a.nlg = nlg;
  a.chunks_total = p.chunks;
  a.chunk = p.chunk;
  a.scale = scale;
  a.S = reinterpret_cast<float*>(w + p.off_S);
  a.part = reinterpret_cast<float2*>(w + p.off_part);
  if (index_loc == KVM_INDEX_DEVICE) {
    a.index = index;
    a.lg_stride = index_cap_blocks * D;
    a.b_first = 0;
    a.nb = (int32_t)n_blocks;
    stored_pass1(dtype, D, a, s);
    KVM_HIP(hipGetLastError());
  } else {
    TiledRes* tr = nullptr;
    KVM_TRY(tiled_take(&tr));
    struct GiveBack {
      TiledRes* r;
      ~GiveBack() { tiled_give_back(r); }
    } give_back{tr};
    const int64_t ntile = (n_blocks + tile_blocks - 1) / tile_blocks;
    const size_t tile_bytes = (size_t)nlg * tile_blocks * D * dtype_bytes(dtype);
    char* stage[2] = {w + p.off_stage, w + p.off_stage + tile_bytes};
    // The side stream starts after the caller's earlier work.
    KVM_HIP(hipEventRecord(tr->used[0], s));
    KVM_HIP(hipStreamWaitEvent(tr->side, tr->used[0], 0));
    KVM_HIP(hipEventRecord(tr->used[1], s));
    for (int64_t t = 0; t < ntile; ++t) {
      const int bi = (int)(t & 1);
      // staging buffer bi is free once the kernel that read it (tile t-2) ran
      KVM_HIP(hipStreamWaitEvent(tr->side, tr->used[bi], 0));
      KVM_HIP(hipMemcpyAsync(stage[bi], (const char*)index + (size_t)t * tile_bytes, tile_bytes,
                             hipMemcpyHostToDevice, tr->side));
      KVM_HIP(hipEventRecord(tr->h2d[bi], tr->side));
      KVM_HIP(hipStreamWaitEvent(s, tr->h2d[bi], 0));
      a.index = stage[bi];
      a.lg_stride = tile_blocks * D;
      a.b_first = (int32_t)(t * tile_blocks);
      a.nb = (int32_t)std::min<int64_t>(tile_blocks, n_blocks - t * tile_blocks);
      stored_pass1(dtype, D, a, s);
      KVM_HIP(hipGetLastError());
      KVM_HIP(hipEventRecord(tr->used[bi], s));
    }
  }
  if (!stored_on_mfma(dtype, TG)) {            // else pass 1 wrote the partials itself
    KernelTimer tm("score_stored_stats", s);
    score_stored_stats<<<dim3((uint32_t)((int64_t)nlg * p.chunks)), dim3(256), 0, s>>>(
        a.S, (int32_t)n_blocks, TG, p.chunk, p.chunks, a.part);
    KVM_HIP(hipGetLastError());
  }
  const int64_t nl = (int64_t)nlg * TG;
  { KernelTimer tm("score_stored_lse", s);
  score_stored_lse<<<dim3((uint32_t)nl), dim3(64), 0, s>>>(
      a.part, nlg, p.chunks, TG, reinterpret_cast<float*>(w + p.off_lse)); }
  KVM_HIP(hipGetLastError());
  const size_t shm2 = (size_t)nlg * TG * sizeof(float);
  { KernelTimer tm("score_stored_pass2", s);
  const dim3 g2((uint32_t)((n_blocks + 255) / 256));
  const float* lse = reinterpret_cast<const float*>(w + p.off_lse);
#define KVM_P2(C)                                                                       \
  score_stored_pass2<C><<<g2, dim3(256), shm2, s>>>(a.S, lse, nlg, TG, (int32_t)n_blocks, \
                                                    inv_lh, scores)
  switch (TG) {
    case 1: KVM_P2(1); break;
    case 2: KVM_P2(2); break;
    case 3: KVM_P2(3); break;
    case 4: KVM_P2(4); break;
    case 5: KVM_P2(5); break;
    case 6: KVM_P2(6); break;
    case 7: KVM_P2(7); break;
    case 8: KVM_P2(8); break;
    default: KVM_P2(0); break;
  }
#undef KVM_P2
  }
  KVM_HIP(hipGetLastError());
  return KVM_OK;
}

extern "C" int kvm_score_blocks(const kvm_dims* dims, int32_t dtype, const void* q,
                                int32_t n_q_tokens, const void* index, int64_t index_cap_blocks,
                                int64_t n_blocks, int32_t index_loc, int64_t tile_blocks,
                                float* scores, void* ws, size_t ws_bytes, void* stream) {
  return kvm::guarded([&] {
    return kvm_score_blocks_body(dims, dtype, q, n_q_tokens, index, index_cap_blocks, n_blocks,
                                 index_loc, tile_blocks, scores, ws, ws_bytes, stream);
  });
}
