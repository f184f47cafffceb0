/*
 * kvm.h - C ABI of libkvm: the per-step working-set update of attention-space
 * block retrieval (KVMem, "Virtualizing Million-Token Agent Workspaces on a
 * Consumer GPU"), for AMD Instinct MI355X (gfx950).
 *
 * Four calls make one agent step (KVMem Sec. 4.2: one update after prefill,
 * before decode):
 *   kvm_build_index    Mean-K index rows of completed blocks       (Sec. 4.3, Sec. 5)
 *   kvm_score_blocks   block relevance R_b, Eq. (10)                (Sec. 4.3, Sec. 5)
 *   kvm_select         sink + recent + top-k, chronological order    (Sec. 4.3)
 *   kvm_rematerialize  delta plan, H2D of misses, re-RoPE K, copy V  (Sec. 4.4, Fig. 3)
 *
 * Conventions shared by every entry point
 *  - Plain pointers and sizes only. "device" pointers are HIP device memory of
 *    the current device; "pinned host" pointers come from hipHostMalloc (or an
 *    equivalent page-locked allocation).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). All
 *    device work is enqueued on it; calls return once the work is enqueued.
 *    No entry point synchronises the device; only kvm_rematerialize waits for
 *    `stream` (to read the selection) and kvm_ctx_sync waits for ctx work.
 *  - kvm_build_index, kvm_score_blocks with KVM_INDEX_DEVICE, kvm_select and
 *    kvm_select_noalloc enqueue kernels only (no allocation, copy, memset or
 *    wait), so a caller may capture them into a HIP graph and replay it.
 *  - The caller owns every buffer it passes (inputs, outputs, workspaces,
 *    pools). The library never frees caller memory and allocates device memory
 *    only inside kvm_ctx_create.
 *  - Return value: KVM_OK or a negative kvm_status. Argument validation is
 *    synchronous and leaves outputs untouched. HIP errors return KVM_EHIP;
 *    the text is in kvm_last_error() (thread-local). No C++ exception crosses
 *    this interface: every entry point catches them; host allocation and
 *    thread-creation failures return KVM_ENOMEM, anything else KVM_EINTERNAL.
 *  - Element types: KVM_F32 (IEEE binary32), KVM_BF16 (bfloat16 bit patterns)
 *    or KVM_FP8_E4M3 (OCP FP8 E4M3FN bytes: bias 7, 3 mantissa bits, largest
 *    finite 448, no infinities; the KV-cache format the pages' engine runs).
 *    With FP8 K/V the Mean-K index and the queries are bf16, so scoring takes
 *    KVM_BF16; re-RoPE decodes FP8 exactly, rotates in fp32 and re-encodes
 *    (nearest, ties to even, saturating at +-448); V is copied byte for byte.
 *    Supported head_dim: 64 and 128; block_tokens: 32.
 */
#ifndef KVM_H
#define KVM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVM_OK = 0,
  KVM_EINVAL = -1,  /* bad shape, pointer, alignment or enum value; also a
                       pointer argument whose byte range is not inside one
                       allocation made through HIP (device, managed or pinned
                       host memory), or device memory where pinned host
                       memory is required, checked before any work is queued
                       (allocators that sub-allocate are checked against their
                       segment; memory without a reported range, such as
                       virtual-memory mappings, skips the extent check) */
  KVM_ENOMEM = -2,  /* workspace, pool or record capacity too small */
  KVM_EHIP = -3,    /* a HIP runtime call failed; see kvm_last_error() */
  KVM_ERANGE = -4,  /* budget < sink + recent, block id out of range, block
                       without a source, NaN or negative score */
  KVM_ENOTSUP = -5, /* valid but unsupported combination (dtype, head_dim) */
  KVM_EINTERNAL = -6 /* unexpected host-side failure inside the library (an
                        exception other than memory or thread exhaustion,
                        which are KVM_ENOMEM); see kvm_last_error() */
} kvm_status;

typedef enum { KVM_F32 = 0, KVM_BF16 = 1, KVM_FP8_E4M3 = 2 } kvm_dtype;

/* Where kvm_score_blocks finds the index. */
typedef enum { KVM_INDEX_DEVICE = 0, KVM_INDEX_HOST_TILED = 1 } kvm_index_loc;

/* Where a block's lower-tier raw K/V copy lives (KVMem Sec. 5 block records). */
typedef enum { KVM_SRC_NONE = 0, KVM_SRC_HOST_PINNED = 1, KVM_SRC_DEVICE = 2 } kvm_src_loc;

typedef struct {
  int32_t n_layers;     /* L: scored attention layers */
  int32_t n_kv_heads;   /* Hkv */
  int32_t n_q_heads;    /* Hq, a multiple of Hkv; query head h uses KV head h / (Hq/Hkv) */
  int32_t head_dim;     /* d */
  int32_t block_tokens; /* B: tokens per logical block (32) */
} kvm_dims;

/* Version of this interface (major*100 + minor): 104. */
int kvm_version(void);

/* Text of the last error on the calling thread ("" if none). */
const char* kvm_last_error(void);

/* ------------------------------------------------------------------------ */
/* Mean-K index build / append.
 * KVMem Sec. 4.3: a block is represented, per layer and KV head, by the mean of
 * its position-independent (pre-RoPE) K vectors; Sec. 5: each completed block
 * is indexed while its K is still on the GPU, so appending is the same call.
 *
 * k_raw   device, block-major raw K: block i at (char*)k_raw + i*k_block_stride,
 *         each block [L][Hkv][B][d] contiguous in `dtype`.
 * index   device, [L][Hkv][index_cap_blocks][d] in `dtype` (bf16 for
 *         KVM_FP8_E4M3 K); the call writes rows [first_block, first_block +
 *         n_blocks) of every (l, g) and nothing else.
 * Result: index[l][g][first_block+i][t] = round(mean_j k_raw[i][l][g][j][t]),
 *         the sum formed exactly (float64; fp32 for FP8 K, whose 32 values sum
 *         exactly there) and rounded once to nearest-even, so the stored mean
 *         is the correctly rounded block mean.
 * Errors: KVM_EINVAL (null pointer, n_blocks < 0, stride smaller than a block,
 *         first_block + n_blocks > index_cap_blocks), KVM_ENOTSUP (head_dim,
 *         block_tokens). n_blocks == 0 is a no-op. */
int kvm_build_index(const kvm_dims* dims, int32_t dtype, const void* k_raw,
                    int64_t k_block_stride, int64_t first_block, int64_t n_blocks,
                    void* index, int64_t index_cap_blocks, void* stream);

/* ------------------------------------------------------------------------ */
/* Block relevance, KVMem Sec. 4.3 Eq. (10) (tiled form: Sec. 5):
 *   R_b = 1/(L*Hq) * sum_l sum_h sum_m softmax_b( q[l][h][m] . kbar[l][g(h)][b] / sqrt(d) )
 * with the softmax over all n_blocks indexed blocks for each fixed (l, m, h)
 * and g(h) = h / (Hq/Hkv). sum_b R_b = n_q_tokens.
 *
 * q       device, pre-RoPE queries [L][Hq][n_q_tokens][d] in `dtype`.
 *         dtype KVM_FP8_E4M3 scores E4M3 queries against an E4M3 index (the
 *         FP8 scoring ablation; both from kvm_quantize_e4m3): the products are
 *         exact and the sums and softmax run in fp32/fp64 as for bf16. It
 *         runs on the matrix cores only and needs d = 128 and either
 *         T*G <= 64 (stored-score form, device or host-tiled index) or a
 *         device index, else KVM_ENOTSUP (and kvm_score_ws_bytes returns 0).
 * index   KVM_INDEX_DEVICE: device [L][Hkv][index_cap_blocks][d];
 *         KVM_INDEX_HOST_TILED: pinned host, tile-major, tile_blocks a
 *         positive multiple of 512: tile t (blocks
 *         [t*tile_blocks, (t+1)*tile_blocks)) is [L][Hkv][tile_blocks][d] at
 *         element offset t*L*Hkv*tile_blocks*d (the last tile is full-sized,
 *         rows past n_blocks are ignored). Tiles are streamed through two device
 *         staging buffers in `ws`; the softmax normalisation is global and the
 *         partial sums are grouped the same way, so the result is bit-identical
 *         to the resident form.
 * scores  device float[n_blocks] (R_b).
 * ws      device workspace of at least kvm_score_ws_bytes(...) bytes.
 * Forms: bf16 (d = 64 or 128) and FP8 (d = 128) with T*G >= 64 and the index
 *         in HBM run two matrix-core passes over the index; every other case stores the scores
 *         in `ws` in one pass over the index (matrix cores for bf16 and FP8 with
 *         T*G <= 64, vector units otherwise). The vector form needs
 *         (T*G*d + 8)*4 <= 65536 and L*Hkv*T*G*4 <= 65536 bytes (shared memory),
 *         else KVM_ENOTSUP: e.g. fp32, or a host-tiled index, with T*G up to 255 at
 *         d = 64.
 * Errors: KVM_EINVAL (shapes, null pointers, n_blocks < 1, n_q_tokens < 1),
 *         KVM_ENOMEM (ws_bytes too small), KVM_ENOTSUP (dtype/head_dim, or the
 *         T*G limits above). */
size_t kvm_score_ws_bytes(const kvm_dims* dims, int32_t dtype, int32_t n_q_tokens,
                          int64_t n_blocks, int32_t index_loc, int64_t tile_blocks);

int kvm_score_blocks(const kvm_dims* dims, int32_t dtype, const void* q, int32_t n_q_tokens,
                     const void* index, int64_t index_cap_blocks, int64_t n_blocks,
                     int32_t index_loc, int64_t tile_blocks, float* scores, void* ws,
                     size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* FP8 E4M3 (OCP E4M3FN) conversion for the FP8 scoring ablation (the pages'
 * engine runs an FP8 KV cache, KVMem Sec. 6.1): dst[i] = the E4M3 byte nearest
 * to src[i], ties to even, saturating at +-448 (infinities too), the sign kept
 * on zero; NaN inputs give an unspecified byte.
 * src       device, n values of src_dtype (KVM_F32 or KVM_BF16).
 * dst       device, n bytes, 4-byte aligned; caller-owned.
 * Errors: KVM_EINVAL (null pointer, dtype, n < 1, alignment). */
int kvm_quantize_e4m3(const void* src, int32_t src_dtype, int64_t n, void* dst, void* stream);

/* ------------------------------------------------------------------------ */
/* Default selector and compact positions, KVMem Sec. 4.3 (sink and recent
 * regions always kept, the rest of the budget to the largest R_b, then
 * chronological order) and Sec. 4.4 / Sec. 5 (contiguous compact positions).
 *
 * scores    device float[n_blocks], finite and >= 0.
 * sel       device int32[budget_blocks]: ascending block ids; the first *n_sel
 *           entries are valid.
 * n_sel     device int32[1]: min(n_blocks, budget_blocks), or KVM_ERANGE (-4)
 *           if a score is NaN or negative (detected on the device; sel is then
 *           unspecified and kvm_rematerialize reports KVM_ERANGE).
 * base_pos  device int32[budget_blocks]: base_pos[i] = i * block_tokens.
 * Selection: blocks [0, n_sink) and [n_blocks - n_recent, n_blocks) always;
 *           k = budget - n_sink - n_recent more from the rest by descending
 *           score, exact ties to the lower block id; every block when
 *           n_blocks <= budget_blocks.
 * ws        device workspace of at least kvm_select_ws_bytes(n_blocks) bytes.
 * Errors: KVM_ERANGE (n_sink + n_recent > budget_blocks), KVM_EINVAL (null
 * pointers, n_blocks < 1, budget_blocks < 1), KVM_ENOMEM. */
size_t kvm_select_ws_bytes(int64_t n_blocks);

int kvm_select(const float* scores, int64_t n_blocks, int32_t n_sink, int32_t n_recent,
               int32_t budget_blocks, int32_t block_tokens, int32_t* sel, int32_t* n_sel,
               int32_t* base_pos, void* ws, size_t ws_bytes, void* stream);

/* kvm_select without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation). Same arguments, results and errors as kvm_select,
 * minus ws/ws_bytes: the selection's scratch (control words, digit
 * histograms, per-chunk counts) is a fixed array of
 * KVM_SELECT_NOALLOC_SCRATCH_BYTES in the library's device code, one per GPU,
 * held until the process ends, so n_blocks is limited to
 * KVM_SELECT_NOALLOC_MAX_BLOCKS (larger: KVM_ENOMEM, nothing enqueued). The
 * call allocates nothing. Every call on one GPU shares that GPU's array (the
 * kernels reset what must start at zero): calls that overlap on one GPU, on
 * different streams or threads, race and give undefined selections; order
 * them on one stream. Not timed by kvm_profile_*. */
#define KVM_SELECT_NOALLOC_SCRATCH_BYTES 65536
#define KVM_SELECT_NOALLOC_MAX_BLOCKS 31326208LL   /* 7648 chunks of 4096 blocks */

int kvm_select_noalloc(const float* scores, int64_t n_blocks, int32_t n_sink,
                       int32_t n_recent, int32_t budget_blocks, int32_t block_tokens,
                       int32_t* sel, int32_t* n_sel, int32_t* base_pos, void* stream);

/* ------------------------------------------------------------------------ */
/* Working-set context: block records, the bounded GPU page pool and the
 * rematerialization data plane (KVMem Sec. 4.4, Sec. 5, Fig. 3).
 *
 * Pool (caller-owned device memory, n_slots pages each [L][Hkv][B][d] in dtype):
 *   k_view    K encoded at the block's current compact position (what attention reads)
 *   v_view    V, a verbatim copy of the block's raw V
 *   k_shadow  the block's raw pre-RoPE K when its lower-tier copy is not in
 *             device memory (the re-encode source for hits whose compact
 *             position changes); blocks with a KVM_SRC_DEVICE copy are
 *             re-encoded from that copy instead. Unused with delta_limit > 0.
 * The ctx owns only host-side state, a side stream, events, a pinned staging
 * ring, a small device job list and the RoPE cos/sin table (fp64 angles,
 * rounded to fp32; positions [0, max_pos)). */
typedef struct {
  kvm_dims dims;
  int32_t dtype;
  int32_t rope_layout;    /* 0: pairs (2t, 2t+1); 1: pairs (t, t + d/2) */
  double rope_theta;      /* base of theta_t = base^(-2t/d), e.g. 10000 */
  int32_t max_pos;        /* compact positions must stay below this */
  int32_t n_slots;        /* pool pages */
  void* k_view;
  void* v_view;
  void* k_shadow;
  int64_t max_blocks;     /* block-record capacity (block ids < max_blocks) */
  int32_t batch_blocks;   /* misses per H2D batch / event (default 64 if <= 0) */
  int32_t staging_blocks; /* pinned ring capacity in blocks for gathered sources (>= 2*batch) */
  int32_t delta_limit;    /* 0: every re-encode reads raw K (k_shadow required).
                             n > 0: bounded delta re-RoPE (KVMem Sec. 4.4): a resident
                             block whose compact position changes has its K page
                             rotated in place by the shift, at most n times in a row;
                             the next change rebuilds K from the block's raw K (its
                             lower-tier copy, which must then exist) and resets the
                             count. k_shadow is unused and may be NULL; staged raw K
                             lands in the K page and is rotated there. */
} kvm_ctx_desc;

typedef struct kvm_ctx kvm_ctx;

typedef struct {
  int32_t n_sel;        /* blocks in the new execution view */
  int32_t hits;         /* selected blocks already resident in the pool */
  int32_t misses;       /* selected blocks staged in this call */
  int32_t rotated;      /* blocks whose K was (re)encoded this call */
  int32_t evicted;      /* resident blocks whose page was reclaimed */
  int32_t batches;      /* H2D batches (events) issued */
  int64_t h2d_bytes;    /* bytes copied host -> device */
  int64_t d2d_bytes;    /* bytes read + written by the remat kernels */
  int32_t deltas;       /* delta-mode rotations in place by a position shift */
  int32_t rebuilds;     /* delta-mode re-encodes from raw K after the limit */
} kvm_remat_stats;

/* Host-gather callback for lower tiers that are not pinned (pageable or
 * procedural stores): write block `block`'s raw K (which=0) or V (which=1),
 * [L][Hkv][B][d] in dtype, to `dst` (pinned). Return 0 on success. Called from
 * library worker threads, possibly concurrently for different blocks. */
typedef int (*kvm_gather_fn)(void* user, int64_t block, int32_t which, void* dst);

int kvm_ctx_create(const kvm_ctx_desc* desc, kvm_ctx** out);
void kvm_ctx_destroy(kvm_ctx* ctx);

/* Record the lower-tier copy of blocks [first_block, first_block + n_blocks):
 * block first_block+i has raw K at (char*)k_base + i*block_stride and raw V at
 * (char*)v_base + i*block_stride, in pinned host memory (KVM_SRC_HOST_PINNED,
 * staged by DMA straight into the destination page) or device memory
 * (KVM_SRC_DEVICE, read by the remat kernel directly, also for later
 * re-encodes while the block stays resident: the memory must stay valid until
 * the block's source is changed or the ctx is destroyed). Changing the source
 * of a resident block that relies on its device copy reclaims its page. */
int kvm_ctx_set_source(kvm_ctx* ctx, int64_t first_block, int64_t n_blocks, const void* k_base,
                       const void* v_base, int64_t block_stride, int32_t loc);

/* Record blocks [first_block, first_block + n_blocks) as served by a host
 * gather callback (packed through the pinned staging ring, KVMem Sec. 4.4). */
int kvm_ctx_set_gather(kvm_ctx* ctx, int64_t first_block, int64_t n_blocks, kvm_gather_fn fn,
                       void* user);

/* Register freshly prefilled blocks as GPU-resident (KVMem Sec. 5: new blocks
 * start in their original frame; here their K page is marked stale so the next
 * selection encodes it). Copies raw K and V (device, block stride as above)
 * into pool pages on `stream`: a free page, else the page of the least recently
 * used resident block outside the current view (the last selection and the
 * blocks registered since), ties to the lower block id; a page of the current
 * view is never taken. All or nothing: KVM_ENOMEM, with nothing changed, when
 * the blocks do not fit. A block already resident is refreshed in its page.
 * If a copy cannot be queued, the call's blocks lose their pages (KVM_EHIP). */
int kvm_ctx_register_resident(kvm_ctx* ctx, int64_t first_block, int64_t n_blocks,
                              const void* k_raw, const void* v_raw, int64_t block_stride,
                              void* stream);

/* The same for a set of blocks that need not be consecutive (KVMem Sec. 4.4:
 * blocks staged back into the GPU tier, or prefilled blocks of several
 * chunks): blocks (host int64[n_blocks], strictly ascending, each below
 * max_blocks) name the blocks; the raw K and V of blocks[i] sit at
 * k_raw / v_raw + i * block_stride (device). Same page rule, all or nothing.
 * Both registration calls copy with one kernel launch per 448 blocks when
 * k_raw, v_raw and block_stride are multiples of 16 bytes (else one copy per
 * page). Errors: KVM_EINVAL (a list entry out of range or not ascending,
 * block_stride below the page size, or sources that are not device memory of
 * the needed size), KVM_ENOMEM and KVM_EHIP as above. */
int kvm_ctx_register_resident_list(kvm_ctx* ctx, const int64_t* blocks, int64_t n_blocks,
                                   const void* k_raw, const void* v_raw, int64_t block_stride,
                                   void* stream);

/* Mean-K index rows from K that already carries RoPE (KVMem Sec. 5: during
 * prefill RoPE is removed from the K of completed blocks and their Mean-K is
 * formed while that K is still on the GPU). k_rope: device, block-major
 * [n_blocks][L][Hkv][B][d] in the ctx dtype, consecutive blocks `block_stride`
 * bytes apart; token j of block i sits at original position
 * pos0 + B*i + j. Each token is rotated back by R_{-p} with the (cos, sin) of
 * the ctx's table (fp32 values of the float64 functions at float64 angles,
 * the same layout and base as re-RoPE), in float64; the block mean is rounded
 * once (round-to-nearest-even) into index rows [first_block, first_block +
 * n_blocks) of the index [L][Hkv][index_cap_blocks][d]. Enqueued on `stream`.
 * Errors: KVM_EINVAL (pointers, alignment, stride, capacity), KVM_ERANGE
 * (positions beyond the ctx's max_pos or pos0 < 0). */
int kvm_ctx_build_index_rope(kvm_ctx* ctx, const void* k_rope, int64_t block_stride,
                             int64_t first_block, int64_t n_blocks, int64_t pos0, void* index,
                             int64_t index_cap_blocks, void* stream);

/* Make the execution view for a selection (KVMem Sec. 4.4, Sec. 5, Fig. 3):
 * reads n_sel/sel from the device (one small copy, then waits for `stream`),
 * plans hits / misses / evictions against the pool (a miss takes a free page,
 * else the page of the least recently used resident block outside the new
 * view, ties to the lower block id), stages misses H2D on the side streams in
 * event-tracked batches, and enqueues on `stream` the kernels that write
 * k_view = RoPE(raw K, compact position) for misses and for hits whose
 * position changed, and v_view = raw V for misses. page_table_dev (device
 * int32[n_sel]) receives the pool page of sel[i]. Selected block i occupies
 * positions [i*B, i*B + B). Returns once everything is enqueued; later work on
 * `stream` sees the finished view. n_sel = 0 is an empty view: nothing is
 * staged or launched and resident pages stay. stats_host may be NULL.
 * Errors: KVM_ERANGE (selection invalid, a miss without a source, or a gather
 * callback that failed; n_sel reported as KVM_ERANGE by kvm_select), KVM_ENOMEM
 * (pool smaller than the view), KVM_EHIP, KVM_EINTERNAL. An error after
 * planning drains the ctx's streams and `stream` and rolls the block records
 * back: every resident block then holds what its record says (blocks whose
 * pages were not completed are no longer resident), and a retry with the same
 * selection stages only what is missing. */
int kvm_rematerialize(kvm_ctx* ctx, const int32_t* sel_dev, const int32_t* n_sel_dev,
                      int32_t* page_table_dev, kvm_remat_stats* stats_host, void* stream);

/* Wait for the ctx's side-stream work (H2D batches). */
int kvm_ctx_sync(kvm_ctx* ctx);

/* Debug aid (race detection). With on != 0, later kvm_rematerialize calls
 * issue every host-to-device copy on the caller's stream, in issue order,
 * instead of the two side streams, so no copy runs alongside a kernel (each
 * copy is issued before the wait and the kernel that consume it, so the
 * order stays valid). The view, page table and stats must come out identical
 * to the overlapped mode's: a difference points at a missing wait. Slower
 * (no H2D/compute overlap). The call first waits for the ctx's side streams.
 * Errors: KVM_EINVAL (ctx NULL), KVM_EHIP. */
int kvm_ctx_set_serialized(kvm_ctx* ctx, int32_t on);

/* Inspection: pool page of `block` (or -1) and its baked compact position
 * (-1 = K page stale). */
int kvm_ctx_block_state(kvm_ctx* ctx, int64_t block, int32_t* slot, int32_t* baked_pos);

/* Inspection (delta mode): delta rotations applied to `block`'s K page since
 * it was last encoded from raw K (0 when not resident). */
int kvm_ctx_block_deltas(kvm_ctx* ctx, int64_t block, int32_t* n_delta);

/* Reclaim the pool pages of resident blocks [first_block, first_block + n_blocks)
 * (KVMem Sec. 4.4: a page can be reclaimed at once because the block keeps a
 * valid lower-tier copy; the block becomes a miss for later selections).
 * Blocks that are not resident are skipped. Host-side bookkeeping only. */
int kvm_ctx_evict(kvm_ctx* ctx, int64_t first_block, int64_t n_blocks);

/* ------------------------------------------------------------------------ */
/* Host-tier admission (KVMem Sec. 4.4, hierarchical reuse): replay a trace of
 * agent steps against a bounded host tier and count where GPU misses come
 * from. Host memory only, no device work.
 *
 * Policies: KVM_TIER_LRU (evict the least recently touched block) and
 * KVM_TIER_LRFU (recency and cumulative frequency: a block touched at
 * t_1 < ... < t_k is worth sum_i 2^(-lambda (t - t_i)); evict the least
 * worth; lambda = 0 is LFU, lambda = 1 orders like LRU). Ties evict the lowest
 * block id.
 * Trace (three CSR lists over n_steps steps; offsets int64[n_steps + 1]
 * starting at 0, each step a strictly ascending list of block ids >= 0):
 *   new:  blocks prefilled at the step, staged out to the host (admitted);
 *   sel:  the step's selection (every block touched once per step);
 *   miss: selected blocks the GPU pool lacked (must be in sel): a host copy
 *         is a host hit, else an NVMe read that admits the block.
 * Admission into a full host tier first demotes the block with the lowest
 * worth to NVMe. out: int32[n_steps][3] = host hits, NVMe reads, demotions.
 * Errors: KVM_EINVAL (pointers, policy, capacity < 1, lambda < 0, malformed
 * lists, a miss outside its selection). */
enum { KVM_TIER_LRU = 0, KVM_TIER_LRFU = 1 };
typedef struct {
  int32_t policy;
  int32_t host_blocks;   /* host-tier capacity in blocks */
  double lambda;         /* LRFU decay per step */
} kvm_tier_policy;

int kvm_tier_simulate(const kvm_tier_policy* policy, int32_t n_steps, const int64_t* new_off,
                      const int32_t* new_blk, const int64_t* sel_off, const int32_t* sel_blk,
                      const int64_t* miss_off, const int32_t* miss_blk, int32_t* out);

/* ------------------------------------------------------------------------ */
/* Measured rates (measurement aid; not on the hot path). Runs one untimed and
 * one timed kernel on `stream`, waits for them and returns in *rate:
 *  KVM_RATE_COPY       bytes read + written per second by a STREAM-style copy
 *                      of n bytes from scratch to scratch + n (n a multiple of
 *                      16, scratch >= 2n bytes, device, 16-byte aligned): one
 *                      16-byte word per thread, one-wave workgroups,
 *                      non-temporal loads and stores;
 *  KVM_RATE_MFMA_BF16  bf16 matrix flop/s of a register-only
 *                      v_mfma_f32_32x32x16_bf16 loop, n iterations of two
 *                      MFMAs per wave (8 waves per SIMD);
 *  KVM_RATE_EXP        v_exp_f32 results per second, n iterations of eight;
 *  KVM_RATE_SCORE_MIX  score elements per second of the score passes'
 *                      instruction mix (per MFMA: two fused scale-and-shifts,
 *                      two exps, two adds; 128 elements per MFMA and wave; two
 *                      waves per SIMD), n iterations of two such slots.
 * The ALU kinds write one float per thread to scratch (>= 2 MiB). Errors:
 * KVM_EINVAL, KVM_EHIP. The figures bound what the score passes (MFMA and
 * VALU), Mean-K build and rematerialization (HBM) can reach on this GPU. */
enum { KVM_RATE_COPY = 0, KVM_RATE_MFMA_BF16 = 1, KVM_RATE_EXP = 2, KVM_RATE_SCORE_MIX = 3 };

int kvm_measure_rate(int32_t kind, int64_t n, void* scratch, size_t scratch_bytes, double* rate,
                     void* stream);

/* ------------------------------------------------------------------------ */
/* Kernel timing (tracing aid). While enabled, every kernel launch of the
 * library is bracketed by a HIP event pair on its stream. kvm_profile_read
 * waits for the recorded events and returns, per kernel name, the number of
 * launches and their summed duration since profiling was (re)enabled; *n is
 * the number of distinct kernels (entries beyond `max` are not written). */
typedef struct {
  char name[48];
  int64_t launches;
  double total_ms;
} kvm_kernel_stat;

int kvm_profile_enable(int32_t on);
int kvm_profile_read(kvm_kernel_stat* out, int32_t max, int32_t* n);

#ifdef __cplusplus
}
#endif

#endif /* KVM_H */
