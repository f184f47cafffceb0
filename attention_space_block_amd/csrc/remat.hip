// Rematerialization data plane (KVMem Sec. 4.4 and Fig. 3; Sec. 5 block
// records and delta plans).
//
// Device side: one fused streaming kernel. Each job names a pool page (slot),
// the block's new compact base position and where its raw K (and V) come
// from. The kernel reads raw K, rotates every (x_a, x_b) pair by the angle
// p * theta_t with cos/sin from a precomputed fp32 table (angles formed in
// float64 on the host), and writes bf16/fp32 K (one round-to-nearest-even)
// into the page's K view; for device-resident sources it also copies V
// verbatim. Pages are contiguous [L][Hkv][B][d] spans, so every job is a long
// coalesced stream: HBM-bound, 2 x page bytes per rotated block (plus 2 x page
// bytes when V is copied). Raw K is read where it already sits in HBM: the
// page's shadow (filled by DMA, gather or registration) or the block's
// device-resident lower-tier copy.
//
// Host side: the planner turns a selection into hits, misses and evictions
// over the bounded page pool (LRU among pages outside the new view), stages
// misses from pinned host memory with DMA straight into their pages on a side
// stream (batches tracked by events; the caller's stream waits per batch and
// rotates that batch while the next one transfers), or through a pinned,
// double-buffered staging ring filled by host gather workers.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <condition_variable>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

#include "common.hpp"
#include "profile.hpp"

namespace kvm {

struct RematJob {
  const char* src_k;  // raw pre-RoPE K of the block (device)
  const char* src_v;  // raw V (device) when flags & JOB_COPY_V
  int32_t slot;
  int32_t pos;        // compact position of token 0 of the block
  int32_t flags;
  int32_t pad;
};
// JOB_DELTA: rotate every token by the same signed shift `pos` (an in-place
// delta re-RoPE) instead of by its absolute position pos + j. JOB_K_ONLY is
// host-side only: a staged rebuild that moves raw K but keeps the V page.
enum { JOB_COPY_V = 2, JOB_DELTA = 4, JOB_K_ONLY = 8 };

// (l, g) units of 32 token rows handled by one workgroup
static constexpr int REMAT_UNITS = 8;
// Units per workgroup scale inversely with the element size, so a thread holds
// the same bytes of rows in every dtype: FP8 rows are half as long (16 units;
// a thread's (cos, sin) pairs then serve as many bytes as in bf16), fp32 rows
// twice as long (4 units; 8 would take all 256 registers, one wave per SIMD)
static constexpr int REMAT_UNITS_FP8 = 16;
static constexpr int REMAT_UNITS_F32 = 4;
static constexpr int remat_units(int elem_bytes) {
  return elem_bytes == 1 ? REMAT_UNITS_FP8 : elem_bytes == 4 ? REMAT_UNITS_F32 : REMAT_UNITS;
}

struct RematArgs {
  const RematJob* jobs;
  int32_t n_jobs;
  int32_t wg_per_job;        // ceil(L * Hkv / units) workgroups per block
  int32_t rows_per_page;     // L * Hkv * B
  int64_t page_bytes;
  char* k_view;
  char* v_view;
  char* k_shadow;
  const float2* table;       // [max_pos][d/2] (cos, sin)
};

template <typename T>
__device__ __forceinline__ void unpack(const uint4& v, float* x);
template <>
__device__ __forceinline__ void unpack<uint16_t>(const uint4& v, float* x) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void unpack<float>(const uint4& v, float* x) {
  x[0] = __uint_as_float(v.x);
  x[1] = __uint_as_float(v.y);
  x[2] = __uint_as_float(v.z);
  x[3] = __uint_as_float(v.w);
}

template <>
__device__ __forceinline__ void unpack<uint8_t>(const uint4& v, float* x) {
  fp8x4_to_f32(v.x, x);
  fp8x4_to_f32(v.y, x + 4);
  fp8x4_to_f32(v.z, x + 8);
  fp8x4_to_f32(v.w, x + 12);
}

template <typename T>
__device__ __forceinline__ uint4 pack(const float* x);
template <>
__device__ __forceinline__ uint4 pack<uint16_t>(const float* x) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = (uint32_t)f32_to_bf16(x[2 * i]) | ((uint32_t)f32_to_bf16(x[2 * i + 1]) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}
template <>
__device__ __forceinline__ uint4 pack<uint8_t>(const float* x) {
  return make_uint4(f32x4_to_fp8(x), f32x4_to_fp8(x + 4), f32x4_to_fp8(x + 8),
                    f32x4_to_fp8(x + 12));
}
template <>
__device__ __forceinline__ uint4 pack<float>(const float* x) {
  return make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                    __float_as_uint(x[3]));
}

// Work split: a flat grid; workgroup w handles UNITS consecutive (l, g) units
// (32 token rows each) of job w / units_per_wg_count, so concurrently running
// workgroups stream neighbouring bytes of the same page (DRAM locality like a
// plain copy). A thread always sees the same token index j of its rows, so its
// (cos, sin) pairs for position pos + j are loaded once into registers.
// Each thread owns two 16-byte pieces of a row:
// LAYOUT 0 (pairs (2t, 2t+1)): pieces [t0, t0+P) and [t0+P, t0+2P);
// LAYOUT 1 (pairs (t, t+d/2)): pieces [t0, t0+P) and [t0+d/2, t0+d/2+P).
// All loads of a workgroup's rows are issued before the first store; loads and
// stores are plain (cached) ones, faster here than the non-temporal forms.
template <typename T, int D, int LAYOUT, bool DELTA>
__global__ __launch_bounds__(256) void remat_kernel(RematArgs a) {
  constexpr int P = 16 / sizeof(T);              // elements per piece
  constexpr int TPR = D / (2 * P);               // threads per row
  constexpr int RPI = 256 / TPR;                 // rows per workgroup pass
  constexpr int ROW_BYTES = D * sizeof(T);
  constexpr int HALF = D / 2;
  constexpr int ROWS = remat_units(sizeof(T)) * 32;   // rows per workgroup
  constexpr int NR = ROWS / RPI;                 // rows per thread
  constexpr int NJ = RPI >= 32 ? 1 : 32 / RPI;   // distinct token indices per thread
  constexpr int NC = P;                          // (cos, sin) pairs per piece pair
  const int32_t jid = blockIdx.x / a.wg_per_job;
  const int32_t wpart = blockIdx.x % a.wg_per_job;
  if (jid >= a.n_jobs) return;
  const RematJob job = a.jobs[jid];
  const int trow = threadIdx.x / TPR;
  const int tcol = threadIdx.x % TPR;
  const int t0 = LAYOUT == 0 ? tcol * 2 * P : tcol * P;            // first element
  const int off1 = LAYOUT == 0 ? P : D / 2;                         // second piece offset
  // (cos, sin) of the pairs this thread rotates, for each of its token indices;
  // launches of delta jobs turn every token by the job's signed shift instead
  // (table entry |shift|, sin negated for a negative shift)
  const int32_t shift = job.pos < 0 ? -job.pos : job.pos;
  const float ssign = DELTA && job.pos < 0 ? -1.0f : 1.0f;
  float2 cs[NJ][NC];
#pragma unroll
  for (int s = 0; s < NJ; ++s) {
    const int j = (trow + s * RPI) & 31;
    const float2* row = a.table + (int64_t)(DELTA ? shift : job.pos + j) * HALF;
#pragma unroll
    for (int q = 0; q < NC; ++q) {
      cs[s][q] = LAYOUT == 0 ? row[t0 / 2 + q] : row[t0 + q];
      if (DELTA) cs[s][q].y *= ssign;
    }
  }
  const int64_t page = (int64_t)job.slot * a.page_bytes;
  const int64_t row0 = (int64_t)wpart * ROWS;
  const bool copyv = (job.flags & JOB_COPY_V) != 0;
  uint4 k0[NR], k1[NR], v0[NR], v1[NR];
#pragma unroll
  for (int u = 0; u < NR; ++u) {
    if (row0 + trow + u * RPI >= a.rows_per_page) continue;   // ragged last workgroup
    const int64_t b0 = (row0 + trow + u * RPI) * ROW_BYTES + (int64_t)t0 * sizeof(T);
    k0[u] = ld_plain(job.src_k + b0);
    k1[u] = ld_plain(job.src_k + b0 + (int64_t)off1 * sizeof(T));
    if (copyv) {
      v0[u] = ld_plain(job.src_v + b0);
      v1[u] = ld_plain(job.src_v + b0 + (int64_t)off1 * sizeof(T));
    }
  }
  char* kv = a.k_view + page;
  char* vv = a.v_view + page;
#pragma unroll
  for (int u = 0; u < NR; ++u) {
    if (row0 + trow + u * RPI >= a.rows_per_page) continue;
    const int64_t b0 = (row0 + trow + u * RPI) * ROW_BYTES + (int64_t)t0 * sizeof(T);
    const int64_t b1 = b0 + (int64_t)off1 * sizeof(T);
    const float2* c = cs[u % NJ];
    float x0[P], x1[P], y0[P], y1[P];
    unpack<T>(k0[u], x0);
    unpack<T>(k1[u], x1);
    if (LAYOUT == 0) {
#pragma unroll
      for (int q = 0; q < P / 2; ++q) {
        const float2 c0 = c[q];
        const float2 c1 = c[P / 2 + q];
        y0[2 * q] = x0[2 * q] * c0.x - x0[2 * q + 1] * c0.y;
        y0[2 * q + 1] = x0[2 * q] * c0.y + x0[2 * q + 1] * c0.x;
        y1[2 * q] = x1[2 * q] * c1.x - x1[2 * q + 1] * c1.y;
        y1[2 * q + 1] = x1[2 * q] * c1.y + x1[2 * q + 1] * c1.x;
      }
    } else {
#pragma unroll
      for (int q = 0; q < P; ++q) {
        y0[q] = x0[q] * c[q].x - x1[q] * c[q].y;
        y1[q] = x0[q] * c[q].y + x1[q] * c[q].x;
      }
    }
    st_plain(kv + b0, pack<T>(y0));
    st_plain(kv + b1, pack<T>(y1));
    if (copyv) {
      st_plain(vv + b0, v0[u]);
      st_plain(vv + b1, v1[u]);
    }
  }
}

static void launch_remat(int32_t dtype, int32_t d, int32_t layout, bool delta,
                         const RematArgs& a, hipStream_t s) {
  const int64_t grid = (int64_t)a.n_jobs * a.wg_per_job;
  if (grid <= 0) return;
  dim3 g((uint32_t)grid), b(256);
  KernelTimer tm("remat", s);
#define KVM_REMAT(T, D, LAY)                                                 \
  do {                                                                       \
    if (delta) remat_kernel<T, D, LAY, true><<<g, b, 0, s>>>(a);             \
    else remat_kernel<T, D, LAY, false><<<g, b, 0, s>>>(a);                  \
  } while (0)
  if (dtype == KVM_FP8_E4M3) {
    if (d == 128) { if (layout == 0) KVM_REMAT(uint8_t, 128, 0); else KVM_REMAT(uint8_t, 128, 1); }
    else { if (layout == 0) KVM_REMAT(uint8_t, 64, 0); else KVM_REMAT(uint8_t, 64, 1); }
  } else if (dtype == KVM_BF16) {
    if (d == 128) { if (layout == 0) KVM_REMAT(uint16_t, 128, 0); else KVM_REMAT(uint16_t, 128, 1); }
    else { if (layout == 0) KVM_REMAT(uint16_t, 64, 0); else KVM_REMAT(uint16_t, 64, 1); }
  } else {
    if (d == 128) { if (layout == 0) KVM_REMAT(float, 128, 0); else KVM_REMAT(float, 128, 1); }
    else { if (layout == 0) KVM_REMAT(float, 64, 0); else KVM_REMAT(float, 64, 1); }
  }
#undef KVM_REMAT
}

// ---------------------------------------------------------------------------
// Host-side block manager.

struct BlockRec {
  int32_t slot = -1;
  int32_t baked = -1;        // compact position encoded in the K page (-1: stale)
  int64_t last_used = -1;    // step of the last selection that contained it
  int32_t src = KVM_SRC_NONE;
  int32_t gather = -1;       // index into ctx->gathers for gathered sources
  const char* src_k = nullptr;
  const char* src_v = nullptr;
  bool raw_in_shadow = false;  // the page's shadow holds the raw K (else the device source)
  bool page_raw = false;       // delta mode: the K page holds raw K, not yet rotated
  int32_t n_delta = 0;         // delta mode: in-place shifts since the last encode from raw K
};

struct Gather {
  kvm_gather_fn fn;
  void* user;
};

class WorkerPool {
 public:
  explicit WorkerPool(int n) {
    for (int i = 0; i < n; ++i) th_.emplace_back([this] { loop(); });
  }
  ~WorkerPool() {
    {
      std::lock_guard<std::mutex> g(m_);
      stop_ = true;
    }
    cv_.notify_all();
    for (auto& t : th_) t.join();
  }
  // Run f(i) for i in [0, n) on the workers; returns when all are done.
  void run(int n, const std::function<void(int)>& f) {
    if (n <= 0) return;
    {
      std::lock_guard<std::mutex> g(m_);
      f_ = &f;
      n_ = n;
      next_ = 0;
      done_ = 0;
      ++gen_;
    }
    cv_.notify_all();
    std::unique_lock<std::mutex> lk(m_);
    done_cv_.wait(lk, [&] { return done_ == n_; });
    f_ = nullptr;
  }

 private:
  void loop() {
    uint64_t seen = 0;
    for (;;) {
      std::unique_lock<std::mutex> lk(m_);
      cv_.wait(lk, [&] { return stop_ || (gen_ != seen && next_ < n_); });
      if (stop_) return;
      while (next_ < n_) {
        const int i = next_++;
        const std::function<void(int)>* f = f_;
        lk.unlock();
        (*f)(i);
        lk.lock();
        if (++done_ == n_) done_cv_.notify_all();
      }
      seen = gen_;
    }
  }
  std::vector<std::thread> th_;
  std::mutex m_;
  std::condition_variable cv_, done_cv_;
  const std::function<void(int)>* f_ = nullptr;
  int n_ = 0, next_ = 0, done_ = 0;
  uint64_t gen_ = 0;
  bool stop_ = false;
};

}  // namespace kvm

struct kvm_ctx {
  kvm_ctx_desc d;
  int64_t page_bytes = 0;
  int device = 0;
  std::vector<kvm::BlockRec> rec;
  std::vector<int64_t> slot_block;
  std::vector<int32_t> free_slots;
  std::vector<kvm::Gather> gathers;
  int64_t step = 0;
  float2* d_table = nullptr;
  kvm::RematJob* d_jobs = nullptr;
  kvm::RematJob* h_jobs = nullptr;   // pinned
  int32_t* h_sel = nullptr;          // pinned [n_slots + 1]
  int32_t* h_page = nullptr;         // pinned [n_slots]
  hipStream_t side = nullptr;        // H2D of K pages (and of gathered pages)
  hipStream_t side_v = nullptr;      // H2D of V pages from pinned sources
  std::vector<hipEvent_t> batch_ev;  // H2D batches (side stream)
  std::vector<hipEvent_t> batch_ev_v;  // H2D batches (side_v)
  std::vector<hipEvent_t> ring_ev;   // ring half reuse
  char* ring = nullptr;              // pinned [2][batch][2][page]
  kvm::WorkerPool* pool = nullptr;
};

namespace kvm {

static int ensure_events(std::vector<hipEvent_t>& v, size_t n) {
  while (v.size() < n) {
    hipEvent_t e;
    KVM_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
    v.push_back(e);
  }
  return KVM_OK;
}

static void destroy(kvm_ctx* c) {
  if (!c) return;
  delete c->pool;
  for (auto e : c->batch_ev) (void)hipEventDestroy(e);
  for (auto e : c->batch_ev_v) (void)hipEventDestroy(e);
  for (auto e : c->ring_ev) (void)hipEventDestroy(e);
  if (c->side) (void)hipStreamDestroy(c->side);
  if (c->side_v) (void)hipStreamDestroy(c->side_v);
  if (c->d_table) (void)hipFree(c->d_table);
  if (c->d_jobs) (void)hipFree(c->d_jobs);
  if (c->h_jobs) (void)hipHostFree(c->h_jobs);
  if (c->h_sel) (void)hipHostFree(c->h_sel);
  if (c->h_page) (void)hipHostFree(c->h_page);
  if (c->ring) (void)hipHostFree(c->ring);
  delete c;
}

// Pick a page for a miss: a free page, else the least recently used resident
// block outside the new view (last_used < step).
static int32_t take_slot(kvm_ctx* c, std::vector<std::pair<int64_t, int32_t>>& lru, size_t& lru_pos,
                         int32_t* evicted) {
  if (!c->free_slots.empty()) {
    int32_t s = c->free_slots.back();
    c->free_slots.pop_back();
    return s;
  }
  while (lru_pos < lru.size()) {
    const int32_t s = lru[lru_pos++].second;
    const int64_t b = c->slot_block[s];
    if (b < 0) return s;
    BlockRec& r = c->rec[b];
    if (r.last_used >= c->step) continue;  // in the new view
    r.slot = -1;
    r.baked = -1;
    r.raw_in_shadow = false;
    r.page_raw = false;
    r.n_delta = 0;
    ++*evicted;
    return s;
  }
  return -1;
}

// A resident page whose re-encode source is the block's device-resident
// lower-tier copy must not outlive a change of that source: reclaim it.
static void release_if_unbacked(kvm_ctx* c, BlockRec& r) {
  // in delta mode a page's K is self-contained; only rebuilds read the source
  if (r.slot < 0 || r.raw_in_shadow || c->d.delta_limit > 0) return;
  c->slot_block[r.slot] = -1;
  c->free_slots.push_back(r.slot);
  r.slot = -1;
  r.baked = -1;
}

}  // namespace kvm

extern "C" int kvm_ctx_create(const kvm_ctx_desc* desc, kvm_ctx** out) {
  using namespace kvm;
  clear_error();
  KVM_CHECK_ARG(desc && out, "null pointer");
  int rc = check_dims(&desc->dims, desc->dtype);
  if (rc) return rc;
  KVM_CHECK_ARG(desc->delta_limit >= 0, "delta_limit");
  KVM_CHECK_ARG(desc->n_slots > 0 && desc->k_view && desc->v_view &&
                    (desc->k_shadow || desc->delta_limit > 0),
                "pool pointers / n_slots");
  KVM_CHECK_ARG(desc->max_blocks > 0 && desc->max_pos > 0, "max_blocks / max_pos");
  KVM_CHECK_ARG(desc->rope_layout == 0 || desc->rope_layout == 1, "rope_layout");
  KVM_CHECK_ARG(desc->rope_theta > 1.0, "rope_theta");
  KVM_CHECK_ARG(((uintptr_t)desc->k_view | (uintptr_t)desc->v_view | (uintptr_t)desc->k_shadow) %
                        16 == 0,
                "pool pointers must be 16-byte aligned");
  {
    const kvm_dims& d0 = desc->dims;
    const size_t pool = (size_t)desc->n_slots * d0.n_layers * d0.n_kv_heads * d0.block_tokens *
                        d0.head_dim * dtype_bytes(desc->dtype);
    KVM_CHECK_RANGE(desc->k_view, pool, RANGE_DEVICE, "k_view");
    KVM_CHECK_RANGE(desc->v_view, pool, RANGE_DEVICE, "v_view");
    if (desc->k_shadow) KVM_CHECK_RANGE(desc->k_shadow, pool, RANGE_DEVICE, "k_shadow");
  }
  kvm_ctx* c = new kvm_ctx();
  c->d = *desc;
  if (c->d.batch_blocks <= 0) c->d.batch_blocks = 64;
  if (c->d.staging_blocks < 2 * c->d.batch_blocks) c->d.staging_blocks = 2 * c->d.batch_blocks;
  const kvm_dims& dm = desc->dims;
  c->page_bytes = (int64_t)dm.n_layers * dm.n_kv_heads * dm.block_tokens * dm.head_dim *
                  dtype_bytes(desc->dtype);
  c->rec.resize((size_t)desc->max_blocks);
  c->slot_block.assign((size_t)desc->n_slots, -1);
  for (int32_t s = desc->n_slots - 1; s >= 0; --s) c->free_slots.push_back(s);
  auto fail = [&](int code) {
    destroy(c);
    return code;
  };
#define KVM_HIP_C(call)                                                              \
  do {                                                                               \
    hipError_t e_ = (call);                                                          \
    if (e_ != hipSuccess) {                                                          \
      set_error("%s failed: %s", #call, hipGetErrorString(e_));                     \
      return fail(e_ == hipErrorOutOfMemory ? KVM_ENOMEM : KVM_EHIP);                \
    }                                                                                \
  } while (0)
  KVM_HIP_C(hipGetDevice(&c->device));
  // RoPE table: angle p * theta_t in float64, cos/sin rounded once to fp32.
  const int half = dm.head_dim / 2;
  std::vector<float2> table((size_t)desc->max_pos * half);
  std::vector<double> theta(half);
  for (int t = 0; t < half; ++t) theta[t] = std::pow(desc->rope_theta, -2.0 * t / dm.head_dim);
  {
    const int nth = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
    std::vector<std::thread> th;
    for (int w = 0; w < nth; ++w)
      th.emplace_back([&, w] {
        for (int64_t p = w; p < desc->max_pos; p += nth)
          for (int t = 0; t < half; ++t) {
            const double ang = (double)p * theta[t];
            table[(size_t)p * half + t] = make_float2((float)std::cos(ang), (float)std::sin(ang));
          }
      });
    for (auto& x : th) x.join();
  }
  KVM_HIP_C(hipMalloc(&c->d_table, table.size() * sizeof(float2)));
  KVM_HIP_C(hipMemcpy(c->d_table, table.data(), table.size() * sizeof(float2),
                      hipMemcpyHostToDevice));
  KVM_HIP_C(hipMalloc(&c->d_jobs, (size_t)desc->n_slots * sizeof(RematJob)));
  KVM_HIP_C(hipHostMalloc(&c->h_jobs, (size_t)desc->n_slots * sizeof(RematJob),
                          hipHostMallocDefault));
  KVM_HIP_C(hipHostMalloc(&c->h_sel, ((size_t)desc->n_slots + 1) * sizeof(int32_t),
                          hipHostMallocDefault));
  KVM_HIP_C(hipHostMalloc(&c->h_page, (size_t)desc->n_slots * sizeof(int32_t),
                          hipHostMallocDefault));
  KVM_HIP_C(hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking));
  KVM_HIP_C(hipStreamCreateWithFlags(&c->side_v, hipStreamNonBlocking));
#undef KVM_HIP_C
  *out = c;
  return KVM_OK;
}

extern "C" void kvm_ctx_destroy(kvm_ctx* ctx) {
  if (!ctx) return;
  (void)hipStreamSynchronize(ctx->side);
  (void)hipStreamSynchronize(ctx->side_v);
  kvm::destroy(ctx);
}

extern "C" int kvm_ctx_build_index_rope(kvm_ctx* c, const void* k_rope, int64_t block_stride,
                                        int64_t first_block, int64_t n_blocks, int64_t pos0,
                                        void* index, int64_t index_cap_blocks, void* stream) {
  using namespace kvm;
  clear_error();
  KVM_CHECK_ARG(c, "ctx is NULL");
  KVM_CHECK_ARG(n_blocks >= 0 && first_block >= 0, "negative block range");
  if (n_blocks == 0) return KVM_OK;
  KVM_CHECK_ARG(k_rope && index, "null pointer");
  KVM_CHECK_ARG(block_stride >= c->page_bytes, "block_stride %lld < block bytes %lld",
                (long long)block_stride, (long long)c->page_bytes);
  KVM_CHECK_ARG(block_stride % 16 == 0 && ((uintptr_t)k_rope % 16) == 0 &&
                    ((uintptr_t)index % 16) == 0,
                "k_rope, index and stride must be 16-byte aligned");
  KVM_CHECK_ARG(first_block + n_blocks <= index_cap_blocks, "rows beyond index capacity");
  const kvm_dims& dm = c->d.dims;
  if (pos0 < 0 || pos0 + (int64_t)dm.block_tokens * n_blocks > (int64_t)c->d.max_pos) {
    set_error("positions [%lld, %lld) outside the RoPE table [0, %d)", (long long)pos0,
              (long long)(pos0 + (int64_t)dm.block_tokens * n_blocks), c->d.max_pos);
    return KVM_ERANGE;
  }
  KVM_CHECK_RANGE(k_rope, (size_t)((n_blocks - 1) * block_stride + c->page_bytes), RANGE_DEVICE,
                  "k_rope");
  KVM_CHECK_RANGE(index,
                  (size_t)dm.n_layers * dm.n_kv_heads * index_cap_blocks * dm.head_dim *
                      dtype_bytes(index_dtype(c->d.dtype)),
                  RANGE_DEVICE, "index");
  return launch_build_rope(c->d.dtype, dm.head_dim, c->d.rope_layout, k_rope, block_stride,
                           n_blocks, dm.n_layers * dm.n_kv_heads, pos0, c->d_table,
                           first_block, index_cap_blocks, index, as_stream(stream));
}

extern "C" int kvm_ctx_set_source(kvm_ctx* c, int64_t first_block, int64_t n_blocks,
                                  const void* k_base, const void* v_base, int64_t block_stride,
                                  int32_t loc) {
  using namespace kvm;
  clear_error();
  KVM_CHECK_ARG(c, "ctx is NULL");
  KVM_CHECK_ARG(first_block >= 0 && n_blocks >= 0 && first_block + n_blocks <= c->d.max_blocks,
                "block range outside the record capacity");
  KVM_CHECK_ARG(loc == KVM_SRC_NONE || loc == KVM_SRC_HOST_PINNED || loc == KVM_SRC_DEVICE,
                "loc");
  if (loc != KVM_SRC_NONE) {
    KVM_CHECK_ARG(k_base && v_base && block_stride >= c->page_bytes, "source pointers/stride");
    KVM_CHECK_ARG(((uintptr_t)k_base | (uintptr_t)v_base | (uintptr_t)block_stride) % 16 == 0,
                  "sources must be 16-byte aligned");
    if (n_blocks > 0) {
      const size_t span = (size_t)((n_blocks - 1) * block_stride + c->page_bytes);
      const RangeKind kind = loc == KVM_SRC_HOST_PINNED ? RANGE_PINNED_HOST : RANGE_DEVICE;
      KVM_CHECK_RANGE(k_base, span, kind, "k source");
      KVM_CHECK_RANGE(v_base, span, kind, "v source");
    }
  }
  for (int64_t i = 0; i < n_blocks; ++i) {
    BlockRec& r = c->rec[first_block + i];
    release_if_unbacked(c, r);
    r.src = loc;
    r.gather = -1;
    r.src_k = loc == KVM_SRC_NONE ? nullptr : (const char*)k_base + i * block_stride;
    r.src_v = loc == KVM_SRC_NONE ? nullptr : (const char*)v_base + i * block_stride;
  }
  return KVM_OK;
}

extern "C" int kvm_ctx_set_gather(kvm_ctx* c, int64_t first_block, int64_t n_blocks,
                                  kvm_gather_fn fn, void* user) {
  using namespace kvm;
  clear_error();
  KVM_CHECK_ARG(c && fn, "null pointer");
  KVM_CHECK_ARG(first_block >= 0 && n_blocks >= 0 && first_block + n_blocks <= c->d.max_blocks,
                "block range outside the record capacity");
  if (!c->ring) {
    const size_t bytes = (size_t)c->d.staging_blocks * 2 * (size_t)c->page_bytes;
    hipError_t e = hipHostMalloc(&c->ring, bytes, hipHostMallocDefault);
    if (e != hipSuccess) {
      c->ring = nullptr;
      set_error("pinned staging ring of %zu bytes: %s", bytes, hipGetErrorString(e));
      return KVM_ENOMEM;
    }
  }
  if (!c->pool) {
    const int n = (int)std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
    c->pool = new WorkerPool(n);
  }
  c->gathers.push_back(Gather{fn, user});
  const int32_t gid = (int32_t)c->gathers.size() - 1;
  for (int64_t i = 0; i < n_blocks; ++i) {
    BlockRec& r = c->rec[first_block + i];
    release_if_unbacked(c, r);
    r.src = KVM_SRC_HOST_PINNED;
    r.gather = gid;
    r.src_k = nullptr;
    r.src_v = nullptr;
  }
  return KVM_OK;
}

extern "C" int kvm_ctx_register_resident(kvm_ctx* c, int64_t first_block, int64_t n_blocks,
                                         const void* k_raw, const void* v_raw,
                                         int64_t block_stride, void* stream) {
  using namespace kvm;
  clear_error();
  KVM_CHECK_ARG(c && k_raw && v_raw, "null pointer");
  KVM_CHECK_ARG(first_block >= 0 && n_blocks >= 0 && first_block + n_blocks <= c->d.max_blocks,
                "block range outside the record capacity");
  KVM_CHECK_ARG(block_stride >= c->page_bytes, "block_stride");
  if (n_blocks > 0) {
    const size_t span = (size_t)((n_blocks - 1) * block_stride + c->page_bytes);
    KVM_CHECK_RANGE(k_raw, span, RANGE_DEVICE, "k_raw");
    KVM_CHECK_RANGE(v_raw, span, RANGE_DEVICE, "v_raw");
  }
  hipStream_t s = as_stream(stream);
  // Only pages of blocks outside the current view (or free pages) are reused.
  std::vector<std::pair<int64_t, int32_t>> lru;
  for (int32_t sl = 0; sl < c->d.n_slots; ++sl) {
    const int64_t b = c->slot_block[sl];
    if (b >= 0) lru.emplace_back(c->rec[b].last_used, sl);
  }
  std::sort(lru.begin(), lru.end());
  size_t lru_pos = 0;
  int32_t evicted = 0;
  for (int64_t i = 0; i < n_blocks; ++i) {
    const int64_t b = first_block + i;
    BlockRec& r = c->rec[b];
    int32_t sl = r.slot;
    if (sl < 0) {
      // reuse: pages not used since before the last step first
      const int64_t saved = c->step;
      c->step = saved + 1;  // everything selected at or before `saved` is evictable
      sl = take_slot(c, lru, lru_pos, &evicted);
      c->step = saved;
      if (sl < 0) {
        set_error("no free pool page for block %lld", (long long)b);
        return KVM_ENOMEM;
      }
      if (c->slot_block[sl] >= 0 && c->slot_block[sl] != b) c->rec[c->slot_block[sl]].slot = -1;
      c->slot_block[sl] = b;
      r.slot = sl;
    }
    r.baked = -1;
    r.last_used = c->step;
    r.n_delta = 0;
    const bool delta = c->d.delta_limit > 0;
    r.raw_in_shadow = !delta;
    r.page_raw = delta;
    char* kdst = (char*)(delta ? c->d.k_view : c->d.k_shadow) + (int64_t)sl * c->page_bytes;
    KVM_HIP(hipMemcpyAsync(kdst, (const char*)k_raw + i * block_stride, c->page_bytes,
                           hipMemcpyDeviceToDevice, s));
    KVM_HIP(hipMemcpyAsync((char*)c->d.v_view + (int64_t)sl * c->page_bytes,
                           (const char*)v_raw + i * block_stride, c->page_bytes,
                           hipMemcpyDeviceToDevice, s));
  }
  return KVM_OK;
}

extern "C" int kvm_ctx_evict(kvm_ctx* c, int64_t first_block, int64_t n_blocks) {
  using namespace kvm;
  clear_error();
  KVM_CHECK_ARG(c, "ctx is NULL");
  KVM_CHECK_ARG(first_block >= 0 && n_blocks >= 0 && first_block + n_blocks <= c->d.max_blocks,
                "block range outside the record capacity");
  for (int64_t b = first_block; b < first_block + n_blocks; ++b) {
    BlockRec& r = c->rec[b];
    if (r.slot < 0) continue;
    c->slot_block[r.slot] = -1;
    c->free_slots.push_back(r.slot);
    r.slot = -1;
    r.baked = -1;
    r.raw_in_shadow = false;
    r.page_raw = false;
    r.n_delta = 0;
  }
  return KVM_OK;
}

extern "C" int kvm_ctx_block_deltas(kvm_ctx* c, int64_t block, int32_t* n_delta) {
  using namespace kvm;
  KVM_CHECK_ARG(c && n_delta && block >= 0 && block < c->d.max_blocks, "block out of range");
  *n_delta = c->rec[block].slot >= 0 ? c->rec[block].n_delta : 0;
  return KVM_OK;
}

extern "C" int kvm_ctx_sync(kvm_ctx* c) {
  using namespace kvm;
  KVM_CHECK_ARG(c, "ctx is NULL");
  KVM_HIP(hipStreamSynchronize(c->side));
  KVM_HIP(hipStreamSynchronize(c->side_v));
  return KVM_OK;
}

extern "C" int kvm_ctx_block_state(kvm_ctx* c, int64_t block, int32_t* slot, int32_t* baked) {
  using namespace kvm;
  KVM_CHECK_ARG(c && block >= 0 && block < c->d.max_blocks, "block out of range");
  if (slot) *slot = c->rec[block].slot;
  if (baked) *baked = c->rec[block].baked;
  return KVM_OK;
}

extern "C" int kvm_rematerialize(kvm_ctx* c, const int32_t* sel_dev, const int32_t* n_sel_dev,
                                 int32_t* page_table_dev, kvm_remat_stats* stats,
                                 void* stream) {
  using namespace kvm;
  clear_error();
  KVM_CHECK_ARG(c && sel_dev && n_sel_dev && page_table_dev, "null pointer");
  KVM_CHECK_RANGE(n_sel_dev, sizeof(int32_t), RANGE_DEVICE, "n_sel");
  hipStream_t s = as_stream(stream);
  const int32_t B = c->d.dims.block_tokens;
  // 1. Read the selection (stream-ordered; waits only for `stream`).
  KVM_HIP(hipMemcpyAsync(c->h_sel, n_sel_dev, sizeof(int32_t), hipMemcpyDeviceToHost, s));
  KVM_HIP(hipStreamSynchronize(s));
  const int32_t n = c->h_sel[0];
  if (n < 0) {
    set_error("selection invalid (n_sel = %d)", n);
    return KVM_ERANGE;
  }
  if (n > c->d.n_slots) {
    set_error("view of %d blocks exceeds the pool (%d pages)", n, c->d.n_slots);
    return KVM_ENOMEM;
  }
  if ((int64_t)n * B > c->d.max_pos) {
    set_error("compact positions up to %lld exceed max_pos %d", (long long)n * B, c->d.max_pos);
    return KVM_ERANGE;
  }
  int32_t* sel = c->h_sel + 1;
  const bool delta_mode = c->d.delta_limit > 0;
  KVM_CHECK_RANGE(sel_dev, (size_t)n * sizeof(int32_t), RANGE_DEVICE, "sel");
  KVM_CHECK_RANGE(page_table_dev, (size_t)n * sizeof(int32_t), RANGE_DEVICE, "page_table");
  if (n > 0) {
    KVM_HIP(hipMemcpyAsync(sel, sel_dev, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToHost, s));
    KVM_HIP(hipStreamSynchronize(s));
  }
  // 2. Validate before touching any state.
  for (int32_t i = 0; i < n; ++i) {
    const int64_t b = sel[i];
    if (b < 0 || b >= c->d.max_blocks || (i > 0 && sel[i] <= sel[i - 1])) {
      set_error("selection entry %d (block %lld) invalid", i, (long long)b);
      return KVM_ERANGE;
    }
    const BlockRec& r = c->rec[b];
    if (r.slot < 0 && r.src == KVM_SRC_NONE) {
      set_error("block %lld is neither resident nor backed by a source", (long long)b);
      return KVM_ERANGE;
    }
    // delta mode: a hit past its delta limit is rebuilt from its raw K
    if (delta_mode && r.slot >= 0 && !r.page_raw && r.baked != i * B &&
        (r.baked < 0 || r.n_delta >= c->d.delta_limit) && r.src == KVM_SRC_NONE) {
      set_error("block %lld needs a rebuild from raw K but has no lower-tier copy",
                (long long)b);
      return KVM_ERANGE;
    }
  }
  // 3. Plan: hits keep their pages; misses take free or LRU pages outside the view.
  c->step += 1;
  for (int32_t i = 0; i < n; ++i) c->rec[sel[i]].last_used = c->step;
  std::vector<std::pair<int64_t, int32_t>> lru;
  for (int32_t sl = 0; sl < c->d.n_slots; ++sl) {
    const int64_t b = c->slot_block[sl];
    if (b >= 0 && c->rec[b].last_used < c->step) lru.emplace_back(c->rec[b].last_used, sl);
  }
  std::sort(lru.begin(), lru.end());
  size_t lru_pos = 0;
  kvm_remat_stats st{};
  st.n_sel = n;
  std::vector<int32_t> hit_jobs, delta_jobs, dev_jobs, dma_miss, gather_miss;
  RematJob* J = c->h_jobs;
  int32_t nj = 0;
  // Where staged raw K lands and is read by the kernel: the page's shadow, or
  // (delta mode) the K page itself, rotated in place.
  auto stage_k = [&](int32_t sl) {
    return (const char*)(delta_mode ? c->d.k_view : c->d.k_shadow) + (int64_t)sl * c->page_bytes;
  };
  auto kpage = [&](int32_t sl) { return (const char*)c->d.k_view + (int64_t)sl * c->page_bytes; };
  // A job whose raw K (and V unless JOB_K_ONLY) comes from host memory.
  auto staged_job = [&](BlockRec& r, int32_t sl, int32_t pos, int32_t flags, int32_t i) {
    J[nj] = RematJob{stage_k(sl), nullptr, sl, pos, flags, i};
    if (r.gather >= 0) gather_miss.push_back(nj++);
    else dma_miss.push_back(nj++);
  };
  for (int32_t i = 0; i < n; ++i) {
    const int64_t b = sel[i];
    BlockRec& r = c->rec[b];
    const int32_t pos = i * B;
    if (r.slot >= 0) {
      ++st.hits;
      c->h_page[i] = r.slot;
      if (r.baked == pos && !r.page_raw) continue;
      if (!delta_mode) {
        // re-encode from the raw K kept in HBM: the page's shadow, or the
        // block's device-resident lower-tier copy
        const char* raw = r.raw_in_shadow
                              ? (const char*)c->d.k_shadow + (int64_t)r.slot * c->page_bytes
                              : r.src_k;
        J[nj] = RematJob{raw, nullptr, r.slot, pos, 0, 0};
        hit_jobs.push_back(nj++);
      } else if (r.page_raw) {
        // freshly registered: raw K sits in the K page, rotate it there
        J[nj] = RematJob{kpage(r.slot), nullptr, r.slot, pos, 0, 0};
        hit_jobs.push_back(nj++);
        r.page_raw = false;
        r.n_delta = 0;
      } else if (r.baked >= 0 && r.n_delta < c->d.delta_limit) {
        // bounded delta re-RoPE: rotate the stored K by the position shift
        J[nj] = RematJob{kpage(r.slot), nullptr, r.slot, pos - r.baked, JOB_DELTA, 0};
        delta_jobs.push_back(nj++);
        r.n_delta += 1;
        ++st.deltas;
      } else {
        // limit reached: rebuild from raw K at the new position, reset the count
        ++st.rebuilds;
        r.n_delta = 0;
        if (r.src == KVM_SRC_DEVICE) {
          J[nj] = RematJob{r.src_k, nullptr, r.slot, pos, 0, 0};
          hit_jobs.push_back(nj++);
        } else {
          staged_job(r, r.slot, pos, JOB_K_ONLY, i);
        }
      }
      r.baked = pos;
      continue;
    }
    ++st.misses;
    const int32_t sl = take_slot(c, lru, lru_pos, &st.evicted);
    if (sl < 0) {
      set_error("pool exhausted while planning (%d pages)", c->d.n_slots);
      return KVM_ENOMEM;  // cannot happen when n <= n_slots
    }
    c->slot_block[sl] = b;
    r.slot = sl;
    r.baked = pos;
    r.page_raw = false;
    r.n_delta = 0;
    c->h_page[i] = sl;
    if (r.src == KVM_SRC_DEVICE) {
      // the lower-tier copy is already in HBM: rotate from it, copy V, and
      // keep reading it for later re-encodes (no shadow copy)
      J[nj] = RematJob{r.src_k, r.src_v, sl, pos, JOB_COPY_V, 0};
      r.raw_in_shadow = false;
      dev_jobs.push_back(nj++);
    } else {
      r.raw_in_shadow = !delta_mode;
      staged_job(r, sl, pos, 0, i);
    }
  }
  // Jobs are grouped: [hits + device misses][delta shifts][DMA misses][gathered misses].
  std::vector<RematJob> ordered;
  ordered.reserve(nj);
  for (int32_t j : hit_jobs) ordered.push_back(J[j]);
  for (int32_t j : dev_jobs) ordered.push_back(J[j]);
  const int32_t n_full = (int32_t)ordered.size();
  for (int32_t j : delta_jobs) ordered.push_back(J[j]);
  const int32_t n_first = (int32_t)ordered.size();
  for (int32_t j : dma_miss) ordered.push_back(J[j]);
  for (int32_t j : gather_miss) ordered.push_back(J[j]);
  std::copy(ordered.begin(), ordered.end(), J);
  // 4. Page table and job list, then the first kernel (no dependency on H2D).
  if (n > 0)
    KVM_HIP(hipMemcpyAsync(page_table_dev, c->h_page, (size_t)n * sizeof(int32_t),
                           hipMemcpyHostToDevice, s));
  if (nj > 0)
    KVM_HIP(hipMemcpyAsync(c->d_jobs, J, (size_t)nj * sizeof(RematJob), hipMemcpyHostToDevice, s));
  const kvm_dims& dm = c->d.dims;
  RematArgs a{};
  a.rows_per_page = dm.n_layers * dm.n_kv_heads * B;
  const int units = remat_units(dtype_bytes(c->d.dtype));
  a.wg_per_job = (dm.n_layers * dm.n_kv_heads + units - 1) / units;
  a.page_bytes = c->page_bytes;
  a.k_view = (char*)c->d.k_view;
  a.v_view = (char*)c->d.v_view;
  a.k_shadow = (char*)c->d.k_shadow;
  a.table = c->d_table;
  auto launch_range = [&](int32_t first, int32_t count, bool delta = false) -> int {
    if (count <= 0) return KVM_OK;
    a.jobs = c->d_jobs + first;
    a.n_jobs = count;
    launch_remat(c->d.dtype, dm.head_dim, c->d.rope_layout, delta, a, s);
    KVM_HIP(hipGetLastError());
    return KVM_OK;
  };
  int rc = launch_range(0, n_full);
  if (rc) return rc;
  rc = launch_range(n_full, n_first - n_full, true);
  if (rc) return rc;
  st.d2d_bytes += (int64_t)(hit_jobs.size() + delta_jobs.size()) * 2 * c->page_bytes +
                  (int64_t)dev_jobs.size() * 4 * c->page_bytes;
  // 5. Misses from pinned host memory: DMA straight into the pages, batched;
  //    K pages on one side stream and V pages on another, so two copy engines
  //    share the transfer (4 MiB copies run at about 50 GB/s on one stream and
  //    56 GB/s on two).
  const int32_t bb = c->d.batch_blocks;
  int32_t cursor = n_first;
  const int32_t n_dma = (int32_t)dma_miss.size();
  const int32_t n_dma_batches = (n_dma + bb - 1) / bb;
  rc = ensure_events(c->batch_ev, (size_t)n_dma_batches + 2 * ((gather_miss.size() + bb - 1) / bb) + 2);
  if (rc) return rc;
  rc = ensure_events(c->batch_ev_v, (size_t)n_dma_batches);
  if (rc) return rc;
  int32_t ev_used = 0;
  if (n_dma > 0) {
    // The side streams must not start before the caller's stream reached this point.
    hipEvent_t start = c->batch_ev[ev_used++];
    KVM_HIP(hipEventRecord(start, s));
    KVM_HIP(hipStreamWaitEvent(c->side, start, 0));
    KVM_HIP(hipStreamWaitEvent(c->side_v, start, 0));
  }
  for (int32_t bi = 0; bi < n_dma_batches; ++bi) {
    const int32_t first = cursor + bi * bb;
    const int32_t cnt = std::min(bb, n_first + n_dma - first);
    int32_t pages_in = 0;
    for (int32_t q = 0; q < cnt; ++q) {
      const RematJob& jb = J[first + q];
      const BlockRec& r = c->rec[sel[jb.pad]];
      KVM_HIP(hipMemcpyAsync((char*)jb.src_k, r.src_k, c->page_bytes, hipMemcpyHostToDevice,
                             c->side));
      ++pages_in;
      if (!(jb.flags & JOB_K_ONLY)) {
        KVM_HIP(hipMemcpyAsync((char*)c->d.v_view + (int64_t)jb.slot * c->page_bytes, r.src_v,
                               c->page_bytes, hipMemcpyHostToDevice, c->side_v));
        ++pages_in;
      }
    }
    hipEvent_t ev = c->batch_ev[ev_used++];
    KVM_HIP(hipEventRecord(ev, c->side));
    KVM_HIP(hipStreamWaitEvent(s, ev, 0));
    hipEvent_t ev_v = c->batch_ev_v[bi];
    KVM_HIP(hipEventRecord(ev_v, c->side_v));
    KVM_HIP(hipStreamWaitEvent(s, ev_v, 0));
    rc = launch_range(first, cnt);
    if (rc) return rc;
    st.h2d_bytes += (int64_t)pages_in * c->page_bytes;
    st.d2d_bytes += (int64_t)cnt * 2 * c->page_bytes;
    ++st.batches;
  }
  cursor += n_dma;
  // 6. Gathered misses: host workers pack raw K/V into a pinned half-ring while
  //    the other half is in flight (double buffering, event-guarded reuse).
  const int32_t n_g = (int32_t)gather_miss.size();
  if (n_g > 0) {
    const int32_t half_blocks = c->d.staging_blocks / 2;
    const int32_t gb = std::min(bb, half_blocks);
    const int32_t n_gb = (n_g + gb - 1) / gb;
    if (ensure_events(c->ring_ev, 2)) return KVM_EHIP;
    bool half_busy[2] = {false, false};
    hipEvent_t start = c->batch_ev[ev_used++];
    KVM_HIP(hipEventRecord(start, s));
    KVM_HIP(hipStreamWaitEvent(c->side, start, 0));
    std::atomic<int> gerr{0};
    for (int32_t bi = 0; bi < n_gb; ++bi) {
      const int h = bi & 1;
      if (half_busy[h]) KVM_HIP(hipEventSynchronize(c->ring_ev[h]));
      const int32_t first = cursor + bi * gb;
      const int32_t cnt = std::min(gb, cursor + n_g - first);
      char* base = c->ring + (size_t)h * half_blocks * 2 * c->page_bytes;
      c->pool->run(cnt * 2, [&](int t) {
        const RematJob& jb = J[first + t / 2];
        if ((t & 1) && (jb.flags & JOB_K_ONLY)) return;   // rebuild: V page is intact
        const int64_t blk = sel[jb.pad];
        const Gather& g = c->gathers[c->rec[blk].gather];
        char* dst = base + ((size_t)(t / 2) * 2 + (t & 1)) * c->page_bytes;
        if (g.fn(g.user, blk, t & 1, dst) != 0) gerr.store(1);
      });
      if (gerr.load()) {
        set_error("host gather callback failed");
        KVM_HIP(hipStreamSynchronize(c->side));
        return KVM_ERANGE;
      }
      int32_t pages_in = 0;
      for (int32_t q = 0; q < cnt; ++q) {
        const RematJob& jb = J[first + q];
        const char* src = base + (size_t)q * 2 * c->page_bytes;
        KVM_HIP(hipMemcpyAsync((char*)jb.src_k, src, c->page_bytes, hipMemcpyHostToDevice,
                               c->side));
        ++pages_in;
        if (!(jb.flags & JOB_K_ONLY)) {
          KVM_HIP(hipMemcpyAsync((char*)c->d.v_view + (int64_t)jb.slot * c->page_bytes,
                                 src + c->page_bytes, c->page_bytes, hipMemcpyHostToDevice,
                                 c->side));
          ++pages_in;
        }
      }
      KVM_HIP(hipEventRecord(c->ring_ev[h], c->side));
      half_busy[h] = true;
      hipEvent_t ev = c->batch_ev[ev_used++];
      KVM_HIP(hipEventRecord(ev, c->side));
      KVM_HIP(hipStreamWaitEvent(s, ev, 0));
      rc = launch_range(first, cnt);
      if (rc) return rc;
      st.h2d_bytes += (int64_t)pages_in * c->page_bytes;
      st.d2d_bytes += (int64_t)cnt * 2 * c->page_bytes;
      ++st.batches;
    }
    // The ring must not be refilled by a later call before its copies finish.
    for (int h = 0; h < 2; ++h)
      if (half_busy[h]) KVM_HIP(hipEventSynchronize(c->ring_ev[h]));
  }
  st.rotated = nj;
  if (stats) *stats = st;
  return KVM_OK;
}
