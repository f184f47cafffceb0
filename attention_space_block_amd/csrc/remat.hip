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
// Host side: the block pool (pool.cpp) turns a selection into hits, misses
// and evictions over the bounded page pool (LRU among pages outside the new
// view) and the data plane (dataplane.cpp) queues the work: misses from pinned
// host memory are copied by DMA straight into their pages on side streams
// (batches tracked by events; the caller's stream waits per batch and rotates
// that batch while the next one transfers), or through a pinned,
// double-buffered staging ring filled by host gather workers. This file holds
// the kernel, the HIP implementation of the data plane's device operations
// and the C entry points.
#include <algorithm>
#include <cmath>
#include <memory>
#include <thread>
#include <vector>

#include "common.hpp"
#include "dataplane.hpp"
#include "pool.hpp"
#include "profile.hpp"

namespace kvm {

// jobs per launch: the grid's y dimension holds them and their V rows
static constexpr int32_t REMAT_JOBS_PER_LAUNCH = 16384;
// (l, g) units a K work item covers with one load of its (cos, sin): FP8
// pieces hold 8 pairs, so one unit per item would read 64 bytes of table per
// 16 bytes of K. FP8 view of the 1M-token workspace with one-wavefront
// workgroups: R = 2 4.26 ms, 4 4.19-4.26, 8 4.33-4.44, 16 4.49.
#ifndef KVM_REMAT_R_FP8
#define KVM_REMAT_R_FP8 4
#endif
#ifndef KVM_REMAT_R_BF16
#define KVM_REMAT_R_BF16 1
#endif
// Threads per workgroup of the remat and registration copies: one wavefront.
// Timed at the 1M-token view (4096 jobs of 4 MiB pages): 64 threads 8.26 ms,
// 256 threads 8.81 ms; a plain device copy moves 6.4 TB/s in 64-thread
// workgroups against 6.1 in 256-thread ones.
static constexpr int REMAT_TPB = 64;
// Pages read from a buffer other than the one written are loaded and stored
// non-temporally (8.16 ms against 8.26 with plain loads for the view above,
// then 8.03 against 8.16 with the stores too; FP8 view 4.20 against 4.38);
// the in-place delta rotation keeps plain loads and stores (5.47 ms against
// 5.74 with non-temporal loads).
template <bool NT>
__device__ __forceinline__ uint4 ld_page(const void* p) {
  return NT ? ld_nt(p) : ld_plain(p);
}
template <bool NT>
__device__ __forceinline__ void st_page(void* p, const uint4& v) {
  if (NT) st_nt(p, v);
  else st_plain(p, v);
}
static constexpr int remat_units_per_item(int elem_bytes) {
  return elem_bytes == 1 ? KVM_REMAT_R_FP8 : elem_bytes == 2 ? KVM_REMAT_R_BF16 : 1;
}

struct RematArgs {
  const RematJob* jobs;
  int32_t n_jobs;
  int32_t first_v;           // jobs [first_v, n_jobs) may copy V (each checks its flag)
  int32_t wg_k;              // workgroups per job for K: ceil(items per page / REMAT_TPB)
  int32_t wg_v;              // workgroups per job for V: ceil(page_bytes / 16 / REMAT_TPB)
  int64_t items;             // K work items per page (one piece or one piece pair, in
                             // R units: ceil(units / R) * 32 * items per row)
  int32_t units;             // (l, g) units per page: L * Hkv
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

// Work split: one 16-byte piece of a page per thread (LAYOUT 0: its pairs
// (2t, 2t+1) lie inside the piece), or one piece and its partner d/2 elements
// on (LAYOUT 1), over a two-dimensional grid: row y < n_jobs of workgroups
// rotates job y's K page in page order, and the rows after them copy the V
// pages of jobs [first_v, n_jobs) that carry JOB_COPY_V (workgroups are
// dispatched x first, so no division maps a workgroup to its job). The
// workgroups in flight then cover one narrow stretch of each page, which the
// DRAM serves best (a plain copy in this shape moves about 6.1-6.6 TB/s,
// against 3.6 TB/s when each thread loads sixteen pieces before storing them);
// each thread reads the (cos, sin) of its pairs from the fp32 table
// (L2-resident: 32 positions of a job span at most 32 table rows). Page loads
// and stores are non-temporal except in the in-place delta rotation (see
// ld_page).
template <typename T, int D, int LAYOUT, bool DELTA, bool COPYV>
__global__ __launch_bounds__(REMAT_TPB) void remat_kernel(RematArgs a) {
  constexpr int P = 16 / sizeof(T);              // elements per piece
  constexpr int ROW_BYTES = D * sizeof(T);
  constexpr int PPR = ROW_BYTES / 16;            // pieces per row
  constexpr int IPR = LAYOUT == 0 ? PPR : PPR / 2;   // work items per row
  constexpr int HALF = D / 2;
  constexpr int NC = LAYOUT == 0 ? P / 2 : P;    // pairs per item
  constexpr int R = remat_units_per_item(sizeof(T));
  // grid: x = workgroup within the page, y = job (rows [n_jobs, ...) copy V)
  const uint32_t part = blockIdx.x;
  if ((int32_t)blockIdx.y >= a.n_jobs) {
    if (!COPYV) return;
    const int32_t jid = a.first_v + ((int32_t)blockIdx.y - a.n_jobs);
    if (jid >= a.n_jobs || (int32_t)part >= a.wg_v) return;
    const RematJob job = a.jobs[jid];
    if ((job.flags & JOB_COPY_V) == 0) return;
    const int64_t off = ((int64_t)part * REMAT_TPB + threadIdx.x) * 16;
    if (off >= a.page_bytes) return;
    st_page<true>(a.v_view + (int64_t)job.slot * a.page_bytes + off, ld_page<true>(job.src_v + off));
    // keeps this path's store its own: merged with the K path's stores, the
    // compiler splits every 16-byte store into a 4- and a 12-byte one
    asm volatile("" ::: "memory");
    return;
  }
  if ((int32_t)part >= a.wg_k) return;
  const RematJob job = a.jobs[blockIdx.y];
  const uint32_t item = part * REMAT_TPB + threadIdx.x;
  if ((int64_t)item >= a.items) return;
  // item -> (group of R (l, g) units, token j, piece p): the thread rotates
  // piece p of token row j in each unit of the group with the same (cos, sin)
  const int p = (int)(item % IPR);
  const uint32_t t = item / IPR;
  const int j = (int)(t & 31);
  const int32_t unit0 = (int32_t)(t >> 5) * R;
  // (cos, sin) of this item's pairs: pair index t0 + q; delta jobs turn every
  // token by the job's signed shift (table entry |shift|, sin negated below 0)
  const int t0 = LAYOUT == 0 ? p * (P / 2) : p * P;
  const int32_t shift = job.pos < 0 ? -job.pos : job.pos;
  const float2* trow = a.table + (int64_t)(DELTA ? shift : job.pos + j) * HALF + t0;
  float2 cs[NC];
#pragma unroll
  for (int q = 0; q < NC; ++q) cs[q] = trow[q];
  if (DELTA && job.pos < 0) {
#pragma unroll
    for (int q = 0; q < NC; ++q) cs[q].y = -cs[q].y;
  }
  char* kv = a.k_view + (int64_t)job.slot * a.page_bytes;
#pragma unroll
  for (int u = 0; u < R; ++u) {
    if (R > 1 && unit0 + u >= a.units) break;
    const int64_t row = (int64_t)(unit0 + u) * 32 + j;
    const int64_t b0 = row * ROW_BYTES + (int64_t)p * 16;
    const uint4 k0 = ld_page<!DELTA>(job.src_k + b0);
    float x0[P], y0[P];
    unpack<T>(k0, x0);
    if (LAYOUT == 0) {
#pragma unroll
      for (int q = 0; q < P / 2; ++q) {
        y0[2 * q] = x0[2 * q] * cs[q].x - x0[2 * q + 1] * cs[q].y;
        y0[2 * q + 1] = x0[2 * q] * cs[q].y + x0[2 * q + 1] * cs[q].x;
      }
      st_page<!DELTA>(kv + b0, pack<T>(y0));
    } else {
      const int64_t b1 = b0 + HALF * (int64_t)sizeof(T);
      const uint4 k1 = ld_page<!DELTA>(job.src_k + b1);
      float x1[P], y1[P];
      unpack<T>(k1, x1);
#pragma unroll
      for (int q = 0; q < P; ++q) {
        y0[q] = x0[q] * cs[q].x - x1[q] * cs[q].y;
        y1[q] = x0[q] * cs[q].y + x1[q] * cs[q].x;
      }
      st_page<!DELTA>(kv + b0, pack<T>(y0));
      st_page<!DELTA>(kv + b1, pack<T>(y1));
    }
  }
}

static void launch_remat(int32_t dtype, int32_t d, int32_t layout, bool delta, bool copy_v,
                         const RematArgs& a, hipStream_t s) {
  const int32_t rows = a.n_jobs + (copy_v ? a.n_jobs - a.first_v : 0);
  if (a.n_jobs <= 0 || rows <= 0) return;
  dim3 g((uint32_t)std::max(a.wg_k, copy_v ? a.wg_v : 0), (uint32_t)rows), b(REMAT_TPB);
  KernelTimer tm("remat", s);
#define KVM_REMAT(T, D, LAY)                                                 \
  do {                                                                       \
    if (delta) remat_kernel<T, D, LAY, true, false><<<g, b, 0, s>>>(a);      \
    else if (copy_v) remat_kernel<T, D, LAY, false, true><<<g, b, 0, s>>>(a); \
    else remat_kernel<T, D, LAY, false, false><<<g, b, 0, s>>>(a);          \
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


// Registration copies: the raw K of listed block i (k_src + i * stride) into
// the K-side page of slot[i] (the shadow page, or the K view page in delta
// mode) and its V into the V view page, byte for byte. A launch takes up to
// REG_MAX blocks; their pages travel in the kernel arguments, so a launch
// needs no upload and leaves no buffer behind whose reuse would have to wait
// for it. Grid: x = 1 KiB stretch of the page, y = block; each thread copies
// one 16-byte piece of K and the same piece of V (the copy shape that moves
// bytes fastest here, as in the remat kernel).
static constexpr int REG_MAX = 448;

struct RegCopyArgs {
  const char* k_src;
  const char* v_src;
  char* k_dst;
  char* v_dst;
  int64_t stride;
  int64_t page_bytes;        // a multiple of 16
  int32_t n;
  int32_t slot[REG_MAX];
};

__global__ __launch_bounds__(REMAT_TPB) void register_copy_kernel(RegCopyArgs a) {
  const int32_t i = (int32_t)blockIdx.y;
  const int64_t off = ((int64_t)blockIdx.x * REMAT_TPB + threadIdx.x) * 16;
  if (i >= a.n || off >= a.page_bytes) return;
  const uint4 k = ld_page<true>(a.k_src + (int64_t)i * a.stride + off);
  const uint4 v = ld_page<true>(a.v_src + (int64_t)i * a.stride + off);
  const int64_t page = (int64_t)a.slot[i] * a.page_bytes;
  st_plain(a.k_dst + page + off, k);
  st_plain(a.v_dst + page + off, v);
}

// Run f(w) for w in [0, n) on up to n threads; a share whose thread cannot be
// started runs on the calling thread.
template <class F>
static void run_threads(int n, const F& f) {
  std::vector<std::thread> th;
  th.reserve((size_t)n);
  for (int w = 0; w < n; ++w) {
    try {
      th.emplace_back(f, w);
    } catch (const std::system_error&) {
      f(w);
    }
  }
  for (auto& t : th) t.join();
}

}  // namespace kvm

struct kvm_ctx {
  kvm_ctx_desc d{};
  int64_t page_bytes = 0;
  int device = 0;
  std::unique_ptr<kvm::BlockPool> pool;
  float2* d_table = nullptr;
  kvm::RematJob* d_jobs = nullptr;
  kvm::RematJob* h_jobs = nullptr;   // pinned [n_slots]
  int32_t* h_sel = nullptr;          // pinned [n_slots + 1]
  int32_t* h_page = nullptr;         // pinned [n_slots]
  hipStream_t side = nullptr;        // H2D of K pages (and of gathered pages)
  hipStream_t side_v = nullptr;      // H2D of V pages from pinned sources
  bool serialized = false;           // debug: every copy on the caller's stream
  std::vector<hipEvent_t> events;    // data-plane events (ids of dataplane.cpp)
  char* ring = nullptr;              // pinned [2][staging/2][2][page]
  std::unique_ptr<kvm::WorkerPool> workers;

  ~kvm_ctx() {
    workers.reset();
    for (auto e : events) (void)hipEventDestroy(e);
    if (side) (void)hipStreamDestroy(side);
    if (side_v) (void)hipStreamDestroy(side_v);
    if (d_table) (void)hipFree(d_table);
    if (d_jobs) (void)hipFree(d_jobs);
    if (h_jobs) (void)hipHostFree(h_jobs);
    if (h_sel) (void)hipHostFree(h_sel);
    if (h_page) (void)hipHostFree(h_page);
    if (ring) (void)hipHostFree(ring);
  }
};

namespace kvm {

// The data plane's device operations on HIP streams and events.
class HipEngine final : public Engine {
 public:
  HipEngine(kvm_ctx* c, hipStream_t s, const RematArgs& a, int32_t* page_table_dev)
      : c_(c), s_(s), a_(a), page_table_(page_table_dev) {}
  int ensure_events(int n) override {
    while ((int)c_->events.size() < n) {
      hipEvent_t e;
      KVM_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
      c_->events.push_back(e);
    }
    return KVM_OK;
  }
  int upload_plan(const RematPlan& p) override {
    // pinned staging of both lists; the previous call's uploads finished
    // before this call read its selection (same stream)
    std::copy(p.page.begin(), p.page.end(), c_->h_page);
    std::copy(p.jobs.begin(), p.jobs.end(), c_->h_jobs);
    if (p.n > 0)
      KVM_HIP(hipMemcpyAsync(page_table_, c_->h_page, (size_t)p.n * sizeof(int32_t),
                             hipMemcpyHostToDevice, s_));
    if (!p.jobs.empty())
      KVM_HIP(hipMemcpyAsync(c_->d_jobs, c_->h_jobs, p.jobs.size() * sizeof(RematJob),
                             hipMemcpyHostToDevice, s_));
    return KVM_OK;
  }
  int h2d(int stream, void* dst, const void* src, size_t bytes) override {
    KVM_HIP(hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, st(stream)));
    return KVM_OK;
  }
  int record(int stream, int ev) override {
    KVM_HIP(hipEventRecord(c_->events[(size_t)ev], st(stream)));
    return KVM_OK;
  }
  int wait(int stream, int ev) override {
    KVM_HIP(hipStreamWaitEvent(st(stream), c_->events[(size_t)ev], 0));
    return KVM_OK;
  }
  int host_wait(int ev) override {
    KVM_HIP(hipEventSynchronize(c_->events[(size_t)ev]));
    return KVM_OK;
  }
  int sync_all() override {
    const hipError_t a = hipStreamSynchronize(s_);
    const hipError_t b = hipStreamSynchronize(c_->side);
    const hipError_t v = hipStreamSynchronize(c_->side_v);
    return a == hipSuccess && b == hipSuccess && v == hipSuccess ? KVM_OK : KVM_EHIP;
  }
  int launch(int32_t first, int32_t n, bool delta, bool copy_v) override {
    const kvm_dims& dm = c_->d.dims;
    // the grid's second dimension holds the jobs (and their V rows): at most
    // REMAT_JOBS_PER_LAUNCH jobs per launch
    for (int32_t c0 = 0; c0 < n; c0 += REMAT_JOBS_PER_LAUNCH) {
      RematArgs a = a_;
      a.jobs = c_->d_jobs + first + c0;
      a.n_jobs = std::min(REMAT_JOBS_PER_LAUNCH, n - c0);
      // V rows start at the first job that copies V (device misses follow the
      // re-encodes in a plan; each job still checks its flag)
      a.first_v = a.n_jobs;
      if (copy_v)
        for (int32_t i = 0; i < a.n_jobs; ++i)
          if (c_->h_jobs[(size_t)(first + c0 + i)].flags & JOB_COPY_V) {
            a.first_v = i;
            break;
          }
      launch_remat(c_->d.dtype, dm.head_dim, c_->d.rope_layout, delta, copy_v, a, s_);
      KVM_HIP(hipGetLastError());
    }
    return KVM_OK;
  }

 private:
  hipStream_t st(int id) const {
    if (id == MAIN || c_->serialized) return s_;
    return id == SIDE_K ? c_->side : c_->side_v;
  }
  kvm_ctx* c_;
  hipStream_t s_;
  RematArgs a_;
  int32_t* page_table_;
};

static int ctx_create(const kvm_ctx_desc* desc, kvm_ctx** out) {
  clear_error();
  KVM_CHECK_ARG(desc && out, "null pointer");
  KVM_TRY(check_dims(&desc->dims, desc->dtype));
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
  const kvm_dims& dm = desc->dims;
  const int64_t page_bytes = (int64_t)dm.n_layers * dm.n_kv_heads * dm.block_tokens *
                             dm.head_dim * dtype_bytes(desc->dtype);
  {
    const size_t pool = (size_t)desc->n_slots * (size_t)page_bytes;
    KVM_CHECK_RANGE(desc->k_view, pool, RANGE_DEVICE, "k_view");
    KVM_CHECK_RANGE(desc->v_view, pool, RANGE_DEVICE, "v_view");
    if (desc->k_shadow) KVM_CHECK_RANGE(desc->k_shadow, pool, RANGE_DEVICE, "k_shadow");
  }
  std::unique_ptr<kvm_ctx> c(new kvm_ctx());
  c->d = *desc;
  if (c->d.batch_blocks <= 0) c->d.batch_blocks = 64;
  if (c->d.staging_blocks < 2 * c->d.batch_blocks) c->d.staging_blocks = 2 * c->d.batch_blocks;
  c->page_bytes = page_bytes;
  PoolLayout L;
  L.k_view = (char*)desc->k_view;
  L.v_view = (char*)desc->v_view;
  L.k_shadow = (char*)desc->k_shadow;
  L.page_bytes = page_bytes;
  L.n_slots = desc->n_slots;
  L.block_tokens = dm.block_tokens;
  L.delta_limit = desc->delta_limit;
  L.max_pos = desc->max_pos;
  L.max_blocks = desc->max_blocks;
  c->pool.reset(new BlockPool(L));
#define KVM_HIP_C(call)                                                              \
  do {                                                                               \
    hipError_t e_ = (call);                                                          \
    if (e_ != hipSuccess) {                                                          \
      set_error("%s failed: %s", #call, hipGetErrorString(e_));                     \
      return e_ == hipErrorOutOfMemory ? KVM_ENOMEM : KVM_EHIP;                      \
    }                                                                                \
  } while (0)
  KVM_HIP_C(hipGetDevice(&c->device));
  // RoPE table: angle p * theta_t in float64, cos/sin rounded once to fp32.
  const int half = dm.head_dim / 2;
  std::vector<float2> table((size_t)desc->max_pos * half);
  std::vector<double> theta(half);
  for (int t = 0; t < half; ++t) theta[t] = std::pow(desc->rope_theta, -2.0 * t / dm.head_dim);
  {
    const int nth = (int)std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
    const int64_t max_pos = desc->max_pos;
    run_threads(nth, [&table, &theta, half, nth, max_pos](int w) {
      for (int64_t p = w; p < max_pos; p += nth)
        for (int t = 0; t < half; ++t) {
          const double ang = (double)p * theta[t];
          table[(size_t)p * half + t] = make_float2((float)std::cos(ang), (float)std::sin(ang));
        }
    });
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
  *out = c.release();
  return KVM_OK;
}

static int ctx_build_index_rope(kvm_ctx* c, const void* k_rope, int64_t block_stride,
                                int64_t first_block, int64_t n_blocks, int64_t pos0,
                                void* index, int64_t index_cap_blocks, void* stream) {
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

static int ctx_set_source(kvm_ctx* c, int64_t first_block, int64_t n_blocks, const void* k_base,
                          const void* v_base, int64_t block_stride, int32_t loc) {
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
  return c->pool->set_source(first_block, n_blocks, (const char*)k_base, (const char*)v_base,
                             block_stride, loc);
}

static int ctx_set_gather(kvm_ctx* c, int64_t first_block, int64_t n_blocks, kvm_gather_fn fn,
                          void* user) {
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
  if (!c->workers) {
    const int n = (int)std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
    c->workers.reset(new WorkerPool(n));
  }
  return c->pool->set_gather(first_block, n_blocks, fn, user);
}

// Registration of blocks ids[0..n) (strictly ascending) whose raw K and V
// sit at k_raw / v_raw + i * block_stride (device): pages by the pool's rule,
// then the copies on `stream` (one kernel launch per REG_MAX blocks when
// sources, stride and pages are 16-byte aligned, else one copy per page).
static int ctx_register(kvm_ctx* c, const int64_t* ids, int64_t n, const void* k_raw,
                        const void* v_raw, int64_t block_stride, void* stream) {
  KVM_CHECK_ARG(k_raw && v_raw, "null pointer");
  KVM_CHECK_ARG(block_stride >= c->page_bytes, "block_stride");
  for (int64_t i = 0; i < n; ++i)
    KVM_CHECK_ARG(ids[i] >= 0 && ids[i] < c->d.max_blocks && (i == 0 || ids[i] > ids[i - 1]),
                  "block list entry %lld (block %lld): out of range or not ascending",
                  (long long)i, (long long)ids[i]);
  if (n == 0) return KVM_OK;
  const size_t span = (size_t)((n - 1) * block_stride + c->page_bytes);
  KVM_CHECK_RANGE(k_raw, span, RANGE_DEVICE, "k_raw");
  KVM_CHECK_RANGE(v_raw, span, RANGE_DEVICE, "v_raw");
  hipStream_t s = as_stream(stream);
  std::vector<int32_t> slots;
  KVM_TRY(c->pool->register_list(ids, n, &slots));
  // raw K lands in the shadow page (in delta mode in the K page, rotated at
  // the block's first selection); V in the V page
  char* kdst = (char*)(c->d.delta_limit > 0 ? c->d.k_view : c->d.k_shadow);
  char* vdst = (char*)c->d.v_view;
  const bool aligned = ((uintptr_t)k_raw % 16 == 0) && ((uintptr_t)v_raw % 16 == 0) &&
                       block_stride % 16 == 0 && c->page_bytes % 16 == 0;
  hipError_t e = hipSuccess;
  int64_t at = 0;
  if (aligned) {
    RegCopyArgs a{};
    a.k_dst = kdst;
    a.v_dst = vdst;
    a.stride = block_stride;
    a.page_bytes = c->page_bytes;
    const uint32_t parts = (uint32_t)((c->page_bytes / 16 + REMAT_TPB - 1) / REMAT_TPB);
    KernelTimer tm("register_copy", s);
    for (; at < n && e == hipSuccess; at += REG_MAX) {
      a.n = (int32_t)std::min<int64_t>(REG_MAX, n - at);
      a.k_src = (const char*)k_raw + at * block_stride;
      a.v_src = (const char*)v_raw + at * block_stride;
      for (int32_t j = 0; j < a.n; ++j) a.slot[j] = slots[(size_t)(at + j)];
      register_copy_kernel<<<dim3(parts, (uint32_t)a.n), dim3(REMAT_TPB), 0, s>>>(a);
      e = hipGetLastError();
    }
  } else {
    for (; at < n && e == hipSuccess; ++at) {
      const int64_t off = (int64_t)slots[(size_t)at] * c->page_bytes;
      e = hipMemcpyAsync(kdst + off, (const char*)k_raw + at * block_stride, c->page_bytes,
                         hipMemcpyDeviceToDevice, s);
      if (e == hipSuccess)
        e = hipMemcpyAsync(vdst + off, (const char*)v_raw + at * block_stride, c->page_bytes,
                           hipMemcpyDeviceToDevice, s);
    }
  }
  if (e != hipSuccess) {
    c->pool->release_list(ids, n);
    set_error("registering %lld blocks: %s", (long long)n, hipGetErrorString(e));
    return KVM_EHIP;
  }
  return KVM_OK;
}

static int ctx_register_resident(kvm_ctx* c, int64_t first_block, int64_t n_blocks,
                                 const void* k_raw, const void* v_raw, int64_t block_stride,
                                 void* stream) {
  clear_error();
  KVM_CHECK_ARG(c, "ctx is NULL");
  KVM_CHECK_ARG(first_block >= 0 && n_blocks >= 0 && first_block + n_blocks <= c->d.max_blocks,
                "block range outside the record capacity");
  std::vector<int64_t> ids((size_t)n_blocks);
  for (int64_t i = 0; i < n_blocks; ++i) ids[(size_t)i] = first_block + i;
  return ctx_register(c, ids.data(), n_blocks, k_raw, v_raw, block_stride, stream);
}

static int ctx_register_resident_list(kvm_ctx* c, const int64_t* blocks, int64_t n_blocks,
                                      const void* k_raw, const void* v_raw, int64_t block_stride,
                                      void* stream) {
  clear_error();
  KVM_CHECK_ARG(c, "ctx is NULL");
  KVM_CHECK_ARG(n_blocks >= 0 && n_blocks <= c->d.max_blocks && (blocks || n_blocks == 0),
                "block list");
  return ctx_register(c, blocks, n_blocks, k_raw, v_raw, block_stride, stream);
}

static int rematerialize(kvm_ctx* c, const int32_t* sel_dev, const int32_t* n_sel_dev,
                         int32_t* page_table_dev, kvm_remat_stats* stats, void* stream) {
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
  KVM_CHECK_RANGE(sel_dev, (size_t)n * sizeof(int32_t), RANGE_DEVICE, "sel");
  KVM_CHECK_RANGE(page_table_dev, (size_t)n * sizeof(int32_t), RANGE_DEVICE, "page_table");
  if (n > 0) {
    KVM_HIP(hipMemcpyAsync(sel, sel_dev, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToHost, s));
    KVM_HIP(hipStreamSynchronize(s));
  }
  // 2. Validate, plan and queue; a failure part way is rolled back.
  const kvm_dims& dm = c->d.dims;
  RematArgs a{};
  // work items per page: one 16-byte piece (interleaved pairs) or one piece
  // pair (half-split pairs) of every row
  const int32_t R = remat_units_per_item(dtype_bytes(c->d.dtype));
  a.units = dm.n_layers * dm.n_kv_heads;
  const int64_t ppr = (int64_t)dm.head_dim * dtype_bytes(c->d.dtype) / 16;
  a.items = (int64_t)((a.units + R - 1) / R) * B * (c->d.rope_layout == 0 ? ppr : ppr / 2);
  a.wg_k = (int32_t)((a.items + REMAT_TPB - 1) / REMAT_TPB);
  a.wg_v = (int32_t)((c->page_bytes / 16 + REMAT_TPB - 1) / REMAT_TPB);
  a.page_bytes = c->page_bytes;
  a.k_view = (char*)c->d.k_view;
  a.v_view = (char*)c->d.v_view;
  a.k_shadow = (char*)c->d.k_shadow;
  a.table = c->d_table;
  HipEngine eng(c, s, a, page_table_dev);
  StagingConfig cfg;
  cfg.batch_blocks = c->d.batch_blocks;
  cfg.staging_blocks = c->d.staging_blocks;
  cfg.ring = c->ring;
  cfg.workers = c->workers.get();
  return apply_selection(eng, *c->pool, sel, n, cfg, stats);
}

}  // namespace kvm

extern "C" int kvm_ctx_create(const kvm_ctx_desc* desc, kvm_ctx** out) {
  return kvm::guarded([&] { return kvm::ctx_create(desc, out); });
}

extern "C" void kvm_ctx_destroy(kvm_ctx* ctx) {
  if (!ctx) return;
  (void)hipStreamSynchronize(ctx->side);
  (void)hipStreamSynchronize(ctx->side_v);
  delete ctx;
}

extern "C" int kvm_ctx_build_index_rope(kvm_ctx* c, const void* k_rope, int64_t block_stride,
                                        int64_t first_block, int64_t n_blocks, int64_t pos0,
                                        void* index, int64_t index_cap_blocks, void* stream) {
  return kvm::guarded([&] {
    return kvm::ctx_build_index_rope(c, k_rope, block_stride, first_block, n_blocks, pos0, index,
                                     index_cap_blocks, stream);
  });
}

extern "C" int kvm_ctx_set_source(kvm_ctx* c, int64_t first_block, int64_t n_blocks,
                                  const void* k_base, const void* v_base, int64_t block_stride,
                                  int32_t loc) {
  return kvm::guarded([&] {
    return kvm::ctx_set_source(c, first_block, n_blocks, k_base, v_base, block_stride, loc);
  });
}

extern "C" int kvm_ctx_set_gather(kvm_ctx* c, int64_t first_block, int64_t n_blocks,
                                  kvm_gather_fn fn, void* user) {
  return kvm::guarded([&] { return kvm::ctx_set_gather(c, first_block, n_blocks, fn, user); });
}

extern "C" int kvm_ctx_register_resident(kvm_ctx* c, int64_t first_block, int64_t n_blocks,
                                         const void* k_raw, const void* v_raw,
                                         int64_t block_stride, void* stream) {
  return kvm::guarded([&] {
    return kvm::ctx_register_resident(c, first_block, n_blocks, k_raw, v_raw, block_stride,
                                      stream);
  });
}

extern "C" int kvm_ctx_register_resident_list(kvm_ctx* c, const int64_t* blocks,
                                              int64_t n_blocks, const void* k_raw,
                                              const void* v_raw, int64_t block_stride,
                                              void* stream) {
  return kvm::guarded([&] {
    return kvm::ctx_register_resident_list(c, blocks, n_blocks, k_raw, v_raw, block_stride,
                                           stream);
  });
}

extern "C" int kvm_ctx_evict(kvm_ctx* c, int64_t first_block, int64_t n_blocks) {
  using namespace kvm;
  return guarded([&]() -> int {
    clear_error();
    KVM_CHECK_ARG(c, "ctx is NULL");
    KVM_CHECK_ARG(first_block >= 0 && n_blocks >= 0 && first_block + n_blocks <= c->d.max_blocks,
                  "block range outside the record capacity");
    return c->pool->evict(first_block, n_blocks);
  });
}

extern "C" int kvm_ctx_block_deltas(kvm_ctx* c, int64_t block, int32_t* n_delta) {
  using namespace kvm;
  return guarded([&]() -> int {
    KVM_CHECK_ARG(c && n_delta && block >= 0 && block < c->d.max_blocks, "block out of range");
    const BlockRec& r = c->pool->rec(block);
    *n_delta = r.slot >= 0 ? r.n_delta : 0;
    return KVM_OK;
  });
}

extern "C" int kvm_ctx_sync(kvm_ctx* c) {
  using namespace kvm;
  return guarded([&]() -> int {
    KVM_CHECK_ARG(c, "ctx is NULL");
    KVM_HIP(hipStreamSynchronize(c->side));
    KVM_HIP(hipStreamSynchronize(c->side_v));
    return KVM_OK;
  });
}

extern "C" int kvm_ctx_set_serialized(kvm_ctx* c, int32_t on) {
  using namespace kvm;
  return guarded([&]() -> int {
    KVM_CHECK_ARG(c, "ctx is NULL");
    // earlier side-stream copies must not overlap work of the other mode
    KVM_HIP(hipStreamSynchronize(c->side));
    KVM_HIP(hipStreamSynchronize(c->side_v));
    c->serialized = on != 0;
    return KVM_OK;
  });
}

extern "C" int kvm_ctx_block_state(kvm_ctx* c, int64_t block, int32_t* slot, int32_t* baked) {
  using namespace kvm;
  return guarded([&]() -> int {
    KVM_CHECK_ARG(c && block >= 0 && block < c->d.max_blocks, "block out of range");
    const BlockRec& r = c->pool->rec(block);
    if (slot) *slot = r.slot;
    if (baked) *baked = r.baked;
    return KVM_OK;
  });
}

extern "C" int kvm_rematerialize(kvm_ctx* c, const int32_t* sel_dev, const int32_t* n_sel_dev,
                                 int32_t* page_table_dev, kvm_remat_stats* stats_host,
                                 void* stream) {
  return kvm::guarded([&] {
    return kvm::rematerialize(c, sel_dev, n_sel_dev, page_table_dev, stats_host, stream);
  });
}
