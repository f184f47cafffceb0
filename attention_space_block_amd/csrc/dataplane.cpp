// Sequencing of one rematerialization's device work (KVMem Sec. 4.4, Fig. 3),
// host only.
#include "dataplane.hpp"

#include <algorithm>
#include <atomic>

namespace kvm {

WorkerPool::WorkerPool(int n) {
  try {
    for (int i = 0; i < n; ++i) th_.emplace_back([this] { loop(); });
  } catch (...) {
    // no half-built pool: stop and join the workers that did start
    {
      std::lock_guard<std::mutex> g(m_);
      stop_ = true;
    }
    cv_.notify_all();
    for (auto& t : th_) t.join();
    throw;
  }
}

WorkerPool::~WorkerPool() {
  {
    std::lock_guard<std::mutex> g(m_);
    stop_ = true;
  }
  cv_.notify_all();
  for (auto& t : th_) t.join();
}

void WorkerPool::run(int n, const std::function<void(int)>& f) {
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

void WorkerPool::loop() {
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

namespace {
// Event ids: 0 start, 1 and 2 the ring halves, then two per DMA batch (SIDE_K,
// SIDE_V) and one per gathered batch.
enum { EV_START = 0, EV_RING0 = 1, EV_FIRST_BATCH = 3 };
}  // namespace

int plan_events(const RematPlan& p, const StagingConfig& cfg) {
  const int32_t bb = cfg.batch_blocks;
  const int32_t gb = std::min(bb, std::max(1, cfg.staging_blocks / 2));
  return EV_FIRST_BATCH + 2 * ((p.n_dma + bb - 1) / bb) + (p.n_gather + gb - 1) / gb;
}

int run_plan(Engine& e, const BlockPool& pool, RematPlan& p, const int32_t* sel,
             const StagingConfig& cfg, PlanProgress* prog) {
  const PoolLayout& L = pool.layout();
  const int64_t pb = L.page_bytes;
  *prog = PlanProgress{};
  KVM_TRY(e.ensure_events(plan_events(p, cfg)));
  // Copies into pages must not start before the caller's stream reached this
  // call (earlier work may still read the pages being replaced). The staged
  // pages are disjoint from the pages the first launches write, so the copies
  // run alongside them.
  const bool staged = p.n_dma + p.n_gather > 0;
  if (staged) {
    KVM_TRY(e.record(Engine::MAIN, EV_START));
    KVM_TRY(e.wait(Engine::SIDE_K, EV_START));
    KVM_TRY(e.wait(Engine::SIDE_V, EV_START));
  }
  auto launch = [&](int32_t first, int32_t n, bool delta, bool copy_v = false) -> int {
    if (n <= 0) return KVM_OK;
    const int rc = e.launch(first, n, delta, copy_v);
    if (rc) {
      prog->unknown = n;
      return rc;
    }
    prog->done = first + n;
    return KVM_OK;
  };
  // 1. Hits re-encoded from raw K in HBM and misses from device sources (one
  //    launch: split into a K-only and a K+V launch it was slower, 9.7 against
  //    9.3 ms at the 1M-token view), then delta shifts. Staged batches below
  //    never copy V on the device (their V pages arrive by DMA), so they run
  //    the K-only kernel.
  KVM_TRY(launch(0, p.n_full, false, p.n_full > p.n_reencode));
  KVM_TRY(launch(p.n_full, p.n_delta, true));
  const int32_t bb = cfg.batch_blocks;
  int ev = EV_FIRST_BATCH;
  // 2. Misses from pinned host memory: DMA straight into the pages, batched;
  //    K pages on SIDE_K and V pages on SIDE_V (two copy engines); the
  //    caller's stream waits per batch and rotates it while the next transfers.
  const int32_t first_dma = p.n_full + p.n_delta;
  for (int32_t first = first_dma; first < first_dma + p.n_dma; first += bb) {
    const int32_t cnt = std::min(bb, first_dma + p.n_dma - first);
    int32_t pages_in = 0;
    for (int32_t q = 0; q < cnt; ++q) {
      const RematJob& jb = p.jobs[(size_t)(first + q)];
      const BlockRec& r = pool.rec(sel[jb.pad]);
      KVM_TRY(e.h2d(Engine::SIDE_K, (void*)jb.src_k, r.src_k, (size_t)pb));
      ++pages_in;
      if (!(jb.flags & JOB_K_ONLY)) {
        KVM_TRY(e.h2d(Engine::SIDE_V, L.v_view + (int64_t)jb.slot * pb, r.src_v, (size_t)pb));
        ++pages_in;
      }
    }
    KVM_TRY(e.record(Engine::SIDE_K, ev));
    KVM_TRY(e.wait(Engine::MAIN, ev));
    KVM_TRY(e.record(Engine::SIDE_V, ev + 1));
    KVM_TRY(e.wait(Engine::MAIN, ev + 1));
    ev += 2;
    KVM_TRY(launch(first, cnt, false));
    p.st.h2d_bytes += (int64_t)pages_in * pb;
    ++p.st.batches;
  }
  // 3. Gathered misses: host workers pack raw K/V into one half of the pinned
  //    ring while the other half is in flight; a half is refilled only after
  //    the event of the copies that read it.
  if (p.n_gather > 0) {
    const int32_t half_blocks = cfg.staging_blocks / 2;
    const int32_t gb = std::min(bb, half_blocks);
    const int32_t first_g = first_dma + p.n_dma;
    bool half_busy[2] = {false, false};
    int rc = KVM_OK;
    for (int32_t bi = 0, first = first_g; first < first_g + p.n_gather; ++bi, first += gb) {
      const int h = bi & 1;
      if (half_busy[h]) {
        rc = e.host_wait(EV_RING0 + h);
        if (rc) break;
      }
      const int32_t cnt = std::min(gb, first_g + p.n_gather - first);
      char* base = cfg.ring + (size_t)h * half_blocks * 2 * pb;
      std::atomic<int> gerr{0};
      cfg.workers->run(cnt * 2, [&](int t) {
        const RematJob& jb = p.jobs[(size_t)(first + t / 2)];
        if ((t & 1) && (jb.flags & JOB_K_ONLY)) return;   // rebuild: the V page is intact
        const int64_t blk = sel[jb.pad];
        const Gather& g = pool.gathers()[(size_t)pool.rec(blk).gather];
        char* dst = base + ((size_t)(t / 2) * 2 + (t & 1)) * pb;
        if (g.fn(g.user, blk, t & 1, dst) != 0) gerr.store(1);
      });
      if (gerr.load()) {
        set_error("host gather callback failed");
        rc = KVM_ERANGE;
        break;
      }
      int32_t pages_in = 0;
      for (int32_t q = 0; q < cnt && !rc; ++q) {
        const RematJob& jb = p.jobs[(size_t)(first + q)];
        const char* src = base + (size_t)q * 2 * pb;
        rc = e.h2d(Engine::SIDE_K, (void*)jb.src_k, src, (size_t)pb);
        ++pages_in;
        if (!rc && !(jb.flags & JOB_K_ONLY)) {
          rc = e.h2d(Engine::SIDE_K, L.v_view + (int64_t)jb.slot * pb, src + pb, (size_t)pb);
          ++pages_in;
        }
      }
      if (!rc) rc = e.record(Engine::SIDE_K, EV_RING0 + h);
      if (rc) break;
      half_busy[h] = true;
      rc = e.record(Engine::SIDE_K, ev);
      if (!rc) rc = e.wait(Engine::MAIN, ev);
      if (rc) break;
      ++ev;
      rc = launch(first, cnt, false);
      if (rc) break;
      p.st.h2d_bytes += (int64_t)pages_in * pb;
      ++p.st.batches;
    }
    // The ring must not be refilled by a later call before its copies finish.
    for (int h = 0; h < 2; ++h)
      if (half_busy[h]) {
        const int rc2 = e.host_wait(EV_RING0 + h);
        if (!rc) rc = rc2;
      }
    if (rc) return rc;
  }
  return KVM_OK;
}

int apply_selection(Engine& e, BlockPool& pool, const int32_t* sel, int32_t n,
                    const StagingConfig& cfg, kvm_remat_stats* st) {
  KVM_TRY(pool.validate(sel, n));
  RematPlan plan;
  KVM_TRY(pool.plan(sel, n, &plan));
  PlanProgress prog;
  int rc = KVM_OK;
  try {
    rc = e.upload_plan(plan);
    if (!rc) rc = run_plan(e, pool, plan, sel, cfg, &prog);
  } catch (...) {
    (void)e.sync_all();
    pool.rollback(plan, prog.done, prog.unknown);
    throw;
  }
  if (rc) {
    (void)e.sync_all();
    pool.rollback(plan, prog.done, prog.unknown);
    return rc;
  }
  if (st) *st = plan.st;
  return KVM_OK;
}

}  // namespace kvm
