// Sequencing of one rematerialization's device work (KVMem Sec. 4.4, Fig. 3:
// packed, pipelined staging of misses overlapped with the GPU scatter and
// re-RoPE), host only.
//
// The order of copies, events and kernel launches is fixed here, against a
// small interface of device operations (Engine). The library implements it
// with HIP streams and events; the host tests implement it with a fake that
// defers every device operation as long as the recorded dependencies allow,
// so a missing wait shows up as wrong page contents or a staging hazard.
#pragma once

#include <stdint.h>

#include <condition_variable>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

#include "pool.hpp"

namespace kvm {

// Device operations in stream order. Streams: MAIN (the caller's stream, where
// the kernels run), SIDE_K and SIDE_V (host-to-device copies). Events are
// small integers; ensure_events(n) makes ids [0, n) usable.
class Engine {
 public:
  enum { MAIN = 0, SIDE_K = 1, SIDE_V = 2 };
  virtual ~Engine() = default;
  virtual int ensure_events(int n) = 0;
  // Queue, on MAIN, the upload of the plan's page table and job list (the
  // kernels read the job list from the device).
  virtual int upload_plan(const RematPlan& p) = 0;
  // Asynchronous copy from pinned host memory to device memory on `stream`.
  virtual int h2d(int stream, void* dst, const void* src, size_t bytes) = 0;
  virtual int record(int stream, int event) = 0;
  virtual int wait(int stream, int event) = 0;         // `stream` waits for `event`
  virtual int host_wait(int event) = 0;                // the host waits for `event`
  virtual int sync_all() = 0;                          // the host waits for all three streams
  // Remat kernel over jobs [first, first + n) of the device job list, on MAIN;
  // jobs that copy V (JOB_COPY_V) only in launches with copy_v.
  virtual int launch(int32_t first, int32_t n, bool delta, bool copy_v) = 0;
};

// Host workers that run the gather callbacks of one batch concurrently.
class WorkerPool {
 public:
  explicit WorkerPool(int n);
  ~WorkerPool();
  // Run f(i) for i in [0, n) on the workers; returns when all are done.
  void run(int n, const std::function<void(int)>& f);

 private:
  void loop();
  std::vector<std::thread> th_;
  std::mutex m_;
  std::condition_variable cv_, done_cv_;
  const std::function<void(int)>* f_ = nullptr;
  int n_ = 0, next_ = 0, done_ = 0;
  uint64_t gen_ = 0;
  bool stop_ = false;
};

struct StagingConfig {
  int32_t batch_blocks = 64;    // misses per copy batch (one event per batch and stream)
  int32_t staging_blocks = 128; // pinned ring capacity in blocks (two halves)
  char* ring = nullptr;         // pinned [2][staging_blocks / 2][2][page] (gathered sources)
  WorkerPool* workers = nullptr;
};

// Progress of run_plan, for a rollback after a failure: jobs [0, done) ran,
// jobs [done, done + unknown) may have run.
struct PlanProgress {
  int32_t done = 0;
  int32_t unknown = 0;
};

// Number of events run_plan may use for a plan.
int plan_events(const RematPlan& p, const StagingConfig& cfg);

// Queue the device work of a plan whose job list is already on the device:
// re-encode launches first, then the misses batch by batch, each batch's
// kernel after its copies (DMA straight into the pages for pinned sources, K
// on SIDE_K and V on SIDE_V; gathered sources through the two ring halves,
// each refilled only after the copies that read it). Adds h2d bytes and
// batches to p.st. On error returns the status with `prog` set.
int run_plan(Engine& e, const BlockPool& pool, RematPlan& p, const int32_t* sel,
             const StagingConfig& cfg, PlanProgress* prog);

// One working-set update once the selection is on the host: validate it,
// plan it against the pool, queue the plan's upload and device work. On a
// failure after planning (or an exception) every stream is drained and the
// block records are rolled back (BlockPool::rollback), so every resident
// block's page is what its record says; a retry re-stages the rest. *st
// receives the statistics on success.
int apply_selection(Engine& e, BlockPool& pool, const int32_t* sel, int32_t n,
                    const StagingConfig& cfg, kvm_remat_stats* st);

}  // namespace kvm
