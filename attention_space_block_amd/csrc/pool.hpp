// Block records and the bounded GPU page pool (KVMem Sec. 4.4 working sets and
// Sec. 5 block records), host only.
//
// A BlockPool keeps one record per block (its pool page, the compact position
// its K page is encoded at, its lower-tier source) and plans one working-set
// update: selected blocks that hold a page are hits (re-encoded only when
// their compact position changed), the others are misses that take a free
// page or the page of the least recently used block outside the new view
// (ties to the lower block id). The plan is a list of jobs for the device
// (one per block whose page must be written) grouped by where their raw K
// comes from, plus an undo log, so a failure while the jobs are being queued
// can be rolled back to a state in which every resident block's page is what
// its record says.
//
// Nothing here touches the device; job source pointers are device addresses
// formed from the pool layout and never dereferenced on the host.
#pragma once

#include <stdint.h>

#include <vector>

#include "host_common.hpp"

namespace kvm {

// One block's page write, as the remat kernel reads it.
struct RematJob {
  const char* src_k;  // raw pre-RoPE K of the block (device)
  const char* src_v;  // raw V (device) when flags & JOB_COPY_V
  int32_t slot;
  int32_t pos;        // compact position of token 0, or the signed shift of a delta job
  int32_t flags;
  int32_t pad;        // staged jobs: index of the block in the selection
};
// JOB_DELTA: rotate every token by the same signed shift `pos` (an in-place
// delta re-RoPE) instead of by its absolute position pos + j. JOB_K_ONLY is
// host-side only: a staged rebuild that moves raw K but keeps the V page.
enum { JOB_COPY_V = 2, JOB_DELTA = 4, JOB_K_ONLY = 8 };

struct BlockRec {
  int32_t slot = -1;
  int32_t baked = -1;        // compact position encoded in the K page (-1: stale)
  int64_t last_used = -1;    // step of the last selection (or registration) that touched it
  int32_t src = KVM_SRC_NONE;
  int32_t gather = -1;       // index into the gather table for gathered sources
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

// Device addresses of the caller's page pool and the sizes the planner needs.
struct PoolLayout {
  char* k_view = nullptr;
  char* v_view = nullptr;
  char* k_shadow = nullptr;
  int64_t page_bytes = 0;
  int32_t n_slots = 0;
  int32_t block_tokens = 32;
  int32_t delta_limit = 0;
  int32_t max_pos = 0;
  int64_t max_blocks = 0;
};

// How a job's raw K reaches the device, which decides the job's group.
enum JobKind {
  JK_REENCODE = 0,   // hit re-encoded from raw K already in HBM (shadow, device source,
                     // or the raw K page of a freshly registered block in delta mode)
  JK_DEVICE_MISS,    // miss whose lower-tier copy is in HBM (K rotated, V copied)
  JK_DELTA,          // hit rotated in place by its position shift
  JK_DMA,            // miss or rebuild staged by DMA from pinned host memory
  JK_GATHER,         // miss or rebuild staged through the pinned ring by a gather callback
};

struct RematPlan {
  int32_t n = 0;                       // blocks in the new view
  std::vector<RematJob> jobs;          // [full][delta][dma][gather]
  std::vector<int64_t> job_block;      // block of each job
  std::vector<int8_t> job_kind;        // JobKind of each job
  int32_t n_full = 0, n_delta = 0, n_dma = 0, n_gather = 0;
  int32_t n_reencode = 0;              // the first n_full jobs: re-encodes, then device misses
  std::vector<int32_t> page;           // page table [n]
  kvm_remat_stats st{};
  struct Undo {
    int64_t block;
    BlockRec rec;
  };
  std::vector<Undo> undo;              // records before planning, one per job
};

class BlockPool {
 public:
  explicit BlockPool(const PoolLayout& layout);   // may throw std::bad_alloc

  const PoolLayout& layout() const { return L_; }
  int64_t step() const { return step_; }
  const BlockRec& rec(int64_t b) const { return rec_[(size_t)b]; }
  const std::vector<Gather>& gathers() const { return gathers_; }

  // Record the lower-tier copy of blocks [first, first + n) (pointers already
  // checked by the caller). A resident block that relied on its old device
  // copy loses its page.
  int set_source(int64_t first, int64_t n, const char* k_base, const char* v_base,
                 int64_t stride, int32_t loc);
  int set_gather(int64_t first, int64_t n, kvm_gather_fn fn, void* user);

  // Freshly prefilled blocks ids[0..n) (strictly ascending, checked by the
  // caller) become resident at the current step: a free page, else the page
  // of the least recently used block outside the current view. All or
  // nothing: KVM_ENOMEM and no change when they do not fit. slots[i] receives
  // block ids[i]'s page.
  int register_list(const int64_t* ids, int64_t n, std::vector<int32_t>* slots);
  // The same for the range [first, first + n).
  int register_blocks(int64_t first, int64_t n, std::vector<int32_t>* slots);
  // Undo a registration after its copies could not be queued: the blocks
  // lose their pages (the pages' contents are unknown).
  void release_list(const int64_t* ids, int64_t n);
  void release(int64_t first, int64_t n);

  int evict(int64_t first, int64_t n);

  // Check a selection (ascending ids, each resident or backed by a source)
  // before any state changes.
  int validate(const int32_t* sel, int32_t n) const;
  // Plan the working-set update for a validated selection; changes the
  // records (undo log in the plan).
  int plan(const int32_t* sel, int32_t n, RematPlan* p);
  // Restore a consistent state after the plan's device work failed part way:
  // jobs [0, done) completed, jobs [done, done + unknown) may or may not have
  // run, the rest never started. Hits whose page was not written get their
  // old record back; hits whose page may have been written are marked stale
  // (their raw K is intact), or in delta mode, where the page itself was
  // being rotated, lose their page; misses and staged blocks that did not
  // complete lose their page.
  void rollback(const RematPlan& p, int32_t done, int32_t unknown);

 private:
  int32_t take_slot(std::vector<std::pair<int64_t, int64_t>>& lru, size_t& pos,
                    int32_t* evicted);
  void free_slot_of(BlockRec& r);
  void release_if_unbacked(BlockRec& r);
  std::vector<std::pair<int64_t, int64_t>> lru_outside_view() const;

  PoolLayout L_;
  std::vector<BlockRec> rec_;
  std::vector<int64_t> slot_block_;
  std::vector<int32_t> free_slots_;
  std::vector<Gather> gathers_;
  int64_t step_ = 0;
};

}  // namespace kvm
