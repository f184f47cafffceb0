// Block records, the bounded page pool and the working-set plan (KVMem Sec.
// 4.4, Sec. 5), host only.
#include "pool.hpp"

#include <algorithm>

namespace kvm {

BlockPool::BlockPool(const PoolLayout& layout) : L_(layout) {
  rec_.resize((size_t)L_.max_blocks);
  slot_block_.assign((size_t)L_.n_slots, -1);
  free_slots_.reserve((size_t)L_.n_slots);
  for (int32_t s = L_.n_slots - 1; s >= 0; --s) free_slots_.push_back(s);
}

void BlockPool::free_slot_of(BlockRec& r) {
  if (r.slot >= 0) {
    slot_block_[(size_t)r.slot] = -1;
    free_slots_.push_back(r.slot);
  }
  r.slot = -1;
  r.baked = -1;
  r.raw_in_shadow = false;
  r.page_raw = false;
  r.n_delta = 0;
}

// A resident page whose re-encode source is the block's device-resident
// lower-tier copy must not outlive a change of that source: reclaim it.
void BlockPool::release_if_unbacked(BlockRec& r) {
  // in delta mode a page's K is self-contained; only rebuilds read the source
  if (r.slot < 0 || r.raw_in_shadow || L_.delta_limit > 0) return;
  free_slot_of(r);
}

// Resident blocks outside the current view, least recently used first (ties
// to the lower block id): the eviction order.
std::vector<std::pair<int64_t, int64_t>> BlockPool::lru_outside_view() const {
  std::vector<std::pair<int64_t, int64_t>> lru;
  for (int32_t sl = 0; sl < L_.n_slots; ++sl) {
    const int64_t b = slot_block_[(size_t)sl];
    if (b >= 0 && rec_[(size_t)b].last_used < step_) lru.emplace_back(rec_[(size_t)b].last_used, b);
  }
  std::sort(lru.begin(), lru.end());
  return lru;
}

// A free page, else the page of the next block in `lru` that is still
// resident and outside the current view (evicting it); -1 if none.
int32_t BlockPool::take_slot(std::vector<std::pair<int64_t, int64_t>>& lru, size_t& pos,
                             int32_t* evicted) {
  if (!free_slots_.empty()) {
    const int32_t s = free_slots_.back();
    free_slots_.pop_back();
    return s;
  }
  while (pos < lru.size()) {
    const int64_t b = lru[pos++].second;
    BlockRec& r = rec_[(size_t)b];
    if (r.slot < 0 || r.last_used >= step_) continue;
    const int32_t s = r.slot;
    r.slot = -1;
    r.baked = -1;
    r.raw_in_shadow = false;
    r.page_raw = false;
    r.n_delta = 0;
    slot_block_[(size_t)s] = -1;
    ++*evicted;
    return s;
  }
  return -1;
}

int BlockPool::set_source(int64_t first, int64_t n, const char* k_base, const char* v_base,
                          int64_t stride, int32_t loc) {
  for (int64_t i = 0; i < n; ++i) {
    BlockRec& r = rec_[(size_t)(first + i)];
    release_if_unbacked(r);
    r.src = loc;
    r.gather = -1;
    r.src_k = loc == KVM_SRC_NONE ? nullptr : k_base + i * stride;
    r.src_v = loc == KVM_SRC_NONE ? nullptr : v_base + i * stride;
  }
  return KVM_OK;
}

int BlockPool::set_gather(int64_t first, int64_t n, kvm_gather_fn fn, void* user) {
  gathers_.push_back(Gather{fn, user});
  const int32_t gid = (int32_t)gathers_.size() - 1;
  for (int64_t i = 0; i < n; ++i) {
    BlockRec& r = rec_[(size_t)(first + i)];
    release_if_unbacked(r);
    r.src = KVM_SRC_HOST_PINNED;
    r.gather = gid;
    r.src_k = nullptr;
    r.src_v = nullptr;
  }
  return KVM_OK;
}

int BlockPool::register_list(const int64_t* ids, int64_t n, std::vector<int32_t>* slots) {
  slots->assign((size_t)n, -1);
  if (n <= 0) return KVM_OK;
  // Room: free pages plus pages of resident blocks outside the current view
  // (blocks of this list are being refreshed, not evicted).
  std::vector<std::pair<int64_t, int64_t>> lru;
  for (const auto& e : lru_outside_view())
    if (!std::binary_search(ids, ids + n, e.second)) lru.push_back(e);
  int64_t need = 0;
  for (int64_t i = 0; i < n; ++i) need += rec_[(size_t)ids[i]].slot < 0;
  if (need > (int64_t)free_slots_.size() + (int64_t)lru.size()) {
    set_error("registering %lld blocks needs %lld free pages; %zu are free and %zu hold blocks "
              "outside the current view",
              (long long)n, (long long)need, free_slots_.size(), lru.size());
    return KVM_ENOMEM;
  }
  size_t pos = 0;
  int32_t evicted = 0;
  const bool delta = L_.delta_limit > 0;
  for (int64_t i = 0; i < n; ++i) {
    const int64_t b = ids[i];
    BlockRec& r = rec_[(size_t)b];
    if (r.slot < 0) {
      const int32_t sl = take_slot(lru, pos, &evicted);
      slot_block_[(size_t)sl] = b;          // room was checked above, so sl >= 0
      r.slot = sl;
    }
    r.baked = -1;
    r.last_used = step_;
    r.n_delta = 0;
    r.raw_in_shadow = !delta;
    r.page_raw = delta;
    (*slots)[(size_t)i] = r.slot;
  }
  return KVM_OK;
}

int BlockPool::register_blocks(int64_t first, int64_t n, std::vector<int32_t>* slots) {
  std::vector<int64_t> ids((size_t)(n > 0 ? n : 0));
  for (int64_t i = 0; i < n; ++i) ids[(size_t)i] = first + i;
  return register_list(ids.data(), n, slots);
}

void BlockPool::release_list(const int64_t* ids, int64_t n) {
  for (int64_t i = 0; i < n; ++i) free_slot_of(rec_[(size_t)ids[i]]);
}

void BlockPool::release(int64_t first, int64_t n) {
  for (int64_t b = first; b < first + n; ++b) free_slot_of(rec_[(size_t)b]);
}

int BlockPool::evict(int64_t first, int64_t n) {
  for (int64_t b = first; b < first + n; ++b) {
    BlockRec& r = rec_[(size_t)b];
    if (r.slot >= 0) free_slot_of(r);
  }
  return KVM_OK;
}

int BlockPool::validate(const int32_t* sel, int32_t n) const {
  const bool delta_mode = L_.delta_limit > 0;
  const int32_t B = L_.block_tokens;
  for (int32_t i = 0; i < n; ++i) {
    const int64_t b = sel[i];
    if (b < 0 || b >= L_.max_blocks || (i > 0 && sel[i] <= sel[i - 1])) {
      set_error("selection entry %d (block %lld) invalid", i, (long long)b);
      return KVM_ERANGE;
    }
    const BlockRec& r = rec_[(size_t)b];
    if (r.slot < 0 && r.src == KVM_SRC_NONE) {
      set_error("block %lld is neither resident nor backed by a source", (long long)b);
      return KVM_ERANGE;
    }
    // delta mode: a hit past its delta limit is rebuilt from its raw K
    if (delta_mode && r.slot >= 0 && !r.page_raw && r.baked != i * B &&
        (r.baked < 0 || r.n_delta >= L_.delta_limit) && r.src == KVM_SRC_NONE) {
      set_error("block %lld needs a rebuild from raw K but has no lower-tier copy",
                (long long)b);
      return KVM_ERANGE;
    }
  }
  return KVM_OK;
}

int BlockPool::plan(const int32_t* sel, int32_t n, RematPlan* p) {
  const bool delta_mode = L_.delta_limit > 0;
  const int32_t B = L_.block_tokens;
  const int64_t pb = L_.page_bytes;
  *p = RematPlan{};
  if (n > L_.n_slots) {
    set_error("view of %d blocks exceeds the pool (%d pages)", n, L_.n_slots);
    return KVM_ENOMEM;
  }
  p->n = n;
  p->page.assign((size_t)n, -1);
  kvm_remat_stats& st = p->st;
  st.n_sel = n;
  // 1. The new view is the current view from here on: none of it is evicted.
  step_ += 1;
  for (int32_t i = 0; i < n; ++i) rec_[(size_t)sel[i]].last_used = step_;
  std::vector<std::pair<int64_t, int64_t>> lru = lru_outside_view();
  size_t lru_pos = 0;
  // 2. One job per page to write, in selection order, then grouped.
  std::vector<RematJob> J;
  std::vector<int64_t> jb;
  std::vector<int8_t> jk;
  std::vector<RematPlan::Undo> undo;
  J.reserve((size_t)n);
  auto push = [&](const RematJob& j, int64_t b, int kind, const BlockRec& before) {
    J.push_back(j);
    jb.push_back(b);
    jk.push_back((int8_t)kind);
    undo.push_back(RematPlan::Undo{b, before});
  };
  // where staged raw K lands: the page's shadow, or (delta mode) the K page itself
  auto stage_k = [&](int32_t sl) {
    return (const char*)(delta_mode ? L_.k_view : L_.k_shadow) + (int64_t)sl * pb;
  };
  auto kpage = [&](int32_t sl) { return (const char*)L_.k_view + (int64_t)sl * pb; };
  auto staged_kind = [&](const BlockRec& r) { return r.gather >= 0 ? JK_GATHER : JK_DMA; };
  for (int32_t i = 0; i < n; ++i) {
    const int64_t b = sel[i];
    BlockRec& r = rec_[(size_t)b];
    const int32_t pos = i * B;
    if (r.slot >= 0) {
      ++st.hits;
      p->page[(size_t)i] = r.slot;
      if (r.baked == pos && !r.page_raw) continue;
      const BlockRec before = r;
      if (!delta_mode) {
        // re-encode from the raw K kept in HBM: the page's shadow, or the
        // block's device-resident lower-tier copy
        const char* raw = r.raw_in_shadow ? (const char*)L_.k_shadow + (int64_t)r.slot * pb
                                          : r.src_k;
        push(RematJob{raw, nullptr, r.slot, pos, 0, 0}, b, JK_REENCODE, before);
      } else if (r.page_raw) {
        // freshly registered: raw K sits in the K page, rotate it there
        push(RematJob{kpage(r.slot), nullptr, r.slot, pos, 0, 0}, b, JK_REENCODE, before);
        r.page_raw = false;
        r.n_delta = 0;
      } else if (r.baked >= 0 && r.n_delta < L_.delta_limit) {
        // bounded delta re-RoPE: rotate the stored K by the position shift
        push(RematJob{kpage(r.slot), nullptr, r.slot, pos - r.baked, JOB_DELTA, 0}, b, JK_DELTA,
             before);
        r.n_delta += 1;
        ++st.deltas;
      } else {
        // limit reached: rebuild from raw K at the new position, reset the count
        ++st.rebuilds;
        r.n_delta = 0;
        if (r.src == KVM_SRC_DEVICE)
          push(RematJob{r.src_k, nullptr, r.slot, pos, 0, 0}, b, JK_REENCODE, before);
        else
          push(RematJob{stage_k(r.slot), nullptr, r.slot, pos, JOB_K_ONLY, i}, b, staged_kind(r),
               before);
      }
      r.baked = pos;
      continue;
    }
    ++st.misses;
    const BlockRec before = r;
    // a page is always found: n <= n_slots and no other block is in the view
    const int32_t sl = take_slot(lru, lru_pos, &st.evicted);
    slot_block_[(size_t)sl] = b;
    r.slot = sl;
    r.baked = pos;
    r.page_raw = false;
    r.n_delta = 0;
    p->page[(size_t)i] = sl;
    if (r.src == KVM_SRC_DEVICE) {
      // the lower-tier copy is already in HBM: rotate from it, copy V, and
      // keep reading it for later re-encodes (no shadow copy)
      r.raw_in_shadow = false;
      push(RematJob{r.src_k, r.src_v, sl, pos, JOB_COPY_V, 0}, b, JK_DEVICE_MISS, before);
    } else {
      r.raw_in_shadow = !delta_mode;
      push(RematJob{stage_k(sl), nullptr, sl, pos, 0, i}, b, staged_kind(r), before);
    }
  }
  // 3. Group: [hit re-encodes][device misses][delta shifts][DMA][gathered].
  static const int order[] = {JK_REENCODE, JK_DEVICE_MISS, JK_DELTA, JK_DMA, JK_GATHER};
  int32_t count[5] = {0, 0, 0, 0, 0};
  for (int k : order)
    for (size_t j = 0; j < J.size(); ++j)
      if (jk[j] == k) {
        p->jobs.push_back(J[j]);
        p->job_block.push_back(jb[j]);
        p->job_kind.push_back(jk[j]);
        p->undo.push_back(undo[j]);
        ++count[k];
      }
  p->n_reencode = count[JK_REENCODE];
  p->n_full = count[JK_REENCODE] + count[JK_DEVICE_MISS];
  p->n_delta = count[JK_DELTA];
  p->n_dma = count[JK_DMA];
  p->n_gather = count[JK_GATHER];
  st.rotated = (int32_t)p->jobs.size();
  st.d2d_bytes = (int64_t)(count[JK_REENCODE] + count[JK_DELTA] + count[JK_DMA] +
                           count[JK_GATHER]) * 2 * pb +
                 (int64_t)count[JK_DEVICE_MISS] * 4 * pb;
  return KVM_OK;
}

void BlockPool::rollback(const RematPlan& p, int32_t done, int32_t unknown) {
  const bool delta_mode = L_.delta_limit > 0;
  for (size_t j = (size_t)std::max(done, 0); j < p.jobs.size(); ++j) {
    const bool maybe_ran = (int64_t)j < (int64_t)done + unknown;
    const int64_t b = p.job_block[j];
    BlockRec& r = rec_[(size_t)b];
    const BlockRec& before = p.undo[j].rec;
    const int kind = p.job_kind[j];
    const bool was_hit = before.slot >= 0;
    if (!was_hit || kind == JK_DMA || kind == JK_GATHER) {
      // a miss, or a staged rebuild (in delta mode its raw K is staged into
      // the K page itself): the page is incomplete
      free_slot_of(r);
      continue;
    }
    if (!maybe_ran) {
      // the page was not touched: the old record is right again
      const int64_t used = r.last_used;
      r = before;
      r.last_used = used;
    } else if (!delta_mode) {
      // K may or may not be at the new position; its raw K is intact
      const int64_t used = r.last_used;
      r = before;
      r.last_used = used;
      r.baked = -1;
    } else {
      // an in-place rotation that may have happened: the K page is unknown
      free_slot_of(r);
    }
  }
}

}  // namespace kvm
