// Host-only driver of the block pool and the rematerialization data plane
// (attention_space_block_amd/csrc/pool.cpp, dataplane.cpp) and of the host
// tier simulation (tier.cpp), built with a plain C++ compiler and its address
// and undefined-behaviour sanitizers by tests/test_host_sanitized.py.
//
// A fake Engine stands in for the GPU. It queues every device operation and
// runs it only when the host has to wait for it, kernels as early and copies
// as late as the recorded events allow, so a missing wait shows up as a wrong
// page or as a hazard: a kernel that runs while a copy into its source is
// still queued, or a host worker that refills a staging half while a copy
// from it is still queued. Pages are small tagged records (kind, block,
// position, then a pattern derived from them) instead of K/V data.
//
// Commands on stdin, one per line; one result line per command on stdout.
//   pool <n_slots> <max_blocks> <delta_limit> <batch> <staging> <seed>
//   src <first> <n> <loc>          lower-tier copies: 1 pinned host, 2 device
//   gather <first> <n>             lower tier served by a gather callback
//   reg <first> <n>                -> reg <rc>
//   evict <first> <n>              -> evict <rc>
//   fail <launch|h2d|gather> <k>   the next selection fails at the k-th such op
//   corrupt <block>                flip one byte of the block's V source
//   sel <n> <b0> ... <bn-1>        -> sel <rc> <hits> <misses> <evicted> <rotated>
//                                     <h2d_pages> <batches> <view_errors>
//   check                          -> check <errors>: every resident page against its record
//   state                          -> state <block> ... (resident blocks, ascending)
//   oom <max_blocks>               -> oom <rc>: a pool too large for the host
//   tier <policy> <cap> <lambda> <steps>, then per step three lines
//        "<n> <ids...>" (new, selected, missed) -> tier <hits> <nvme> <demoted> per step
// Hazards print "error <text>" lines as they happen.
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <chrono>
#include <deque>
#include <functional>
#include <iostream>
#include <memory>
#include <mutex>
#include <random>
#include <sstream>
#include <string>
#include <thread>
#include <vector>

#include "dataplane.hpp"
#include "pool.hpp"

using namespace kvm;

namespace {

constexpr int64_t PAGE = 64;                 // bytes per fake page
enum { RAWK = 1, RAWV = 2, ENCK = 3 };

void make_page(char* p, int64_t kind, int64_t block, int64_t pos) {
  int64_t w[PAGE / 8];
  w[0] = kind;
  w[1] = block;
  w[2] = pos;
  for (int i = 3; i < PAGE / 8; ++i) w[i] = (kind * 1000003 + block * 7919 + pos * 31) ^ (i * 0x9e37);
  memcpy(p, w, PAGE);
}

bool page_is(const char* p, int64_t kind, int64_t block, int64_t pos) {
  char want[PAGE];
  make_page(want, kind, block, pos);
  return memcmp(p, want, PAGE) == 0;
}

std::mutex g_out_mu;
std::atomic<int> g_errors{0};

void error(const std::string& s) {
  std::lock_guard<std::mutex> g(g_out_mu);
  printf("error %s\n", s.c_str());
  fflush(stdout);
  ++g_errors;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const char* x = (const char*)a;
  const char* y = (const char*)b;
  return x < y + nb && y < x + na;
}

struct Op {
  enum Type { H2D, RECORD, WAIT, LAUNCH, UPLOAD, CALL } type;
  void* dst = nullptr;
  const void* src = nullptr;
  size_t bytes = 0;
  uint64_t rid = 0;        // RECORD: its id; WAIT: the record it waits for (0: none)
  int32_t first = 0, n = 0;
  bool delta = false;
  bool copy_v = false;      // LAUNCH: the launch may copy V
  std::vector<RematJob> jobs;   // UPLOAD: the job list as queued
  std::function<void()> call;   // CALL: the caller's later work on MAIN
};

class FakeEngine final : public Engine {
 public:
  FakeEngine(const PoolLayout& L, uint32_t seed) : L_(L), rng_(seed) {}

  int fail_launch = 0, fail_h2d = 0;   // fail the k-th op of the kind (1-based; 0: never)

  int ensure_events(int n) override {
    if ((int)last_rid_.size() < n) last_rid_.resize((size_t)n, 0);
    return KVM_OK;
  }
  int upload_plan(const RematPlan& p) override {
    Op o;
    o.type = Op::UPLOAD;
    o.jobs = p.jobs;
    push(MAIN, std::move(o));
    return KVM_OK;
  }
  int h2d(int stream, void* dst, const void* src, size_t bytes) override {
    if (fail_h2d > 0 && --fail_h2d == 0) {
      set_error("injected copy failure");
      return KVM_EHIP;
    }
    Op o;
    o.type = Op::H2D;
    o.dst = dst;
    o.src = src;
    o.bytes = bytes;
    push(stream, std::move(o));
    return KVM_OK;
  }
  int record(int stream, int ev) override {
    Op o;
    o.type = Op::RECORD;
    o.rid = ++rid_;
    last_rid_.at((size_t)ev) = o.rid;
    push(stream, std::move(o));
    return KVM_OK;
  }
  int wait(int stream, int ev) override {
    Op o;
    o.type = Op::WAIT;
    o.rid = last_rid_.at((size_t)ev);
    push(stream, std::move(o));
    return KVM_OK;
  }
  int host_wait(int ev) override {
    const uint64_t want = last_rid_.at((size_t)ev);
    while (want && !done(want))
      if (!step(std::max(0, stream_of_record(want)))) {
        error("host wait on an event that can never complete");
        return KVM_EHIP;
      }
    return KVM_OK;
  }
  int sync_all() override {
    while (step()) {
    }
    for (auto& q : q_)
      if (!q.empty()) {
        error("streams deadlocked");
        return KVM_EHIP;
      }
    return KVM_OK;
  }
  int launch(int32_t first, int32_t n, bool delta, bool copy_v) override {
    if (fail_launch > 0 && --fail_launch == 0) {
      set_error("injected launch failure");
      return KVM_EHIP;
    }
    Op o;
    o.type = Op::LAUNCH;
    o.first = first;
    o.n = n;
    o.delta = delta;
    o.copy_v = copy_v;
    push(MAIN, std::move(o));
    return KVM_OK;
  }

  // Queue `f` on MAIN as the caller's later work and run until MAIN has run it
  // (side-stream ops run only as far as MAIN's waits need them).
  int run_on_main(std::function<void()> f) {
    Op o;
    o.type = Op::CALL;
    o.call = std::move(f);
    push(MAIN, std::move(o));
    while (!q_[MAIN].empty())
      if (!step()) {
        error("the caller's stream can never reach its later work");
        return KVM_EHIP;
      }
    return KVM_OK;
  }

  // The host is about to write [p, p + bytes) (a gather worker filling the
  // staging ring): no queued copy may still read it.
  void host_write(const void* p, size_t bytes) {
    std::lock_guard<std::mutex> g(mu_);
    for (auto& q : q_)
      for (auto& o : q)
        if (o.type == Op::H2D && overlap(o.src, o.bytes, p, bytes))
          error("staging memory refilled while a copy from it is still queued");
  }

 private:
  void push(int stream, Op&& o) {
    std::lock_guard<std::mutex> g(mu_);
    q_[stream].push_back(std::move(o));
  }
  bool done(uint64_t rid) const { return done_set(rid); }
  bool done_set(uint64_t rid) const {
    return rid < completed_.size() && completed_[(size_t)rid];
  }
  bool runnable(int s) const {
    if (q_[s].empty()) return false;
    const Op& o = q_[s].front();
    return o.type != Op::WAIT || o.rid == 0 || done_set(o.rid);
  }
  // Stream holding the not yet executed RECORD with id `rid` (-1: none).
  int stream_of_record(uint64_t rid) const {
    for (int s = 0; s < 3; ++s)
      for (const Op& o : q_[s])
        if (o.type == Op::RECORD && o.rid == rid) return s;
    return -1;
  }
  // The stream whose head op must run next for stream `s` to advance: `s`
  // itself when runnable, else (following waits) the stream that records the
  // event it waits for.
  int needed_for(int s) const {
    for (int depth = 0; depth < 4 && s >= 0 && !q_[s].empty(); ++depth) {
      if (runnable(s)) return s;
      s = stream_of_record(q_[s].front().rid);
    }
    return -1;
  }
  // Run one queued op: only what `target` (MAIN unless the host waits on
  // another stream) needs next, so kernels run as early and copies as late
  // as the events allow, with an occasional random pick among the runnable
  // streams.
  bool step(int target = MAIN) {
    std::vector<int> ready;
    for (int s = 0; s < 3; ++s)
      if (runnable(s)) ready.push_back(s);
    if (ready.empty()) return false;
    int pick = needed_for(target);
    if (pick < 0 || (ready.size() > 1 && (rng_() % 5) == 0)) pick = ready[rng_() % ready.size()];
    Op o;
    {
      std::lock_guard<std::mutex> g(mu_);
      o = std::move(q_[pick].front());
      q_[pick].pop_front();
    }
    exec(o);
    return true;
  }
  void exec(const Op& o) {
    switch (o.type) {
      case Op::RECORD:
        if (completed_.size() <= o.rid) completed_.resize((size_t)o.rid + 1, false);
        completed_[(size_t)o.rid] = true;
        break;
      case Op::WAIT:
        break;
      case Op::CALL:
        o.call();
        break;
      case Op::UPLOAD:
        dev_jobs_ = o.jobs;
        break;
      case Op::H2D:
        memcpy(o.dst, o.src, o.bytes);
        break;
      case Op::LAUNCH:
        for (int32_t j = o.first; j < o.first + o.n; ++j) kernel(dev_jobs_.at((size_t)j), o.delta, o.copy_v);
        break;
    }
  }
  bool copy_pending_into(const void* p, size_t bytes) {
    std::lock_guard<std::mutex> g(mu_);
    for (auto& q : q_)
      for (auto& o : q)
        if (o.type == Op::H2D && overlap(o.dst, o.bytes, p, bytes)) return true;
    return false;
  }
  // The remat kernel on tagged pages.
  void kernel(const RematJob& jb, bool delta, bool copy_v) {
    if ((jb.flags & JOB_COPY_V) && !copy_v) error("a job that copies V in a K-only launch");
    char* kv = L_.k_view + (int64_t)jb.slot * PAGE;
    char* vv = L_.v_view + (int64_t)jb.slot * PAGE;
    if (copy_pending_into(jb.src_k, PAGE) || ((jb.flags & JOB_COPY_V) && copy_pending_into(jb.src_v, PAGE)))
      error("kernel ran while a copy into its source was still queued");
    int64_t w[3];
    memcpy(w, jb.src_k, sizeof(w));
    if (delta) {
      if (w[0] != ENCK) error("delta job on a page that holds no encoded K");
      make_page(kv, ENCK, w[1], w[2] + jb.pos);
    } else {
      if (!page_is((const char*)jb.src_k, RAWK, w[1], -1)) error("kernel source is not raw K");
      make_page(kv, ENCK, w[1], jb.pos);
    }
    if (jb.flags & JOB_COPY_V) memcpy(vv, jb.src_v, PAGE);
  }

  PoolLayout L_;
  std::mt19937 rng_;
  std::mutex mu_;
  std::deque<Op> q_[3];
  std::vector<uint64_t> last_rid_;
  std::vector<bool> completed_;
  uint64_t rid_ = 0;
  std::vector<RematJob> dev_jobs_;
};

struct World {
  PoolLayout L;
  std::vector<char> kview, vview, shadow;         // the "device" page pool
  std::vector<char> pin_k, pin_v, dev_k, dev_v;   // lower tiers
  std::vector<char> ring;
  std::unique_ptr<BlockPool> pool;
  std::unique_ptr<FakeEngine> eng;
  std::unique_ptr<WorkerPool> workers;
  StagingConfig cfg;
  std::vector<int32_t> src_loc;                   // per block: 0 none, 1 pinned, 2 device, 3 gather
  std::atomic<int> gather_calls{0};
  int fail_gather = 0;
  std::mt19937 rng;
};

World* g_world = nullptr;

int gather_fn(void* user, int64_t block, int32_t which, void* dst) {
  World* w = (World*)user;
  const int k = ++w->gather_calls;
  if (w->fail_gather > 0 && k == w->fail_gather) return 1;
  // an injected delay, so the workers finish in a shuffled order
  std::this_thread::sleep_for(std::chrono::microseconds((block * 37 + which * 11) % 50));
  w->eng->host_write(dst, PAGE);
  make_page((char*)dst, which == 0 ? RAWK : RAWV, block, -1);
  return 0;
}

// Every resident block's pages must be what its record says.
int check_world(World& w) {
  int bad = 0;
  const PoolLayout& L = w.L;
  for (int64_t b = 0; b < L.max_blocks; ++b) {
    const BlockRec& r = w.pool->rec(b);
    if (r.slot < 0) continue;
    const char* kv = L.k_view + (int64_t)r.slot * PAGE;
    const char* vv = L.v_view + (int64_t)r.slot * PAGE;
    if (r.page_raw) {
      if (!page_is(kv, RAWK, b, -1)) ++bad, error("raw K page of block " + std::to_string(b));
    } else if (r.baked >= 0) {
      if (!page_is(kv, ENCK, b, r.baked)) ++bad, error("K page of block " + std::to_string(b));
    }
    if (!page_is(vv, RAWV, b, -1)) ++bad, error("V page of block " + std::to_string(b));
    if (r.raw_in_shadow && !page_is(L.k_shadow + (int64_t)r.slot * PAGE, RAWK, b, -1))
      ++bad, error("shadow of block " + std::to_string(b));
  }
  return bad;
}

void cmd_pool(World& w, std::istringstream& in) {
  int64_t n_slots, max_blocks, delta, batch, staging, seed;
  in >> n_slots >> max_blocks >> delta >> batch >> staging >> seed;
  w.kview.assign((size_t)(n_slots * PAGE), 0);
  w.vview.assign((size_t)(n_slots * PAGE), 0);
  w.shadow.assign((size_t)(n_slots * PAGE), 0);
  w.pin_k.assign((size_t)(max_blocks * PAGE), 0);
  w.pin_v.assign((size_t)(max_blocks * PAGE), 0);
  w.dev_k.assign((size_t)(max_blocks * PAGE), 0);
  w.dev_v.assign((size_t)(max_blocks * PAGE), 0);
  for (int64_t b = 0; b < max_blocks; ++b) {
    make_page(&w.pin_k[(size_t)(b * PAGE)], RAWK, b, -1);
    make_page(&w.pin_v[(size_t)(b * PAGE)], RAWV, b, -1);
    make_page(&w.dev_k[(size_t)(b * PAGE)], RAWK, b, -1);
    make_page(&w.dev_v[(size_t)(b * PAGE)], RAWV, b, -1);
  }
  w.L = PoolLayout{};
  w.L.k_view = w.kview.data();
  w.L.v_view = w.vview.data();
  w.L.k_shadow = w.shadow.data();
  w.L.page_bytes = PAGE;
  w.L.n_slots = (int32_t)n_slots;
  w.L.block_tokens = 32;
  w.L.delta_limit = (int32_t)delta;
  w.L.max_pos = 1 << 30;
  w.L.max_blocks = max_blocks;
  w.pool.reset(new BlockPool(w.L));
  w.eng.reset(new FakeEngine(w.L, (uint32_t)seed));
  w.workers.reset(new WorkerPool(4));
  w.cfg.batch_blocks = (int32_t)batch;
  w.cfg.staging_blocks = (int32_t)staging;
  w.ring.assign((size_t)(staging * 2 * PAGE), 0);
  w.cfg.ring = w.ring.data();
  w.cfg.workers = w.workers.get();
  w.src_loc.assign((size_t)max_blocks, 0);
  w.rng.seed((uint32_t)seed);
  printf("pool ok\n");
}

void cmd_sel(World& w, std::istringstream& in) {
  int32_t n;
  in >> n;
  std::vector<int32_t> sel((size_t)n);
  for (auto& b : sel) in >> b;
  kvm_remat_stats st{};
  w.gather_calls = 0;
  const int rc = apply_selection(*w.eng, *w.pool, sel.data(), n, w.cfg, &st);
  w.eng->fail_launch = w.eng->fail_h2d = 0;
  w.fail_gather = 0;
  int view_errors = 0;
  if (rc == KVM_OK) {
    // the caller's later work on its stream (attention over the view) must
    // see every page of the view finished
    w.eng->run_on_main([&] {
      for (int32_t i = 0; i < n; ++i) {
        const BlockRec& r = w.pool->rec(sel[(size_t)i]);
        if (r.slot < 0) {
          ++view_errors;
          error("selected block " + std::to_string(sel[(size_t)i]) + " has no page");
          continue;
        }
        if (!page_is(w.L.k_view + (int64_t)r.slot * PAGE, ENCK, sel[(size_t)i], (int64_t)i * 32))
          ++view_errors, error("view K of block " + std::to_string(sel[(size_t)i]));
        if (!page_is(w.L.v_view + (int64_t)r.slot * PAGE, RAWV, sel[(size_t)i], -1))
          ++view_errors, error("view V of block " + std::to_string(sel[(size_t)i]));
      }
    });
  }
  (void)w.eng->sync_all();
  printf("sel %d %d %d %d %d %lld %d %d\n", rc, st.hits, st.misses, st.evicted, st.rotated,
         (long long)(st.h2d_bytes / PAGE), st.batches, view_errors);
}

void cmd_tier(std::istringstream& in) {
  kvm_tier_policy pol{};
  int32_t steps;
  in >> pol.policy >> pol.host_blocks >> pol.lambda >> steps;
  std::vector<int64_t> off[3];
  std::vector<int32_t> blk[3];
  for (int i = 0; i < 3; ++i) off[i].push_back(0);
  std::string line;
  for (int32_t t = 0; t < steps; ++t)
    for (int i = 0; i < 3; ++i) {
      std::getline(std::cin, line);
      std::istringstream ls(line);
      int64_t m;
      ls >> m;
      for (int64_t j = 0; j < m; ++j) {
        int32_t b;
        ls >> b;
        blk[i].push_back(b);
      }
      off[i].push_back((int64_t)blk[i].size());
    }
  std::vector<int32_t> out((size_t)std::max(steps, 1) * 3, 0);
  for (int i = 0; i < 3; ++i) blk[i].push_back(0);   // never an empty array
  const int rc = kvm_tier_simulate(&pol, steps, off[0].data(), blk[0].data(), off[1].data(),
                                   blk[1].data(), off[2].data(), blk[2].data(), out.data());
  printf("tier %d", rc);
  for (int32_t t = 0; t < steps; ++t)
    printf(" %d %d %d", out[(size_t)t * 3], out[(size_t)t * 3 + 1], out[(size_t)t * 3 + 2]);
  printf("\n");
}

}  // namespace

int main() {
  World w;
  g_world = &w;
  std::string line;
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    std::string cmd;
    in >> cmd;
    if (cmd.empty()) continue;
    if (cmd == "end") break;
    if (cmd == "pool") {
      cmd_pool(w, in);
    } else if (cmd == "src") {
      int64_t first, n;
      int32_t loc;
      in >> first >> n >> loc;
      const std::vector<char>& K = loc == 1 ? w.pin_k : w.dev_k;
      const std::vector<char>& V = loc == 1 ? w.pin_v : w.dev_v;
      const int rc = w.pool->set_source(first, n, K.data() + first * PAGE, V.data() + first * PAGE,
                                        PAGE, loc == 1 ? KVM_SRC_HOST_PINNED : KVM_SRC_DEVICE);
      printf("src %d\n", rc);
    } else if (cmd == "gather") {
      int64_t first, n;
      in >> first >> n;
      printf("gather %d\n", w.pool->set_gather(first, n, gather_fn, &w));
    } else if (cmd == "reg") {
      int64_t first, n;
      in >> first >> n;
      std::vector<int32_t> slots;
      const int rc = w.pool->register_blocks(first, n, &slots);
      if (rc == KVM_OK) {
        const bool delta = w.L.delta_limit > 0;
        for (int64_t i = 0; i < n; ++i) {
          // the registration's device copies (stream ordered before later work)
          char* kd = (delta ? w.L.k_view : w.L.k_shadow) + (int64_t)slots[(size_t)i] * PAGE;
          make_page(kd, RAWK, first + i, -1);
          make_page(w.L.v_view + (int64_t)slots[(size_t)i] * PAGE, RAWV, first + i, -1);
        }
      }
      printf("reg %d\n", rc);
    } else if (cmd == "regl") {
      int64_t n;
      in >> n;
      std::vector<int64_t> ids((size_t)n);
      for (auto& x : ids) in >> x;
      std::vector<int32_t> slots;
      const int rc = w.pool->register_list(ids.data(), n, &slots);
      if (rc == KVM_OK) {
        const bool delta = w.L.delta_limit > 0;
        for (int64_t i = 0; i < n; ++i) {
          char* kd = (delta ? w.L.k_view : w.L.k_shadow) + (int64_t)slots[(size_t)i] * PAGE;
          make_page(kd, RAWK, ids[(size_t)i], -1);
          make_page(w.L.v_view + (int64_t)slots[(size_t)i] * PAGE, RAWV, ids[(size_t)i], -1);
        }
      }
      printf("regl %d\n", rc);
    } else if (cmd == "evict") {
      int64_t first, n;
      in >> first >> n;
      printf("evict %d\n", w.pool->evict(first, n));
    } else if (cmd == "fail") {
      std::string what;
      int k;
      in >> what >> k;
      if (what == "launch") w.eng->fail_launch = k;
      else if (what == "h2d") w.eng->fail_h2d = k;
      else if (what == "gather") w.fail_gather = k;
      printf("fail ok\n");
    } else if (cmd == "corrupt") {
      int64_t b;
      in >> b;
      w.pin_v[(size_t)(b * PAGE + 40)] ^= 1;
      w.dev_v[(size_t)(b * PAGE + 40)] ^= 1;
      printf("corrupt ok\n");
    } else if (cmd == "sel") {
      cmd_sel(w, in);
    } else if (cmd == "check") {
      printf("check %d\n", check_world(w));
    } else if (cmd == "state") {
      printf("state");
      for (int64_t b = 0; b < w.L.max_blocks; ++b)
        if (w.pool->rec(b).slot >= 0) printf(" %lld", (long long)b);
      printf("\n");
    } else if (cmd == "oom") {
      int64_t mb;
      in >> mb;
      PoolLayout L = w.L;
      L.max_blocks = mb;
      std::unique_ptr<BlockPool> p;
      const int rc = guarded([&] {
        p.reset(new BlockPool(L));
        return KVM_OK;
      });
      printf("oom %d\n", rc);
    } else if (cmd == "tier") {
      cmd_tier(in);
    } else {
      printf("unknown %s\n", cmd.c_str());
    }
    fflush(stdout);
  }
  printf("errors %d\n", g_errors.load());
  return 0;
}
