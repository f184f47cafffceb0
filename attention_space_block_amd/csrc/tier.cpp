// Host-tier admission and eviction over a trace of agent steps (KVMem
// Sec. 4.4, hierarchical reuse): evicted GPU blocks reload from host memory
// when it holds them, else from NVMe; host memory is bounded and keeps blocks
// with strong recent or cumulative retrieval. The recency-and-frequency
// weighting is LRFU (Lee et al., IEEE Trans. Computers 2001): a block touched
// at t_1 < ... < t_k is worth sum_i 2^(-lambda (t - t_i)), kept incrementally,
// and compared through the time-invariant key log2(crf) + lambda * t_last.
// LRU (key t_last) is the recency-only baseline. Host C++ only: an ordered
// set of (key, block) gives the eviction victim in O(log n).
#include <cmath>
#include <set>
#include <utility>
#include <vector>

#include "host_common.hpp"

namespace kvm {
namespace {

struct TierSim {
  int32_t policy;
  int32_t cap;
  double lam;
  std::vector<int32_t> last;
  std::vector<double> crf, key;
  std::vector<char> in_host;
  std::set<std::pair<double, int32_t>> host;

  void touch(int32_t b, int32_t t) {
    if (last[b] == t) return;
    if (policy == KVM_TIER_LRFU)
      crf[b] = last[b] < 0 ? 1.0 : 1.0 + std::pow(2.0, -lam * (double)(t - last[b])) * crf[b];
    last[b] = t;
    const double k = policy == KVM_TIER_LRU ? (double)t : std::log2(crf[b]) + lam * (double)t;
    if (in_host[b]) {
      host.erase({key[b], b});
      host.insert({k, b});
    }
    key[b] = k;
  }
  int admit(int32_t b) {
    if (in_host[b]) return 0;
    int demoted = 0;
    if ((int32_t)host.size() >= cap) {
      const int32_t v = host.begin()->second;
      host.erase(host.begin());
      in_host[v] = 0;
      demoted = 1;
    }
    host.insert({key[b], b});
    in_host[b] = 1;
    return demoted;
  }
};

int check_csr(int32_t n_steps, const int64_t* off, const int32_t* blk, int32_t* max_id,
              const char* what) {
  if (!off || (off[n_steps] > 0 && !blk)) {
    set_error("%s: null offsets or blocks", what);
    return KVM_EINVAL;
  }
  if (off[0] != 0) {
    set_error("%s: offsets must start at 0", what);
    return KVM_EINVAL;
  }
  for (int32_t t = 0; t < n_steps; ++t) {
    if (off[t + 1] < off[t]) {
      set_error("%s: offsets decrease at step %d", what, t);
      return KVM_EINVAL;
    }
    for (int64_t i = off[t]; i < off[t + 1]; ++i) {
      if (blk[i] < 0 || (i > off[t] && blk[i] <= blk[i - 1])) {
        set_error("%s: step %d is not a strictly ascending list of block ids", what, t);
        return KVM_EINVAL;
      }
      if (blk[i] > *max_id) *max_id = blk[i];
    }
  }
  return KVM_OK;
}

}  // namespace
}  // namespace kvm

static int kvm_tier_simulate_body(const kvm_tier_policy* pol, int32_t n_steps,
                                 const int64_t* new_off, const int32_t* new_blk,
                                 const int64_t* sel_off, const int32_t* sel_blk,
                                 const int64_t* miss_off, const int32_t* miss_blk, int32_t* out) {
  using namespace kvm;
  clear_error();
  KVM_CHECK_ARG(pol && out && n_steps >= 0, "null pointer or negative step count");
  KVM_CHECK_ARG(pol->policy == KVM_TIER_LRU || pol->policy == KVM_TIER_LRFU, "policy");
  KVM_CHECK_ARG(pol->host_blocks >= 1, "host_blocks must be >= 1");
  KVM_CHECK_ARG(std::isfinite(pol->lambda) && pol->lambda >= 0.0, "lambda must be >= 0");
  int32_t max_id = -1;
  int rc = check_csr(n_steps, new_off, new_blk, &max_id, "new");
  if (rc) return rc;
  rc = check_csr(n_steps, sel_off, sel_blk, &max_id, "sel");
  if (rc) return rc;
  rc = check_csr(n_steps, miss_off, miss_blk, &max_id, "miss");
  if (rc) return rc;
  TierSim s{pol->policy, pol->host_blocks, pol->lambda, {}, {}, {}, {}, {}};
  const size_t n = (size_t)max_id + 1;
  s.last.assign(n, -1);
  s.crf.assign(n, 0.0);
  s.key.assign(n, 0.0);
  s.in_host.assign(n, 0);
  for (int32_t t = 0; t < n_steps; ++t) {
    const int32_t step = t + 1;
    int32_t hits = 0, nvme = 0, dem = 0;
    for (int64_t i = new_off[t]; i < new_off[t + 1]; ++i) {
      s.touch(new_blk[i], step);
      dem += s.admit(new_blk[i]);
    }
    for (int64_t i = sel_off[t]; i < sel_off[t + 1]; ++i) s.touch(sel_blk[i], step);
    for (int64_t i = miss_off[t]; i < miss_off[t + 1]; ++i) {
      const int32_t b = miss_blk[i];
      if (s.last[b] != step) {
        set_error("miss %d at step %d is not in that step's selection", b, t);
        return KVM_EINVAL;
      }
      if (s.in_host[b]) {
        ++hits;
      } else {
        ++nvme;
        dem += s.admit(b);
      }
    }
    out[3 * t] = hits;
    out[3 * t + 1] = nvme;
    out[3 * t + 2] = dem;
  }
  return KVM_OK;
}

extern "C" int kvm_tier_simulate(const kvm_tier_policy* pol, int32_t n_steps,
                                 const int64_t* new_off, const int32_t* new_blk,
                                 const int64_t* sel_off, const int32_t* sel_blk,
                                 const int64_t* miss_off, const int32_t* miss_blk, int32_t* out) {
  return kvm::guarded([&] {
    return kvm_tier_simulate_body(pol, n_steps, new_off, new_blk, sel_off, sel_blk, miss_off,
                                  miss_blk, out);
  });
}
