// Per-kernel launch timing with HIP events (off unless enabled).
// Each instrumented launch records an event pair on its own stream; reading
// the profile waits for those events and accumulates durations per kernel.
#include <mutex>
#include <string>
#include <vector>

#include "common.hpp"
#include "profile.hpp"

namespace kvm {

namespace {
struct Pending {
  const char* name;
  hipEvent_t a, b;
};
struct Total {
  std::string name;
  int64_t launches = 0;
  double ms = 0.0;
};
std::mutex g_mu;
bool g_on = false;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_free;
std::vector<Total> g_tot;

hipEvent_t get_event() {
  if (!g_free.empty()) {
    hipEvent_t e = g_free.back();
    g_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

KernelTimer::KernelTimer(const char* name, hipStream_t s) : name_(name), s_(s) {
  if (!name_) return;   // untimed launch
  std::lock_guard<std::mutex> g(g_mu);
  if (!g_on) return;
  a_ = get_event();
  b_ = get_event();
  if (a_ && b_) (void)hipEventRecord((hipEvent_t)a_, s_);
}

KernelTimer::~KernelTimer() {
  if (!a_ || !b_) return;
  (void)hipEventRecord((hipEvent_t)b_, s_);
  std::lock_guard<std::mutex> g(g_mu);
  g_pending.push_back(Pending{name_, (hipEvent_t)a_, (hipEvent_t)b_});
}

}  // namespace kvm

static int kvm_profile_enable_body(int32_t on) {
  using namespace kvm;
  std::lock_guard<std::mutex> g(g_mu);
  g_on = on != 0;
  if (g_on) g_tot.clear();
  return KVM_OK;
}

extern "C" int kvm_profile_enable(int32_t on) {
  return kvm::guarded([&] {
    return kvm_profile_enable_body(on);
  });
}

static int kvm_profile_read_body(kvm_kernel_stat* out, int32_t max, int32_t* n) {
  using namespace kvm;
  clear_error();
  KVM_CHECK_ARG(n != nullptr && (out != nullptr || max == 0), "null pointer");
  std::lock_guard<std::mutex> g(g_mu);
  for (auto& p : g_pending) {
    KVM_HIP(hipEventSynchronize(p.b));
    float ms = 0.0f;
    KVM_HIP(hipEventElapsedTime(&ms, p.a, p.b));
    Total* t = nullptr;
    for (auto& x : g_tot)
      if (x.name == p.name) t = &x;
    if (!t) {
      g_tot.push_back(Total{p.name, 0, 0.0});
      t = &g_tot.back();
    }
    t->launches += 1;
    t->ms += ms;
    g_free.push_back(p.a);
    g_free.push_back(p.b);
  }
  g_pending.clear();
  *n = (int32_t)g_tot.size();
  for (int32_t i = 0; i < max && i < (int32_t)g_tot.size(); ++i) {
    memset(out[i].name, 0, sizeof(out[i].name));
    strncpy(out[i].name, g_tot[i].name.c_str(), sizeof(out[i].name) - 1);
    out[i].launches = g_tot[i].launches;
    out[i].total_ms = g_tot[i].ms;
  }
  return KVM_OK;
}

extern "C" int kvm_profile_read(kvm_kernel_stat* out, int32_t max, int32_t* n) {
  return kvm::guarded([&] {
    return kvm_profile_read_body(out, max, n);
  });
}
