// Opt-in kernel timing: event pairs on the launch stream, summed per kind.
#include "profile.hpp"

#include <mutex>
#include <vector>

namespace etpc {
namespace {

struct Rec {
  int kind;
  hipEvent_t a, b;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

ProfScope::ProfScope(int kind, hipStream_t s) : kind_(kind), s_(s) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on) return;
  a_ = take_event();
  b_ = take_event();
  if (a_ && b_ && hipEventRecord(a_, s_) != hipSuccess) a_ = nullptr;
}

ProfScope::~ProfScope() {
  if (!a_ || !b_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (hipEventRecord(b_, s_) == hipSuccess) g_recs.push_back(Rec{kind_, a_, b_});
}

}  // namespace etpc

extern "C" {

etpc_status etpc_profile_enable(int32_t enable) {
  std::lock_guard<std::mutex> lk(etpc::g_mu);
  for (auto& r : etpc::g_recs) {
    (void)hipEventSynchronize(r.b);
    etpc::g_pool.push_back(r.a);
    etpc::g_pool.push_back(r.b);
  }
  etpc::g_recs.clear();
  etpc::g_on = enable != 0;
  return ETPC_OK;
}

etpc_status etpc_profile_read(int32_t kind, double* total_ms, int64_t* launches) {
  if (kind < 0 || kind >= ETPC_KIND_COUNT) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "unknown kernel kind");
  std::lock_guard<std::mutex> lk(etpc::g_mu);
  double t = 0.0;
  int64_t n = 0;
  for (auto& r : etpc::g_recs) {
    if (r.kind != kind) continue;
    ETPC_HIP(hipEventSynchronize(r.b));
    float ms = 0.f;
    ETPC_HIP(hipEventElapsedTime(&ms, r.a, r.b));
    t += ms;
    ++n;
  }
  if (total_ms) *total_ms = t;
  if (launches) *launches = n;
  return ETPC_OK;
}

}  // extern "C"
