// Optional per-kernel timing with HIP events recorded on the stream each
// kernel is launched on (benchmark instrumentation; off by default).
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"

namespace mtgr {
namespace {

struct Rec {
  const char* name;
  hipEvent_t a, b;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t get_event() {
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

bool profiling_enabled() {
  std::lock_guard<std::mutex> lk(g_mu);
  return g_on;
}

ProfScope::ProfScope(const char* name, hipStream_t s) : name_(name), stream_(s), begin_(nullptr) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on) return;
  begin_ = get_event();
  if (begin_ && hipEventRecord((hipEvent_t)begin_, s) != hipSuccess) begin_ = nullptr;
}

ProfScope::~ProfScope() {
  if (!begin_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t e = get_event();
  if (!e || hipEventRecord(e, stream_) != hipSuccess) return;
  g_recs.push_back(Rec{name_, (hipEvent_t)begin_, e});
}

}  // namespace mtgr

using namespace mtgr;

extern "C" {

int mtgr_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto& r : g_recs) {
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_recs.clear();
  g_on = on != 0;
  return MTGR_OK;
}

int mtgr_profile_summary(int max_entries, const char** names, double* total_ms, int32_t* launches) {
  std::lock_guard<std::mutex> lk(g_mu);
  std::vector<std::string> keys;
  std::vector<double> ms;
  std::vector<int32_t> cnt;
  for (auto& r : g_recs) {
    if (hipEventSynchronize(r.b) != hipSuccess) return MTGR_ERR_HIP;
    float t = 0.f;
    if (hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) return MTGR_ERR_HIP;
    size_t i = 0;
    for (; i < keys.size(); ++i)
      if (keys[i] == r.name) break;
    if (i == keys.size()) {
      keys.push_back(r.name);
      ms.push_back(0.0);
      cnt.push_back(0);
    }
    ms[i] += t;
    cnt[i] += 1;
  }
  int n = (int)keys.size();
  for (int i = 0; i < n && i < max_entries; ++i) {
    // names point at the static literals passed to ProfScope
    for (auto& r : g_recs)
      if (keys[i] == r.name) { names[i] = r.name; break; }
    total_ms[i] = ms[i];
    launches[i] = cnt[i];
  }
  return n;
}

}  // extern "C"
