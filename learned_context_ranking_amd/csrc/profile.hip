// Opt-in per-kernel timing (measurement only, off by default). While enabled, each kernel
// the library launches is bracketed by two HIP events recorded on the stream it is
// launched on; collecting waits for the recorded events and sums the elapsed times per
// kernel name. Disabled, a launch site costs one relaxed atomic load.
#include <hip/hip_runtime.h>
#include <string.h>

#include <atomic>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/sas.h"
#include "sas_kernels.h"

namespace sas {
namespace {

struct Rec {
  const char* name;
  hipEvent_t a, b;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Rec> g_recs;          // launches recorded since the last collect
std::vector<hipEvent_t> g_pool;   // events ready for reuse

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

ProfScope::ProfScope(const char* name, hipStream_t st) : name_(name), st_(st), a_(nullptr) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  a_ = take_event();
  if (a_ != nullptr && hipEventRecord((hipEvent_t)a_, st) != hipSuccess) {
    g_pool.push_back((hipEvent_t)a_);
    a_ = nullptr;
  }
}

ProfScope::~ProfScope() {
  if (a_ == nullptr) return;
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t b = take_event();
  if (b == nullptr || hipEventRecord(b, st_) != hipSuccess) {
    g_pool.push_back((hipEvent_t)a_);
    if (b != nullptr) g_pool.push_back(b);
    return;
  }
  g_recs.push_back(Rec{name_, (hipEvent_t)a_, b});
}

}  // namespace sas

extern "C" {

sas_status sas_profile_enable(int on) {
  sas::g_on.store(on != 0, std::memory_order_relaxed);
  return SAS_OK;
}

int sas_profile_collect(int max, char* names, int name_len, int* launches, double* total_ms) {
  using namespace sas;
  std::lock_guard<std::mutex> lk(g_mu);
  std::map<std::string, std::pair<int, double>> acc;
  std::vector<std::string> order;
  int rc = 0;
  for (const Rec& r : g_recs) {
    float ms = 0.0f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) rc = -1;
    auto it = acc.find(r.name);
    if (it == acc.end()) {
      order.push_back(r.name);
      acc[r.name] = {1, (double)ms};
    } else {
      it->second.first += 1;
      it->second.second += ms;
    }
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_recs.clear();
  if (rc != 0) return -1;
  int n = 0;
  for (const std::string& k : order) {
    if (n >= max) break;
    if (names != nullptr && name_len > 0) {
      strncpy(names + (size_t)n * name_len, k.c_str(), (size_t)name_len - 1);
      names[(size_t)n * name_len + name_len - 1] = '\0';
    }
    if (launches != nullptr) launches[n] = acc[k].first;
    if (total_ms != nullptr) total_ms[n] = acc[k].second;
    ++n;
  }
  return n;
}

}  // extern "C"
