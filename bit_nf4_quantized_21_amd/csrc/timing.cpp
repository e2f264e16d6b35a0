// Per-kernel HIP-event timing (support facility for benchmarks).
#include "timing.hpp"

#include <atomic>
#include <cstdio>
#include <map>
#include <mutex>
#include <vector>

namespace qlora {

namespace {
struct Record {
  const char* name;
  hipEvent_t start, stop;
};
std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Record> g_recs;        // events in use, in launch order
std::vector<hipEvent_t> g_free;    // recycled events
}  // namespace

bool timing_enabled() { return g_on.load(std::memory_order_relaxed); }
void timing_enable(bool on) { g_on.store(on, std::memory_order_relaxed); }

static hipEvent_t take_event() {
  if (!g_free.empty()) {
    hipEvent_t e = g_free.back();
    g_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

KernelTimer::KernelTimer(const char* name, hipStream_t s) : s_(s) {
  if (!timing_enabled()) return;
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t a = take_event(), b = take_event();
  if (!a || !b) return;
  if (hipEventRecord(a, s) != hipSuccess) return;
  g_recs.push_back(Record{name, a, b});
  slot_ = (int)g_recs.size() - 1;
}

KernelTimer::~KernelTimer() {
  if (slot_ < 0) return;
  std::lock_guard<std::mutex> lk(g_mu);
  (void)hipEventRecord(g_recs[slot_].stop, s_);
}

std::string timing_collect(hipError_t* err) {
  std::lock_guard<std::mutex> lk(g_mu);
  std::map<std::string, std::pair<long, double>> acc;
  *err = hipSuccess;
  for (const Record& r : g_recs) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess) *err = e;
    auto& a = acc[r.name];
    a.first += 1;
    a.second += ms;
    g_free.push_back(r.start);
    g_free.push_back(r.stop);
  }
  g_recs.clear();
  std::string out;
  char line[256];
  for (const auto& kv : acc) {
    std::snprintf(line, sizeof(line), "%s %ld %.6f\n", kv.first.c_str(), kv.second.first, kv.second.second);
    out += line;
  }
  return out;
}

}  // namespace qlora
