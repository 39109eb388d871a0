#include "trace.hpp"

#include <atomic>
#include <map>
#include <mutex>
#include <stdio.h>
#include <string>
#include <vector>

#include "../../include/dspark.h"

namespace dspark {

namespace {
struct Rec {
  const char* name;
  hipEvent_t a, b;
};
std::atomic<bool> g_on{false};
std::mutex g_mu;
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
void recycle_all() {
  for (auto& r : g_recs) {
    if (r.a) g_pool.push_back(r.a);
    if (r.b) g_pool.push_back(r.b);
  }
  g_recs.clear();
}
}  // namespace

bool trace_on() { return g_on.load(std::memory_order_relaxed); }

int trace_begin(const char* name, hipStream_t stream) {
  if (!trace_on()) return -1;
  std::lock_guard<std::mutex> lk(g_mu);
  Rec r{name, get_event(), get_event()};
  if (!r.a || !r.b) return -1;
  if (hipEventRecord(r.a, stream) != hipSuccess) return -1;
  g_recs.push_back(r);
  return (int)g_recs.size() - 1;
}

void trace_end(int slot, hipStream_t stream) {
  if (slot < 0) return;
  std::lock_guard<std::mutex> lk(g_mu);
  // a failed record makes dspark_trace_summary report DSPARK_EHIP
  if (slot < (int)g_recs.size()) (void)hipEventRecord(g_recs[slot].b, stream);
}

}  // namespace dspark

extern "C" {

int dspark_trace_enable(int on) {
  std::lock_guard<std::mutex> lk(dspark::g_mu);
  dspark::recycle_all();
  dspark::g_on.store(on != 0);
  if (!on) {   // tracing stops: every event is destroyed (none outlives it)
    for (hipEvent_t e : dspark::g_pool) (void)hipEventDestroy(e);
    dspark::g_pool.clear();
  }
  return DSPARK_OK;
}

int dspark_trace_summary(char* buf, size_t len) {
  using namespace dspark;
  std::lock_guard<std::mutex> lk(g_mu);
  std::map<std::string, std::pair<long, double>> agg;
  for (auto& r : g_recs) {
    if (hipEventSynchronize(r.b) != hipSuccess) return DSPARK_EHIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return DSPARK_EHIP;
    auto& e = agg[r.name];
    e.first += 1;
    e.second += ms;
  }
  std::string out;
  char line[256];
  for (auto& kv : agg) {
    snprintf(line, sizeof(line), "%s %ld %.6f\n", kv.first.c_str(), kv.second.first,
             kv.second.second);
    out += line;
  }
  if (buf && len) {
    snprintf(buf, len, "%s", out.c_str());
  }
  return (int)out.size();
}

}  // extern "C"
