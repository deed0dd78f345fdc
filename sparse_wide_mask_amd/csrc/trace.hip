// Opt-in kernel timing: while enabled, every launch the library makes is
// bracketed by two HIP events on the launch stream.  Reading the trace waits on
// the recorded events and aggregates per kernel name.  Off by default; when off
// a launch pays one relaxed atomic load.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "internal.h"

namespace wide {
namespace {

struct Rec {
  const char* name;
  hipEvent_t start, stop;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Rec> g_open;  // the launch currently being bracketed, one per thread is enough here
std::vector<Rec> g_recs;

struct Agg {
  std::string name;
  int launches = 0;
  double total_ms = 0.0;
};
std::vector<Agg> g_aggs;

}  // namespace

TraceScope::TraceScope(const char* name, hipStream_t s) : s_(s), active_(g_on.load(std::memory_order_relaxed)) {
  if (!active_) return;
  hipEvent_t a, b;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) {
    active_ = false;
    return;
  }
  (void)hipEventRecord(a, s_);
  std::lock_guard<std::mutex> lk(g_mu);
  g_open.push_back({name, a, b});
}

TraceScope::~TraceScope() {
  if (!active_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  Rec r = g_open.back();
  g_open.pop_back();
  (void)hipEventRecord(r.stop, s_);
  g_recs.push_back(r);
}

}  // namespace wide

extern "C" {

int wide_trace_enable(int on) {
  wide::g_on.store(on != 0);
  return 0;
}

// Waits for the recorded events, folds them into per-kernel totals and returns
// the number of distinct kernels.  Returns -1 if an event query fails.
int wide_trace_collect(void) {
  using namespace wide;
  std::lock_guard<std::mutex> lk(g_mu);
  for (Rec& r : g_recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
      return -1;
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
    Agg* a = nullptr;
    for (Agg& x : g_aggs)
      if (x.name == r.name) a = &x;
    if (!a) {
      g_aggs.push_back(Agg{r.name});
      a = &g_aggs.back();
    }
    a->launches += 1;
    a->total_ms += ms;
  }
  g_recs.clear();
  return (int)g_aggs.size();
}

int wide_trace_get(int i, char* name, int name_len, int* launches, double* total_ms) {
  using namespace wide;
  std::lock_guard<std::mutex> lk(g_mu);
  if (i < 0 || i >= (int)g_aggs.size() || !name || name_len < 1 || !launches || !total_ms) return 1;
  std::strncpy(name, g_aggs[i].name.c_str(), name_len - 1);
  name[name_len - 1] = 0;
  *launches = g_aggs[i].launches;
  *total_ms = g_aggs[i].total_ms;
  return 0;
}

void wide_trace_reset(void) {
  using namespace wide;
  std::lock_guard<std::mutex> lk(g_mu);
  for (Rec& r : g_recs) {
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  g_recs.clear();
  g_aggs.clear();
}

}  // extern "C"
