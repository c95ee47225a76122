// Per-kernel timing with HIP events (off by default).
//
// When enabled, every kernel launch of the library (or only those of one
// name, see kvs_trace_only) is bracketed by two events recorded on the launch
// stream, so the elapsed time between them is that
// launch's duration on the GPU.  kvs_trace_summary waits for the recorded
// events, aggregates count / total / min / max per kernel name and returns the
// events to a pool, so steady-state tracing creates no new events.
#include <hip/hip_runtime.h>

#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "kvs_trace.h"

namespace kvs {
namespace {

struct Rec {
  const char* name;
  hipEvent_t a, b;
};

std::mutex g_mu;
bool g_on = false;
std::string g_only;  // record only launches of this name when not empty
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t take() {
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

TraceScope::TraceScope(const char* name, hipStream_t st) : name_(name), st_(st) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on || (!g_only.empty() && g_only != name_)) return;
  a_ = take();
  b_ = take();
  if (!a_ || !b_ || hipEventRecord(static_cast<hipEvent_t>(a_), st_) != hipSuccess) {
    if (a_) g_pool.push_back(static_cast<hipEvent_t>(a_));
    if (b_) g_pool.push_back(static_cast<hipEvent_t>(b_));
    a_ = b_ = nullptr;
  }
}

TraceScope::~TraceScope() {
  if (!a_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (hipEventRecord(static_cast<hipEvent_t>(b_), st_) == hipSuccess) {
    g_recs.push_back(Rec{name_, static_cast<hipEvent_t>(a_), static_cast<hipEvent_t>(b_)});
  } else {
    g_pool.push_back(static_cast<hipEvent_t>(a_));
    g_pool.push_back(static_cast<hipEvent_t>(b_));
  }
}

}  // namespace kvs

using namespace kvs;

extern "C" {

int kvs_trace_enable(int on) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_on = on != 0;
  return KVS_OK;
}

int kvs_trace_only(const char* name) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_only = name ? name : "";
  return KVS_OK;
}

int kvs_trace_summary(kvs_trace_entry* out, int max_entries, int* n_entries) {
  if (!n_entries || (max_entries > 0 && !out)) return KVS_E_NULL;
  std::vector<Rec> recs;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    recs.swap(g_recs);
  }
  std::map<std::string, kvs_trace_entry> agg;
  std::vector<std::string> order;
  int status = KVS_OK;
  for (const Rec& r : recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
      status = KVS_E_HIP;
      continue;
    }
    auto it = agg.find(r.name);
    if (it == agg.end()) {
      kvs_trace_entry e;
      std::memset(&e, 0, sizeof(e));
      std::strncpy(e.name, r.name, sizeof(e.name) - 1);
      e.min_ms = ms;
      e.max_ms = ms;
      it = agg.emplace(r.name, e).first;
      order.push_back(r.name);
    }
    kvs_trace_entry& e = it->second;
    e.count += 1;
    e.total_ms += ms;
    if (ms < e.min_ms) e.min_ms = ms;
    if (ms > e.max_ms) e.max_ms = ms;
  }
  {
    std::lock_guard<std::mutex> lk(g_mu);
    for (const Rec& r : recs) {
      g_pool.push_back(r.a);
      g_pool.push_back(r.b);
    }
  }
  int n = 0;
  for (const std::string& name : order) {
    if (n < max_entries) out[n] = agg[name];
    ++n;
  }
  *n_entries = n;
  return status;
}

}  // extern "C"
