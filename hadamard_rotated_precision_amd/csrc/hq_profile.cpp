// hq_profile.cpp — optional launch instrumentation of libhq: when enabled for a set of kernel
// kinds, each launch of those kinds gets two HIP events and its algorithmic work (ops for the
// GEMM, bytes for streaming kernels). The GEMM and prologue kernels hand the events to
// hipExtLaunchKernel, which stamps them with the kernel's own start and end on its stream
// (no extra packets between launches); other launches are bracketed by two event records on
// the launch's stream. Nothing is recorded while disabled (the default).
#include "../../include/hq.h"

#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "hq_internal.hpp"

namespace hq {
namespace {

struct Rec {
  int kind;
  double units;
  hipEvent_t a, b;
};

std::mutex g_mu;
bool g_on = false;
uint32_t g_mask = 0;
std::vector<Rec> g_recs;
std::vector<hq_profile_record> g_done;   // per-launch results of the last hq_profile_stop
std::vector<hipEvent_t> g_pool;
size_t g_next = 0;

hipEvent_t take_event() {
  if (g_next == g_pool.size()) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    g_pool.push_back(e);
  }
  return g_pool[g_next++];
}

}  // namespace

int prof_begin(int kind, double units, hipStream_t st) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on || !(g_mask & (1u << kind))) return -1;
  Rec r{kind, units, take_event(), take_event()};
  if (!r.a || !r.b || hipEventRecord(r.a, st) != hipSuccess) return -1;
  g_recs.push_back(r);
  return static_cast<int>(g_recs.size() - 1);
}

int prof_open(int kind, double units) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on || !(g_mask & (1u << kind))) return -1;
  Rec r{kind, units, take_event(), take_event()};
  if (!r.a || !r.b) return -1;
  g_recs.push_back(r);
  return static_cast<int>(g_recs.size() - 1);
}

void prof_events(int idx, hipEvent_t* a, hipEvent_t* b) {
  *a = *b = nullptr;
  if (idx < 0) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (idx < static_cast<int>(g_recs.size())) {
    *a = g_recs[idx].a;
    *b = g_recs[idx].b;
  }
}

void prof_end(int idx, hipStream_t st) {
  if (idx < 0) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (idx < static_cast<int>(g_recs.size())) (void)hipEventRecord(g_recs[idx].b, st);
}

}  // namespace hq

extern "C" {

hq_status hq_profile_start(uint32_t kind_mask) {
  std::lock_guard<std::mutex> lk(hq::g_mu);
  hq::g_recs.clear();
  hq::g_done.clear();
  hq::g_next = 0;
  hq::g_mask = kind_mask;
  hq::g_on = kind_mask != 0;
  return HQ_OK;
}

hq_status hq_profile_stop(hq_profile_stat* stats, int32_t n_stats) {
  std::lock_guard<std::mutex> lk(hq::g_mu);
  hq::g_on = false;
  if (!stats && n_stats > 0) return HQ_ERR_NULL;
  for (int32_t i = 0; i < n_stats; ++i) {
    stats[i].kind = i;
    stats[i].count = 0;
    stats[i].total_ms = 0.0;
    stats[i].units = 0.0;
  }
  hq_status st = HQ_OK;
  hq::g_done.clear();
  for (const auto& r : hq::g_recs) {
    float ms = 0.0f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
      st = HQ_ERR_LAUNCH;
      continue;
    }
    hq::g_done.push_back(hq_profile_record{r.kind, 0, static_cast<double>(ms), r.units});
    if (r.kind < n_stats) {
      stats[r.kind].count += 1;
      stats[r.kind].total_ms += ms;
      stats[r.kind].units += r.units;
    }
  }
  hq::g_recs.clear();
  hq::g_next = 0;
  return st;
}

int32_t hq_profile_records(hq_profile_record* out, int32_t cap) {
  std::lock_guard<std::mutex> lk(hq::g_mu);
  const int32_t n = static_cast<int32_t>(hq::g_done.size());
  if (out)
    for (int32_t i = 0; i < n && i < cap; ++i) out[i] = hq::g_done[i];
  return n;
}

}  // extern "C"
