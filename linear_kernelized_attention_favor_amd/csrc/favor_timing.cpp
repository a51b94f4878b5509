// Per-kernel event timing behind favor_timing_start / favor_timing_stop.
// Host code only; the launchers call timing_before / timing_after around
// each kernel, which cost one thread-local test while recording is off.
#include <cstdint>
#include <cstring>
#include <vector>

#include <hip/hip_runtime.h>

#include "favor.h"
#include "favor_internal.h"

namespace favor {
namespace {

struct Record {
  const char* name;
  hipEvent_t start, stop;
};

struct Timing {
  bool on = false;
  hipError_t err = hipSuccess;     // first failure while recording
  hipEvent_t pending = nullptr;    // start event of the kernel being launched
  std::vector<hipEvent_t> pool;    // events free for reuse
  std::vector<Record> recs;
};

thread_local Timing g_t;

hipEvent_t take_event() {
  if (!g_t.pool.empty()) {
    hipEvent_t e = g_t.pool.back();
    g_t.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  const hipError_t r = hipEventCreate(&e);
  if (r != hipSuccess) {
    if (g_t.err == hipSuccess) g_t.err = r;
    return nullptr;
  }
  return e;
}

}  // namespace

void timing_before(hipStream_t st) {
  if (!g_t.on) return;
  hipEvent_t e = take_event();
  if (!e) return;
  const hipError_t r = hipEventRecord(e, st);
  if (r != hipSuccess) {
    if (g_t.err == hipSuccess) g_t.err = r;
    g_t.pool.push_back(e);
    return;
  }
  g_t.pending = e;
}

void timing_after(hipStream_t st, const char* kernel) {
  if (!g_t.on || !g_t.pending) return;
  hipEvent_t e = take_event();
  if (!e) return;
  const hipError_t r = hipEventRecord(e, st);
  if (r != hipSuccess) {
    if (g_t.err == hipSuccess) g_t.err = r;
    g_t.pool.push_back(e);
    return;
  }
  g_t.recs.push_back(Record{kernel, g_t.pending, e});
  g_t.pending = nullptr;
}

}  // namespace favor

extern "C" {

int favor_timing_start(void) {
  using favor::g_t;
  for (const auto& r : g_t.recs) {
    g_t.pool.push_back(r.start);
    g_t.pool.push_back(r.stop);
  }
  g_t.recs.clear();
  if (g_t.pending) g_t.pool.push_back(g_t.pending);
  g_t.pending = nullptr;
  g_t.err = hipSuccess;
  g_t.on = true;
  return FAVOR_OK;
}

int favor_timing_stop(int32_t max_kernels, const char** names, float* ms, int32_t* launches,
                      int32_t* n_kernels) {
  using favor::g_t;
  g_t.on = false;
  if (!n_kernels || (max_kernels > 0 && (!names || !ms || !launches))) return FAVOR_ERR_NULL;
  if (g_t.err != hipSuccess) return favor::record_hip_error(g_t.err);
  std::vector<const char*> nm;
  std::vector<double> tot;
  std::vector<int32_t> cnt;
  for (const auto& r : g_t.recs) {
    hipError_t e = hipEventSynchronize(r.stop);
    float t = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&t, r.start, r.stop);
    if (e != hipSuccess) return favor::record_hip_error(e);
    size_t k = 0;
    while (k < nm.size() && std::strcmp(nm[k], r.name) != 0) ++k;
    if (k == nm.size()) {
      nm.push_back(r.name);
      tot.push_back(0.0);
      cnt.push_back(0);
    }
    tot[k] += t;
    cnt[k] += 1;
  }
  *n_kernels = static_cast<int32_t>(nm.size());
  for (size_t k = 0; k < nm.size() && static_cast<int32_t>(k) < max_kernels; ++k) {
    names[k] = nm[k];
    ms[k] = static_cast<float>(tot[k]);
    launches[k] = cnt[k];
  }
  return FAVOR_OK;
}

}  // extern "C"
