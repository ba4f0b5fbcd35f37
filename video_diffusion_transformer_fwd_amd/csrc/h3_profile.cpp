// Per-stage timing of the path with HIP events recorded on the launch stream around each
// launch of the selected stages.  Host-side state, not thread-safe (one profiling session
// per process at a time).
#include <hip/hip_runtime.h>

#include <vector>

#include "h3_internal.h"

namespace h3 {

namespace {
struct ProfState {
  bool on = false;
  uint32_t mask = 0;
  std::vector<hipEvent_t> events;  // begin/end pairs
  std::vector<int> stage;          // stage of each pair
  int used_pairs = 0;
  bool overflow = false;
};
ProfState g_prof;
}  // namespace

ProfScope::ProfScope(int st, hipStream_t s) : stage_(st), stream_(s), pair_(-1) {
  if (!g_prof.on || !(g_prof.mask & (1u << st))) return;
  if (static_cast<size_t>(g_prof.used_pairs) * 2 + 2 > g_prof.events.size()) {
    g_prof.overflow = true;
    return;
  }
  pair_ = g_prof.used_pairs++;
  g_prof.stage[pair_] = st;
  hipEventRecord(g_prof.events[2 * pair_], s);
}

ProfScope::~ProfScope() {
  if (pair_ >= 0) hipEventRecord(g_prof.events[2 * pair_ + 1], stream_);
}

}  // namespace h3

using namespace h3;

extern "C" {

int32_t h3_profile_begin(uint32_t stage_mask, int32_t max_launches) {
  if (g_prof.on) return fail(H3_EINVAL, "h3_profile_begin: a session is already open");
  if (max_launches < 1 || max_launches > (1 << 20))
    return fail(H3_EINVAL, "h3_profile_begin: max_launches must be in [1, 2^20]");
  g_prof = ProfState{};
  g_prof.events.resize(2 * static_cast<size_t>(max_launches));
  g_prof.stage.resize(max_launches);
  for (auto &e : g_prof.events) {
    if (hipEventCreate(&e) != hipSuccess) {
      for (auto &x : g_prof.events)
        if (x) hipEventDestroy(x);
      g_prof = ProfState{};
      return fail(H3_EHIP, "h3_profile_begin: hipEventCreate failed");
    }
  }
  g_prof.mask = stage_mask;
  g_prof.on = true;
  return H3_OK;
}

int32_t h3_profile_end(double *ms_per_stage, int32_t *launches_per_stage) {
  if (!g_prof.on) return fail(H3_EINVAL, "h3_profile_end: no open session");
  int32_t rc = H3_OK;
  if (ms_per_stage && launches_per_stage) {
    for (int i = 0; i < H3_ST_COUNT; ++i) {
      ms_per_stage[i] = 0.0;
      launches_per_stage[i] = 0;
    }
    for (int p = 0; p < g_prof.used_pairs; ++p) {
      float ms = 0.f;
      if (hipEventSynchronize(g_prof.events[2 * p + 1]) != hipSuccess ||
          hipEventElapsedTime(&ms, g_prof.events[2 * p], g_prof.events[2 * p + 1]) != hipSuccess) {
        rc = fail(H3_EHIP, "h3_profile_end: event query failed");
        break;
      }
      ms_per_stage[g_prof.stage[p]] += ms;
      launches_per_stage[g_prof.stage[p]] += 1;
    }
  } else {
    hipDeviceSynchronize();
  }
  const bool overflow = g_prof.overflow;
  for (auto &e : g_prof.events) hipEventDestroy(e);
  g_prof = ProfState{};
  if (rc == H3_OK && overflow) rc = fail(H3_EINVAL, "h3_profile_end: more launches than max_launches");
  return rc;
}

}  // extern "C"
