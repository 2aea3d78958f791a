// Opt-in kernel timing with HIP events on the launch stream (spd_profile_*).
#include <vector>

#include "spd_internal.h"

namespace spd {
namespace {

constexpr int kMaxLaunches = 1024;

struct Profile {
  bool active = false;
  bool failed = false;
  std::vector<hipEvent_t> ev[SPD_K_COUNT];   // 2 per launch: start, stop
  int used[SPD_K_COUNT] = {};
};

thread_local Profile g_prof;

hipEvent_t event_at(int k, int i) {
  auto &v = g_prof.ev[k];
  while (static_cast<int>(v.size()) <= i) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) {
      g_prof.failed = true;
      return nullptr;
    }
    v.push_back(e);
  }
  return v[i];
}

}  // namespace

void prof_start(int k, hipStream_t st) {
  if (!g_prof.active || k < 0 || k >= SPD_K_COUNT || g_prof.used[k] >= kMaxLaunches) return;
  hipEvent_t e = event_at(k, 2 * g_prof.used[k]);
  if (e && hipEventRecord(e, st) != hipSuccess) g_prof.failed = true;
}

void prof_stop(int k, hipStream_t st) {
  if (!g_prof.active || k < 0 || k >= SPD_K_COUNT || g_prof.used[k] >= kMaxLaunches) return;
  hipEvent_t e = event_at(k, 2 * g_prof.used[k] + 1);
  if (e && hipEventRecord(e, st) != hipSuccess) g_prof.failed = true;
  ++g_prof.used[k];
}

}  // namespace spd

using namespace spd;

extern "C" spd_status spd_profile_begin(void) {
  g_prof.active = true;
  g_prof.failed = false;
  for (int k = 0; k < SPD_K_COUNT; ++k) {
    g_prof.used[k] = 0;
    event_at(k, 127);   // create a first batch of events outside any timed region
  }
  return g_prof.failed ? SPD_ERR_HIP : SPD_OK;
}

extern "C" spd_status spd_profile_end(int64_t *launches, double *total_ms) {
  if (!launches || !total_ms) return SPD_ERR_INVALID_ARG;
  spd_status st = g_prof.failed ? SPD_ERR_HIP : SPD_OK;
  for (int k = 0; k < SPD_K_COUNT; ++k) {
    double sum = 0.0;
    for (int i = 0; i < g_prof.used[k]; ++i) {
      hipEvent_t a = g_prof.ev[k][2 * i], b = g_prof.ev[k][2 * i + 1];
      float ms = 0.0f;
      if (hipEventSynchronize(b) != hipSuccess || hipEventElapsedTime(&ms, a, b) != hipSuccess) {
        st = SPD_ERR_HIP;
        continue;
      }
      sum += ms;
    }
    launches[k] = g_prof.used[k];
    total_ms[k] = sum;
    g_prof.used[k] = 0;
  }
  g_prof.active = false;
  return st;
}
