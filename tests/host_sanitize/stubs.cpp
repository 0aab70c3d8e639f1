// Host-only stand-ins for the kernel launchers and the few runtime calls the
// C ABI makes, so that the ABI's argument checks and geometry can run under
// AddressSanitizer and UndefinedBehaviorSanitizer on a machine without a GPU.
// Every launcher checks the geometry it receives and counts the call, or,
// while g_fail_launch is set, reports a launch failure as the runtime would.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "kara_device.h"

int g_launches = 0;
int g_fail_launch = 0;   // when set, every launcher reports a launch failure without counting a launch

static void check_geo(const kara::Geo& g, const char* who) {
  const bool ok = g.S >= 1 && g.Lyr >= 1 && g.Hkv >= 1 && g.G >= 1 && g.Hq == g.G * g.Hkv && g.GW == g.G * g.W &&
                  g.GWp >= g.GW && g.GWp % 32 == 0 && g.bs == (1 << g.bs_shift) && g.B >= 1 && g.B <= g.W &&
                  g.nblocks >= 1 && g.max_blocks >= 1 && isfinite(g.alpha) && g.alpha > 0.f;
  if (!ok) {
    fprintf(stderr, "%s: inconsistent geometry\n", who);
    abort();
  }
  ++g_launches;
}

namespace kara {
bool fused_score_supported(const Geo& g, int dtype) { return dtype == KARA_BF16 && g.D == 128 && g.W <= 1024; }
// staged-key scorer: 256 keys, 128 for fp32 rows of head_dim 128
bool small_score_supported(const Geo& g, int dtype) {
  if (fused_score_supported(g, dtype)) return false;
  if (dtype == KARA_BF16) return g.D == 64 && g.W <= 256;
  return g.W <= (g.D == 64 ? 256 : 128);
}
bool pipeline_supported(const Geo& g, int dtype) {
  return fused_score_supported(g, dtype) || small_score_supported(g, dtype);
}
hipError_t launch_score(const Geo& g, int, const void*, const void*, const int32_t*, const int32_t*, float*, float*,
                        hipStream_t) {
  if (g_fail_launch) return hipErrorLaunchFailure;
  check_geo(g, "launch_score");
  return hipSuccess;
}
size_t score_workspace_bytes(const Geo& g, int dtype) {
  if (pipeline_supported(g, dtype)) return 0;
  return (size_t)g.S * g.Lyr * g.Hkv * (size_t)g.GWp * sizeof(float);
}
hipError_t launch_select(const Geo& g, int, const float*, int32_t*, uint8_t*, hipStream_t) {
  if (g_fail_launch) return hipErrorLaunchFailure;
  check_geo(g, "launch_select");
  return hipSuccess;
}
hipError_t launch_compact(const Geo& g, int, void*, void*, int32_t*, const int32_t*, int32_t*, const int32_t*,
                          int32_t*, int32_t*, int max_freed, const int32_t*, hipStream_t) {
  if (g_fail_launch) return hipErrorLaunchFailure;
  check_geo(g, "launch_compact");
  if (max_freed != (g.W + g.bs - 1) / g.bs + 1) abort();
  return hipSuccess;
}
hipError_t launch_validate(const Geo& g, const int32_t*, const int32_t*, int32_t*, hipStream_t) {
  if (g_fail_launch) return hipErrorLaunchFailure;
  check_geo(g, "launch_validate");
  return hipSuccess;
}
size_t decode_attn_workspace_bytes(const Geo&) { return 0; }
int decode_attn_splits(const Geo&) { return 1; }
hipError_t launch_decode_attn(const Geo& g, int, const void*, const void*, const void*, const int32_t*,
                              const int32_t*, float*, float*, hipStream_t) {
  if (g_fail_launch) return hipErrorLaunchFailure;
  check_geo(g, "launch_decode_attn");
  return hipSuccess;
}
hipError_t launch_pipeline_any(const Geo& g, int dtype, const void*, void*, void*, int32_t*, const int32_t*, float*,
                               int32_t*, uint8_t*, int32_t*, int32_t*, int32_t*, int, int32_t*, hipStream_t) {
  if (g_fail_launch) return hipErrorLaunchFailure;
  check_geo(g, "launch_pipeline_any");
  if (!pipeline_supported(g, dtype)) abort();
  return hipSuccess;
}
hipError_t launch_pipeline_noalloc(const Geo& g, int dtype, const void*, void*, void*, int32_t*, const int32_t*,
                                   float*, int32_t*, uint8_t*, int32_t*, int32_t*, int32_t*, int, hipStream_t) {
  if (g_fail_launch) return hipErrorLaunchFailure;
  check_geo(g, "launch_pipeline_noalloc");
  if (!pipeline_supported(g, dtype)) abort();
  return hipSuccess;
}
}  // namespace kara

extern "C" {
hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t* d) {
  *d = 0;
  return hipSuccess;
}
int roctxRangePushA(const char*) { return 0; }
int roctxRangePop() { return 0; }
}
