// Host-only stand-ins for the launchers and size queries that the library's
// HIP sources define, so that api.cpp and slot_cache.cpp link into a CPU
// program under AddressSanitizer and UndefinedBehaviorSanitizer.  Launches do
// nothing except the staging copy, which copies at once (as the runtime stub
// does) so that the expert cache's slot contents can be checked; every launch
// is a failure-injection point of the runtime stub.  Workspace sizes are
// plausible stand-ins: the checks here are of the host code's argument and
// state handling, never of results.
#include <cstring>

#include "../../int4_routed_expert_route_amd/csrc/kernels.h"

extern "C" int stub_failing(void);

namespace moe {

namespace {
hipError_t launched() { return stub_failing() ? hipErrorLaunchFailure : hipSuccess; }
}  // namespace

size_t route_workspace_bytes(int T, int d, int E) { return 256 + (size_t)T * (size_t)(E + d) * 4; }
hipError_t route_scratch(void** out) {
  static unsigned char scratch[4096];
  *out = scratch;
  return hipSuccess;
}
hipError_t launch_route(const float*, const float*, float, const float*, const float*, int, int, int, int, float*,
                        int32_t*, float*, void*, hipStream_t) {
  return launched();
}
hipError_t launch_rms_rescale(const float*, int, int, float, float*, hipStream_t) { return launched(); }
size_t permute_workspace_bytes(int n_pairs, int E) { return n_pairs > 1024 ? (size_t)64 * E * 4 : 0; }
hipError_t launch_permute(const int32_t*, int, int, int32_t*, int32_t*, int32_t*, int32_t*, void*, size_t,
                          hipStream_t) {
  return launched();
}

bool gemv_supported(int d, int f, int k) { return d % 64 == 0 && f % 64 == 0 && k >= 1 && k <= 8; }
size_t gemv_workspace_bytes(int call, int T, int d, int k, bool grouped) {
  return grouped || call == 3 ? (size_t)T * k * d * 4 : 0;
}
hipError_t launch_gateup_fp32(GateupArgs, hipStream_t) { return launched(); }
hipError_t launch_down_fp32(DownArgs, void*, hipStream_t) { return launched(); }
hipError_t launch_combine(const float*, const float*, const float*, float*, int, int, int, hipStream_t) {
  return launched();
}

bool mfma_supported(int d, int f) { return d % 128 == 0 && f % 128 == 0; }
size_t mfma_act_bytes(int T, int f, int k) { return (size_t)T * k * f * 2 + (size_t)T * k * (f / 64); }
size_t mfma_workspace_bytes(int, int T, int d, int, int E, int k) {
  return 4096 + (size_t)E * 64 + (size_t)T * k * d * 4;
}
hipError_t launch_gateup_mfma(bool, const float*, const int32_t*, const int32_t*, const int32_t*, int,
                              const uint8_t*, int64_t, int, int, int, int, int, int64_t, int64_t, int64_t, int64_t,
                              void*, void*, hipStream_t) {
  return launched();
}
hipError_t launch_down_mfma(bool, const void*, const int32_t*, const int32_t*, const int32_t*, int, const uint8_t*,
                            int64_t, int, int, int, int, int, int64_t, int64_t, const float*, const float*, float*,
                            void*, hipStream_t) {
  return launched();
}

hipError_t launch_stage_copy(const StageCopyArgs& a, hipStream_t) {
  if (stub_failing()) return hipErrorLaunchFailure;
  for (int i = 0; i < a.n; ++i) std::memmove(a.dst[i], a.src[i], (size_t)a.bytes);
  return hipSuccess;
}
// The device-resident cache is not driven here.
hipError_t launch_cache_step(const CacheStepArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_stage_misses(const uint8_t*, uint8_t*, int, int, int, int64_t, int64_t, const int32_t*,
                               const int32_t*, hipStream_t) {
  return hipErrorNotSupported;
}

bool decode_fused_supported(int d, int f, int E, int k, int cus, int* G, int* rpw) {
  if (d > 3072 || f > 768 || E > 256 || k > 8 || k * f / 32 > cus) return false;
  *G = k * f / 32;
  *rpw = 1;
  return true;
}
size_t decode_fused_workspace_bytes(int L, int d, int, int E, int k) {
  return 4096 + (size_t)L * (size_t)(d + E + k) * 64;
}
hipError_t launch_decode_fused(float*, int, const float*, float, const float*, const float*, const int32_t*, int,
                               const uint8_t*, int64_t, int64_t, int, int, int, int, int64_t, int64_t, int64_t,
                               int64_t, int64_t, int64_t, int32_t*, float*, float*, void*, int, int, hipStream_t) {
  return launched();
}

size_t shared_expert_workspace_bytes(int T, int f_sh) { return (size_t)T * f_sh * 4; }
hipError_t launch_shared_expert_bf16(const uint16_t*, const uint16_t*, const float*, const float*, int, int, int,
                                     float*, void*, hipStream_t) {
  return launched();
}
hipError_t launch_shared_gemv_bf16(const uint16_t*, const float*, int, int, int, float*, hipStream_t) {
  return launched();
}

}  // namespace moe
