// Internal launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ---- one-shot kernel timing events (api.cpp); take_profile_events returns
// true and clears the arm when `call` was armed on this thread.
bool take_profile_events(int call, hipEvent_t* start, hipEvent_t* stop);

// ---- routing (route.hip)
size_t route_workspace_bytes(int T, int d, int E);
// moe_route_noalloc: a static device array per GPU instead of a caller's workspace
constexpr size_t kRouteScratchBytes = (size_t)16 << 20;
constexpr int kMaxScratchDevices = 64;
hipError_t route_scratch(void** out);
hipError_t launch_route(const float* x, const float* norm_w, float eps, const float* router_w,
                        const float* router_bias, int T, int d, int E, int k, float* h_out,
                        int32_t* topk_idx, float* topk_w, void* ws, hipStream_t s);
hipError_t launch_rms_rescale(const float* x, int T, int d, float eps, float* out, hipStream_t s);

// ---- pair permutation (permute.hip)
// Workspace of the two-launch path (0: one workgroup walks every pair).
size_t permute_workspace_bytes(int n_pairs, int E);
hipError_t launch_permute(const int32_t* topk_idx, int n_pairs, int E, int32_t* counts, int32_t* offsets,
                          int32_t* sorted_pair, int32_t* pair_pos, void* ws, size_t ws_bytes, hipStream_t s);

// ---- fp32 dequant-GEMV (q4_gemv.hip)
struct GateupArgs {
  const float* h;
  const int32_t* topk_idx;
  const int32_t* slot_of_expert;
  int n_slots;
  const uint8_t* arena;
  int64_t slot_stride;
  const int32_t* offsets;
  const int32_t* sorted_pair;
  const uint8_t* pair_mask;
  int mask_value;
  int T, d, f, E, k;
  int64_t off_q0, off_q1, off_sb0, off_sb1;  // gate and up sections
  float* act;
  int n_rb;  // set by the launcher
  int nck;   // set by the launcher: chunks per lane
};

struct DownArgs {
  const float* act;
  const int32_t* topk_idx;
  const float* topk_w;
  const int32_t* slot_of_expert;
  int n_slots;
  const uint8_t* arena;
  int64_t slot_stride;
  const int32_t* offsets;
  const int32_t* sorted_pair;
  const float* residual;
  float* y;
  int T, d, f, E, k;
  int64_t off_q, off_sb;  // down sections
  float* pair_out;        // grouped path: per-pair outputs (workspace), set by the launcher
  int n_rb;               // set by the launcher
  int nck;                // set by the launcher: chunks per lane
};

bool gemv_supported(int d, int f, int k);
size_t gemv_workspace_bytes(int call, int T, int d, int k, bool grouped);
hipError_t launch_gateup_fp32(GateupArgs a, hipStream_t s);
hipError_t launch_down_fp32(DownArgs a, void* ws, hipStream_t s);

// rank-ordered gather combine of per-pair outputs (q4_gemv.hip)
hipError_t launch_combine(const float* pair_out, const float* topk_w, const float* residual, float* y, int T,
                          int d, int k, hipStream_t s);

// ---- grouped int4 GEMM on MFMA for batched prefill (q4_grouped_mfma.hip).
// act for these calls is block-scaled: 16-bit values [T*k][f], then int8
// exponents [T*k][f/64]; element (p, c) = value * 2^exp[p][c/64].
bool mfma_supported(int d, int f);
size_t mfma_act_bytes(int T, int f, int k);
size_t mfma_workspace_bytes(int call, int T, int d, int f, int E, int k);
hipError_t launch_gateup_mfma(bool direct, const float* h, const int32_t* offsets, const int32_t* sorted_pair,
                              const int32_t* slot_of_expert, int n_slots, const uint8_t* arena, int64_t slot_stride,
                              int T, int d, int f, int E, int k, int64_t off_q0, int64_t off_q1, int64_t off_sb0,
                              int64_t off_sb1, void* act_out, void* ws, hipStream_t s);
hipError_t launch_down_mfma(bool direct, const void* act_in, const int32_t* offsets, const int32_t* sorted_pair,
                            const int32_t* slot_of_expert, int n_slots, const uint8_t* arena, int64_t slot_stride,
                            int T, int d, int f, int E, int k, int64_t off_q, int64_t off_sb, const float* topk_w,
                            const float* residual, float* y, void* ws, hipStream_t s);

// ---- device-pulled staging of expert blobs (stage_copy.hip): copy i moves
// `bytes` (a multiple of 16) from src[i] (device-mapped pinned host memory,
// 16-byte aligned) to dst[i] (device, 16-byte aligned)
constexpr int kMaxStageCopies = 32;
struct StageCopyArgs {
  const uint8_t* src[kMaxStageCopies];
  uint8_t* dst[kMaxStageCopies];
  int n;
  int64_t bytes;
};
hipError_t launch_stage_copy(const StageCopyArgs& a, hipStream_t s);

// ---- the expert cache on the device (cache_device.hip): one layer step of
// the eviction rule (policy 0 LRU, 1 LFU over every step), then the copies of
// its misses from the device-mapped pinned pool.  Pointers are this layer's.
struct CacheStepArgs {
  int E, S, k, policy;
  int64_t step, blob;
  const int32_t* sel;    // [k] chosen experts
  int32_t* table;        // [E] slot of each expert, -1 absent
  int32_t* slot_expert;  // [S] expert of each slot, -1 empty
  int64_t* stamp;        // [S] last step each slot was used, -1 never
  int64_t* count;        // [E] use counts (LFU)
  uint8_t* hit_mask;     // [k] out
  int32_t* miss;         // [k][2] out: (expert, slot) installs in order
  int32_t* n_miss;       // [1] out
  int64_t* stats;        // [3] cumulative hits, misses, staged bytes
  uint32_t* err;         // set when a selection is out of range or repeats an expert
};
hipError_t launch_cache_step(const CacheStepArgs& a, hipStream_t s);
hipError_t launch_stage_misses(const uint8_t* pool_dev, uint8_t* arena, int E, int S, int k, int64_t blob,
                               int64_t stride, const int32_t* miss, const int32_t* n_miss, hipStream_t s);

// ---- fused batch-1 decode through many layers (decode_fused.hip)
bool decode_fused_supported(int d, int f, int E, int k, int cus, int* G, int* rpw);
size_t decode_fused_workspace_bytes(int L, int d, int f, int E, int k);
constexpr int kDecodeErrOffset = 384;  // byte offset of the error word in the workspace
hipError_t launch_decode_fused(float* x_io, int L, const float* norm_w, float eps, const float* router_w,
                               const float* router_bias, const int32_t* slot_tables, int n_slots,
                               const uint8_t* arena, int64_t layer_stride, int64_t slot_stride, int d, int f, int E,
                               int k, int64_t off_gq, int64_t off_uq, int64_t off_dq, int64_t off_gsb, int64_t off_usb,
                               int64_t off_dsb, int32_t* topk_idx, float* topk_w, float* x_next, void* ws, int G,
                               int rpw, hipStream_t s);

// ---- bf16 shared-path GEMV (shared_gemv.hip)
size_t shared_expert_workspace_bytes(int T, int f_sh);
hipError_t launch_shared_expert_bf16(const uint16_t* w_gu, const uint16_t* w_down, const float* h,
                                     const float* residual, int T, int d, int f_sh, float* out, void* ws,
                                     hipStream_t s);
hipError_t launch_shared_gemv_bf16(const uint16_t* w, const float* h, int T, int rows, int cols,
                                   float* out, hipStream_t s);

}  // namespace moe
