// Fused int4 dequant-GEMV for the selected experts (decode and small batches).
//
// The routed experts' projections are INT4 with affine groups of 64 columns,
// one scale and one bias per group ("Optimizing a 14.3 GB model for an 8 GB
// machine", section "Vectorization helped when it respected the storage
// layout").  Once expert reads are explicit these matvecs are the largest GPU
// cost of a decode step, and the kernel that won on the pages gave the GPU many
// independent workgroups instead of making lanes cooperate on one expert (same
// page, section "MoE needed parallel work, reuse, and coarse overlap").  The
// same section's four-groups-at-a-time lesson (shorter dependency chains) is
// what the per-lane multi-group loop below keeps.
//
// gfx950 design (batch-1 decode moves ~27 MB per layer, ~3.4 us at 8 TB/s, so
// every wave puts all of its bytes in flight in one round trip and the VALU
// cost per weight has to stay well under the ~4 ops/weight the CUs can issue
// at that bandwidth):
//  * A wave owns R rows of one matrix; its 64 lanes are P K-parts x R rows
//    (gate/up: 8 x 8, down: 4 x 16).  In the blob layout the 16-byte chunks of
//    64 consecutive rows sit side by side, so each 128-bit load instruction
//    reads P runs of R*16 bytes.  Every lane issues all of its nibble and
//    (scale, bias) loads before it computes anything.
//  * Dequant without converts, in exact integer arithmetic: each 64-column
//    group of the activation row is scaled by a power of two that puts its
//    largest magnitude in [2^13, 2^14) and rounded to integers (16-bit fixed
//    point per group, relative error <= 2^-14 of the group maximum), held as
//    four balanced base-16 digits.  v_dot8_i32_i4 multiplies eight weight
//    nibbles (xor 8 makes them the signed q - 8) with eight digits at once, so
//    8 weights cost 1 xor and 4 dot8: exact int32 sums per group.
//  * Group-factored dequant: sum_c (s q_c + b) x_c = s * 2^e * sum_c (q_c - 8) x_c
//    + (b + 8 s) * sum_c x_c, with the fp32 group sum for the second term.
//  * The activation row is staged once per workgroup in LDS as digit words,
//    each K-part at its own bank offset so the parts' broadcast reads do not
//    conflict; group sums and group exponents are reduced during the staging.
//  * K-parts are summed with cross-lane shuffles; gate and up (two waves of
//    one workgroup) meet in LDS, so GELU(gate) * up needs no global sync.
//  * Down: a workgroup holds the k experts of one token for 16 output rows, one
//    wave each, and sums them in rank order in LDS (deterministic combine).
//    The grouped path writes per-pair outputs and a gather kernel combines them,
//    again in rank order.
#include "common.h"
#include "kernels.h"
#include "q4_lane.h"

namespace moe {

namespace {

using namespace lane;

constexpr int kMBGrouped = 4;  // tokens per pass over the loaded weights (grouped path)

struct Members {
  int expert;  // may be out of range: the blob lookup then fails
  int count;
  int first;   // ungrouped: the pair itself; grouped: index into sorted_pair
};

__device__ __forceinline__ Members resolve_group(int group, const int32_t* __restrict__ topk_idx,
                                                 const int32_t* __restrict__ offsets,
                                                 const uint8_t* __restrict__ pair_mask,
                                                 int mask_value, int n_pairs) {
  Members m;
  if (offsets == nullptr) {
    m.expert = topk_idx[group];
    m.count = 1;
    m.first = group;
    if (pair_mask && (int)pair_mask[group] != mask_value) m.count = 0;
  } else {
    int a = offsets[group], b = offsets[group + 1];
    a = max(0, min(a, n_pairs));
    b = max(a, min(b, n_pairs));
    m.expert = group;
    m.count = b - a;
    m.first = a;
  }
  return m;
}

__device__ __forceinline__ int member_pair(const Members& m, int i, const int32_t* __restrict__ sorted_pair,
                                           bool grouped, int n_pairs) {
  if (!grouped) return m.first;
  const int p = sorted_pair[m.first + i];
  return (p >= 0 && p < n_pairs) ? p : -1;
}

// The expert's blob through the slot table, or nullptr if it is not resident.
__device__ __forceinline__ const uint8_t* expert_blob(int expert, int E, const int32_t* __restrict__ slot_of_expert,
                                                      int n_slots, const uint8_t* arena, int64_t slot_stride) {
  if (expert < 0 || expert >= E) return nullptr;
  const int slot = slot_of_expert[expert];
  if (slot < 0 || slot >= n_slots) return nullptr;
  return arena + (int64_t)slot * slot_stride;
}

// XCD-aware block mapping.  Workgroups are dispatched round-robin over the 8
// XCDs (block b runs on XCD b % 8), and every XCD has its own L2.  The `per`
// workgroups that cover one 64-row tile read neighbouring halves of the same
// 128-byte lines (scale/bias words), so they are given block ids with equal
// b % 8: the lines are then fetched from HBM once, into one L2.
constexpr int kXcds = 8;
struct TileSub {
  int tile, sub;
};
__device__ __forceinline__ TileSub xcd_tile_map(int b, int n_tiles, int per) {
  const int span = kXcds * per;
  const int full = (n_tiles * per) / span * span;
  if (b < full) return TileSub{(b / span) * kXcds + b % kXcds, (b / kXcds) % per};
  return TileSub{b / per, b % per};
}

// ------------------------------------------------------------------ gate/up

// Workgroup = 2 x RB waves: (gate, up) x RB blocks of R rows of one expert
// group; lanes = P parts x R rows.  The staged activation row is shared by all
// 2 * RB waves.
#ifndef MOE_GATEUP_RB
#define MOE_GATEUP_RB 2
#endif
constexpr int kGateRB = MOE_GATEUP_RB;

template <int P, int GPP, int MB, bool GROUPED>
__global__ __launch_bounds__(2 * kGateRB * kWave) void k_gateup(GateupArgs a) {
  constexpr int R = kWave / P;
  constexpr int GMAX = P * GPP;
  constexpr int NT = 2 * kGateRB * kWave;
  constexpr int NPASS = (8 * GMAX + NT - 1) / NT;
  __shared__ XRow<P, GMAX> xs[MB];
  __shared__ float g_lds[MB][kGateRB][R];
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int mat = wave / kGateRB;  // 0: gate, 1: up
  const int rbi = wave % kGateRB;
  const int lane = tid % kWave;
  const int j = lane / R, r = lane % R;
  const int n_pairs = a.T * a.k;
  constexpr int kPer = kTileRows / (kGateRB * R);  // workgroups per 64-row tile
  const int tiles_per_group = a.f / kTileRows;
  const TileSub ts = xcd_tile_map(blockIdx.x, a.n_rb / kPer * (GROUPED ? a.E : a.T * a.k), kPer);
  const int group = ts.tile / tiles_per_group;
  const int row0 = (ts.tile % tiles_per_group) * kTileRows + ts.sub * (kGateRB * R) + rbi * R;
  const Members m = resolve_group(group, a.topk_idx, GROUPED ? a.offsets : nullptr, a.pair_mask, a.mask_value,
                                  n_pairs);
  if (m.count <= 0) return;
  const uint8_t* blob = expert_blob(m.expert, a.E, a.slot_of_expert, a.n_slots, a.arena, a.slot_stride);
  const bool ok = blob != nullptr;
  if (!ok) blob = a.arena;  // keep the loads in bounds; the outputs become NaN
  const int G = a.d / kGroup;
  const Part pt = part_of<P>(j, G);
  const int trow = (row0 % kTileRows) + r;
  const int64_t tile = (int64_t)(row0 / kTileRows);
  const uint8_t* qbase = blob + (mat ? a.off_q1 : a.off_q0) + tile * (kTileRows * a.d / 2) + trow * 16;
  const uint8_t* sbase = blob + (mat ? a.off_sb1 : a.off_sb0) + tile * (kTileRows * G * 4) + trow * 4;
  LaneSlice<GPP> w;
  if constexpr (!GROUPED) {
    // one token: activation loads, then every weight load, then compute as
    // the weights arrive (in issue order)
    const int p = m.first;
    StageRegs<NPASS> sr;
    stage_load<NPASS>(sr, a.h + (int64_t)(p / a.k) * a.d, G, tid, NT);
    load_lane<GPP>(w, qbase, sbase, pt, G);
    stage_store<P, GMAX, NPASS>(xs[0], sr, G, tid, NT);
    __syncthreads();
    float v = lane_dot<P, GPP, GMAX>(w, xs[0], j, pt, G, a.nck);
    if (!ok) v = f32_nan();
    if (mat == 0 && j == 0) g_lds[0][rbi][r] = v;
    __syncthreads();
    if (mat == 1 && j == 0) a.act[(int64_t)p * a.f + row0 + r] = gelu_tanh(g_lds[0][rbi][r]) * v;
  } else {
    load_lane<GPP>(w, qbase, sbase, pt, G);
    for (int i0 = 0; i0 < m.count; i0 += MB) {
      const int nm = min(MB, m.count - i0);
      int pm[MB];
      StageRegs<NPASS> sr[MB];
#pragma unroll
      for (int t = 0; t < MB; ++t) {
        pm[t] = t < nm ? member_pair(m, i0 + t, a.sorted_pair, true, n_pairs) : -1;
        if (pm[t] >= 0) stage_load<NPASS>(sr[t], a.h + (int64_t)(pm[t] / a.k) * a.d, G, tid, NT);
      }
#pragma unroll
      for (int t = 0; t < MB; ++t)
        if (pm[t] >= 0) stage_store<P, GMAX, NPASS>(xs[t], sr[t], G, tid, NT);
      __syncthreads();
      float u[MB];
#pragma unroll
      for (int t = 0; t < MB; ++t) {
        u[t] = 0.0f;
        if (pm[t] >= 0) {
          float v = lane_dot<P, GPP, GMAX>(w, xs[t], j, pt, G, a.nck);
          if (!ok) v = f32_nan();
          if (mat == 0 && j == 0) g_lds[t][rbi][r] = v;
          u[t] = v;
        }
      }
      __syncthreads();
      if (mat == 1 && j == 0) {
#pragma unroll
        for (int t = 0; t < MB; ++t)
          if (pm[t] >= 0) a.act[(int64_t)pm[t] * a.f + row0 + r] = gelu_tanh(g_lds[t][rbi][r]) * u[t];
      }
      if (i0 + MB < m.count) __syncthreads();
    }
  }
}

// ------------------------------------------------------------------ down + combine

constexpr int kDownP = 4;              // down: lanes = 4 K-parts x 16 rows
constexpr int kDownR = kWave / kDownP;

// Ungrouped: workgroup = k waves (the k experts of token t) x 16 output rows.
template <int GPP>
__global__ __launch_bounds__(1024) void k_down_token(DownArgs a) {
  constexpr int GMAX = kDownP * GPP;
  __shared__ XRow<kDownP, GMAX> xs[16];
  __shared__ float o_lds[16][kDownR];
  const int tid = threadIdx.x;
  const int jr = tid / kWave;  // rank of the expert this wave runs
  const int lane = tid % kWave;
  const int j = lane / kDownR, r = lane % kDownR;
  constexpr int kPer = kTileRows / kDownR;
  const int tiles_per_tok = a.d / kTileRows;
  const TileSub ts = xcd_tile_map(blockIdx.x, a.T * tiles_per_tok, kPer);
  const int t = ts.tile / tiles_per_tok;
  const int row0 = (ts.tile % tiles_per_tok) * kTileRows + ts.sub * kDownR;
  const int p = t * a.k + jr;
  const uint8_t* blob = expert_blob(a.topk_idx[p], a.E, a.slot_of_expert, a.n_slots, a.arena, a.slot_stride);
  const bool ok = blob != nullptr;
  if (!ok) blob = a.arena;
  const int G = a.f / kGroup;
  const Part pt = part_of<kDownP>(j, G);
  const int trow = (row0 % kTileRows) + r;
  const int64_t tile = (int64_t)(row0 / kTileRows);
  constexpr int NPASS = (8 * GMAX + kWave - 1) / kWave;
  StageRegs<NPASS> sr;
  LaneSlice<GPP> w;
  stage_load<NPASS>(sr, a.act + (int64_t)p * a.f, G, lane, kWave);
  if constexpr (GPP >= 7) {
    // 16 waves leave 128 VGPRs a wave: the activations reach LDS before the
    // weight slice is loaded, so the two are never in registers together
    stage_store<kDownP, GMAX, NPASS>(xs[jr], sr, G, lane, kWave);
    load_lane<GPP>(w, blob + a.off_q + tile * (kTileRows * a.f / 2) + trow * 16,
                   blob + a.off_sb + tile * (kTileRows * G * 4) + trow * 4, pt, G);
  } else {
    load_lane<GPP>(w, blob + a.off_q + tile * (kTileRows * a.f / 2) + trow * 16,
                   blob + a.off_sb + tile * (kTileRows * G * 4) + trow * 4, pt, G);
    stage_store<kDownP, GMAX, NPASS>(xs[jr], sr, G, lane, kWave);
  }
  __syncthreads();
  float v = lane_dot<kDownP, GPP, GMAX>(w, xs[jr], j, pt, G, a.nck);
  if (!ok) v = f32_nan();
  if (j == 0) o_lds[jr][r] = v;
  __syncthreads();
  if (jr == 0 && j == 0) {
    const int row = row0 + r;
    float y = a.residual ? a.residual[(int64_t)t * a.d + row] : 0.0f;
    for (int jj = 0; jj < a.k; ++jj) y = fmaf(a.topk_w[t * a.k + jj], o_lds[jj][r], y);
    a.y[(int64_t)t * a.d + row] = y;
  }
}

// Grouped: workgroup = 1 wave x 16 output rows of one expert, all its pairs;
// per-pair outputs go to pair_out[p][row].
template <int GPP, int MB>
__global__ __launch_bounds__(kWave) void k_down_grouped(DownArgs a) {
  constexpr int GMAX = kDownP * GPP;
  __shared__ XRow<kDownP, GMAX> xs[MB];
  const int lane = threadIdx.x;
  const int j = lane / kDownR, r = lane % kDownR;
  const int n_pairs = a.T * a.k;
  constexpr int kPer = kTileRows / kDownR;
  const int tiles_per_e = a.d / kTileRows;
  const TileSub ts = xcd_tile_map(blockIdx.x, a.E * tiles_per_e, kPer);
  const int e = ts.tile / tiles_per_e;
  const int row0 = (ts.tile % tiles_per_e) * kTileRows + ts.sub * kDownR;
  const Members m = resolve_group(e, a.topk_idx, a.offsets, nullptr, 0, n_pairs);
  if (m.count <= 0) return;
  const uint8_t* blob = expert_blob(m.expert, a.E, a.slot_of_expert, a.n_slots, a.arena, a.slot_stride);
  const bool ok = blob != nullptr;
  if (!ok) blob = a.arena;
  const int G = a.f / kGroup;
  const Part pt = part_of<kDownP>(j, G);
  const int trow = (row0 % kTileRows) + r;
  const int64_t tile = (int64_t)(row0 / kTileRows);
  constexpr int NPASS = (8 * GMAX + kWave - 1) / kWave;
  LaneSlice<GPP> w;
  load_lane<GPP>(w, blob + a.off_q + tile * (kTileRows * a.f / 2) + trow * 16,
                 blob + a.off_sb + tile * (kTileRows * G * 4) + trow * 4, pt, G);
  for (int i0 = 0; i0 < m.count; i0 += MB) {
    const int nm = min(MB, m.count - i0);
    int pm[MB];
    StageRegs<NPASS> sr[MB];
#pragma unroll
    for (int t = 0; t < MB; ++t) {
      pm[t] = t < nm ? member_pair(m, i0 + t, a.sorted_pair, true, n_pairs) : -1;
      if (pm[t] >= 0) stage_load<NPASS>(sr[t], a.act + (int64_t)pm[t] * a.f, G, lane, kWave);
    }
#pragma unroll
    for (int t = 0; t < MB; ++t)
      if (pm[t] >= 0) stage_store<kDownP, GMAX, NPASS>(xs[t], sr[t], G, lane, kWave);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < MB; ++t) {
      if (pm[t] >= 0) {
        float v = lane_dot<kDownP, GPP, GMAX>(w, xs[t], j, pt, G, a.nck);
        if (!ok) v = f32_nan();
        if (j == 0) a.pair_out[(int64_t)pm[t] * a.d + row0 + r] = v;
      }
    }
    if (i0 + MB < m.count) __syncthreads();
  }
}

// y[t][i] = residual[t][i] + sum_j w[t][j] * pair_out[t*k+j][i], j in rank order.
__global__ __launch_bounds__(256) void k_combine(DownArgs a) {
  const int64_t n4 = (int64_t)a.T * a.d / 4;
  const int64_t i4 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i4 >= n4) return;
  const int t = (int)(i4 * 4 / a.d);
  const int col = (int)(i4 * 4 - (int64_t)t * a.d);
  float4 y = a.residual ? reinterpret_cast<const float4*>(a.residual)[i4] : make_float4(0.f, 0.f, 0.f, 0.f);
  for (int jj = 0; jj < a.k; ++jj) {
    const float wj = a.topk_w[t * a.k + jj];
    const float4 o = *reinterpret_cast<const float4*>(a.pair_out + (int64_t)(t * a.k + jj) * a.d + col);
    y.x = fmaf(wj, o.x, y.x);
    y.y = fmaf(wj, o.y, y.y);
    y.z = fmaf(wj, o.z, y.z);
    y.w = fmaf(wj, o.w, y.w);
  }
  reinterpret_cast<float4*>(a.y)[i4] = y;
}

}  // namespace

// ------------------------------------------------------------------ host side

constexpr int kGateP = 8;  // gate/up: lanes = 8 K-parts x 8 rows

// Groups per K-part: the smallest instantiated count covering the row's groups
// (gate/up 2816 columns: 44 groups / 8 parts -> 6; down 704 columns: 11 / 4 -> 3).
static int pick_gpp(int groups, int parts) {
  static const int opts[] = {1, 2, 3, 4, 6, 8};
  const int need = (groups + parts - 1) / parts;
  for (int o : opts)
    if (o >= need) return o;
  return -1;
}

bool gemv_supported(int d, int f, int k) {
  return pick_gpp(d / kGroup, kGateP) > 0 && pick_gpp(f / kGroup, kDownP) > 0 && k <= 16;
}

size_t gemv_workspace_bytes(int call, int T, int d, int k, bool grouped) {
  if (call == MOE_CALL_DOWN_COMBINE && grouped) return round256((int64_t)T * k * d * 4);
  return 0;
}

#define MOE_GPP_SWITCH(GPPV, CASE)        \
  switch (GPPV) {                         \
    CASE(1)                               \
    CASE(2)                               \
    CASE(3)                               \
    CASE(4)                               \
    CASE(6)                               \
    CASE(8)                               \
    default: return hipErrorInvalidValue; \
  }

hipError_t launch_gateup_fp32(GateupArgs a, hipStream_t s) {
  const bool grouped = a.offsets != nullptr;
  constexpr int R = kWave / kGateP;
  if (a.f % (kGateRB * R)) return hipErrorInvalidValue;
  a.n_rb = a.f / (kGateRB * R);
  const int n_groups = grouped ? a.E : a.T * a.k;
  const int grid = n_groups * a.n_rb;
  a.nck = 2 * pick_gpp(a.d / kGroup, kGateP);
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  take_profile_events(MOE_CALL_GATEUP, &ev0, &ev1);
#define MOE_GATEUP_CASE(N)                                                                      \
  case N:                                                                                       \
    if (grouped)                                                                                \
      launch_maybe_timed((k_gateup<kGateP, N, kMBGrouped, true>), grid, 2 * kGateRB * kWave, s, ev0, ev1, a); \
    else                                                                                                       \
      launch_maybe_timed((k_gateup<kGateP, N, 1, false>), grid, 2 * kGateRB * kWave, s, ev0, ev1, a);         \
    break;
  MOE_GPP_SWITCH(pick_gpp(a.d / kGroup, kGateP), MOE_GATEUP_CASE)
#undef MOE_GATEUP_CASE
  return hipGetLastError();
}

hipError_t launch_down_fp32(DownArgs a, void* ws, hipStream_t s) {
  const bool grouped = a.offsets != nullptr;
  a.n_rb = a.d / kDownR;
  a.pair_out = reinterpret_cast<float*>(ws);
  a.nck = 2 * pick_gpp(a.f / kGroup, kDownP);
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  take_profile_events(MOE_CALL_DOWN_COMBINE, &ev0, &ev1);
  if (!grouped) {
    const int grid = a.T * a.n_rb;
#define MOE_DOWN_CASE(N)                                                       \
  case N:                                                                      \
    launch_maybe_timed((k_down_token<N>), grid, a.k * kWave, s, ev0, ev1, a); \
    break;
    MOE_GPP_SWITCH(pick_gpp(a.f / kGroup, kDownP), MOE_DOWN_CASE)
#undef MOE_DOWN_CASE
    return hipGetLastError();
  }
  const int grid = a.E * a.n_rb;
#define MOE_DOWNG_CASE(N)                                                              \
  case N:                                                                              \
    launch_maybe_timed((k_down_grouped<N, kMBGrouped>), grid, kWave, s, ev0, ev1, a); \
    break;
  MOE_GPP_SWITCH(pick_gpp(a.f / kGroup, kDownP), MOE_DOWNG_CASE)
#undef MOE_DOWNG_CASE
  const int64_t n4 = (int64_t)a.T * a.d / 4;
  hipLaunchKernelGGL(k_combine, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

#undef MOE_GPP_SWITCH

hipError_t launch_combine(const float* pair_out, const float* topk_w, const float* residual, float* y, int T,
                          int d, int k, hipStream_t s) {
  DownArgs a{};
  a.pair_out = const_cast<float*>(pair_out);
  a.topk_w = topk_w;
  a.residual = residual;
  a.y = y;
  a.T = T;
  a.d = d;
  a.k = k;
  const int64_t n4 = (int64_t)T * d / 4;
  hipLaunchKernelGGL(k_combine, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
