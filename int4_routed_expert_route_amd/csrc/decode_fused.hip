// Batch-1 decode through many routed MoE layers in one persistent launch.
//
// One token per step goes through every layer in order: router, softmax over
// the experts, top-k, the selected experts' int4 gated FFN and the
// gate-weighted combine ("Optimizing a 14.3 GB model for an 8 GB machine":
// routed MoE per layer; TurboFieldfare video transcript: the router naming its
// experts).  The separate calls (moe_route, moe_expert_q4_gateup,
// moe_expert_q4_down_combine) cost three kernel launches per layer, and at
// batch 1 each of them is dominated by its fixed start/drain time, not by its
// ~27 MB of weights.  Here the layers run inside one kernel, in two phases per
// layer:
//
//   gate/up phase  every workgroup reduces the router partials of the layer
//                  (written by the previous phase), takes the top-k and the
//                  weights, stages h = RMSNorm(x) in LDS and computes 32 act
//                  columns of one selected expert (k * f/32 workgroups);
//   down phase     workgroup g owns d/G output rows: the k experts' down rows,
//                  the rank-ordered combine with the residual, and the next
//                  layer's router partials over its rows (sum_i Wr[e][i] w[i] y[i]
//                  and sum_i y[i]^2), so the next router needs no phase of its own.
//
// There is no device-wide barrier.  Every value one workgroup hands to another
// (act, router partials, sums of squares, the next layer's input) is written
// once per launch, through to memory, in a region of its own, encoded so that
// a zero word means "not written yet"; the reader loads the value itself with
// coherent loads until it is nonzero.  A barrier would cost the writer's wait
// for its stores, a flag round trip and then the data round trip; polling the
// data costs one round trip after the last write lands.  Two sets of regions
// alternate between launches: a launch clears, as it goes, its own entries of
// the set the previous launch used, which the next launch then finds zeroed.
// Weights that the down phase needs (the chosen experts' down rows, into
// registers, and the next layer's router rows, into LDS) are requested as the
// phase begins and arrive while it waits for the act values, so the gate/up
// phase streams only the gate and up rows.  Every wait is bounded: a
// value that never arrives (a workgroup that never became resident) sets the
// error word and the kernel runs out instead of hanging.  The int4 dot
// products are those of the decode GEMV kernels (exact integer v_dot8_i32_i4
// of the nibbles against 16-bit fixed point activations per group).
#include "common.h"
#include "kernels.h"
#include "q4_lane.h"

// Stage timeline (a build option for measurement, off in the library): with
// MOE_DECODE_TIMELINE defined, thread 0 of every workgroup records the global
// 100 MHz clock (s_memrealtime) at the end of each stage of each layer of
// the last launch; moe_debug_decode_timeline() copies the table to the host.
#ifdef MOE_DECODE_TIMELINE
namespace moe {
constexpr int kTlLayers = 64, kTlGroups = 256, kTlStages = 12;
__device__ uint64_t g_decode_timeline[kTlLayers][kTlGroups][kTlStages];
}  // namespace moe
#define DECODE_TL(layer, stage)                                                                       \
  do {                                                                                                \
    if (threadIdx.x == 0 && (layer) < moe::kTlLayers)                                                 \
      moe::g_decode_timeline[(layer)][blockIdx.x][(stage)] = __builtin_amdgcn_s_memrealtime();        \
  } while (0)
#else
#define DECODE_TL(layer, stage) \
  do {                          \
  } while (0)
#endif

namespace moe {

namespace {

using namespace lane;

constexpr int kFWaves = 8;
constexpr int kFThreads = kFWaves * kWave;
// gate/up phase: the workgroup's 32 act columns x 16 K-parts; wave w holds
// columns 16 (w % 2) .. +15 and K-parts 4 (w / 2) .. +3, lane = 4 parts x 16
// columns, and each lane computes the gate row and the up row of its column
// (one read of the activations for both).  (Spreading a layer over all 256
// compute units, 22 columns each, measured slower in every stage: more
// requests in flight, weight lines split between workgroups and more
// pollers of each exchange.)
constexpr int kGP = 16, kGPW = 4, kGR = kWave / kGPW, kGGPP = 3, kGGMAX = kGP * kGGPP;  // d/64 <= 48
constexpr int kActCols = 2 * kGR;                                                        // 32 act columns
// down phase: one wave per selected expert; lanes 4 K-parts x 16 rows
constexpr int kDP = 4, kDR = kWave / kDP, kDGPP = 3, kDGMAX = kDP * kDGPP;  // f/64 <= 12
constexpr int kMaxE = 256;
constexpr int kPartBatch = 12;         // float4 loads in flight per thread when summing router partials
constexpr uint32_t kSpinLimit = 300000u;  // polling rounds (~1 us each) per wait at most
// Router partials are reduced in two steps: workgroup q < E/4 (a reducer)
// sums column quad q (experts 4q..4q+3) over every workgroup's row of
// partials and publishes the 4 sums; then every workgroup reads the E sums.
// A coherent load brings ~23 GB/s into one compute unit, so what bounds the
// exchange is the bytes each workgroup reads: 16 bytes per row for a reducer
// and 4 bytes per expert for everyone, where every workgroup reading every
// row of partials (~90 KB) took ~5 us.

struct FusedArgs {
  float* x_io;  // [L+1][d]
  int L;
  const float* norm_w;       // [L][d] or null
  float eps;
  const float* router_w;     // [L][E][d]
  const float* router_bias;  // [L][E] or null
  const int32_t* slot_tables;  // [L][E]
  int n_slots;
  const uint8_t* arena;
  int64_t layer_stride, slot_stride;
  int d, f, E, k;
  int64_t off_gq, off_uq, off_dq, off_gsb, off_usb, off_dsb;
  int32_t* topk_idx;  // [L][k]
  float* topk_w;      // [L][k]
  float* x_next;      // [d] or null
  uint64_t* launches; // launches run on this workspace (its parity picks the region set)
  uint64_t* sig;      // shape signature of the launches that use this workspace (0: none yet)
  uint64_t my_sig;
  uint32_t* err;      // 1: a wait timed out; 2: the workspace was used with other shapes
  // Two sets of per-layer regions (set 1 at set_floats after set 0), each
  // region on its own 256-byte boundary; encoded values, 0 = not written yet.
  uint32_t* regions;
  int64_t set_floats;
  int64_t act_off, part_off, ss_off, xs_off, qs_off;  // region offsets inside a set (words)
  int act_ls, part_ls, ss_ls, xs_ls, qs_ls;  // words per layer: [k][f] act, [G][epad] router
                                             // partials, [G] sums of squares, [d] layer input,
                                             // [E] router sums (summed partials)
  int epad;      // E rounded up to 32: each workgroup's partials fill whole 128-byte lines
  int G, rpw;    // workgroups, down rows per workgroup (a multiple of 4, at most 16)
  int nck_g, nck_d;
};

constexpr int kRsrcWord3F = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kRsrcWord3F);
}
// Plain loads (the caller's input token, which no workgroup writes).
__device__ __forceinline__ float ldn(__amdgpu_buffer_rsrc_t r, int idx) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, idx * 4, 0, 0));
}
__device__ __forceinline__ float4 ldn4(__amdgpu_buffer_rsrc_t r, int idx) {  // idx % 4 == 0
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, idx * 4, 0, 0));
}
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Values handed between workgroups travel as the complement of their bits,
// NaNs made canonical first: no value encodes to zero, and a zero word (the
// zero-filled workspace, or an entry cleared by the previous launch) is one
// that has not been written yet.
__device__ __forceinline__ uint32_t enc(float v) {
  return ~(v != v ? 0x7FC00000u : __builtin_bit_cast(uint32_t, v));
}
__device__ __forceinline__ float dec(uint32_t u) { return __builtin_bit_cast(float, ~u); }
__device__ __forceinline__ float4 dec4(u32x4_t u) { return make_float4(dec(u.x), dec(u.y), dec(u.z), dec(u.w)); }
__device__ __forceinline__ bool ready4(u32x4_t u) { return u.x != 0u && u.y != 0u && u.z != 0u && u.w != 0u; }

// Stores written through to memory (sc1) and coherent (sc1) loads, which see
// what other XCDs wrote in this launch.
constexpr int kSc1 = 16;
__device__ __forceinline__ void st_e(__amdgpu_buffer_rsrc_t r, int idx, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(enc(v), r, idx * 4, 0, kSc1);
}
__device__ __forceinline__ void st_e4(__amdgpu_buffer_rsrc_t r, int idx, float4 v) {  // idx % 4 == 0
  const u32x4_t u = {enc(v.x), enc(v.y), enc(v.z), enc(v.w)};
  __builtin_amdgcn_raw_buffer_store_b128(u, r, idx * 4, 0, kSc1);
}
__device__ __forceinline__ void st_zero4(__amdgpu_buffer_rsrc_t r, int idx) {  // idx % 4 == 0
  const u32x4_t z = {0u, 0u, 0u, 0u};
  __builtin_amdgcn_raw_buffer_store_b128(z, r, idx * 4, 0, kSc1);
}
__device__ __forceinline__ uint32_t ldc(__amdgpu_buffer_rsrc_t r, int idx) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, idx * 4, 0, kSc1);
}
__device__ __forceinline__ u32x4_t ldc4(__amdgpu_buffer_rsrc_t r, int idx) {  // idx % 4 == 0
  return __builtin_amdgcn_raw_buffer_load_b128(r, idx * 4, 0, kSc1);
}

// Re-load an encoded word (or four) until it has been written.  A wait that
// outlasts kSpinLimit rounds, or any wait after one in this workgroup did,
// gives up: the error word is set and the value decodes to NaN.
__device__ __forceinline__ bool give_up(const FusedArgs& a, uint32_t& spins, volatile int* s_fail) {
  if (*s_fail) return true;
  if (++spins > kSpinLimit) {
    __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_fail = 1;
    return true;
  }
  __builtin_amdgcn_s_sleep(1);
  asm volatile("" ::: "memory");  // the next load is a new load
  return false;
}
// Waits for N words (or N groups of four) at once: every round re-issues the
// loads of all entries not written yet, so a wait costs one round trip after
// the last write lands, however many entries it covers.
template <int N>
__device__ __forceinline__ void wait_all(const FusedArgs& a, __amdgpu_buffer_rsrc_t r, const int (&idx)[N],
                                         uint32_t (&v)[N], volatile int* s_fail) {
  uint32_t spins = 0;
  for (;;) {
    bool pend = false;
#pragma unroll
    for (int c = 0; c < N; ++c) pend |= v[c] == 0u;
    if (!pend || give_up(a, spins, s_fail)) return;
#pragma unroll
    for (int c = 0; c < N; ++c)
      if (v[c] == 0u) v[c] = ldc(r, idx[c]);
  }
}
template <int N>
__device__ __forceinline__ void wait_all4(const FusedArgs& a, __amdgpu_buffer_rsrc_t r, const int (&idx)[N],
                                          u32x4_t (&v)[N], volatile int* s_fail) {
  uint32_t spins = 0;
  for (;;) {
    bool pend = false;
#pragma unroll
    for (int c = 0; c < N; ++c) pend |= !ready4(v[c]);
    if (!pend || give_up(a, spins, s_fail)) return;
#pragma unroll
    for (int c = 0; c < N; ++c)
      if (!ready4(v[c])) v[c] = ldc4(r, idx[c]);
  }
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
__device__ __forceinline__ lds_ptr_t to_lds(void* p) { return (lds_ptr_t)(p); }

// Threads that share one expert in the sums over experts (E <= 256).
__device__ __forceinline__ int threads_per_expert(int E) { return E <= 64 ? 8 : (E <= 128 ? 4 : 2); }

// The region words of one set that this workgroup writes for `layer` are
// cleared for the launch after next (the one that uses that set again):
// its act columns, its row of router partials and its sum of squares, and
// its rows of the layer input (layer >= 1).  `clear_last` adds the sum of
// squares of the last output.
__device__ __forceinline__ void clear_own(const FusedArgs& a, int t, __amdgpu_buffer_rsrc_t r, int layer,
                                          int act0, int r0, int nr, bool clear_last) {
  const int g = blockIdx.x;
  const int na = 32 / 4, np = a.epad / 4, nx = (nr + 3) / 4;
  if (t < na) st_zero4(r, (int)a.act_off + layer * a.act_ls + act0 + 4 * t);
  else if (t < na + np) st_zero4(r, (int)a.part_off + layer * a.part_ls + g * a.epad + 4 * (t - na));
  else if (t < na + np + nx) {
    if (layer >= 1) st_zero4(r, (int)a.xs_off + layer * a.xs_ls + r0 + 4 * (t - na - np));
  } else if (t == na + np + nx) {
    __builtin_amdgcn_raw_buffer_store_b32(0u, r, ((int)a.ss_off + layer * a.ss_ls + g) * 4, 0, kSc1);
    if (clear_last)
      __builtin_amdgcn_raw_buffer_store_b32(0u, r, ((int)a.ss_off + (layer + 1) * a.ss_ls + g) * 4, 0, kSc1);
  } else if (t == na + np + nx + 1 && g < (a.E + 3) / 4) {
    st_zero4(r, (int)a.qs_off + layer * a.qs_ls + 4 * g);  // this reducer's 4 router sums
  }
}

// Copies into LDS (no registers held while in flight): router rows
// [r0, r0 + 16) of every expert of `layer` into rw[e*4 + 0..3] (float4
// units) and the norm weight over the same rows into rnw[0..3].  Rows past d
// read a clamped address; the values that use them are masked.
__device__ __forceinline__ void router_rows_to_lds(const FusedArgs& a, int t, int layer, int r0, float4* rw,
                                                   float4* rnw) {
  const int wave = __builtin_amdgcn_readfirstlane(t / kWave), lane = t % kWave;
  const __amdgpu_buffer_rsrc_t r = rsrc_of(a.router_w + (int64_t)layer * a.E * a.d, (int64_t)a.E * a.d * 4);
  const int row = min(r0 + 4 * (lane % 4), a.d - 4);
  for (int n = wave; n * 16 < a.E; n += kFWaves) {
    const int e = min(n * 16 + lane / 4, a.E - 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, to_lds(&rw[n * kWave]), 16, (e * a.d + row) * 4, 0, 0, 0);
  }
  if (a.norm_w && wave == kFWaves - 1) {
    const __amdgpu_buffer_rsrc_t rn = rsrc_of(a.norm_w + (int64_t)layer * a.d, (int64_t)a.d * 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rn, to_lds(rnw), 16, min(r0 + 4 * min(lane, 3), a.d - 4) * 4, 0, 0, 0);
  }
}

// Router partials of `layer` over this workgroup's rows, from the router rows
// in LDS and z = w * y (w the norm weight, 1 without one; z = 0 past the
// rows): part[g][e] = sum_i Wr[e][r0 + i] * z[i], plus sumsq[g] = sum_i y[i]^2.
// The row of E values goes out as whole 128-byte lines (s_pe holds zeros past
// E).  Fixed summation order, the same in every launch.
__device__ __forceinline__ void write_partials(const FusedArgs& a, int t, int layer, const float4* rw, const float* z,
                                               const float* y, float* s_pe, __amdgpu_buffer_rsrc_t rc) {
  const int g = blockIdx.x;
  if (layer < a.L) {
    const int tq = threads_per_expert(a.E), rpt = kDR / tq;
    const int e = t / tq, q = t % tq;
    float s = 0.0f;
    if (e < a.E) {
      const float* w = reinterpret_cast<const float*>(rw) + e * kDR + q * rpt;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < rpt) s = fmaf(w[i], z[q * rpt + i], s);
    }
    s = group_sum_dpp(s, tq);
    if (e < a.E && q == 0) s_pe[e] = s;
  }
  if (t < kWave) {
    const float v = t < kDR ? y[t] : 0.0f;
    const float ss = wave_sum_dpp(v * v);
    if (t == 0) st_e(rc, (int)a.ss_off + layer * a.ss_ls + g, ss);
  }
  __syncthreads();
  if (layer < a.L && t < a.epad / 4)
    st_e4(rc, (int)a.part_off + layer * a.part_ls + g * a.epad + 4 * t, reinterpret_cast<const float4*>(s_pe)[t]);
}

__global__ __launch_bounds__(kFThreads) void k_decode_fused(FusedArgs a) {
  __shared__ XRow<kGP, kGGMAX> xh;             // h of the current layer (gate/up phase)
  __shared__ XRow<kDP, kDGMAX> xa[kFWaves];    // act rows of the selected experts (down phase)
  __shared__ float4 s_rw[kMaxE * kDR / 4];     // next layer's router rows over this workgroup's rows
  __shared__ float4 s_rnw[kWave];              // next layer's norm weight over the rows (first 4 used)
  __shared__ float4 s_logit4[kMaxE / 4 + 1];   // logits
  __shared__ uint4 s_key4[kMaxE / 2 + 2];      // rank keys (logit, then lower id), zeros past E
  __shared__ float4 s_pe4[kMaxE / 4];          // this workgroup's router partials (zeros past E)
  __shared__ float4 s_red4[kFThreads];         // router partial sums per (slice, quad of experts)
  __shared__ int s_table[kMaxE];               // this layer's slot per expert
  __shared__ float s_val[16];
  __shared__ int s_idx[16];
  __shared__ float s_w[16];
  __shared__ float2 s_gu[kGP / kGPW][kActCols];  // (gate, up) partial sums per part block and column
  __shared__ float s_o[kFWaves][kDR];          // down outputs per expert rank
  __shared__ float s_y[kDR], s_z[kDR];         // this workgroup's rows of the layer input / output, norm weight * rows
  __shared__ uint64_t s_launch;
  __shared__ float s_inv;                      // 1/rms of the current layer input
  __shared__ int s_stop;                       // the workspace belongs to other shapes
  __shared__ int s_fail;                       // a wait of this workgroup gave up
  const int t0 = threadIdx.x;
  const int g = blockIdx.x;
  const int t = t0, lane = t0 % kWave;
  if (t == 0) {
    const uint64_t sig = __hip_atomic_load(a.sig, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_launch = __hip_atomic_load(a.launches, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_stop = (sig != 0u && sig != a.my_sig) ? 1 : 0;
    s_fail = 0;
    if (s_stop) __hip_atomic_store(a.err, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  float* s_logit = reinterpret_cast<float*>(s_logit4);
  float* s_pe = reinterpret_cast<float*>(s_pe4);
  uint64_t* s_key = reinterpret_cast<uint64_t*>(s_key4);
  if (t < 4) s_key[a.E + t] = 0;
  if (t >= a.E && t < a.epad) s_pe[t] = 0.0f;
  __syncthreads();
  if (s_stop) return;  // regions laid out for other shapes: nothing is read or written
  const uint64_t launch = s_launch;
  const int set = (int)(launch & 1u);
  const int Gd = a.d / kGroup, Gf = a.f / kGroup;
  const int r0 = g * a.rpw, nr = max(0, min(a.rpw, a.d - r0));
  const int jr0 = g / (a.f / kActCols), c00 = (g % (a.f / kActCols)) * kActCols;  // gate/up expert rank, act columns
  const __amdgpu_buffer_rsrc_t rX = rsrc_of(a.x_io, (int64_t)(a.L + 1) * a.d * 4);
  // this launch's region set, and the one the previous launch used (cleared for the next)
  const __amdgpu_buffer_rsrc_t rc = rsrc_of(a.regions + set * a.set_floats, a.set_floats * 4);
  const __amdgpu_buffer_rsrc_t ro = rsrc_of(a.regions + (1 - set) * a.set_floats, a.set_floats * 4);
  const int tq = threads_per_expert(a.E);

  // ---- prologue: router partials of layer 0 over this workgroup's rows of x_io[0]
  if (t < kDR) s_y[t] = t < nr ? ldn(rX, r0 + t) : 0.0f;
  router_rows_to_lds(a, t, 0, r0, s_rw, s_rnw);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (t < kDR) s_z[t] = t < nr ? s_y[t] * (a.norm_w ? reinterpret_cast<const float*>(s_rnw)[t] : 1.0f) : 0.0f;
  __syncthreads();
  write_partials(a, t, 0, s_rw, s_z, s_y, s_pe, rc);

  for (int l = 0; l < a.L; ++l) {
    DECODE_TL(l, 0);  // layer start
    // Thread-derived indices are recomputed from an opaque copy of the thread
    // id every layer: hoisted out of the loop they would hold hundreds of
    // registers for the whole launch.
    int tid = t0;
    asm volatile("" : "+v"(tid));
    const int t = tid, lane = t % kWave, wave = __builtin_amdgcn_readfirstlane(t / kWave);
    // ================= gate/up phase =================
    // Everything that does not depend on the routing goes out at once: the
    // slot table, the router bias, the sums of squares, x and the norm
    // weight, then the router partials.
    // the slot table goes to LDS only after the waits below: storing it now
    // would wait for this load, and with it for every store still in flight
    const int stbl = t < a.E ? a.slot_tables[(int64_t)l * a.E + t] : -1;
    const float bias = (a.router_bias && t < a.E) ? a.router_bias[(int64_t)l * a.E + t] : 0.0f;
    const int nq = (a.E + 3) / 4;
    // the sums of squares (G <= 256 words): wave 1 alone polls them and
    // shares 1/rms through LDS (every wave polling them multiplied the
    // coherent requests of the wait eightfold)
    uint32_t ssu[4] = {1u, 1u, 1u, 1u};
    int ssi[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      ssi[c] = (int)a.ss_off + l * a.ss_ls + min(lane + c * kWave, a.G - 1);
      if (wave == 1) ssu[c] = ldc(rc, ssi[c]);
    }
    constexpr int NPASSG = (8 * kGGMAX + kFThreads - 1) / kFThreads;
    StageRegs<NPASSG> xr, nwr;
    const float* nw = a.norm_w ? a.norm_w + (int64_t)l * a.d : nullptr;
    const int xs0 = (int)a.xs_off + l * a.xs_ls;
    u32x4_t xu[2 * NPASSG];
    int xi[2 * NPASSG];
#pragma unroll
    for (int ps = 0; ps < NPASSG; ++ps) {
      const int wi = min(ps * kFThreads + t, 8 * Gd - 1);
      xi[2 * ps] = xs0 + wi * 8;
      xi[2 * ps + 1] = xs0 + wi * 8 + 4;
      if (l == 0) {
        xr.a[ps] = ldn4(rX, wi * 8);
        xr.b[ps] = ldn4(rX, wi * 8 + 4);
      } else {
        xu[2 * ps] = ldc4(rc, xi[2 * ps]);
        xu[2 * ps + 1] = ldc4(rc, xi[2 * ps + 1]);
      }
      nwr.a[ps] = nw ? *reinterpret_cast<const float4*>(nw + wi * 8) : make_float4(1.f, 1.f, 1.f, 1.f);
      nwr.b[ps] = nw ? *reinterpret_cast<const float4*>(nw + wi * 8 + 4) : make_float4(1.f, 1.f, 1.f, 1.f);
    }
    if (g < nq) {
      // reducer of quad g: row t of the partials (16 bytes), summed in row
      // order by wave 0 (a fixed order, the same in every launch)
      u32x4_t pv[1] = {{1u, 1u, 1u, 1u}};
      int pix[1] = {(int)a.part_off + l * a.part_ls + min(t, a.G - 1) * a.epad + 4 * g};
      if (t < a.G) {
        pv[0] = ldc4(rc, pix[0]);
        wait_all4<1>(a, rc, pix, pv, &s_fail);
        s_red4[t] = dec4(pv[0]);
      }
      __syncthreads();
      DECODE_TL(l, 8);  // reducer: its column of every row of partials has arrived
      if (wave == 0) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int r = lane; r < a.G; r += kWave) {
          const float4 u = s_red4[r];
          acc.x += u.x;
          acc.y += u.y;
          acc.z += u.z;
          acc.w += u.w;
        }
        acc.x = wave_sum_dpp(acc.x);
        acc.y = wave_sum_dpp(acc.y);
        acc.z = wave_sum_dpp(acc.z);
        acc.w = wave_sum_dpp(acc.w);
        if (lane == 0) st_e4(rc, (int)a.qs_off + l * a.qs_ls + 4 * g, acc);
        DECODE_TL(l, 9);  // reducer: its 4 sums written
      }
    }
    // every workgroup: the E router sums, 4 per thread
    u32x4_t qv[1] = {{1u, 1u, 1u, 1u}};
    int qix[1] = {(int)a.qs_off + l * a.qs_ls + 4 * min(t, nq - 1)};
    if (t < nq) qv[0] = ldc4(rc, qix[0]);
    if (wave == 1) {
      wait_all<4>(a, rc, ssi, ssu, &s_fail);
      float ss = 0.0f;
#pragma unroll
      for (int c = 0; c < 4; ++c) ss += lane + c * kWave < a.G ? dec(ssu[c]) : 0.0f;
      ss = wave_sum_dpp(ss);
      if (lane == 0) s_inv = a.norm_w ? 1.0f / sqrtf(ss / (float)a.d + a.eps) : 1.0f;
    }
    if (l > 0) {
      wait_all4<2 * NPASSG>(a, rc, xi, xu, &s_fail);
#pragma unroll
      for (int ps = 0; ps < NPASSG; ++ps) {
        xr.a[ps] = dec4(xu[2 * ps]);
        xr.b[ps] = dec4(xu[2 * ps + 1]);
      }
    }
    if (t < nq) {
      wait_all4<1>(a, rc, qix, qv, &s_fail);
      s_pe4[t] = dec4(qv[0]);  // the E sums (s_pe is free until the partials are written)
    }
    DECODE_TL(l, 10);  // thread 0: the router sums of its quad have arrived
    if (t < a.E) s_table[t] = stbl;
    __syncthreads();
    DECODE_TL(l, 1);  // router sums, sums of squares and x have arrived
    const float inv = s_inv;
    if (t < a.E) {
      const float lg = s_pe[t] * inv + bias + 0.0f;  // + 0: -0 becomes +0
      s_logit[t] = lg;
      // one unsigned key orders (larger logit, then lower id): the float's
      // bits made monotone, then the complement of the id
      const uint32_t u = __builtin_bit_cast(uint32_t, lg);
      const uint32_t mono = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
      s_key[t] = ((uint64_t)mono << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)t);
    }
    __syncthreads();
    {
      // rank of expert e = experts with a larger logit, or an equal one and a
      // lower id = experts with a larger key (tq threads per expert, each
      // over a quarter/half/eighth of the keys, two per LDS read)
      const int e = t / tq, q = t % tq;
      int beats = 0;
      float v = 0.0f;
      if (e < a.E) {
        v = s_logit[e];
        const uint64_t kv = s_key[e];
        const int span = ((a.E + tq - 1) / tq + 3) / 4 * 4, j0 = q * span, j1 = min(a.E, j0 + span);
#pragma unroll 8
        for (int jj = j0; jj < j1; jj += 2) {
          const uint4 u = s_key4[jj / 2];
          beats += (((uint64_t)u.y << 32 | u.x) > kv) ? 1 : 0;
          beats += (((uint64_t)u.w << 32 | u.z) > kv) ? 1 : 0;
        }
      }
      beats = group_sum_dpp(beats, tq);
      if (e < a.E && q == 0 && beats < a.k) {
        s_idx[beats] = e;
        s_val[beats] = v;
      }
    }
    __syncthreads();
    DECODE_TL(l, 2);  // top-k known
    // this workgroup's expert (rank jr) and act columns [c0, c0 + 32)
    const int jr = g / (a.f / kActCols);
    const int c0 = (g % (a.f / kActCols)) * kActCols;
    const uint8_t* larena = a.arena + (int64_t)l * a.layer_stride;
    const int layer_expert = s_idx[jr];
    const int slot = (layer_expert >= 0 && layer_expert < a.E) ? s_table[layer_expert] : -1;
    const bool ok = slot >= 0 && slot < a.n_slots;
    const uint8_t* blob = larena + (ok ? (int64_t)slot * a.slot_stride : 0);
    const int cb = wave % 2, pb = wave / 2;
    const int j = pb * kGPW + lane / kGR, r = lane % kGR;
    const Part pt = part_of<kGP>(j, Gd);
    const int row = c0 + cb * kGR + r;
    LaneSlice<kGGPP> wg, wu;
    {
      const int64_t tile = row / kTileRows;
      const int trow = row % kTileRows;
      const int64_t qo = tile * (kTileRows * a.d / 2) + trow * 16, so = tile * (kTileRows * Gd * 4) + trow * 4;
      load_lane<kGGPP>(wg, blob + a.off_gq + qo, blob + a.off_gsb + so, pt, Gd);
      load_lane<kGGPP>(wu, blob + a.off_uq + qo, blob + a.off_usb + so, pt, Gd);
    }
    {
      // h = x * inv * w in 8-column words: thread t stages word t
      StageRegs<NPASSG> sr;
#pragma unroll
      for (int ps = 0; ps < NPASSG; ++ps) {
        const float4 xa4 = xr.a[ps], xb4 = xr.b[ps], na = nwr.a[ps], nb = nwr.b[ps];
        sr.a[ps] = make_float4(xa4.x * inv * na.x, xa4.y * inv * na.y, xa4.z * inv * na.z, xa4.w * inv * na.w);
        sr.b[ps] = make_float4(xb4.x * inv * nb.x, xb4.y * inv * nb.y, xb4.z * inv * nb.z, xb4.w * inv * nb.w);
      }
      stage_store<kGP, kGGMAX, NPASSG>(xh, sr, Gd, t, kFThreads);
    }
    __syncthreads();
    DECODE_TL(l, 3);  // h staged in LDS, gate/up weight loads issued
    {
      const float2 v = lane_dot2<kGP, kGPW, kGGPP, kGGMAX>(wg, wu, xh, j, pt, Gd, a.nck_g);
      if (lane < kGR) s_gu[pb][cb * kGR + r] = v;
      __syncthreads();
      DECODE_TL(l, 4);  // gate/up dot products done
      if (t < kActCols) {
        // the part blocks in a fixed order
        float gs = 0.0f, us = 0.0f;
#pragma unroll
        for (int q = 0; q < kGP / kGPW; ++q) {
          gs += s_gu[q][t].x;
          us += s_gu[q][t].y;
        }
        const float v2 = ok ? gelu_tanh(gs) * us : f32_nan();
        st_e(rc, (int)a.act_off + l * a.act_ls + jr * a.f + c0 + t, v2);
      }
    }
    if (wave == kFWaves - 1) {
      // weights: softmax over the chosen logits (largest first), off the
      // gate/up critical path (the down phase reads them)
      const float m = s_val[0];
      const float ex = lane < a.k ? expf(s_val[lane < a.k ? lane : 0] - m) : 0.0f;
      const float sum = wave_sum(ex);
      if (lane < a.k) {
        s_w[lane] = ex / sum;
        if (g == 0) {
          a.topk_idx[(int64_t)l * a.k + lane] = s_idx[lane];
          a.topk_w[(int64_t)l * a.k + lane] = ex / sum;
        }
      }
    } else if (wave == kFWaves - 2) {
      // this workgroup's entries of the other set for this layer are cleared
      // for the launch after next
      clear_own(a, lane + kWave, ro, l, jr0 * a.f + c00, r0, nr, l + 1 == a.L);
    } else if (wave == kFWaves - 3) {
      clear_own(a, lane, ro, l, jr0 * a.f + c00, r0, nr, l + 1 == a.L);
    } else if (wave == kFWaves - 4) {
      clear_own(a, lane + 2 * kWave, ro, l, jr0 * a.f + c00, r0, nr, l + 1 == a.L);
    }

    // ================= down phase =================
    {
      const int jw = wave;  // expert rank of this wave
      const bool wave_on = jw < a.k && nr > 0;
      const int jd = lane / kDR, rd = lane % kDR;
      const Part pd = part_of<kDP>(jd, Gf);
      const int ed = wave_on ? s_idx[jw] : -1;
      const int sd = (ed >= 0 && ed < a.E) ? s_table[ed] : -1;
      const bool ok2 = sd >= 0 && sd < a.n_slots;
      // The expert's down rows go straight to registers and the next layer's
      // router rows to LDS: both arrive while the act values are awaited,
      // which leaves the gate/up phase only its own weights to stream.
      LaneSlice<kDGPP> wd;
      if (wave_on) {
        const uint8_t* blob2 = larena + (ok2 ? (int64_t)sd * a.slot_stride : 0);
        const int rowd = r0 + min(rd, nr - 1);
        const int64_t tile = rowd / kTileRows;
        const int trow = rowd % kTileRows;
        const int64_t qo = tile * (kTileRows * a.f / 2) + trow * 16, so = tile * (kTileRows * Gf * 4) + trow * 4;
        load_lane<kDGPP>(wd, blob2 + a.off_dq + qo, blob2 + a.off_dsb + so, pd, Gf);
      }
      if (l + 1 < a.L) router_rows_to_lds(a, t, l + 1, r0, s_rw, s_rnw);
      constexpr int NPASS = (8 * kDGMAX + kWave - 1) / kWave;
      StageRegs<NPASS> sr;
      if (wave_on) {
        const int ab = (int)a.act_off + l * a.act_ls + jw * a.f;
        u32x4_t au[2 * NPASS];
        int ai[2 * NPASS];
#pragma unroll
        for (int ps = 0; ps < NPASS; ++ps) {
          const int wi = min(ps * kWave + lane, 8 * Gf - 1);
          ai[2 * ps] = ab + wi * 8;
          ai[2 * ps + 1] = ab + wi * 8 + 4;
          au[2 * ps] = ldc4(rc, ai[2 * ps]);
          au[2 * ps + 1] = ldc4(rc, ai[2 * ps + 1]);
        }
        wait_all4<2 * NPASS>(a, rc, ai, au, &s_fail);
#pragma unroll
        for (int ps = 0; ps < NPASS; ++ps) {
          sr.a[ps] = dec4(au[2 * ps]);
          sr.b[ps] = dec4(au[2 * ps + 1]);
        }
      }
      // the residual: this workgroup's rows of the layer input
      const float xres = (t < nr) ? s_y[t] : 0.0f;
      if (wave_on) stage_store<kDP, kDGMAX, NPASS>(xa[jw], sr, Gf, lane, kWave);
      __builtin_amdgcn_s_waitcnt(0);  // this wave's router-row copies have landed in LDS
      __syncthreads();
      DECODE_TL(l, 5);  // act values arrived, down rows and next router rows landed
      if (wave_on) {
        float v = lane_dot<kDP, kDGPP, kDGMAX>(wd, xa[jw], jd, pd, Gf, a.nck_d);
        if (!ok2) v = f32_nan();
        if (jd == 0) s_o[jw][rd] = v;
      }
      __syncthreads();
      DECODE_TL(l, 6);  // down dot products done
      if (t < kDR) {
        float y = 0.0f, z = 0.0f;
        if (t < nr) {
          y = xres;
          for (int jj = 0; jj < a.k; ++jj) y = fmaf(s_w[jj], s_o[jj][t], y);
          a.x_io[(int64_t)(l + 1) * a.d + r0 + t] = y;
          z = y * ((a.norm_w && l + 1 < a.L) ? reinterpret_cast<const float*>(s_rnw)[t] : 1.0f);
        }
        s_y[t] = y;
        s_z[t] = z;
      }
      __syncthreads();
      // the next layer's input rows for the other workgroups, then its router partials
      if (l + 1 < a.L && t < nr / 4)
        st_e4(rc, (int)a.xs_off + (l + 1) * a.xs_ls + r0 + 4 * t, reinterpret_cast<const float4*>(s_y)[t]);
      write_partials(a, t, l + 1, s_rw, s_z, s_y, s_pe, rc);
      DECODE_TL(l, 7);  // combine done, next layer input and router partials written
    }
  }

  // unit-RMS rescale of the last output for the next decode step
  if (a.x_next) {
    uint32_t su[4];
    int si[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      si[c] = (int)a.ss_off + a.L * a.ss_ls + min(lane + c * kWave, a.G - 1);
      su[c] = ldc(rc, si[c]);
    }
    wait_all<4>(a, rc, si, su, &s_fail);
    float ss = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) ss += lane + c * kWave < a.G ? dec(su[c]) : 0.0f;
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)a.d + a.eps);
    if (t < nr) a.x_next[r0 + t] = s_y[t] * inv;
  }
  // the next launch on this workspace uses the other set (every workgroup
  // read the count before it wrote anything that workgroup 0 waited for)
  if (g == 0 && t == 0) {
    __hip_atomic_store(a.sig, a.my_sig, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.launches, launch + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace

// ------------------------------------------------------------------ host side

bool decode_fused_supported(int d, int f, int E, int k, int cus, int* G_out, int* rpw_out) {
  if (d % kGroup || f % kGroup || d / kGroup > kGGMAX || f / kGroup > kDGMAX || E > kMaxE || k > kFWaves)
    return false;
  const int G = k * (f / kActCols);
  const int rpw = ((d + G - 1) / G + 3) / 4 * 4;  // router rows go to LDS in 16-byte pieces
  if (G > cus || G > 256 || rpw > kDR) return false;
  *G_out = G;
  *rpw_out = rpw;
  return true;
}

namespace {
// Workspace: a 512-byte header (launch count at 0, shape signature at 8, error
// word at kDecodeErrOffset), then two region sets of set_floats words each.
struct FusedLayout {
  int act_ls, part_ls, ss_ls, xs_ls, qs_ls;  // words per layer region, multiples of 64 (256 bytes)
  int epad;
  int64_t act_off, part_off, ss_off, xs_off, qs_off, set_floats;  // words inside a set
  int64_t regions_off, bytes;
};
FusedLayout fused_layout(int L, int d, int f, int E, int k) {
  const int G = k * (f / kActCols);
  auto r64 = [](int64_t n) { return (int)((n + 63) / 64 * 64); };
  FusedLayout o;
  o.act_ls = r64((int64_t)k * f);
  o.epad = (E + 31) / 32 * 32;
  o.part_ls = r64((int64_t)G * o.epad);
  o.ss_ls = r64(G);
  o.xs_ls = r64(d);
  o.qs_ls = r64(E + 3);
  o.act_off = 0;
  o.part_off = o.act_off + (int64_t)L * o.act_ls;
  o.ss_off = o.part_off + (int64_t)L * o.part_ls;
  o.xs_off = o.ss_off + (int64_t)(L + 1) * o.ss_ls;
  o.qs_off = o.xs_off + (int64_t)L * o.xs_ls;
  o.set_floats = o.qs_off + (int64_t)L * o.qs_ls;
  o.regions_off = 512;
  o.bytes = o.regions_off + 2 * o.set_floats * 4;
  return o;
}
}  // namespace

size_t decode_fused_workspace_bytes(int L, int d, int f, int E, int k) {
  return (size_t)fused_layout(L, d, f, E, k).bytes;
}

hipError_t launch_decode_fused(float* x_io, int L, const float* norm_w, float eps, const float* router_w,
                               const float* router_bias, const int32_t* slot_tables, int n_slots,
                               const uint8_t* arena, int64_t layer_stride, int64_t slot_stride, int d, int f, int E,
                               int k, int64_t off_gq, int64_t off_uq, int64_t off_dq, int64_t off_gsb, int64_t off_usb,
                               int64_t off_dsb, int32_t* topk_idx, float* topk_w, float* x_next, void* ws, int G,
                               int rpw, hipStream_t s) {
  FusedArgs a{};
  a.x_io = x_io;
  a.L = L;
  a.norm_w = norm_w;
  a.eps = eps;
  a.router_w = router_w;
  a.router_bias = router_bias;
  a.slot_tables = slot_tables;
  a.n_slots = n_slots;
  a.arena = arena;
  a.layer_stride = layer_stride;
  a.slot_stride = slot_stride;
  a.d = d; a.f = f; a.E = E; a.k = k;
  a.off_gq = off_gq; a.off_uq = off_uq; a.off_dq = off_dq;
  a.off_gsb = off_gsb; a.off_usb = off_usb; a.off_dsb = off_dsb;
  a.topk_idx = topk_idx;
  a.topk_w = topk_w;
  a.x_next = x_next;
  char* c = reinterpret_cast<char*>(ws);
  a.launches = reinterpret_cast<uint64_t*>(c);
  a.sig = reinterpret_cast<uint64_t*>(c + 8);
  a.err = reinterpret_cast<uint32_t*>(c + kDecodeErrOffset);
  const FusedLayout lay = fused_layout(L, d, f, E, k);
  a.regions = reinterpret_cast<uint32_t*>(c + lay.regions_off);
  a.set_floats = lay.set_floats;
  a.act_off = lay.act_off;
  a.part_off = lay.part_off;
  a.ss_off = lay.ss_off;
  a.xs_off = lay.xs_off;
  a.qs_off = lay.qs_off;
  a.qs_ls = lay.qs_ls;
  a.act_ls = lay.act_ls;
  a.part_ls = lay.part_ls;
  a.ss_ls = lay.ss_ls;
  a.xs_ls = lay.xs_ls;
  a.epad = lay.epad;
  // the shapes that fix the region layout, never 0
  uint64_t sig = 1469598103934665603ull;
  for (int64_t v : {(int64_t)L, (int64_t)d, (int64_t)f, (int64_t)E, (int64_t)k, (int64_t)G, (int64_t)rpw}) {
    sig ^= (uint64_t)v;
    sig *= 1099511628211ull;
  }
  a.my_sig = sig | 1u;
  a.G = G;
  a.rpw = rpw;
  a.nck_g = 2 * kGGPP;
  a.nck_d = 2 * kDGPP;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  take_profile_events(MOE_CALL_DECODE_LAYERS, &ev0, &ev1);
  launch_maybe_timed(k_decode_fused, G, kFThreads, s, ev0, ev1, a);
  return hipGetLastError();
}

}  // namespace moe

#ifdef MOE_DECODE_TIMELINE
// The timeline of the last launch: uint64 [64][256][12] (layer, workgroup, stage).
extern "C" int moe_debug_decode_timeline(uint64_t* host_out) {
  return (int)hipMemcpyFromSymbol(host_out, HIP_SYMBOL(moe::g_decode_timeline), sizeof(moe::g_decode_timeline), 0,
                                  hipMemcpyDeviceToHost);
}
#endif
