// Fused int4 dequant-GEMV for the selected experts (decode and small batches).
//
// The routed experts' projections are INT4 with affine groups of 64 columns,
// one scale and one bias per group ("Optimizing a 14.3 GB model for an 8 GB
// machine", section "Vectorization helped when it respected the storage
// layout").  Once expert reads are explicit, these matvecs are the largest GPU
// cost of a decode step, and the kernel that won on the pages gave the GPU many
// independent workgroups that claim rows until the dispatch is done (same page,
// section "MoE needed parallel work, reuse, and coarse overlap").
//
// gfx950 design
//  * One blob row tile = 64 rows = one row per lane.  Inside a tile the 16-byte
//    column chunks of the 64 rows are adjacent, so every 128-bit load of a wave
//    reads 1 KiB of contiguous HBM, and a lane's (scale, bias) pairs are 4-byte
//    loads that also coalesce to 256 bytes per group.
//  * A task is (expert group, row tile, K-slice).  A wave issues all of its
//    slice's nibble and pair loads up front, so several KiB per wave are in
//    flight, then dequantises in registers.
//  * Group-factored dequant: sum_c (s q_c + b) x_c = s * sum_c q_c x_c + b * sum_c x_c,
//    so each weight costs one byte extract, one int->float convert and one FMA;
//    the per-group x sums come from a 16-lane shuffle reduction.
//  * The activations x are wave-uniform and read through uniform loads.
//  * K-slices of the same (group, tile) write fp32 partials; the last task to
//    arrive (device-scope counter) sums them in slice order and finishes the row
//    (GELU * up, or the rank-ordered combine), so results are deterministic.
//  * Tasks beyond the grid are claimed from an atomic counter (persistent
//    workgroups).  Counters are returned to zero by the last arrival.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kMBGrouped = 4;  // tokens per pass over the loaded weights (grouped path)

// Activations are read-only for the whole kernel and wave-uniform at every use
// in the dot products; reading them through the constant address space lets
// the compiler fetch them with scalar loads into SGPR operands of the FMAs.
typedef __attribute__((address_space(4))) const float cfloat;
__device__ __forceinline__ const cfloat* uniform_ptr(const float* p) { return (const cfloat*)p; }

// Dot of 8 nibbles (one 32-bit word: columns 0..7, even column = low nibble)
// with 8 consecutive x values.  The masks are kept opaque to the optimiser so
// that the byte extracts map onto v_cvt_f32_ubyte{0,1,2,3}: 3 bit operations,
// 8 converts and 8 FMAs per 8 weights.
__device__ __forceinline__ float dot8(uint32_t w, const cfloat* x, float acc) {
  uint32_t lo = w & 0x0F0F0F0Fu;
  uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;
  asm volatile("" : "+v"(lo));
  asm volatile("" : "+v"(hi));
  acc = fmaf((float)(lo & 0xffu), x[0], acc);
  acc = fmaf((float)(hi & 0xffu), x[1], acc);
  acc = fmaf((float)((lo >> 8) & 0xffu), x[2], acc);
  acc = fmaf((float)((hi >> 8) & 0xffu), x[3], acc);
  acc = fmaf((float)((lo >> 16) & 0xffu), x[4], acc);
  acc = fmaf((float)((hi >> 16) & 0xffu), x[5], acc);
  acc = fmaf((float)(lo >> 24), x[6], acc);
  acc = fmaf((float)(hi >> 24), x[7], acc);
  return acc;
}

// Sums of x over the groups of a K-slice for one token: lanes 16g..16g+15 load
// group g's 64 values as float4 and reduce; result broadcast to all lanes.
template <int G>
__device__ __forceinline__ void group_sums(const float* __restrict__ x, int ngroups, float (&out)[G]) {
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int gb = 0; gb < (G + 3) / 4; ++gb) {
    const int g = gb * 4 + lane / 16;
    float s = 0.0f;
    if (g < ngroups) {
      float4 v = reinterpret_cast<const float4*>(x + g * kGroup)[lane % 16];
      s = (v.x + v.y) + (v.z + v.w);
    }
    s = sum16(s);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (gb * 4 + q < G) out[gb * 4 + q] = __shfl(s, q * 16, kWave);
  }
}

struct Members {
  int expert;  // -1: nothing to do
  int count;
  int first;   // mode A: the pair itself; mode B: index into sorted_pair
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

__device__ __forceinline__ int member_pair(const Members& m, int i,
                                           const int32_t* __restrict__ sorted_pair, bool grouped,
                                           int n_pairs) {
  if (!grouped) return m.first;
  int p = sorted_pair[m.first + i];
  return (p >= 0 && p < n_pairs) ? p : -1;
}

// Resolve the expert's blob through the slot table; nullptr if not resident.
__device__ __forceinline__ const uint8_t* expert_blob(int expert, int E,
                                                      const int32_t* __restrict__ slot_of_expert,
                                                      int n_slots, const uint8_t* arena,
                                                      int64_t slot_stride) {
  if (expert < 0 || expert >= E) return nullptr;
  int slot = slot_of_expert[expert];
  if (slot < 0 || slot >= n_slots) return nullptr;
  return arena + (int64_t)slot * slot_stride;
}

// ------------------------------------------------------------------ gate/up

// Loads of one K-slice of one matrix tile: NCH 16-byte nibble chunks and NCH/2
// (scale, bias) pairs for this lane's row.
template <int NCH>
struct SliceRegs {
  uint4 q[NCH];
  uint32_t sb[NCH / 2];
};

template <int NCH>
__device__ __forceinline__ void load_slice(SliceRegs<NCH>& r, const uint8_t* q, const uint8_t* sb) {
#pragma unroll
  for (int c = 0; c < NCH; ++c) r.q[c] = *reinterpret_cast<const uint4*>(q + c * 1024);
#pragma unroll
  for (int g = 0; g < NCH / 2; ++g) r.sb[g] = *reinterpret_cast<const uint32_t*>(sb + g * 256);
}

// Dequantised dot of the slice with one token's x: sum_g s_g * (q . x)_g + b_g * xsum_g.
template <int NCH>
__device__ __forceinline__ float slice_dot(const SliceRegs<NCH>& r, const float* x, const float* xs) {
  const cfloat* xc = uniform_ptr(x);
  float acc = 0.0f;
#pragma unroll
  for (int g = 0; g < NCH / 2; ++g) {
    float d = 0.0f;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const uint4 w = r.q[2 * g + cc];
      const cfloat* xw = xc + (2 * g + cc) * kChunkCols;
      d = dot8(w.x, xw + 0, d);
      d = dot8(w.y, xw + 8, d);
      d = dot8(w.z, xw + 16, d);
      d = dot8(w.w, xw + 24, d);
    }
    acc = fmaf(half_lo(r.sb[g]), d, fmaf(half_hi(r.sb[g]), xs[g], acc));
  }
  return acc;
}

// Gate and up slices against the same x in one pass, so every x value is used
// twice right after it is loaded.
template <int NCH>
__device__ __forceinline__ void slice_dot2(const SliceRegs<NCH>& r0, const SliceRegs<NCH>& r1,
                                           const float* x, const float* xs, float& out0, float& out1) {
  const cfloat* xc = uniform_ptr(x);
  float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
  for (int g = 0; g < NCH / 2; ++g) {
    float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const uint4 w0 = r0.q[2 * g + cc];
      const uint4 w1 = r1.q[2 * g + cc];
      const cfloat* xw = xc + (2 * g + cc) * kChunkCols;
      d0 = dot8(w0.x, xw + 0, d0);
      d1 = dot8(w1.x, xw + 0, d1);
      d0 = dot8(w0.y, xw + 8, d0);
      d1 = dot8(w1.y, xw + 8, d1);
      d0 = dot8(w0.z, xw + 16, d0);
      d1 = dot8(w1.z, xw + 16, d1);
      d0 = dot8(w0.w, xw + 24, d0);
      d1 = dot8(w1.w, xw + 24, d1);
    }
    acc0 = fmaf(half_lo(r0.sb[g]), d0, fmaf(half_hi(r0.sb[g]), xs[g], acc0));
    acc1 = fmaf(half_lo(r1.sb[g]), d1, fmaf(half_hi(r1.sb[g]), xs[g], acc1));
  }
  out0 = acc0;
  out1 = acc1;
}

template <int NCH, int MB>
__global__ __launch_bounds__(kWave) void k_gateup_fp32(GateupArgs a) {
  constexpr int G = NCH / 2;
  const int lane = threadIdx.x;
  const int n_pairs = a.T * a.k;
  const bool grouped = a.offsets != nullptr;
  int task = blockIdx.x;
  while (task < a.ntasks) {
    const int ks = task % a.nks;
    const int rt = (task / a.nks) % a.n_rt;
    const int group = task / (a.nks * a.n_rt);
    const Members m = resolve_group(group, a.topk_idx, a.offsets, a.pair_mask, a.mask_value, n_pairs);
    if (m.count > 0) {
      const uint8_t* blob = expert_blob(m.expert, a.E, a.slot_of_expert, a.n_slots, a.arena, a.slot_stride);
      const bool ok = blob != nullptr;
      if (!ok) blob = a.arena;  // keep the loads in bounds; outputs become NaN
      const int c0 = ks * NCH;
      const int64_t tile_q = (int64_t)rt * (kTileRows * a.d / 2) + (int64_t)c0 * 1024 + lane * 16;
      const int64_t tile_sb = (int64_t)rt * (kTileRows * (a.d / kGroup) * 4) + (int64_t)(c0 / 2) * 256 + lane * 4;
      SliceRegs<NCH> rg, ru;
      load_slice(rg, blob + a.off_q0 + tile_q, blob + a.off_sb0 + tile_sb);
      load_slice(ru, blob + a.off_q1 + tile_q, blob + a.off_sb1 + tile_sb);
      for (int i0 = 0; i0 < m.count; i0 += MB) {
        const int nm = min(MB, m.count - i0);
#pragma unroll
        for (int j = 0; j < MB; ++j) {
          if (j < nm) {
            const int p = member_pair(m, i0 + j, a.sorted_pair, grouped, n_pairs);
            if (p < 0) continue;
            const float* x = a.h + (int64_t)(p / a.k) * a.d + (int64_t)c0 * kChunkCols;
            float xs[G];
            group_sums<G>(x, G, xs);
            float g, u;
            slice_dot2<NCH>(rg, ru, x, xs, g, u);
            if (!ok) { g = f32_nan(); u = f32_nan(); }
            if (a.nks == 1) {
              a.act[(int64_t)p * a.f + rt * kTileRows + lane] = gelu_tanh(g) * u;
            } else {
              float* dst = a.partial + (((int64_t)p * a.n_rt + rt) * a.nks + ks) * (2 * kTileRows);
              dst[lane] = g;
              dst[kTileRows + lane] = u;
            }
          }
        }
      }
      // the last K-slice of this (group, tile) to arrive finishes its rows
      if (a.nks > 1) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        uint32_t* ctr = a.counters + (int64_t)group * a.n_rt + rt;
        uint32_t ticket = 0;
        if (lane == 0) ticket = arrive(ctr);
        ticket = __builtin_amdgcn_readfirstlane(ticket);
        if (ticket == (uint32_t)a.nks - 1) {
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
          for (int i = 0; i < m.count; ++i) {
            const int p = member_pair(m, i, a.sorted_pair, grouped, n_pairs);
            if (p < 0) continue;
            const float* src = a.partial + ((int64_t)p * a.n_rt + rt) * a.nks * (2 * kTileRows);
            float g = 0.0f, u = 0.0f;
            for (int s = 0; s < a.nks; ++s) {
              g += src[s * 2 * kTileRows + lane];
              u += src[s * 2 * kTileRows + kTileRows + lane];
            }
            a.act[(int64_t)p * a.f + rt * kTileRows + lane] = gelu_tanh(g) * u;
          }
          if (lane == 0) reset_counter(ctr);
        }
      }
    }
    if (!a.persistent) break;
    int next = 0;
    if (lane == 0) next = (int)atomicAdd(a.claim, 1u) + (int)gridDim.x;
    task = __builtin_amdgcn_readfirstlane(next);
  }
  if (a.persistent && lane == 0) {
    uint32_t done = arrive(a.claim + 1);
    if (done == gridDim.x - 1) {
      reset_counter(a.claim);
      reset_counter(a.claim + 1);
    }
  }
}

// ------------------------------------------------------------------ down + combine

template <int NCH, int MB>
__global__ __launch_bounds__(kWave) void k_down_fp32(DownArgs a) {
  constexpr int G = NCH / 2;
  const int lane = threadIdx.x;
  const int n_pairs = a.T * a.k;
  const bool grouped = a.offsets != nullptr;
  int task = blockIdx.x;
  while (task < a.ntasks) {
    const int ks = task % a.nks;
    const int rt = (task / a.nks) % a.n_rt;
    const int group = task / (a.nks * a.n_rt);
    const Members m = resolve_group(group, a.topk_idx, a.offsets, nullptr, 0, n_pairs);
    if (m.count > 0) {
      const uint8_t* blob = expert_blob(m.expert, a.E, a.slot_of_expert, a.n_slots, a.arena, a.slot_stride);
      const bool ok = blob != nullptr;
      if (!ok) blob = a.arena;
      const int c0 = ks * NCH;
      const int64_t tile_q = (int64_t)rt * (kTileRows * a.f / 2) + (int64_t)c0 * 1024 + lane * 16;
      const int64_t tile_sb = (int64_t)rt * (kTileRows * (a.f / kGroup) * 4) + (int64_t)(c0 / 2) * 256 + lane * 4;
      SliceRegs<NCH> rd;
      load_slice(rd, blob + a.off_q + tile_q, blob + a.off_sb + tile_sb);
      for (int i0 = 0; i0 < m.count; i0 += MB) {
        const int nm = min(MB, m.count - i0);
#pragma unroll
        for (int j = 0; j < MB; ++j) {
          if (j < nm) {
            const int p = member_pair(m, i0 + j, a.sorted_pair, grouped, n_pairs);
            if (p < 0) continue;
            const float* x = a.act + (int64_t)p * a.f + (int64_t)c0 * kChunkCols;
            float xs[G];
            group_sums<G>(x, G, xs);
            float o = slice_dot<NCH>(rd, x, xs);
            if (!ok) o = f32_nan();
            a.partial[(((int64_t)p * a.n_rt + rt) * a.nks + ks) * kTileRows + lane] = o;
          }
        }
      }
    }
    // every task of a row tile arrives, empty ones included; the last combines
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    uint32_t* ctr = a.counters + rt;
    uint32_t ticket = 0;
    if (lane == 0) ticket = arrive(ctr);
    ticket = __builtin_amdgcn_readfirstlane(ticket);
    if (ticket == (uint32_t)(a.n_groups * a.nks) - 1) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      const int row = rt * kTileRows + lane;
      for (int t = 0; t < a.T; ++t) {
        float yv = a.residual ? a.residual[(int64_t)t * a.d + row] : 0.0f;
        for (int j = 0; j < a.k; ++j) {
          const int p = t * a.k + j;
          const float* src = a.partial + ((int64_t)p * a.n_rt + rt) * a.nks * kTileRows;
          float o = 0.0f;
          for (int s = 0; s < a.nks; ++s) o += src[s * kTileRows + lane];
          yv = fmaf(a.topk_w[p], o, yv);
        }
        a.y[(int64_t)t * a.d + row] = yv;
      }
      if (lane == 0) reset_counter(ctr);
    }
    if (!a.persistent) break;
    int next = 0;
    if (lane == 0) next = (int)atomicAdd(a.claim, 1u) + (int)gridDim.x;
    task = __builtin_amdgcn_readfirstlane(next);
  }
  if (a.persistent && lane == 0) {
    uint32_t done = arrive(a.claim + 1);
    if (done == gridDim.x - 1) {
      reset_counter(a.claim);
      reset_counter(a.claim + 1);
    }
  }
}

}  // namespace

// ------------------------------------------------------------------ host side

// Chunks per K-slice: the largest supported even count that divides the row.
// Gate/up rows (2816 columns = 88 chunks) take 8-chunk slices (256 columns),
// down rows (704 columns = 22 chunks) are read whole.
static int pick_nch(int nch_total, const int* options, int n) {
  for (int i = 0; i < n; ++i)
    if (nch_total % options[i] == 0) return options[i];
  return 2;
}
static int gateup_nch(int d) {
  static const int opts[] = {8, 4, 2};
  return pick_nch(d / kChunkCols, opts, 3);
}
static int down_nch(int f) {
  static const int opts[] = {22, 16, 12, 8, 4, 2};
  return pick_nch(f / kChunkCols, opts, 6);
}

static int ceil_div(int a, int b) { return (a + b - 1) / b; }

GemvPlan plan_gateup(int T, int d, int f, int E, int k, bool grouped) {
  GemvPlan p;
  p.nch = gateup_nch(d);
  p.nks = (d / kChunkCols) / p.nch;
  p.n_rt = f / kTileRows;
  p.n_groups = grouped ? E : T * k;
  p.ntasks = p.n_groups * p.n_rt * p.nks;
  p.partial_floats = p.nks > 1 ? (size_t)T * k * p.n_rt * p.nks * 2 * kTileRows : 0;
  p.counters = p.nks > 1 ? (size_t)p.n_groups * p.n_rt : 0;
  return p;
}

GemvPlan plan_down(int T, int d, int f, int E, int k, bool grouped) {
  GemvPlan p;
  p.nch = down_nch(f);
  p.nks = (f / kChunkCols) / p.nch;
  p.n_rt = d / kTileRows;
  p.n_groups = grouped ? E : T * k;
  p.ntasks = p.n_groups * p.n_rt * p.nks;
  p.partial_floats = (size_t)T * k * p.n_rt * p.nks * kTileRows;
  p.counters = (size_t)p.n_rt;
  return p;
}

// Workspace: [claim counters 256 B][task counters][partials], all 256-B aligned.
size_t gemv_workspace_bytes(const GemvPlan& p) {
  size_t b = 256;
  b += round256((int64_t)p.counters * 4);
  b += round256((int64_t)p.partial_floats * 4);
  return b;
}

static void carve(void* ws, const GemvPlan& p, uint32_t** claim, uint32_t** counters, float** partial) {
  char* c = reinterpret_cast<char*>(ws);
  *claim = reinterpret_cast<uint32_t*>(c);
  *counters = reinterpret_cast<uint32_t*>(c + 256);
  *partial = reinterpret_cast<float*>(c + 256 + round256((int64_t)p.counters * 4));
}

static int grid_for(const GemvPlan& p, int max_resident) {
  if (max_resident > 0 && p.ntasks > max_resident) return max_resident;
  return p.ntasks;
}

hipError_t launch_gateup_fp32(GateupArgs a, const GemvPlan& p, void* ws, int max_resident, hipStream_t s) {
  carve(ws, p, &a.claim, &a.counters, &a.partial);
  a.nks = p.nks;
  a.n_rt = p.n_rt;
  a.ntasks = p.ntasks;
  const int grid = grid_for(p, max_resident);
  a.persistent = grid < p.ntasks;
  const bool grouped = a.offsets != nullptr;
#define MOE_GATEUP_CASE(N)                                                                    \
  case N:                                                                                     \
    if (grouped)                                                                              \
      hipLaunchKernelGGL((k_gateup_fp32<N, kMBGrouped>), dim3(grid), dim3(kWave), 0, s, a);  \
    else                                                                                      \
      hipLaunchKernelGGL((k_gateup_fp32<N, 1>), dim3(grid), dim3(kWave), 0, s, a);           \
    break;
  switch (p.nch) {
    MOE_GATEUP_CASE(2)
    MOE_GATEUP_CASE(4)
    MOE_GATEUP_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef MOE_GATEUP_CASE
  return hipGetLastError();
}

hipError_t launch_down_fp32(DownArgs a, const GemvPlan& p, void* ws, int max_resident, hipStream_t s) {
  carve(ws, p, &a.claim, &a.counters, &a.partial);
  a.nks = p.nks;
  a.n_rt = p.n_rt;
  a.n_groups = p.n_groups;
  a.ntasks = p.ntasks;
  const int grid = grid_for(p, max_resident);
  a.persistent = grid < p.ntasks;
  const bool grouped = a.offsets != nullptr;
#define MOE_DOWN_CASE(N)                                                                   \
  case N:                                                                                  \
    if (grouped)                                                                           \
      hipLaunchKernelGGL((k_down_fp32<N, kMBGrouped>), dim3(grid), dim3(kWave), 0, s, a); \
    else                                                                                   \
      hipLaunchKernelGGL((k_down_fp32<N, 1>), dim3(grid), dim3(kWave), 0, s, a);          \
    break;
  switch (p.nch) {
    MOE_DOWN_CASE(2)
    MOE_DOWN_CASE(4)
    MOE_DOWN_CASE(8)
    MOE_DOWN_CASE(12)
    MOE_DOWN_CASE(16)
    MOE_DOWN_CASE(22)
    default: return hipErrorInvalidValue;
  }
#undef MOE_DOWN_CASE
  return hipGetLastError();
}

}  // namespace moe
