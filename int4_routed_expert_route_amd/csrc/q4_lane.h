// Lane-level pieces of the int4 dequant-GEMV shared by the decode kernels:
// nibble pairs as fp16 subnormals dotted with fp16 hi/lo activation pairs,
// K-part bookkeeping, per-lane weight loads and the LDS activation row.
#pragma once

#include "common.h"

namespace moe {
namespace lane {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t q, uint32_t x, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, q), __builtin_bit_cast(half2_t, x), acc, false);
}

// Dot of the 8 nibbles of one 32-bit word (columns 0..7, even column = low
// nibble) with 8 activations given as 4 hi and 4 lo fp16 pairs ordered
// (x0,x4) (x1,x5) (x2,x6) (x3,x7).  Result scaled by 2^-24.
__device__ __forceinline__ float dot8(uint32_t w, const uint4 xh, const uint4 xl, float acc) {
  const uint32_t m = 0x000F000Fu;
  uint32_t w4 = w >> 4;
  const uint32_t p0 = w & m;           // columns 0, 4
  const uint32_t p1 = w4 & m;          // columns 1, 5
  const uint32_t p2 = (w >> 8) & m;    // columns 2, 6
  const uint32_t p3 = (w4 >> 8) & m;   // columns 3, 7
  acc = dot2(p0, xh.x, acc);
  acc = dot2(p1, xh.y, acc);
  acc = dot2(p2, xh.z, acc);
  acc = dot2(p3, xh.w, acc);
  acc = dot2(p0, xl.x, acc);
  acc = dot2(p1, xl.y, acc);
  acc = dot2(p2, xl.z, acc);
  acc = dot2(p3, xl.w, acc);
  return acc;
}

// K-part j of a row with G groups split over P parts: groups [g0, g0 + ng).
struct Part {
  int g0, ng;
};
template <int P>
__device__ __forceinline__ Part part_of(int j, int G) {
  const int base = G / P, rem = G % P;
  return Part{j * base + min(j, rem), base + (j < rem ? 1 : 0)};
}
template <int P>
__device__ __forceinline__ int part_of_group(int g, int G) {
  const int base = G / P, rem = G % P;
  const int big = rem * (base + 1);  // groups covered by the first `rem` (longer) parts
  return g < big ? g / (base + 1) : rem + (g - big) / max(base, 1);
}

// One lane's share of its rows: up to GPP groups (2*GPP chunks) of its K-part
// plus their (scale, bias) words.
template <int GPP>
struct LaneSlice {
  uint4 q[2 * GPP];
  uint32_t sb[GPP];
};

// Every lane issues GPP groups' worth of loads unconditionally (conditional
// loads into registers with a default value make the compiler wait for them
// early).  A part shorter than GPP groups re-reads its last group (a cache hit)
// and lane_dot gives those padding groups a zero scale and bias.  The (scale,
// bias) words go first, so code that only needs them waits for them alone; the
// scheduling barrier keeps later arithmetic below the loads.
template <int GPP>
__device__ __forceinline__ void load_lane(LaneSlice<GPP>& s, const uint8_t* q, const uint8_t* sb, Part pt, int G) {
#pragma unroll
  for (int i = 0; i < GPP; ++i) {
    const int g = max(0, min(pt.g0 + min(i, pt.ng - 1), G - 1));
    s.sb[i] = *reinterpret_cast<const uint32_t*>(sb + (int64_t)g * 256);
  }
#pragma unroll
  for (int i = 0; i < 2 * GPP; ++i) {
    const int c = max(0, min(2 * pt.g0 + min(i, 2 * pt.ng - 1), 2 * G - 1));
    s.q[i] = *reinterpret_cast<const uint4*>(q + (int64_t)c * 1024);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// LDS image of one activation row of G <= GMAX groups: per 8-column word 4 hi
// and 4 lo fp16 pairs (32 bytes); part j's words start 16*j bytes later than
// packed (bank offset); per group its fp32 sum and its power-of-two scale.
template <int P, int GMAX>
struct XRow {
  static constexpr int kWords = GMAX * 8;
  uint4 v[2 * kWords + 2 * P];  // 16-byte units: word w of part j at 2*w + j
  float gsum[GMAX];
  float gscale[GMAX];
};

// Staging of an activation row x[0 .. 64*G) into LDS, split in two so that the
// activation loads can be issued before the weight loads (and waited for on
// their own): stage_load reads this thread's 8-column words into registers,
// stage_store converts them and writes LDS.  `nthreads` threads (a multiple
// of 64) all call both; NPASS >= ceil(8*G / nthreads).
template <int NPASS>
struct StageRegs {
  float4 a[NPASS], b[NPASS];
};

template <int NPASS>
__device__ __forceinline__ void stage_load(StageRegs<NPASS>& sr, const float* __restrict__ x, int G, int tid,
                                           int nthreads) {
  const int nw = G * 8;
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const int wi = min(ps * nthreads + tid, nw - 1);  // clamped: stage_store skips the extra words
    sr.a[ps] = reinterpret_cast<const float4*>(x)[2 * wi];
    sr.b[ps] = reinterpret_cast<const float4*>(x)[2 * wi + 1];
  }
}

template <int P, int GMAX, int NPASS>
__device__ __forceinline__ void stage_store(XRow<P, GMAX>& dst, const StageRegs<NPASS>& sr, int G, int tid,
                                            int nthreads) {
  const int nw = G * 8;
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    if (ps * nthreads >= nw) break;  // uniform
    const int wi = ps * nthreads + tid;
    const bool live = wi < nw;
    const float4 a = sr.a[ps], b = sr.b[ps];
    // group (8 consecutive words = 8 consecutive lanes) sum and max magnitude
    float s = ((a.x + a.y) + (a.z + a.w)) + ((b.x + b.y) + (b.z + b.w));
    float mx = fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                     fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
#pragma unroll
    for (int o = 4; o >= 1; o >>= 1) {
      s += __shfl_xor(s, o, kWave);
      mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
    }
    // 2^-e with max * 2^-e in [2^14, 2^15) (1 for zero or non-finite maxima)
    int e = 0;
    if (mx > 0.0f && mx < INFINITY) e = __builtin_amdgcn_frexp_expf(mx) - 15;
    const float down = __builtin_ldexpf(1.0f, -e);
    if (live) {
      const float xs[8] = {a.x * down, a.y * down, a.z * down, a.w * down,
                           b.x * down, b.y * down, b.z * down, b.w * down};
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const _Float16 h0 = (_Float16)xs[i], h1 = (_Float16)xs[i + 4];
        const _Float16 l0 = (_Float16)(xs[i] - (float)h0), l1 = (_Float16)(xs[i + 4] - (float)h1);
        hi[i] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
        lo[i] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
      }
      const int g = wi / 8;
      const int j = part_of_group<P>(g, G);
      dst.v[2 * wi + j] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      dst.v[2 * wi + j + 1] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
      if ((wi % 8) == 0) {
        dst.gsum[g] = s;
        dst.gscale[g] = __builtin_ldexpf(16777216.0f, e);  // 2^24 * 2^e
      }
    }
  }
}

// sum over the lane's groups of s_g * (q . x)_g + b_g * xsum_g, then over the
// P K-parts (lanes r, r + R, r + 2R, ...).  Every lane runs GPP groups (padding
// groups have zero weights and reuse finite activations).  The next
// 32-column chunk's activations are read from LDS while the current chunk is
// multiplied.
//
// `nck` is 2*GPP passed at run time: the branch on it puts every chunk in its
// own basic block, which keeps the scheduler from hoisting all LDS reads and
// nibble extractions to the top (that needs hundreds of registers).
template <int P, int GPP, int GMAX>
__device__ __forceinline__ float lane_dot(const LaneSlice<GPP>& s, const XRow<P, GMAX>& x, int j, Part pt, int G,
                                          int nck) {
  float acc = 0.0f, d0 = 0.0f, d1 = 0.0f;
  // chunk c's activations live in xb[c & 1]; padding chunks keep the finite
  // values of an earlier chunk (their weights are zero)
  uint4 xb[2][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    xb[0][i] = make_uint4(0u, 0u, 0u, 0u);
    xb[1][i] = make_uint4(0u, 0u, 0u, 0u);
  }
  if (pt.ng > 0) {
    const uint4* xv = &x.v[16 * pt.g0 + j];
#pragma unroll
    for (int i = 0; i < 8; ++i) xb[0][i] = xv[i];
  }
#pragma unroll
  for (int c = 0; c < 2 * GPP; ++c) {
    if (c < nck) {
      if (c + 1 < 2 * GPP && c + 1 < 2 * pt.ng) {
        const uint4* xv = &x.v[16 * (pt.g0 + (c + 1) / 2) + j + 8 * ((c + 1) & 1)];
#pragma unroll
        for (int i = 0; i < 8; ++i) xb[(c + 1) & 1][i] = xv[i];
      }
      const uint4* xc = xb[c & 1];
      // opaque copy: waits for this chunk only and keeps its nibble extraction
      // here (not hoisted out of the token loop)
      uint4 w = s.q[c];
      asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w));
      d0 = dot8(w.x, xc[0], xc[1], d0);
      d1 = dot8(w.y, xc[2], xc[3], d1);
      d0 = dot8(w.z, xc[4], xc[5], d0);
      d1 = dot8(w.w, xc[6], xc[7], d1);
      if (c & 1) {
        const int g = min(pt.g0 + c / 2, G - 1);
        const uint32_t sb = (c / 2 < pt.ng) ? s.sb[c / 2] : 0u;  // padding group: zero scale and bias
        acc = fmaf(half_lo(sb) * x.gscale[g], d0 + d1, fmaf(half_hi(sb), x.gsum[g], acc));
        d0 = 0.0f;
        d1 = 0.0f;
      }
    }
  }
  constexpr int R = kWave / P;
#pragma unroll
  for (int o = R; o < kWave; o <<= 1) acc += __shfl_xor(acc, o, kWave);
  return acc;
}

}  // namespace lane
}  // namespace moe
