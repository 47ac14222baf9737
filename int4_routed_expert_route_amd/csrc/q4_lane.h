// Lane-level pieces of the int4 dequant-GEMV shared by the decode kernels:
// exact integer dot products of the weight nibbles with activations held as
// 16-bit fixed point per group of 64 (a power-of-two scale per group, four
// balanced base-16 digits per value), K-part bookkeeping, per-lane weight
// loads and the LDS activation row.
#pragma once

#include "common.h"

namespace moe {
namespace lane {

// Eight weight nibbles (column i in bits 4i..4i+3 of w, unsigned 0..15)
// against eight activations given as four words of balanced base-16 digits
// (digit k of column i in bits 4i..4i+3 of word k, each in [-8, 7]).  The xor
// turns nibble q into the signed nibble q - 8, so a[k] += sum_i (q_i - 8) *
// digit_k(x_i); every product and sum is an exact integer.
__device__ __forceinline__ void dot8d(uint32_t w, const uint4 xd, int& a0, int& a1, int& a2, int& a3) {
  const int ws = (int)(w ^ 0x88888888u);
  a0 = __builtin_amdgcn_sdot8(ws, (int)xd.x, a0, false);
  a1 = __builtin_amdgcn_sdot8(ws, (int)xd.y, a1, false);
  a2 = __builtin_amdgcn_sdot8(ws, (int)xd.z, a2, false);
  a3 = __builtin_amdgcn_sdot8(ws, (int)xd.w, a3, false);
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

// LDS image of one activation row of G <= GMAX groups: per 8-column word its
// four digit words (16 bytes); part j's words start 16*j bytes later than
// packed (bank offset); per group its fp32 sum and its power-of-two scale
// (NaN when the group holds a non-finite value, so that it propagates).
template <int P, int GMAX>
struct XRow {
  static constexpr int kWords = GMAX * 8;
  uint4 v[kWords + P];  // word w (group w / 8) of part j at w + j
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
    // DPP row operations (the shuffles compiled to LDS permutes)
    s = group_sum_dpp(s, 8);
    mx = group8_max_dpp(mx);
    // 2^-e with max * 2^-e in [2^13, 2^14): every value rounds to an integer
    // of magnitude <= 2^14, which four balanced base-16 digits hold
    const bool finite = mx < INFINITY && fabsf(s) < INFINITY;
    int e = 0;
    if (finite && mx > 0.0f) e = __builtin_amdgcn_frexp_expf(mx) - 14;
    const float down = finite ? __builtin_ldexpf(1.0f, -e) : 0.0f;
    if (live) {
      // balanced digits of v are the base-16 digits of u = v + 0x8888 minus
      // 8, and a nibble n - 8 in two's complement is n ^ 8
      const float xs[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      uint32_t dw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t u = (uint32_t)((int)__builtin_rintf(xs[i] * down) + 0x8888);
#pragma unroll
        for (int k = 0; k < 4; ++k) dw[k] |= __builtin_amdgcn_ubfe(u, 4 * k, 4) << (4 * i);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) dw[k] ^= 0x88888888u;
      const int g = wi / 8;
      const int j = part_of_group<P>(g, G);
      dst.v[wi + j] = make_uint4(dw[0], dw[1], dw[2], dw[3]);
      if ((wi % 8) == 0) {
        dst.gsum[g] = s;
        dst.gscale[g] = finite ? __builtin_ldexpf(1.0f, e) : __builtin_nanf("");
      }
    }
  }
}

// sum over the lane's groups of s_g * (q . x)_g + b_g * xsum_g, then over the
// P K-parts (lanes r, r + R, r + 2R, ...).  Per group the digit sums give
// D = sum_i (q_i - 8) x_i exactly (x_i the group's integers), and
// sum_i (s q_i + b) x_i = s 2^e D + (b + 8 s) xsum.  Every lane runs GPP
// groups (padding groups have zero scale and bias and reuse an earlier
// chunk's activations).  The next 32-column chunk's activations are read
// from LDS while the current chunk is multiplied.
//
// `nck` is 2*GPP passed at run time: the branch on it puts every chunk in its
// own basic block, which keeps the scheduler from hoisting all LDS reads and
// nibble work to the top (that needs hundreds of registers).
template <int P, int GPP, int GMAX>
__device__ __forceinline__ float lane_dot(const LaneSlice<GPP>& s, const XRow<P, GMAX>& x, int j, Part pt, int G,
                                          int nck) {
  float acc = 0.0f;
  int a0 = 0, a1 = 0, a2 = 0, a3 = 0;
  // chunk c's activations (4 words) live in xb[c & 1]
  uint4 xb[2][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xb[0][i] = make_uint4(0u, 0u, 0u, 0u);
    xb[1][i] = make_uint4(0u, 0u, 0u, 0u);
  }
  if (pt.ng > 0) {
    const uint4* xv = &x.v[8 * pt.g0 + j];
#pragma unroll
    for (int i = 0; i < 4; ++i) xb[0][i] = xv[i];
  }
#pragma unroll
  for (int c = 0; c < 2 * GPP; ++c) {
    if (c < nck) {
      if (c + 1 < 2 * GPP && c + 1 < 2 * pt.ng) {
        const uint4* xv = &x.v[8 * (pt.g0 + (c + 1) / 2) + 4 * ((c + 1) & 1) + j];
#pragma unroll
        for (int i = 0; i < 4; ++i) xb[(c + 1) & 1][i] = xv[i];
      }
      const uint4* xc = xb[c & 1];
      // opaque copy: waits for this chunk only and keeps its nibble work here
      // (not hoisted out of the token loop)
      uint4 w = s.q[c];
      asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w));
      dot8d(w.x, xc[0], a0, a1, a2, a3);
      dot8d(w.y, xc[1], a0, a1, a2, a3);
      dot8d(w.z, xc[2], a0, a1, a2, a3);
      dot8d(w.w, xc[3], a0, a1, a2, a3);
      if (c & 1) {
        const int g = min(pt.g0 + c / 2, G - 1);
        const uint32_t sb = (c / 2 < pt.ng) ? s.sb[c / 2] : 0u;  // padding group: zero scale and bias
        const int D = ((a3 * 16 + a2) * 16 + a1) * 16 + a0;
        const float sc = half_lo(sb);
        acc = fmaf(sc * x.gscale[g], (float)D, fmaf(fmaf(8.0f, sc, half_hi(sb)), x.gsum[g], acc));
        a0 = a1 = a2 = a3 = 0;
      }
    }
  }
  constexpr int R = kWave / P;
#pragma unroll
  for (int o = R; o < kWave; o <<= 1) acc += __shfl_xor(acc, o, kWave);
  return acc;
}

// lane_dot for two rows at once (the gate row and the up row of one column)
// that read the same activations: each chunk's activation words are read
// from LDS once for both.  Returns the sums reduced over the PW K-parts a wave
// holds (lanes r, r + 64/PW, ...); the caller adds the other waves' parts.
// P is the number of K-parts of the LDS row layout.
template <int P, int PW, int GPP, int GMAX>
__device__ __forceinline__ float2 lane_dot2(const LaneSlice<GPP>& s0, const LaneSlice<GPP>& s1,
                                            const XRow<P, GMAX>& x, int j, Part pt, int G, int nck) {
  float acc0 = 0.0f, acc1 = 0.0f;
  int a0 = 0, a1 = 0, a2 = 0, a3 = 0, b0 = 0, b1 = 0, b2 = 0, b3 = 0;
  uint4 xb[2][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xb[0][i] = make_uint4(0u, 0u, 0u, 0u);
    xb[1][i] = make_uint4(0u, 0u, 0u, 0u);
  }
  if (pt.ng > 0) {
    const uint4* xv = &x.v[8 * pt.g0 + j];
#pragma unroll
    for (int i = 0; i < 4; ++i) xb[0][i] = xv[i];
  }
#pragma unroll
  for (int c = 0; c < 2 * GPP; ++c) {
    if (c < nck) {
      if (c + 1 < 2 * GPP && c + 1 < 2 * pt.ng) {
        const uint4* xv = &x.v[8 * (pt.g0 + (c + 1) / 2) + 4 * ((c + 1) & 1) + j];
#pragma unroll
        for (int i = 0; i < 4; ++i) xb[(c + 1) & 1][i] = xv[i];
      }
      const uint4* xc = xb[c & 1];
      uint4 w = s0.q[c], u = s1.q[c];
      asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w));
      asm volatile("" : "+v"(u.x), "+v"(u.y), "+v"(u.z), "+v"(u.w));
      dot8d(w.x, xc[0], a0, a1, a2, a3);
      dot8d(u.x, xc[0], b0, b1, b2, b3);
      dot8d(w.y, xc[1], a0, a1, a2, a3);
      dot8d(u.y, xc[1], b0, b1, b2, b3);
      dot8d(w.z, xc[2], a0, a1, a2, a3);
      dot8d(u.z, xc[2], b0, b1, b2, b3);
      dot8d(w.w, xc[3], a0, a1, a2, a3);
      dot8d(u.w, xc[3], b0, b1, b2, b3);
      if (c & 1) {
        const int g = min(pt.g0 + c / 2, G - 1);
        const bool real = c / 2 < pt.ng;  // padding group: zero scale and bias
        const uint32_t sb0 = real ? s0.sb[c / 2] : 0u, sb1 = real ? s1.sb[c / 2] : 0u;
        const float gs = x.gscale[g], gsum = x.gsum[g];
        const int D0 = ((a3 * 16 + a2) * 16 + a1) * 16 + a0, D1 = ((b3 * 16 + b2) * 16 + b1) * 16 + b0;
        const float sc0 = half_lo(sb0), sc1 = half_lo(sb1);
        acc0 = fmaf(sc0 * gs, (float)D0, fmaf(fmaf(8.0f, sc0, half_hi(sb0)), gsum, acc0));
        acc1 = fmaf(sc1 * gs, (float)D1, fmaf(fmaf(8.0f, sc1, half_hi(sb1)), gsum, acc1));
        a0 = a1 = a2 = a3 = 0;
        b0 = b1 = b2 = b3 = 0;
      }
    }
  }
  constexpr int R = kWave / PW;
#pragma unroll
  for (int o = R; o < kWave; o <<= 1) {
    acc0 += __shfl_xor(acc0, o, kWave);
    acc1 += __shfl_xor(acc1, o, kWave);
  }
  return make_float2(acc0, acc1);
}

}  // namespace lane
}  // namespace moe
