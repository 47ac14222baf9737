// Routing: RMSNorm, router matvec, softmax, top-k, renormalisation.
//
// The router is a small fp32 matrix that names k of E experts per token
// (TurboFieldfare video transcript, paragraphs on the router).  The choice is
// taken on fp32 logits: largest first, equal logits to the lower expert id; the
// weights are the softmax over all experts renormalised over the chosen ones,
// which equals the softmax over the chosen logits alone.
#include <hip/hip_ext.h>

#include <mutex>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kSmallT = 8;         // fused single-launch path up to this many tokens
typedef float floatx4r __attribute__((ext_vector_type(4)));
constexpr int kRouteWaves = 4;     // waves per workgroup in the fused path

// Top-k of one token's logits by one wave: k rounds of a wave-wide arg-max
// over one 64-bit key per (logit, expert) (topk_key, wave_max_u64 in common.h).
// Writes idx/w for the token.
// v[i], ok[i]: the logit of expert lane + 64 i and whether that expert exists.
__device__ void wave_topk_vals(float (&v)[4], bool (&ok)[4], int k, int32_t* idx_out, float* w_out) {
  const int lane = threadIdx.x % kWave;
  uint64_t key[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) key[i] = ok[i] ? topk_key(v[i], lane + kWave * i) : 0ull;
  // lane j keeps the j-th choice
  float my_v = 0.0f;
  int my_e = -1;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    const int be = (int)(0xFFFFFFFFu - (uint32_t)best);
    if (best == 0) break;  // fewer than k experts
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (lane + kWave * i == be) key[i] = 0;
    // the chosen logit, back from the key's monotone bits
    const uint32_t mono = (uint32_t)(best >> 32);
    const float bv = __builtin_bit_cast(float, (mono & 0x80000000u) ? (mono & 0x7FFFFFFFu) : ~mono);
    if (lane == j) {
      my_v = bv;
      my_e = be;
    }
  }
  const float m = __shfl(my_v, 0, kWave);
  const float ex = lane < k ? expf(my_v - m) : 0.0f;
  const float s = wave_sum(ex);
  if (lane < k) {
    idx_out[lane] = my_e;
    w_out[lane] = ex / s;
  }
}

__device__ void wave_topk(const float* logits, int E, int k, int32_t* idx_out, float* w_out,
                          bool coherent) {
  const int lane = threadIdx.x % kWave;
  float v[4];
  bool ok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int e = lane + kWave * i;
    ok[i] = e < E;
    v[i] = ok[i] ? (coherent ? load_coherent(logits + e) : logits[e]) : 0.0f;
  }
  wave_topk_vals(v, ok, k, idx_out, w_out);
}

// Top-k of one token's E <= 256 logits by one workgroup of 256 threads.  The
// rank of expert e is the number of experts that beat it (larger logit, or
// equal logit and lower id); 2 threads per expert (E <= 128) or 1 (E <= 256)
// count over halves of the list with 4-wide LDS reads.  No dependent shuffle
// chains.
__device__ void block_topk(const float* logits, int E, int k, int32_t* idx_out, float* w_out) {
  __shared__ float4 s_l4[64];
  __shared__ int s_cnt[256];
  __shared__ float s_val[16];
  __shared__ int s_idx[16];
  float* s_l = reinterpret_cast<float*>(s_l4);
  const int tid = threadIdx.x;
  const int E4 = (E + 3) / 4;
  s_l[tid] = tid < E ? load_coherent(logits + tid) : -INFINITY;
  __syncthreads();
  const int split = E <= 128 ? 2 : 1;
  const int e = tid / split, h = tid % split;
  int cnt = 0;
  if (e < E) {
    const float v = s_l[e];
    const int q0 = h * (E4 / split), q1 = (h + 1 == split) ? E4 : (h + 1) * (E4 / split);
#pragma unroll 4
    for (int q = q0; q < q1; ++q) {
      const float4 o = s_l4[q];
      const int b = 4 * q;
      cnt += (o.x > v || (o.x == v && b + 0 < e)) ? 1 : 0;
      cnt += (o.y > v || (o.y == v && b + 1 < e)) ? 1 : 0;
      cnt += (o.z > v || (o.z == v && b + 2 < e)) ? 1 : 0;
      cnt += (o.w > v || (o.w == v && b + 3 < e)) ? 1 : 0;
    }
  }
  if (split == 2) cnt += __shfl_xor(cnt, 1, kWave);
  if (e < E && h == 0 && cnt < k) {
    s_idx[cnt] = e;
    s_val[cnt] = s_l[e];
  }
  __syncthreads();
  if (tid < kWave) {
    const float m = s_val[0];
    const float ex = tid < k ? expf(s_val[tid] - m) : 0.0f;
    const float sum = wave_sum(ex);
    if (tid < k) {
      idx_out[tid] = s_idx[tid];
      w_out[tid] = ex / sum;
    }
  }
  __syncthreads();
}

// 1 / sqrt(mean(x^2) + eps) of one row, by one wave.
__device__ float wave_rinv(const float* x, int d, float eps) {
  const int lane = threadIdx.x % kWave;
  const float4* x4 = reinterpret_cast<const float4*>(x);
  float s = 0.0f;
  for (int i = lane; i < d / 4; i += kWave) {
    float4 a = x4[i];
    s += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
  }
  s = wave_sum(s);
  return 1.0f / sqrtf(s / (float)d + eps);
}

// Fused path for T <= kSmallT and d <= 4096: every wave computes one expert's
// logit for all tokens, with all of its loads issued before any arithmetic
// (one memory round trip); the last workgroup to finish runs top-k.
// Workgroup 0 also writes h.
constexpr int kMaxV = 16;  // float4 per lane per row (d <= 64 * 4 * 16)

__global__ __launch_bounds__(kRouteWaves * kWave) void k_route_small(
    const float* __restrict__ x, const float* __restrict__ norm_w, float eps,
    const float* __restrict__ router_w, const float* __restrict__ router_bias, int T, int d, int E,
    int k, float* __restrict__ h_out, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ logits, uint32_t* __restrict__ counter) {
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int e = min(blockIdx.x * kRouteWaves + wave, E - 1);
  const bool has_e = blockIdx.x * kRouteWaves + wave < E;
  __shared__ uint32_t s_ticket;
  const int n4 = d / 4;
  const float4* w4 = reinterpret_cast<const float4*>(router_w + (size_t)e * d);
  const float4* nw4 = reinterpret_cast<const float4*>(norm_w);
  float4 wv[kMaxV], nv[kMaxV];
#pragma unroll
  for (int i = 0; i < kMaxV; ++i) {
    const int fi = lane + kWave * i;
    if (fi < n4) {
      wv[i] = w4[fi];
      nv[i] = norm_w ? nw4[fi] : make_float4(1.f, 1.f, 1.f, 1.f);
    }
  }
  const float bias = router_bias ? router_bias[e] : 0.0f;
  for (int t = 0; t < T; ++t) {
    const float4* x4 = reinterpret_cast<const float4*>(x + (size_t)t * d);
    float4 xv[kMaxV];
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxV; ++i) {
      const int fi = lane + kWave * i;
      if (fi < n4) {
        xv[i] = x4[fi];
        ss += xv[i].x * xv[i].x + xv[i].y * xv[i].y + xv[i].z * xv[i].z + xv[i].w * xv[i].w;
      }
    }
    const float rinv = norm_w ? 1.0f / sqrtf(wave_sum(ss) / (float)d + eps) : 1.0f;
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxV; ++i) {
      const int fi = lane + kWave * i;
      if (fi < n4) {
        float4 a = xv[i];
        if (norm_w) {
          a.x = a.x * rinv * nv[i].x; a.y = a.y * rinv * nv[i].y;
          a.z = a.z * rinv * nv[i].z; a.w = a.w * rinv * nv[i].w;
        }
        xv[i] = a;
        acc += a.x * wv[i].x + a.y * wv[i].y + a.z * wv[i].z + a.w * wv[i].w;
      }
    }
    acc = wave_sum(acc);
    if (has_e && lane == 0) store_coherent(logits + (size_t)t * E + e, acc + bias);
    if (blockIdx.x == 0 && wave == (t % kRouteWaves)) {
      float4* h4 = reinterpret_cast<float4*>(h_out + (size_t)t * d);
#pragma unroll
      for (int i = 0; i < kMaxV; ++i) {
        const int fi = lane + kWave * i;
        if (fi < n4) h4[fi] = xv[i];
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    s_ticket = arrive(counter);
  }
  __syncthreads();
  if (s_ticket != gridDim.x - 1) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  for (int t = 0; t < T; ++t)
    block_topk(logits + (size_t)t * E, E, k, topk_idx + (size_t)t * k, topk_w + (size_t)t * k);
  if (threadIdx.x == 0) reset_counter(counter);
}

// ---- larger T: fp32 MFMA router GEMM (split-K), then norm factor + top-k per token

// Router GEMM for many tokens on fp32 MFMA: logits = (x * w) . Wr^T, the
// RMSNorm's 1/rms factor applied per token afterwards (by k_topk, which also
// writes h).  Workgroup = NSUB MFMA row tiles of 16 tokens (2 for many
// tokens, 1 for few, so that enough workgroups exist) x all experts x one K
// slice; wave w owns expert blocks w, w+4, ... (16 experts each).
// Each lane holds 4 consecutive columns of two token rows and of one expert
// row per 16-column chunk and feeds them to v_mfma_f32_16x16x4f32, column j
// of each group of 4 in MFMA j; every router load serves all NSUB token tiles.
// Partial logits of K slice ks go to partial[ks][t][e]; the top-k kernel adds
// the slices in order, so the sums do not depend on scheduling.
constexpr int kRWaves = 4;
// At most 32 K slices: with few tokens a workgroup then loads 6 chunks of 16
// columns (d = 2816) instead of 11, two of them in flight at a time, and the
// router's time is that chain of load round trips (16 slices at 32 tokens:
// 2% slower for the batched step).
constexpr int kMaxSlices = 32;

// token tiles of 16 per workgroup
inline int router_nsub(int T) { return T > 256 ? 2 : 1; }

struct RouterSplit {
  int slices, kslice;
};
inline RouterSplit router_split(int T, int d) {
  const int rt = 16 * router_nsub(T);
  const int tiles = (T + rt - 1) / rt;
  int ks = (512 + tiles - 1) / tiles;  // ~2 workgroups per compute unit
  ks = ks < 1 ? 1 : (ks > kMaxSlices ? kMaxSlices : ks);
  int kslice = (d + ks - 1) / ks;
  kslice = (kslice + 15) / 16 * 16;
  return RouterSplit{(d + kslice - 1) / kslice, kslice};
}

template <int NSUB>
__global__ __launch_bounds__(kRWaves * kWave) void k_router_mfma(const float* __restrict__ x,
                                                                 const float* __restrict__ norm_w,
                                                                 const float* __restrict__ router_w, int T,
                                                                 int d, int E, int kslice,
                                                                 float* __restrict__ partial) {
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int tn = lane % 16, kq = lane / 16;
  const int t0 = blockIdx.x * 16 * NSUB, ks = blockIdx.y;
  const int k_begin = ks * kslice, k_end = min(d, k_begin + kslice);
  const int nb = (E + 15) / 16;
  const float* hrow[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) hrow[s] = x + (size_t)min(t0 + 16 * s + tn, T - 1) * d + kq * 4;
  const float* nrow = norm_w ? norm_w + kq * 4 : nullptr;
  const float* wrow[4];
  bool eok[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int e = (w + b * kRWaves) * 16 + tn;
    eok[b] = (w + b * kRWaves) < nb && e < E;
    wrow[b] = router_w + (size_t)(eok[b] ? e : 0) * d + kq * 4;
  }
  floatx4r acc[NSUB][4];
#pragma unroll
  for (int s = 0; s < NSUB; ++s)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[s][b] = floatx4r{0.f, 0.f, 0.f, 0.f};
  // chunks of 16 columns, loaded two ahead of their MFMAs
  struct Chunk {
    float4 a[NSUB], n, b[4];
  };
  auto load = [&](Chunk& c, int k0) {
#pragma unroll
    for (int s = 0; s < NSUB; ++s) c.a[s] = *reinterpret_cast<const float4*>(hrow[s] + k0);
    c.n = nrow ? *reinterpret_cast<const float4*>(nrow + k0) : make_float4(1.f, 1.f, 1.f, 1.f);
#pragma unroll
    for (int b = 0; b < 4; ++b)
      if (w + b * kRWaves < nb) c.b[b] = *reinterpret_cast<const float4*>(wrow[b] + k0);
  };
  auto mma = [&](const Chunk& c) {
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      const float av[4] = {c.a[s].x * c.n.x, c.a[s].y * c.n.y, c.a[s].z * c.n.z, c.a[s].w * c.n.w};
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if (w + b * kRWaves >= nb) continue;  // wave-uniform
        const float bv[4] = {c.b[b].x, c.b[b].y, c.b[b].z, c.b[b].w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[s][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j], bv[j], acc[s][b], 0, 0, 0);
      }
    }
  };
  Chunk c0, c1, c2;
  if (k_begin < k_end) load(c0, k_begin);
  if (k_begin + 16 < k_end) load(c1, k_begin + 16);
  for (int k0 = k_begin; k0 < k_end; k0 += 48) {
    if (k0 + 32 < k_end) load(c2, k0 + 32);
    mma(c0);
    if (k0 + 16 >= k_end) break;
    if (k0 + 48 < k_end) load(c0, k0 + 48);
    mma(c1);
    if (k0 + 32 >= k_end) break;
    if (k0 + 64 < k_end) load(c1, k0 + 64);
    mma(c2);
  }
  // lane holds C[token 16 s + kq*4 + i][expert tn] of each block
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    if (w + b * kRWaves >= nb || !eok[b]) continue;
    const int e = (w + b * kRWaves) * 16 + tn;
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tt = t0 + 16 * s + kq * 4 + i;
        if (tt < T) partial[((size_t)ks * T + tt) * E + e] = acc[s][b][i];
      }
  }
}

// Per token (one wave, one workgroup): the RMSNorm factor
// r = 1/sqrt(mean(x^2) + eps) from the token's row, logits = r * (sum of the
// K-slice partials in slice order) + bias, top-k and the renormalised weights,
// and h = x * r * w.  A wave issues ~100 vector memory instructions (16 slice
// partials per expert group, the row, the norm weights, the h stores); with one
// wave per workgroup the tokens spread over T compute units instead of T/4,
// whose instruction issue was the limit.
// MS: slices the kernel holds (>= slices): 16 unless there are more, since the
// partials' registers limit how many tokens' waves a SIMD holds.
template <int MS>
__global__ __launch_bounds__(kWave) void k_topk(const float* __restrict__ partial, int slices,
                                              const float* __restrict__ x, const float* __restrict__ norm_w,
                                              float eps, int d, const float* __restrict__ router_bias, int T,
                                              int E, int k, float* __restrict__ h_out,
                                              int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  const int lane = threadIdx.x;
  const int t = blockIdx.x;
  if (t >= T) return;
  // every slice's partial and the token's row go out before the first add (a
  // loop of dependent loads would pay one memory round trip per slice)
  float p[4][MS];
  bool ok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + kWave * i;
    ok[i] = e < E;
    if (kWave * i >= E) continue;  // wave-uniform: no expert of this lane group
    const int ec = min(e, E - 1);
#pragma unroll
    for (int s = 0; s < MS; ++s) p[i][s] = partial[((size_t)min(s, slices - 1) * T + t) * E + ec];
  }
  // the bias, and the token's row with its norm weights: all of it at once
  // when it fits in registers (none of these loads waits for the row's sum)
  float bv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) bv[i] = (router_bias && kWave * i < E) ? router_bias[min(lane + kWave * i, E - 1)] : 0.0f;
  const float4* x4 = reinterpret_cast<const float4*>(x + (size_t)t * d);
  const float4* n4 = reinterpret_cast<const float4*>(norm_w);
  const bool in_regs = d <= kWave * 4 * kMaxV;
  float4 xv[kMaxV], nv[kMaxV];
  float ss = 0.0f;
  if (in_regs) {
#pragma unroll
    for (int i = 0; i < kMaxV; ++i) {
      const int fi = lane + kWave * i;
      if (kWave * i < d / 4) {
        xv[i] = x4[min(fi, d / 4 - 1)];
        if (norm_w) nv[i] = n4[min(fi, d / 4 - 1)];
      }
    }
#pragma unroll
    for (int i = 0; i < kMaxV; ++i)
      if (kWave * i < d / 4 && lane + kWave * i < d / 4)
        ss += xv[i].x * xv[i].x + xv[i].y * xv[i].y + xv[i].z * xv[i].z + xv[i].w * xv[i].w;
  } else {
#pragma unroll 4
    for (int fi = lane; fi < d / 4; fi += kWave) {
      const float4 a = x4[fi];
      ss += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
    }
  }
  const float rinv = norm_w ? 1.0f / sqrtf(wave_sum(ss) / (float)d + eps) : 1.0f;
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float acc = 0.0f;
#pragma unroll
    for (int s = 0; s < MS; ++s)
      if (s < slices) acc += p[i][s];
    acc *= rinv;
    acc += bv[i];
    v[i] = ok[i] ? acc : 0.0f;
  }
  float4* h4 = reinterpret_cast<float4*>(h_out + (size_t)t * d);
  auto put = [&](int fi, float4 a, float4 n) {
    if (norm_w) {
      a.x = a.x * rinv * n.x; a.y = a.y * rinv * n.y;
      a.z = a.z * rinv * n.z; a.w = a.w * rinv * n.w;
    }
    h4[fi] = a;
  };
  if (in_regs) {
#pragma unroll
    for (int i = 0; i < kMaxV; ++i)
      if (lane + kWave * i < d / 4) put(lane + kWave * i, xv[i], norm_w ? nv[i] : xv[i]);
  } else {
#pragma unroll 4
    for (int fi = lane; fi < d / 4; fi += kWave) put(fi, x4[fi], norm_w ? n4[fi] : x4[fi]);
  }
  wave_topk_vals(v, ok, k, topk_idx + (size_t)t * k, topk_w + (size_t)t * k);
}

}  // namespace

size_t route_workspace_bytes(int T, int d, int E) {
  const size_t small = (size_t)T * E * sizeof(float);
  const size_t split = T > kSmallT ? (size_t)router_split(T, d).slices * T * E * sizeof(float) : 0;
  return 256 + (small > split ? small : split);
}

hipError_t launch_route(const float* x, const float* norm_w, float eps, const float* router_w,
                        const float* router_bias, int T, int d, int E, int k, float* h_out,
                        int32_t* topk_idx, float* topk_w, void* ws, hipStream_t s) {
  uint32_t* counter = reinterpret_cast<uint32_t*>(ws);
  float* logits = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + 256);
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  take_profile_events(MOE_CALL_ROUTE, &ev0, &ev1);
  if (T <= kSmallT && d <= kWave * 4 * kMaxV) {
    int grid = (E + kRouteWaves - 1) / kRouteWaves;
    launch_maybe_timed(k_route_small, grid, kRouteWaves * kWave, s, ev0, ev1, x, norm_w, eps, router_w,
                       router_bias, T, d, E, k, h_out, topk_idx, topk_w, logits, counter);
    return hipGetLastError();
  }
  const RouterSplit sp = router_split(T, d);
  const int rt = 16 * router_nsub(T);
  if (router_nsub(T) == 2)
    launch_maybe_timed2(k_router_mfma<2>, dim3((T + rt - 1) / rt, sp.slices), kRWaves * kWave, s, ev0, ev1, x,
                        norm_w, router_w, T, d, E, sp.kslice, logits);
  else
    launch_maybe_timed2(k_router_mfma<1>, dim3((T + rt - 1) / rt, sp.slices), kRWaves * kWave, s, ev0, ev1, x,
                        norm_w, router_w, T, d, E, sp.kslice, logits);
  if (sp.slices <= 16)
    hipLaunchKernelGGL(k_topk<16>, dim3(T), dim3(kWave), 0, s, logits, sp.slices, x, norm_w, eps, d, router_bias,
                       T, E, k, h_out, topk_idx, topk_w);
  else
    hipLaunchKernelGGL(k_topk<kMaxSlices>, dim3(T), dim3(kWave), 0, s, logits, sp.slices, x, norm_w, eps, d,
                       router_bias, T, E, k, h_out, topk_idx, topk_w);
  return hipGetLastError();
}

}  // namespace moe

// Scratch of moe_route_noalloc, for callers that cannot allocate: the route
// kernels' workspace (the fused small path's arrival counter in the first 256
// bytes, then the logits or the split-K partial logits).  One copy per GPU the
// library runs on, held until the process ends.  It is zero when the module
// loads and every launch of the small path leaves its counter at zero again
// (the split path uses no counter), so no call has to clear it.  In host code
// `scratch` only names the symbol: kernels get the device address from
// route_scratch().
static __device__ __align__(256) uint8_t scratch[moe::kRouteScratchBytes];

namespace moe {

// The device address of `scratch` on the current device, looked up with
// hipGetSymbolAddress the first time a device asks and kept per device.
hipError_t route_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  static std::mutex mu;
  static void* ptr[kMaxScratchDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return hipSuccess;
}

__global__ __launch_bounds__(256) void k_rms_rescale(const float* __restrict__ x, int T, int d,
                                                     float eps, float* __restrict__ out) {
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= T) return;
  const float* xt = x + (size_t)t * d;
  float rinv = wave_rinv(xt, d, eps);
  const float4* x4 = reinterpret_cast<const float4*>(xt);
  float4* o4 = reinterpret_cast<float4*>(out + (size_t)t * d);
  for (int i = lane; i < d / 4; i += kWave) {
    float4 a = x4[i];
    a.x *= rinv; a.y *= rinv; a.z *= rinv; a.w *= rinv;
    o4[i] = a;
  }
}

hipError_t launch_rms_rescale(const float* x, int T, int d, float eps, float* out, hipStream_t s) {
  hipLaunchKernelGGL(k_rms_rescale, dim3((T + 3) / 4), dim3(256), 0, s, x, T, d, eps, out);
  return hipGetLastError();
}

}  // namespace moe
