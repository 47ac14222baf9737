// Routing: RMSNorm, router matvec, softmax, top-k, renormalisation.
//
// The router is a small fp32 matrix that names k of E experts per token
// (TurboFieldfare video transcript, paragraphs on the router).  The choice is
// taken on fp32 logits: largest first, equal logits to the lower expert id; the
// weights are the softmax over all experts renormalised over the chosen ones,
// which equals the softmax over the chosen logits alone.
#include <hip/hip_ext.h>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kSmallT = 8;         // fused single-launch path up to this many tokens
constexpr int kRouteWaves = 4;     // waves per workgroup in the fused path

// Top-k of one token's logits by one wave: k rounds of a wave-wide arg-max with
// (larger value, then lower id) order.  Writes idx/w for the token.
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
  // lane j keeps the j-th choice
  float my_v = 0.0f;
  int my_e = -1;
  for (int j = 0; j < k; ++j) {
    // lane-local best
    bool bok = false;
    float bv = 0.0f;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int e = lane + kWave * i;
      bool better = ok[i] && (!bok || v[i] > bv || (v[i] == bv && e < be));
      if (better) { bok = true; bv = v[i]; be = e; }
    }
    // wave butterfly
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      int ook = __shfl_xor((int)bok, o, kWave);
      float ov = __shfl_xor(bv, o, kWave);
      int oe = __shfl_xor(be, o, kWave);
      bool take = ook && (!bok || ov > bv || (ov == bv && oe < be));
      if (take) { bok = true; bv = ov; be = oe; }
    }
    if (lane == j) { my_v = bv; my_e = be; }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (lane + kWave * i == be) ok[i] = false;
  }
  const float m = __shfl(my_v, 0, kWave);
  const float ex = lane < k ? expf(my_v - m) : 0.0f;
  const float s = wave_sum(ex);
  if (lane < k) {
    idx_out[lane] = my_e;
    w_out[lane] = ex / s;
  }
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

// ---- larger T: norm, tiled fp32 router GEMM, then top-k

__global__ __launch_bounds__(256) void k_rmsnorm(const float* __restrict__ x,
                                                 const float* __restrict__ norm_w, float eps, int T,
                                                 int d, float* __restrict__ h_out) {
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= T) return;
  const float* xt = x + (size_t)t * d;
  float rinv = norm_w ? wave_rinv(xt, d, eps) : 1.0f;
  const float4* x4 = reinterpret_cast<const float4*>(xt);
  const float4* n4 = reinterpret_cast<const float4*>(norm_w);
  float4* h4 = reinterpret_cast<float4*>(h_out + (size_t)t * d);
  for (int i = lane; i < d / 4; i += kWave) {
    float4 a = x4[i];
    if (norm_w) {
      float4 n = n4[i];
      a.x = a.x * rinv * n.x; a.y = a.y * rinv * n.y;
      a.z = a.z * rinv * n.z; a.w = a.w * rinv * n.w;
    }
    h4[i] = a;
  }
}

// logits[T][E] = h[T][d] * Wr[E][d]^T (+ bias).  32x32 output tile per
// workgroup of 256 threads (2x2 outputs each), K staged through LDS 64 at a time.
constexpr int kGT = 32, kGE = 32, kGK = 64;

__global__ __launch_bounds__(256) void k_router_gemm(const float* __restrict__ h,
                                                     const float* __restrict__ router_w,
                                                     const float* __restrict__ router_bias, int T,
                                                     int d, int E, float* __restrict__ logits) {
  __shared__ float sh[kGT][kGK + 4];
  __shared__ float sw[kGE][kGK + 4];
  const int t0 = blockIdx.y * kGT, e0 = blockIdx.x * kGE;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;  // 16 x 16 threads, 2x2 each
  float acc[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
  for (int k0 = 0; k0 < d; k0 += kGK) {
    // load 32 rows x 64 cols of each operand: 512 float4 per operand, 2 per thread
    for (int i = threadIdx.x; i < kGT * kGK / 4; i += 256) {
      int r = i / (kGK / 4), c4 = i % (kGK / 4);
      int t = t0 + r, e = e0 + r;
      float4 a = t < T ? *reinterpret_cast<const float4*>(h + (size_t)t * d + k0 + c4 * 4)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
      float4 b = e < E ? *reinterpret_cast<const float4*>(router_w + (size_t)e * d + k0 + c4 * 4)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
      sh[r][c4 * 4 + 0] = a.x; sh[r][c4 * 4 + 1] = a.y; sh[r][c4 * 4 + 2] = a.z; sh[r][c4 * 4 + 3] = a.w;
      sw[r][c4 * 4 + 0] = b.x; sw[r][c4 * 4 + 1] = b.y; sw[r][c4 * 4 + 2] = b.z; sw[r][c4 * 4 + 3] = b.w;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < kGK; ++kk) {
      float a0 = sh[ty * 2 + 0][kk], a1 = sh[ty * 2 + 1][kk];
      float b0 = sw[tx * 2 + 0][kk], b1 = sw[tx * 2 + 1][kk];
      acc[0][0] += a0 * b0; acc[0][1] += a0 * b1;
      acc[1][0] += a1 * b0; acc[1][1] += a1 * b1;
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      int t = t0 + ty * 2 + i, e = e0 + tx * 2 + j;
      if (t < T && e < E) logits[(size_t)t * E + e] = acc[i][j] + (router_bias ? router_bias[e] : 0.f);
    }
}

__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int T, int E, int k,
                                              int32_t* __restrict__ topk_idx,
                                              float* __restrict__ topk_w) {
  const int t = blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= T) return;
  wave_topk(logits + (size_t)t * E, E, k, topk_idx + (size_t)t * k, topk_w + (size_t)t * k, false);
}

}  // namespace

size_t route_workspace_bytes(int T, int E) { return 256 + (size_t)T * E * sizeof(float); }

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
  hipLaunchKernelGGL(k_rmsnorm, dim3((T + 3) / 4), dim3(256), 0, s, x, norm_w, eps, T, d, h_out);
  if (ev0 && ev1)
    hipExtLaunchKernelGGL(k_router_gemm, dim3((E + kGE - 1) / kGE, (T + kGT - 1) / kGT), dim3(256), 0, s,
                          ev0, ev1, 0, h_out, router_w, router_bias, T, d, E, logits);
  else
    hipLaunchKernelGGL(k_router_gemm, dim3((E + kGE - 1) / kGE, (T + kGT - 1) / kGT), dim3(256), 0, s, h_out,
                       router_w, router_bias, T, d, E, logits);
  hipLaunchKernelGGL(k_topk, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, topk_idx, topk_w);
  return hipGetLastError();
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
