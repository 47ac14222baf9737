// Routing: RMSNorm, router matvec, softmax, top-k, renormalisation.
//
// The router is a small fp32 matrix that names k of E experts per token
// (TurboFieldfare video transcript, paragraphs on the router).  The choice is
// taken on fp32 logits: largest first, equal logits to the lower expert id; the
// weights are the softmax over all experts renormalised over the chosen ones,
// which equals the softmax over the chosen logits alone.
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

// Fused path for T <= kSmallT: every wave computes one expert's logit for all
// tokens; the last workgroup to finish runs top-k.  Workgroup 0 writes h.
__global__ __launch_bounds__(kRouteWaves * kWave) void k_route_small(
    const float* __restrict__ x, const float* __restrict__ norm_w, float eps,
    const float* __restrict__ router_w, const float* __restrict__ router_bias, int T, int d, int E,
    int k, float* __restrict__ h_out, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ logits, uint32_t* __restrict__ counter) {
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int e = blockIdx.x * kRouteWaves + wave;
  __shared__ uint32_t s_ticket;
  for (int t = 0; t < T; ++t) {
    const float* xt = x + (size_t)t * d;
    float rinv = norm_w ? wave_rinv(xt, d, eps) : 1.0f;
    if (e < E) {
      const float4* w4 = reinterpret_cast<const float4*>(router_w + (size_t)e * d);
      const float4* x4 = reinterpret_cast<const float4*>(xt);
      const float4* n4 = reinterpret_cast<const float4*>(norm_w);
      float acc = 0.0f;
      for (int i = lane; i < d / 4; i += kWave) {
        float4 a = x4[i];
        float4 b = w4[i];
        if (norm_w) {
          float4 n = n4[i];
          a.x = a.x * rinv * n.x; a.y = a.y * rinv * n.y;
          a.z = a.z * rinv * n.z; a.w = a.w * rinv * n.w;
        }
        acc += a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
      }
      acc = wave_sum(acc);
      if (lane == 0) {
        if (router_bias) acc += router_bias[e];
        store_coherent(logits + (size_t)t * E + e, acc);
      }
    }
    if (blockIdx.x == 0 && wave == (t % kRouteWaves)) {
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
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    release_fence();
    s_ticket = arrive(counter);
  }
  __syncthreads();
  if (s_ticket != gridDim.x - 1) return;
  acquire_fence();
  for (int t = wave; t < T; t += kRouteWaves)
    wave_topk(logits + (size_t)t * E, E, k, topk_idx + (size_t)t * k, topk_w + (size_t)t * k, true);
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
  if (T <= kSmallT) {
    int grid = (E + kRouteWaves - 1) / kRouteWaves;
    hipLaunchKernelGGL(k_route_small, dim3(grid), dim3(kRouteWaves * kWave), 0, s, x, norm_w, eps,
                       router_w, router_bias, T, d, E, k, h_out, topk_idx, topk_w, logits, counter);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_rmsnorm, dim3((T + 3) / 4), dim3(256), 0, s, x, norm_w, eps, T, d, h_out);
  hipLaunchKernelGGL(k_router_gemm, dim3((E + kGE - 1) / kGE, (T + kGT - 1) / kGT), dim3(256), 0, s,
                     h_out, router_w, router_bias, T, d, E, logits);
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
