// Shared path with bf16 weights: the GEMV out[t][r] = sum_c W[r][c] h[t][c]
// (+ residual[t][r]), and the shared expert built from it.  It is the
// always-resident work the GPU runs while expert misses are copied in
// ("Optimizing a 14.3 GB model for an 8 GB machine", section "MoE needed
// parallel work, reuse, and coarse overlap": coarse overlap with the shared MLP;
// TurboFieldfare video transcript, paragraph on the two weight piles: one
// shared expert runs for every token).
// HBM-bound: one wave per row, 16-byte loads of 8 bf16 weights, fp32 FMA, wave
// reduction.  Up to 4 tokens share each weight load.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kSgTok = 4;

template <bool RESID>
__global__ __launch_bounds__(256) void k_shared_gemv_bf16(const uint16_t* __restrict__ w,
                                                          const float* __restrict__ h, int T,
                                                          int rows, int cols,
                                                          const float* __restrict__ residual,
                                                          float* __restrict__ out) {
  const int lane = threadIdx.x % kWave;
  const int r = blockIdx.x * 4 + threadIdx.x / kWave;
  if (r >= rows) return;
  const uint4* wr = reinterpret_cast<const uint4*>(w + (size_t)r * cols);
  const int n8 = cols / 8;
  for (int t0 = 0; t0 < T; t0 += kSgTok) {
    const int nt = min(kSgTok, T - t0);
    float acc[kSgTok] = {0.f, 0.f, 0.f, 0.f};
    for (int i = lane; i < n8; i += kWave) {
      const uint4 q = wr[i];
      const uint32_t u[4] = {q.x, q.y, q.z, q.w};
      float wv[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wv[2 * j] = __uint_as_float(u[j] << 16);
        wv[2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
      }
#pragma unroll
      for (int tt = 0; tt < kSgTok; ++tt) {
        if (tt < nt) {
          const float4* hx = reinterpret_cast<const float4*>(h + (size_t)(t0 + tt) * cols + i * 8);
          const float4 a = hx[0], b = hx[1];
          float s = acc[tt];
          s = fmaf(wv[0], a.x, s); s = fmaf(wv[1], a.y, s); s = fmaf(wv[2], a.z, s); s = fmaf(wv[3], a.w, s);
          s = fmaf(wv[4], b.x, s); s = fmaf(wv[5], b.y, s); s = fmaf(wv[6], b.z, s); s = fmaf(wv[7], b.w, s);
          acc[tt] = s;
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < kSgTok; ++tt) {
      float v = wave_sum(acc[tt]);
      if (tt < nt && lane == 0) {
        if (RESID) v = residual[(size_t)(t0 + tt) * rows + r] + v;
        out[(size_t)(t0 + tt) * rows + r] = v;
      }
    }
  }
}

// The shared expert's gate/up: wave c computes gate row c and up row f + c
// of w_gu [2f][cols] against the same activation loads, then
// act[t][c] = gelu_tanh(gate) * up.
__global__ __launch_bounds__(256) void k_shared_gateup_bf16(const uint16_t* __restrict__ w,
                                                            const float* __restrict__ h, int T, int f,
                                                            int cols, float* __restrict__ act) {
  const int lane = threadIdx.x % kWave;
  const int c = blockIdx.x * 4 + threadIdx.x / kWave;
  if (c >= f) return;
  const uint4* wg = reinterpret_cast<const uint4*>(w + (size_t)c * cols);
  const uint4* wu = reinterpret_cast<const uint4*>(w + (size_t)(f + c) * cols);
  const int n8 = cols / 8;
  for (int t0 = 0; t0 < T; t0 += kSgTok) {
    const int nt = min(kSgTok, T - t0);
    float ag[kSgTok] = {0.f, 0.f, 0.f, 0.f}, au[kSgTok] = {0.f, 0.f, 0.f, 0.f};
    for (int i = lane; i < n8; i += kWave) {
      const uint4 qg = wg[i], qu = wu[i];
      const uint32_t ug[4] = {qg.x, qg.y, qg.z, qg.w}, uu[4] = {qu.x, qu.y, qu.z, qu.w};
      float gv[8], uv[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        gv[2 * j] = __uint_as_float(ug[j] << 16);
        gv[2 * j + 1] = __uint_as_float(ug[j] & 0xffff0000u);
        uv[2 * j] = __uint_as_float(uu[j] << 16);
        uv[2 * j + 1] = __uint_as_float(uu[j] & 0xffff0000u);
      }
#pragma unroll
      for (int tt = 0; tt < kSgTok; ++tt) {
        if (tt < nt) {
          const float4* hx = reinterpret_cast<const float4*>(h + (size_t)(t0 + tt) * cols + i * 8);
          const float4 a = hx[0], b = hx[1];
          const float hv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
          float sg = ag[tt], su = au[tt];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            sg = fmaf(gv[j], hv[j], sg);
            su = fmaf(uv[j], hv[j], su);
          }
          ag[tt] = sg;
          au[tt] = su;
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < kSgTok; ++tt) {
      const float g = wave_sum(ag[tt]), u = wave_sum(au[tt]);
      if (tt < nt && lane == 0) act[(size_t)(t0 + tt) * f + c] = gelu_tanh(g) * u;
    }
  }
}

}  // namespace

size_t shared_expert_workspace_bytes(int T, int f_sh) { return (size_t)T * f_sh * 4; }

hipError_t launch_shared_expert_bf16(const uint16_t* w_gu, const uint16_t* w_down, const float* h,
                                     const float* residual, int T, int d, int f_sh, float* out, void* ws,
                                     hipStream_t s) {
  float* act = reinterpret_cast<float*>(ws);
  hipLaunchKernelGGL(k_shared_gateup_bf16, dim3((f_sh + 3) / 4), dim3(256), 0, s, w_gu, h, T, f_sh, d, act);
  if (residual)
    hipLaunchKernelGGL(k_shared_gemv_bf16<true>, dim3((d + 3) / 4), dim3(256), 0, s, w_down, act, T, d, f_sh,
                       residual, out);
  else
    hipLaunchKernelGGL(k_shared_gemv_bf16<false>, dim3((d + 3) / 4), dim3(256), 0, s, w_down, act, T, d, f_sh,
                       nullptr, out);
  return hipGetLastError();
}

hipError_t launch_shared_gemv_bf16(const uint16_t* w, const float* h, int T, int rows, int cols,
                                   float* out, hipStream_t s) {
  hipLaunchKernelGGL(k_shared_gemv_bf16<false>, dim3((rows + 3) / 4), dim3(256), 0, s, w, h, T, rows, cols, nullptr,
                     out);
  return hipGetLastError();
}

}  // namespace moe
