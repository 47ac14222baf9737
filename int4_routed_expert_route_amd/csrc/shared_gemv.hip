// Shared-path GEMV with bf16 weights, out[t][r] = sum_c W[r][c] h[t][c].
// It is the always-resident work the GPU runs while expert misses are copied in
// ("Optimizing a 14.3 GB model for an 8 GB machine", section "MoE needed
// parallel work, reuse, and coarse overlap": coarse overlap with the shared MLP).
// HBM-bound: one wave per row, 16-byte loads of 8 bf16 weights, fp32 FMA, wave
// reduction.  Up to 4 tokens share each weight load.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kSgTok = 4;

__global__ __launch_bounds__(256) void k_shared_gemv_bf16(const uint16_t* __restrict__ w,
                                                          const float* __restrict__ h, int T,
                                                          int rows, int cols,
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
      const float v = wave_sum(acc[tt]);
      if (tt < nt && lane == 0) out[(size_t)(t0 + tt) * rows + r] = v;
    }
  }
}

}  // namespace

hipError_t launch_shared_gemv_bf16(const uint16_t* w, const float* h, int T, int rows, int cols,
                                   float* out, hipStream_t s) {
  hipLaunchKernelGGL(k_shared_gemv_bf16, dim3((rows + 3) / 4), dim3(256), 0, s, w, h, T, rows, cols, out);
  return hipGetLastError();
}

}  // namespace moe
