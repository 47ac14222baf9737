// Measurement hooks, built only into the measurement variant of the library
// (libmoe_measure.so), never into libmoe.so: kernels that read a known number
// of bytes with each of the load paths the hot kernels use, so that the HBM
// counters (rocprofv3 FETCH_SIZE) can be scaled per load path.
//   mode 0: 128-bit buffer loads into registers (the decode kernels' weights);
//   mode 1: LDS-DMA buffer loads (buffer_load ... lds: the grouped GEMM's
//           weight and activation tiles, the fused decode's router rows).
// Every byte of [src, src + bytes) is read exactly once; a per-workgroup sum
// is written to out so that the loads cannot be dropped.
// Also an issue probe: whether packed fp16 VALU work (the grouped GEMM's
// dequant arithmetic) runs alongside fp16 MFMAs on the same SIMD.
#include "common.h"

namespace moe {
namespace {

constexpr int kMThreads = 256;
constexpr int kMChunk = kMThreads * 16;  // bytes one workgroup reads per step

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__global__ __launch_bounds__(kMThreads) void k_read_vgpr(const uint8_t* src, int64_t bytes, uint32_t* out) {
  uint32_t acc = 0;
  const int64_t steps = bytes / kMChunk;
  for (int64_t s = blockIdx.x; s < steps; s += gridDim.x) {
    const int64_t off = s * kMChunk + threadIdx.x * 16;
    // 32-bit offsets: the source is re-based every 1 GiB of steps
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(src) + (off >> 30 << 30), (short)0, 0x7FFFFFFF, 0x00020000);
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    const u4 v = __builtin_amdgcn_raw_buffer_load_b128(rb, (int)(off & ((1 << 30) - 1)), 0, 0);
    acc += v.x ^ v.y ^ v.z ^ v.w;
  }
  out[blockIdx.x * kMThreads + threadIdx.x] = acc;
}

__global__ __launch_bounds__(kMThreads) void k_read_lds_dma(const uint8_t* src, int64_t bytes, uint32_t* out) {
  __shared__ uint4 stage[kMThreads];
  uint32_t acc = 0;
  const int64_t steps = bytes / kMChunk;
  for (int64_t s = blockIdx.x; s < steps; s += gridDim.x) {
    const int64_t base = s * kMChunk;
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(src) + (base >> 30 << 30), (short)0, 0x7FFFFFFF, 0x00020000);
    const int off = (int)(base & ((1 << 30) - 1)) + (int)threadIdx.x * 16;
    // each wave copies its 64 lanes x 16 bytes into its quarter of the stage
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(&stage[(threadIdx.x / kWave) * kWave]), 16, off, 0, 0,
                                             0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const uint4 v = stage[threadIdx.x];
    acc += v.x ^ v.y ^ v.z ^ v.w;
    __syncthreads();
  }
  out[blockIdx.x * kMThreads + threadIdx.x] = acc;
}

// Issue probe.  A workgroup of 8 waves, two per SIMD (waves w and w + 4
// share a SIMD when waves are dealt round-robin over the four).  Each MFMA
// step is 8 independent v_mfma_f32_16x16x32_f16; each VALU step is
// 8 * kValuPerMfma independent v_pk_fma_f16 (8 dependency chains).
//   mode 1: waves 0-3 run `iters` MFMA steps, waves 4-7 idle;
//   mode 2: waves 4-7 run `iters` VALU steps, waves 0-3 idle;
//   mode 3: both at once (one MFMA wave and one VALU wave per SIMD);
//   mode 4: every wave runs iters / 2 steps with the VALU ops between its
//           MFMAs (the same total work as mode 3, mixed inside each wave).
// Overlap shows as mode 3 (or 4) taking about the longer of modes 1 and 2;
// no overlap as about their sum.
constexpr int kValuPerMfma = 4;
typedef _Float16 f16x8p __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2p __attribute__((ext_vector_type(2)));
typedef float f32x4p __attribute__((ext_vector_type(4)));

template <int MODE>
__global__ __launch_bounds__(512) void k_issue_probe(float* out, int iters) {
  const int wave = threadIdx.x / kWave;
  f16x8p a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(threadIdx.x * 0.001f + i);
    b[i] = (_Float16)(i * 0.5f);
  }
  f32x4p c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = f32x4p{0.f, 0.f, 0.f, 0.f};
  f16x2p v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = f16x2p{(_Float16)(threadIdx.x * 0.01f), (_Float16)i};
  const f16x2p s = {(_Float16)0.999f, (_Float16)0.999f}, t = {(_Float16)0.001f, (_Float16)0.002f};
  const bool do_mfma = MODE == 4 || ((MODE & 1) && wave < 4);
  const bool do_valu = MODE == 4 || ((MODE & 2) && wave >= 4);
  const int n = MODE == 4 ? iters / 2 : iters;
  if (do_mfma && do_valu) {
    for (int it = 0; it < n; ++it) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        c[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c[i], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < kValuPerMfma; ++j) v[(i + j) % 8] = __builtin_elementwise_fma(v[(i + j) % 8], s, t);
      }
    }
  } else if (do_mfma) {
    for (int it = 0; it < n; ++it) {
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c[i], 0, 0, 0);
    }
  } else if (do_valu) {
    for (int it = 0; it < n; ++it) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < kValuPerMfma; ++j) v[(i + j) % 8] = __builtin_elementwise_fma(v[(i + j) % 8], s, t);
    }
  }
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) r += c[i][i % 4] + (float)v[i][0] + (float)v[i][1];
  out[blockIdx.x * blockDim.x + threadIdx.x] = r;
}

}  // namespace
}  // namespace moe

// Issue probe (modes above) over `groups` workgroups of 512 threads; out is
// device memory of groups * 512 floats.  Returns a hipError_t.
extern "C" int moe_debug_issue_probe(int mode, int groups, int iters, float* out, hipStream_t s) {
  if (!out || groups <= 0 || iters <= 0 || mode < 1 || mode > 4) return (int)hipErrorInvalidValue;
  if (mode == 1) hipLaunchKernelGGL(moe::k_issue_probe<1>, dim3(groups), dim3(512), 0, s, out, iters);
  if (mode == 2) hipLaunchKernelGGL(moe::k_issue_probe<2>, dim3(groups), dim3(512), 0, s, out, iters);
  if (mode == 3) hipLaunchKernelGGL(moe::k_issue_probe<3>, dim3(groups), dim3(512), 0, s, out, iters);
  if (mode == 4) hipLaunchKernelGGL(moe::k_issue_probe<4>, dim3(groups), dim3(512), 0, s, out, iters);
  return (int)hipGetLastError();
}

// Reads `bytes` (a multiple of 4096) of device memory once with load path
// `mode`; out is device memory of 1024 * 256 uint32.  Returns a hipError_t.
extern "C" int moe_debug_read(const void* src, int64_t bytes, int mode, uint32_t* out, hipStream_t s) {
  if (!src || !out || bytes <= 0 || bytes % moe::kMChunk || (mode != 0 && mode != 1)) return (int)hipErrorInvalidValue;
  const int grid = 1024;
  if (mode == 0)
    hipLaunchKernelGGL(moe::k_read_vgpr, dim3(grid), dim3(moe::kMThreads), 0, s, static_cast<const uint8_t*>(src),
                       bytes, out);
  else
    hipLaunchKernelGGL(moe::k_read_lds_dma, dim3(grid), dim3(moe::kMThreads), 0, s,
                       static_cast<const uint8_t*>(src), bytes, out);
  return (int)hipGetLastError();
}
