// Measurement hooks, built only into the measurement variant of the library
// (libmoe_measure.so), never into libmoe.so: kernels that read a known number
// of bytes with each of the load paths the hot kernels use, so that the HBM
// counters (rocprofv3 FETCH_SIZE) can be scaled per load path.
//   mode 0: 128-bit buffer loads into registers (the decode kernels' weights);
//   mode 1: LDS-DMA buffer loads (buffer_load ... lds: the grouped GEMM's
//           weight and activation tiles, the fused decode's router rows).
// Every byte of [src, src + bytes) is read exactly once; a per-workgroup sum
// is written to out so that the loads cannot be dropped.
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

}  // namespace
}  // namespace moe

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
