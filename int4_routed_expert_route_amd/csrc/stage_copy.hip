// Device-pulled staging of expert blobs: the GPU reads the pinned host pool
// itself, over PCIe, and writes each blob into its HBM slot.
//
// The pages read each miss explicitly into a preallocated slot and keep
// several reads in flight at once ("Optimizing a 14.3 GB model for an 8 GB
// machine", sections "Explicit reads made expert streaming work" and "MoE
// needed parallel work, reuse, and coarse overlap": bounded parallel reads).
// On MI355X one DMA copy per miss uses one copy engine; this kernel instead
// keeps many 16-byte PCIe reads in flight from every workgroup, for all the
// misses of a step in one launch.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;  // 16-byte loads in flight per thread

__global__ __launch_bounds__(kCopyThreads) void k_stage_copy(StageCopyArgs a) {
  const int i = blockIdx.y;  // copy index
  const uint4* __restrict__ src = reinterpret_cast<const uint4*>(a.src[i]);
  uint4* __restrict__ dst = reinterpret_cast<uint4*>(a.dst[i]);
  const int64_t n16 = a.bytes / 16;
  const int64_t stride = (int64_t)gridDim.x * kCopyThreads;
  for (int64_t j0 = (int64_t)blockIdx.x * kCopyThreads + threadIdx.x; j0 < n16; j0 += stride * kCopyUnroll) {
    uint4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u)
      if (j0 + u * stride < n16) v[u] = src[j0 + u * stride];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u)
      if (j0 + u * stride < n16) dst[j0 + u * stride] = v[u];
  }
}

}  // namespace

hipError_t launch_stage_copy(const StageCopyArgs& a, hipStream_t s) {
  if (a.n < 1 || a.n > kMaxStageCopies || a.bytes % 16) return hipErrorInvalidValue;
  // enough workgroups per copy for ~1 MB of reads in flight each
  const int64_t n16 = a.bytes / 16;
  const int gx = (int)std::min<int64_t>(64, (n16 + kCopyThreads * kCopyUnroll - 1) / (kCopyThreads * kCopyUnroll));
  hipLaunchKernelGGL(k_stage_copy, dim3(std::max(gx, 1), a.n), dim3(kCopyThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
