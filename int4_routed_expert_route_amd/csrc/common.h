// Internal helpers shared by the libmoe HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/libmoe.h"

namespace moe {

constexpr int kWave = 64;
constexpr int kGroup = 64;      // int4 affine group along the input dimension
constexpr int kTileRows = 64;   // rows per blob tile: one row per lane
constexpr int kChunkCols = 32;  // 16 bytes of nibbles

// Byte offsets of the six blob sections (see the blob format in libmoe.h).
struct BlobLayout {
  int64_t gate_q, up_q, down_q, gate_sb, up_sb, down_sb, total;
};

inline __host__ __device__ int64_t round256(int64_t v) { return (v + 255) / 256 * 256; }

inline __host__ BlobLayout blob_layout(int d, int f) {
  BlobLayout b;
  int64_t o = 0;
  b.gate_q = o;  o = round256(o + (int64_t)f * d / 2);
  b.up_q = o;    o = round256(o + (int64_t)f * d / 2);
  b.down_q = o;  o = round256(o + (int64_t)d * f / 2);
  b.gate_sb = o; o = round256(o + (int64_t)f * (d / kGroup) * 4);
  b.up_sb = o;   o = round256(o + (int64_t)f * (d / kGroup) * 4);
  b.down_sb = o; o = round256(o + (int64_t)d * (f / kGroup) * 4);
  b.total = o;
  return b;
}

// ---------------------------------------------------------------- numerics

__device__ __forceinline__ float half_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float half_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// tanh-form GELU in fp32.
__device__ __forceinline__ float gelu_tanh(float z) {
  const float k0 = 0.7978845608028654f;  // sqrt(2/pi)
  const float k1 = 0.044715f;
  return 0.5f * z * (1.0f + tanhf(k0 * (z + k1 * z * z * z)));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Sum over aligned groups of 16 lanes (lanes 16g..16g+15 end with the same value).
__device__ __forceinline__ float sum16(float v) {
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ int wave_bcast(int v, int lane) { return __shfl(v, lane, kWave); }

// Top-k keys: each (logit, expert) is one unsigned 64-bit key, larger for a
// larger logit and then for a lower id (the float's bits made monotone, then
// the complemented id), so "larger logit, ties to the lower id" is a plain
// integer maximum, reduced across a wave with DPP row operations.
__device__ __forceinline__ uint64_t topk_key(float v, int e) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v + 0.0f);  // + 0: -0 becomes +0
  const uint32_t mono = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)mono << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t k) {
  const uint32_t lo = (uint32_t)k, hi = (uint32_t)(k >> 32);
  // lanes the operation does not write keep their own key (the max identity)
  const uint32_t olo = (uint32_t)__builtin_amdgcn_update_dpp((int)lo, (int)lo, CTRL, ROW_MASK, 0xF, false);
  const uint32_t ohi = (uint32_t)__builtin_amdgcn_update_dpp((int)hi, (int)hi, CTRL, ROW_MASK, 0xF, false);
  const uint64_t o = ((uint64_t)ohi << 32) | olo;
  return o > k ? o : k;
}
// One DPP step of a sum: lanes the operation does not write add zero.
template <int CTRL, int ROW_MASK, typename T>
__device__ __forceinline__ T dpp_add_step(T v) {
  const int o = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false);
  return v + __builtin_bit_cast(T, o);
}
// Sum over aligned groups of 2, 4 or 8 lanes (n), every lane of a group ending
// with the group's sum: quad_perm [1,0,3,2], [2,3,0,1], then row_half_mirror.
template <typename T>
__device__ __forceinline__ T group_sum_dpp(T v, int n) {
  if (n >= 2) v = dpp_add_step<0xB1, 0xF>(v);
  if (n >= 4) v = dpp_add_step<0x4E, 0xF>(v);
  if (n >= 8) v = dpp_add_step<0x141, 0xF>(v);
  return v;
}
// Maximum over aligned groups of 8 lanes, in every lane of the group (lanes
// the operation does not write keep their own value, the identity).
template <int CTRL>
__device__ __forceinline__ float dpp_max_stepf(float v) {
  const int o = __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false);
  return fmaxf(v, __builtin_bit_cast(float, o));
}
__device__ __forceinline__ float group8_max_dpp(float v) {
  v = dpp_max_stepf<0xB1>(v);
  v = dpp_max_stepf<0x4E>(v);
  return dpp_max_stepf<0x141>(v);
}
// Sum over a fully active wave by DPP row operations in a fixed order (no LDS
// permutes): groups of 8, row_mirror for rows of 16, then row_bcast:15 and
// :31 leave the total in lane 63, which every lane reads back.
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v = group_sum_dpp(v, 8);
  v = dpp_add_step<0x140, 0xF>(v);
  v = dpp_add_step<0x142, 0xA>(v);
  v = dpp_add_step<0x143, 0xC>(v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
// Maximum of k over the wave, in every lane.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
  k = dpp_max_step<0xB1, 0xF>(k);   // quad_perm [1,0,3,2]
  k = dpp_max_step<0x4E, 0xF>(k);   // quad_perm [2,3,0,1]
  k = dpp_max_step<0x141, 0xF>(k);  // row_half_mirror
  k = dpp_max_step<0x140, 0xF>(k);  // row_mirror: every lane holds its row's maximum
  k = dpp_max_step<0x142, 0xA>(k);  // row_bcast:15 into rows 1 and 3
  k = dpp_max_step<0x143, 0xC>(k);  // row_bcast:31 into rows 2 and 3: lane 63 holds the maximum
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)k, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(k >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// The logit back from a key's monotone bits.
__device__ __forceinline__ float topk_key_value(uint64_t key) {
  const uint32_t mono = (uint32_t)(key >> 32);
  return __builtin_bit_cast(float, (mono & 0x80000000u) ? (mono & 0x7FFFFFFFu) : ~mono);
}
__device__ __forceinline__ int topk_key_expert(uint64_t key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }

__device__ __forceinline__ float f32_nan() { return __builtin_nanf(""); }

// Device-scope (all XCDs) release/acquire helpers for last-arriver reductions.
__device__ __forceinline__ void release_fence() { __atomic_thread_fence(__ATOMIC_RELEASE); }
__device__ __forceinline__ void acquire_fence() { __atomic_thread_fence(__ATOMIC_ACQUIRE); }

__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Arrival counter: returns the number of earlier arrivals (0-based ticket).
__device__ __forceinline__ uint32_t arrive(uint32_t* counter) {
  return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void reset_counter(uint32_t* counter) {
  __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Plain launch, or (when timing events are armed) a launch that records the
// events at the kernel's own begin and end.
template <typename Kernel, typename... Args>
inline void launch_maybe_timed(Kernel k, int grid, int block, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1,
                               Args... args) {
  if (ev0 || ev1)  // either may be null: a timed span over several launches
    hipExtLaunchKernelGGL(k, dim3(grid), dim3(block), 0, s, ev0, ev1, 0, args...);
  else
    hipLaunchKernelGGL(k, dim3(grid), dim3(block), 0, s, args...);
}

template <typename Kernel, typename... Args>
inline void launch_maybe_timed2(Kernel k, dim3 grid, int block, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1,
                                Args... args) {
  if (ev0 && ev1)
    hipExtLaunchKernelGGL(k, grid, dim3(block), 0, s, ev0, ev1, 0, args...);
  else
    hipLaunchKernelGGL(k, grid, dim3(block), 0, s, args...);
}

}  // namespace moe
