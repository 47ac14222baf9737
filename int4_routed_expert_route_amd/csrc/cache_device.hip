// The bounded expert cache run on the device: the eviction rule of one layer
// step and the copies of its misses, with no host round trip.
//
// The pages keep a bounded set of experts per layer in preallocated slots,
// evict by use (LRU, then LFU) and read the misses explicitly into the freed
// slots ("Optimizing a 14.3 GB model for an 8 GB machine", sections "Explicit
// reads made expert streaming work" and "MoE needed parallel work, reuse, and
// coarse overlap").  There the host decides, because the reads come from a
// file.  On MI355X the pool is pinned host memory the GPU can read itself, so
// the rule runs in one wave right after the router, and a copy kernel pulls
// the misses over PCIe: a decode step then never waits for the host.
//
// The rule is the host cache's, step for step: every hit is stamped with the
// step; then each miss, in ascending expert id, takes for LRU the slot with
// the smallest (stamp, slot) (empty slots carry stamp -1), for LFU the lowest
// empty slot, else the slot not used in this step whose expert has the
// smallest (use count, stamp, slot), counts over every step so far.  The
// layer's state is worked on in LDS and written back at the end.
#include <algorithm>
#include <climits>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kCacheMax = 256;  // experts and slots per layer at most

struct Key {  // lexicographic (a, b, c); a = INT64_MAX excludes the slot
  int64_t a, b;
  int c;
};
__device__ __forceinline__ bool less(const Key& x, const Key& y) {
  return x.a != y.a ? x.a < y.a : (x.b != y.b ? x.b < y.b : x.c < y.c);
}
__device__ __forceinline__ Key shfl_key(const Key& k, int o) {
  Key r;
  r.a = __shfl_xor(k.a, o, kWave);
  r.b = __shfl_xor(k.b, o, kWave);
  r.c = __shfl_xor(k.c, o, kWave);
  return r;
}

__global__ __launch_bounds__(kWave) void k_cache_step(CacheStepArgs a) {
  __shared__ int s_se[kCacheMax];        // expert of each slot, -1 empty
  __shared__ int64_t s_st[kCacheMax];    // stamp of each slot, -1 never used
  __shared__ int64_t s_cnt[kCacheMax];   // use count of each expert (LFU)
  __shared__ int s_sel[kCacheMax];
  __shared__ int s_list[kCacheMax];      // misses in ascending expert id
  __shared__ int s_bad;
  const int lane = threadIdx.x;
  const int E = a.E, S = a.S, k = a.k;
  if (lane == 0) s_bad = 0;
  for (int s = lane; s < S; s += kWave) {
    s_se[s] = a.slot_expert[s];
    s_st[s] = a.stamp[s];
  }
  for (int e = lane; e < E; e += kWave) s_cnt[e] = a.policy == 1 ? a.count[e] : 0;
  for (int j = lane; j < k; j += kWave) {
    const int e = a.sel[j];
    s_sel[j] = e;
    if (e < 0 || e >= E) s_bad = 1;
  }
  __syncthreads();
  for (int j = lane; j < k; j += kWave)
    for (int i = 0; i < j; ++i)
      if (s_sel[i] == s_sel[j]) s_bad = 1;
  __syncthreads();
  if (s_bad) {  // a selection the rule cannot take: nothing changes
    if (lane == 0) __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int j = lane; j < k; j += kWave) a.hit_mask[j] = 0;
    if (lane == 0) *a.n_miss = 0;
    return;
  }
  // use counts (this step included), then stamp the hits
  if (a.policy == 1)
    for (int j = lane; j < k; j += kWave) s_cnt[s_sel[j]] += 1;
  __syncthreads();
  int hits = 0;
  for (int j = lane; j < k; j += kWave) {
    const int s = a.table[s_sel[j]];
    const bool hit = s >= 0 && s < S && s_se[s] == s_sel[j];
    a.hit_mask[j] = hit ? 1 : 0;
    if (hit) {
      s_st[s] = a.step;
      ++hits;
    }
  }
  // the misses in ascending expert id (rank by counting)
  for (int j = lane; j < k; j += kWave) {
    const int s = a.table[s_sel[j]];
    const bool miss = !(s >= 0 && s < S && s_se[s] == s_sel[j]);
    if (miss) {
      int r = 0;
      for (int i = 0; i < k; ++i) {
        const int si = a.table[s_sel[i]];
        const bool mi = !(si >= 0 && si < S && s_se[si] == s_sel[i]);
        r += (mi && s_sel[i] < s_sel[j]) ? 1 : 0;
      }
      s_list[r] = s_sel[j];
    }
  }
  hits = (int)wave_sum((float)hits);
  const int n_miss = k - hits;
  __syncthreads();
  for (int r = 0; r < n_miss; ++r) {
    const int e = s_list[r];
    Key best{INT64_MAX, INT64_MAX, INT32_MAX};
    for (int s = lane; s < S; s += kWave) {
      Key key;
      if (a.policy == 0) {
        key = Key{s_st[s], 0, s};
      } else if (s_se[s] < 0) {
        key = Key{-1, 0, s};  // empty slots first, lowest index
      } else if (s_st[s] == a.step) {
        key = Key{INT64_MAX, INT64_MAX, s};  // used in this step: never the victim
      } else {
        key = Key{s_cnt[s_se[s]], s_st[s], s};
      }
      if (less(key, best)) best = key;
    }
    for (int o = 1; o < kWave; o <<= 1) {
      const Key other = shfl_key(best, o);
      if (less(other, best)) best = other;
    }
    const int v = best.c;
    if (lane == 0) {
      const int old = s_se[v];
      if (old >= 0) a.table[old] = -1;
      a.table[e] = v;
      s_se[v] = e;
      s_st[v] = a.step;
      a.miss[2 * r] = e;
      a.miss[2 * r + 1] = v;
    }
    __syncthreads();
  }
  for (int s = lane; s < S; s += kWave) {
    a.slot_expert[s] = s_se[s];
    a.stamp[s] = s_st[s];
  }
  if (a.policy == 1)
    for (int j = lane; j < k; j += kWave) a.count[s_sel[j]] = s_cnt[s_sel[j]];
  if (lane == 0) {
    *a.n_miss = n_miss;
    a.stats[0] += hits;
    a.stats[1] += n_miss;
    a.stats[2] += (int64_t)n_miss * a.blob;
  }
}

// Copy i of the step's miss list: blob of expert miss[2i] from the pinned
// pool (device-mapped) into slot miss[2i + 1]; copies past n_miss do nothing.
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;
__global__ __launch_bounds__(kCopyThreads) void k_stage_misses(const uint8_t* pool_dev, uint8_t* arena, int E,
                                                               int S, int64_t blob, int64_t stride,
                                                               const int32_t* miss, const int32_t* n_miss) {
  const int i = blockIdx.y;
  if (i >= *n_miss) return;
  const int e = miss[2 * i], s = miss[2 * i + 1];
  if (e < 0 || e >= E || s < 0 || s >= S) return;
  const uint4* __restrict__ src = reinterpret_cast<const uint4*>(pool_dev + (int64_t)e * blob);
  uint4* __restrict__ dst = reinterpret_cast<uint4*>(arena + (int64_t)s * stride);
  const int64_t n16 = blob / 16;
  const int64_t step = (int64_t)gridDim.x * kCopyThreads;
  for (int64_t j0 = (int64_t)blockIdx.x * kCopyThreads + threadIdx.x; j0 < n16; j0 += step * kCopyUnroll) {
    uint4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u)
      if (j0 + u * step < n16) v[u] = src[j0 + u * step];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u)
      if (j0 + u * step < n16) dst[j0 + u * step] = v[u];
  }
}

}  // namespace

hipError_t launch_cache_step(const CacheStepArgs& a, hipStream_t s) {
  if (a.E < 1 || a.E > kCacheMax || a.S < 1 || a.S > kCacheMax || a.k < 1 || a.k > a.S) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_cache_step, dim3(1), dim3(kWave), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_stage_misses(const uint8_t* pool_dev, uint8_t* arena, int E, int S, int k, int64_t blob,
                               int64_t stride, const int32_t* miss, const int32_t* n_miss, hipStream_t s) {
  if (blob % 16) return hipErrorInvalidValue;
  const int64_t n16 = blob / 16;
  const int gx = (int)std::min<int64_t>(64, (n16 + kCopyThreads * kCopyUnroll - 1) / (kCopyThreads * kCopyUnroll));
  hipLaunchKernelGGL(k_stage_misses, dim3(std::max(gx, 1), k), dim3(kCopyThreads), 0, s, pool_dev, arena, E, S, blob,
                     stride, miss, n_miss);
  return hipGetLastError();
}

}  // namespace moe
