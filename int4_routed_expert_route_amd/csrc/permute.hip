// Pair permutation: histogram of pairs per expert, exclusive scan, stable
// scatter.  Grouping all pairs of one expert lets the expert kernels read each
// expert's weights once for every token routed to it (the batched routed MoE of
// "Optimizing a 14.3 GB model for an 8 GB machine", section "Splitting the work
// improved attention and prefill").
//
// One workgroup of 1024 threads.  Counts come from LDS atomics (order free);
// the scatter walks the pairs in ascending order, 1024 at a time: inside a wave
// the pairs with equal expert are found with ballots over the expert id bits,
// their rank is a popcount, and wave totals are scanned per expert in LDS, so
// every bucket lists its pairs in ascending pair id without ordered atomics.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / kWave;
constexpr int kMaxE = 256;

__global__ __launch_bounds__(kPermThreads) void k_permute(const int32_t* __restrict__ topk_idx,
                                                          int n_pairs, int E,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ sorted_pair,
                                                          int32_t* __restrict__ pair_pos) {
  __shared__ int s_count[kMaxE];
  __shared__ int s_base[kMaxE];
  __shared__ int s_wave[kPermWaves][kMaxE];
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  for (int e = tid; e < kMaxE; e += kPermThreads) s_count[e] = 0;
  __syncthreads();
  for (int p = tid; p < n_pairs; p += kPermThreads) {
    int e = topk_idx[p];
    if (e >= 0 && e < E) atomicAdd(&s_count[e], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      s_base[e] = run;
      offsets[e] = run;
      counts[e] = s_count[e];
      run += s_count[e];
    }
    offsets[E] = run;
  }
  __syncthreads();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = 0; base < n_pairs; base += kPermThreads) {
    for (int i = tid; i < kPermWaves * kMaxE; i += kPermThreads) (&s_wave[0][0])[i] = 0;
    __syncthreads();
    const int p = base + tid;
    int e = p < n_pairs ? topk_idx[p] : -1;
    if (e < 0 || e >= E) e = -1;
    // lanes holding the same expert id (invalid ids match only each other)
    uint64_t same = __ballot(e >= 0);
    if (e < 0) same = ~same;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint64_t set = __ballot(e >= 0 && ((e >> b) & 1));
      same &= ((e >= 0) && ((e >> b) & 1)) ? set : ~set;
    }
    const int rank = __popcll(same & lt_mask);
    if (e >= 0 && rank == 0) s_wave[wave][e] = __popcll(same);
    __syncthreads();
    // per expert: exclusive scan over the waves of this chunk
    for (int ee = tid; ee < E; ee += kPermThreads) {
      int run = s_base[ee];
      for (int w = 0; w < kPermWaves; ++w) {
        const int c = s_wave[w][ee];
        s_wave[w][ee] = run;
        run += c;
      }
      s_base[ee] = run;
    }
    __syncthreads();
    if (e >= 0) {
      const int pos = s_wave[wave][e] + rank;
      sorted_pair[pos] = p;
      pair_pos[p] = pos;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_permute(const int32_t* topk_idx, int n_pairs, int E, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos, hipStream_t s) {
  if (E > kMaxE) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_permute, dim3(1), dim3(kPermThreads), 0, s, topk_idx, n_pairs, E, counts,
                     offsets, sorted_pair, pair_pos);
  return hipGetLastError();
}

}  // namespace moe
