// Pair permutation: histogram of pairs per expert, exclusive scan, stable
// scatter.  Grouping all pairs of one expert lets the expert kernels read each
// expert's weights once for every token routed to it (the batched routed MoE of
// "Optimizing a 14.3 GB model for an 8 GB machine", section "Splitting the work
// improved attention and prefill").
//
// One workgroup of 1024 threads (16 waves).  Wave w owns a contiguous
// stretch of pair ids and walks it 64 at a time in ascending order: the lanes
// holding the same expert are found with ballots over the expert id bits, a
// lane's rank among them is a popcount, and a wave-private counter per expert
// in LDS gives each pair its position among the wave's pairs of that expert
// (kept in pair_pos meanwhile).  The waves' counts are then scanned per expert
// in wave order and over the experts, and a second walk writes every pair's
// final position: each bucket lists its pairs in ascending pair id, with no
// atomics.  Expert ids are loaded 16 rounds at a time, so each walk pays one
// memory round trip per 1024 pairs of its stretch.
//
// Many pairs (a prefill batch) with a workspace: two launches over chunks of
// 1024 pairs, one workgroup each.  k_perm_chunk ranks each pair among its
// chunk's pairs of the same expert (the same ballot matching, one round per
// wave) and writes the chunk's count per expert; k_perm_scatter sums, per
// expert, the counts of all chunks (the offsets) and of the chunks before its
// own (the chunk's base in the bucket), and writes the final positions.  The
// result is the one-workgroup kernel's, bit for bit: buckets list their pairs
// in ascending pair id.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / kWave;
constexpr int kMaxE = 256;
constexpr int kBatch = 16;  // rounds of 64 pairs whose ids are loaded together
constexpr int kChunk = kPermThreads;  // pairs per workgroup of the two-launch path
constexpr int kMaxChunks = 64;        // T*k <= 65536

// lanes whose expert id equals this lane's (invalid ids, -1, match only each other)
__device__ __forceinline__ uint64_t same_expert(int e) {
  uint64_t same = __ballot(e >= 0);
  if (e < 0) same = ~same;
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const uint64_t set = __ballot(e >= 0 && ((e >> b) & 1));
    same &= ((e >= 0) && ((e >> b) & 1)) ? set : ~set;
  }
  return same;
}

__global__ __launch_bounds__(kPermThreads) void k_permute(const int32_t* __restrict__ topk_idx,
                                                          int n_pairs, int E,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ sorted_pair,
                                                          int32_t* __restrict__ pair_pos) {
  __shared__ int s_cnt[kPermWaves][kMaxE];  // per wave and expert: count, then the wave's base
  __shared__ int s_base[kMaxE];             // per expert: first position of its bucket
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  for (int i = tid; i < kPermWaves * kMaxE; i += kPermThreads) (&s_cnt[0][0])[i] = 0;
  __syncthreads();
  const int seg = ((n_pairs + kPermWaves - 1) / kPermWaves + kWave - 1) / kWave * kWave;
  const int p0 = min(n_pairs, wave * seg), p1 = min(n_pairs, p0 + seg);
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  auto expert_of = [&](int v) { return (v >= 0 && v < E) ? v : -1; };

  // walk 1: position of each pair among its wave's pairs of the same expert.
  // When the wave's pairs fit one batch (every wave of a launch with at most
  // kBatch * kPermThreads pairs), walk 2 takes the experts and the positions
  // from registers instead of reloading them.
  const bool one = p1 - p0 <= kBatch * kWave;
  int k_e[kBatch], k_loc[kBatch];
  for (int b0 = p0; b0 < p1; b0 += kBatch * kWave) {
    int ids[kBatch];
#pragma unroll
    for (int r = 0; r < kBatch; ++r) ids[r] = topk_idx[min(b0 + r * kWave + lane, max(p1 - 1, 0))];
#pragma unroll
    for (int r = 0; r < kBatch; ++r) {
      const int p = b0 + r * kWave + lane;
      if (b0 + r * kWave >= p1) break;  // wave-uniform
      const int e = p < p1 ? expert_of(ids[r]) : -1;
      const uint64_t same = same_expert(e);
      const int rank = __popcll(same & lt_mask);
      int before = 0;
      if (e >= 0) before = s_cnt[wave][e];
      if (e >= 0 && rank == 0) s_cnt[wave][e] = before + __popcll(same);
      k_e[r] = e;
      k_loc[r] = e >= 0 ? before + rank : -1;
      if (p < p1 && (!one || e < 0)) pair_pos[p] = k_loc[r];
    }
  }
  __syncthreads();
  // per expert: the waves' counts become exclusive bases in wave order
  if (tid < E) {
    int run = 0;
    for (int w = 0; w < kPermWaves; ++w) {
      const int c = s_cnt[w][tid];
      s_cnt[w][tid] = run;
      run += c;
    }
    s_base[tid] = run;
  }
  __syncthreads();
  // exclusive scan of the counts over the experts (wave 0, 4 experts per lane)
  if (wave == 0) {
    int c[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane * 4 + i;
      c[i] = e < E ? s_base[e] : 0;
      sum += c[i];
    }
    int incl = sum;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int u = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += u;
    }
    int run = incl - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane * 4 + i;
      if (e < E) {
        s_base[e] = run;
        offsets[e] = run;
        counts[e] = c[i];
      }
      run += c[i];
    }
    if (lane == kWave - 1) offsets[E] = incl;
  }
  __syncthreads();
  // walk 2: final positions
  if (one) {
#pragma unroll
    for (int r = 0; r < kBatch; ++r) {
      const int p = p0 + r * kWave + lane;
      if (p0 + r * kWave >= p1) break;  // wave-uniform
      const int e = k_e[r];             // -1 past p1
      if (e >= 0) {
        const int pos = s_base[e] + s_cnt[wave][e] + k_loc[r];
        sorted_pair[pos] = p;
        pair_pos[p] = pos;
      }
    }
    return;
  }
  for (int b0 = p0; b0 < p1; b0 += kBatch * kWave) {
    int ids[kBatch], loc[kBatch];
#pragma unroll
    for (int r = 0; r < kBatch; ++r) {
      const int p = min(b0 + r * kWave + lane, max(p1 - 1, 0));
      ids[r] = topk_idx[p];
      loc[r] = pair_pos[p];
    }
#pragma unroll
    for (int r = 0; r < kBatch; ++r) {
      const int p = b0 + r * kWave + lane;
      if (b0 + r * kWave >= p1) break;  // wave-uniform
      const int e = p < p1 ? expert_of(ids[r]) : -1;
      if (e >= 0) {
        const int pos = s_base[e] + s_cnt[wave][e] + loc[r];
        sorted_pair[pos] = p;
        pair_pos[p] = pos;
      }
    }
  }
}

// Chunk b = pairs b*kChunk .. +kChunk: each pair's rank among the chunk's pairs
// of its expert (to pair_pos), the chunk's count per expert (to chunk_cnt[b][e]).
__global__ __launch_bounds__(kPermThreads) void k_perm_chunk(const int32_t* __restrict__ topk_idx, int n_pairs,
                                                             int E, int32_t* __restrict__ chunk_cnt,
                                                             int32_t* __restrict__ pair_pos) {
  __shared__ int s_cnt[kPermWaves][kMaxE];  // per wave and expert: count, then the wave's base
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  for (int i = tid; i < kPermWaves * kMaxE; i += kPermThreads) (&s_cnt[0][0])[i] = 0;
  const int p = (int)blockIdx.x * kChunk + tid;
  const int v = p < n_pairs ? topk_idx[p] : -1;
  const int e = (v >= 0 && v < E) ? v : -1;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const uint64_t same = same_expert(e);
  const int rank = __popcll(same & lt_mask);
  __syncthreads();
  if (e >= 0 && rank == 0) s_cnt[wave][e] = __popcll(same);
  __syncthreads();
  // per expert: the waves' counts become exclusive bases in wave order
  if (tid < E) {
    int run = 0;
    for (int w = 0; w < kPermWaves; ++w) {
      const int c = s_cnt[w][tid];
      s_cnt[w][tid] = run;
      run += c;
    }
    chunk_cnt[(int64_t)blockIdx.x * E + tid] = run;
  }
  __syncthreads();
  if (p < n_pairs) pair_pos[p] = e >= 0 ? s_cnt[wave][e] + rank : -1;
}

// Chunk b: bucket bases from every chunk's counts, then final positions.
// Workgroup 0 also writes counts and offsets.
__global__ __launch_bounds__(kPermThreads) void k_perm_scatter(const int32_t* __restrict__ topk_idx, int n_pairs,
                                                               int E, int n_chunks,
                                                               const int32_t* __restrict__ chunk_cnt,
                                                               int32_t* __restrict__ counts,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ sorted_pair,
                                                               int32_t* __restrict__ pair_pos) {
  __shared__ int s_base[kMaxE];   // per expert: this chunk's first position in the bucket
  __shared__ int s_wsum[kMaxE / kWave];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int b = (int)blockIdx.x;
  // this thread's pair (requested first: the count sums below take a while)
  const int p = b * kChunk + tid;
  const int v = p < n_pairs ? topk_idx[p] : -1;
  const int loc = p < n_pairs ? pair_pos[p] : -1;
  int total = 0, before = 0;
  if (tid < E) {
    for (int c = 0; c < n_chunks; ++c) {
      const int n = chunk_cnt[(int64_t)c * E + tid];
      total += n;
      if (c < b) before += n;
    }
  }
  // exclusive scan of the totals over the experts (waves 0..3, then their sums)
  int incl = total;
  if (tid < kMaxE) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int u = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += u;
    }
    if (lane == kWave - 1) s_wsum[wave] = incl;
  }
  __syncthreads();
  if (tid < kMaxE) {
    int off = incl - total;
    for (int w = 0; w < wave; ++w) off += s_wsum[w];
    if (tid < E) {
      s_base[tid] = off + before;
      if (b == 0) {
        offsets[tid] = off;
        counts[tid] = total;
        if (tid == E - 1) offsets[E] = off + total;
      }
    }
  }
  __syncthreads();
  const int e = (v >= 0 && v < E) ? v : -1;
  if (p < n_pairs && e >= 0) {
    const int pos = s_base[e] + loc;
    sorted_pair[pos] = p;
    pair_pos[p] = pos;
  }
}

}  // namespace

size_t permute_workspace_bytes(int n_pairs, int E) {
  return n_pairs > kChunk ? (size_t)kMaxChunks * (size_t)E * sizeof(int32_t) : 0;
}

hipError_t launch_permute(const int32_t* topk_idx, int n_pairs, int E, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos, void* ws, size_t ws_bytes,
                          hipStream_t s) {
  if (E > kMaxE) return hipErrorInvalidValue;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  take_profile_events(MOE_CALL_PERMUTE, &ev0, &ev1);
  const int n_chunks = (n_pairs + kChunk - 1) / kChunk;
  if (n_chunks > 1 && n_chunks <= kMaxChunks && ws && ws_bytes >= permute_workspace_bytes(n_pairs, E)) {
    int32_t* chunk_cnt = static_cast<int32_t*>(ws);
    launch_maybe_timed(k_perm_chunk, n_chunks, kPermThreads, s, ev0, nullptr, topk_idx, n_pairs, E, chunk_cnt,
                       pair_pos);
    launch_maybe_timed(k_perm_scatter, n_chunks, kPermThreads, s, nullptr, ev1, topk_idx, n_pairs, E, n_chunks,
                       static_cast<const int32_t*>(chunk_cnt), counts, offsets, sorted_pair, pair_pos);
    return hipGetLastError();
  }
  launch_maybe_timed(k_permute, 1, kPermThreads, s, ev0, ev1, topk_idx, n_pairs, E, counts, offsets, sorted_pair,
                     pair_pos);
  return hipGetLastError();
}

}  // namespace moe
