// Grouped int4 GEMM on bf16 MFMA for batched prefill.
//
// With many tokens the routed experts are run as batched kernels over all the
// tokens routed to each expert ("Optimizing a 14.3 GB model for an 8 GB
// machine", section "Splitting the work improved attention and prefill": batched
// routed MoE), and the quantised weights go through the matrix hardware as small
// staged dequantised tiles that are thrown away after use (same section: staged
// affine tiles; a direct in-register int4 path was slower there).
//
// gfx950 design
//  * Work item = (expert, 128-row M tile of its sorted pairs) x one N tile.  A
//    one-workgroup scheduler orders experts by pair count, largest first, so the
//    Zipf-skewed big experts start early and the small ones fill the tail.
//  * Workgroup = 4 waves (2 x 2); each wave owns a 64 x 64 block of the 128 x 128
//    output tile = 4 x 4 v_mfma_f32_16x16x32_bf16 tiles, fp32 accumulate.
//  * K steps are one quantisation group (64 columns).  Per step a thread loads
//    64 bytes of activation rows (gathered through sorted_pair) and 16 bytes of
//    nibbles plus one (scale, bias) word; the weights are dequantised in fp32
//    (w = s*q + b, exact), rounded to bf16 and written to LDS.  Two LDS stages:
//    the next step's global loads are in flight while the current one feeds the
//    MFMAs.
//  * Gate/up tile = 64 gate rows + the same 64 up rows, so GELU(gate) * up is
//    computed in the epilogue from accumulators held by the same lane; the
//    activation is stored as bf16 for the down GEMM.  Down writes fp32 per-pair
//    outputs and the rank-ordered gather combine sums them.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// Operand element traits: bf16 (the specified format) or fp16 (three more
// mantissa bits at the same MFMA rate on gfx950).
template <typename ET>
struct Elem;
template <>
struct Elem<__bf16> {
  typedef bf16x8 V8;
  static __device__ __forceinline__ floatx4 mfma(V8 a, V8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Elem<_Float16> {
  typedef f16x8 V8;
  static __device__ __forceinline__ floatx4 mfma(V8 a, V8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDK = BK + 8;  // padded LDS row (bf16): 144 bytes
constexpr int kThreads = 256;

struct Work {
  int expert, m0;
};

// ------------------------------------------------------------------ schedule

__global__ __launch_bounds__(256) void k_mfma_schedule(const int32_t* __restrict__ offsets, int E, int n_pairs,
                                                       int2* __restrict__ work, int* __restrict__ n_work) {
  __shared__ int s_cnt[256];
  __shared__ int s_tiles_by_rank[256];
  __shared__ int s_base_by_rank[257];
  const int t = threadIdx.x;
  int cnt = 0;
  if (t < E) {
    const int a = max(0, min(offsets[t], n_pairs)), b = max(a, min(offsets[t + 1], n_pairs));
    cnt = b - a;
  }
  s_cnt[t] = t < E ? cnt : -1;
  __syncthreads();
  int rank = 0;
  if (t < E) {
    for (int e = 0; e < E; ++e) {
      const int c = s_cnt[e];
      rank += (c > cnt || (c == cnt && e < t)) ? 1 : 0;
    }
    s_tiles_by_rank[rank] = (cnt + BM - 1) / BM;
  }
  __syncthreads();
  if (t == 0) {
    int run = 0;
    for (int r = 0; r < E; ++r) {
      s_base_by_rank[r] = run;
      run += s_tiles_by_rank[r];
    }
    s_base_by_rank[E] = run;
    *n_work = run;
  }
  __syncthreads();
  if (t < E) {
    const int base = s_base_by_rank[rank];
    const int nt = (cnt + BM - 1) / BM;
    for (int i = 0; i < nt; ++i) work[base + i] = make_int2(t, i * BM);
  }
}

// ------------------------------------------------------------------ fp32 -> bf16

template <typename ET>
__global__ __launch_bounds__(256) void k_convert(const float* __restrict__ x, int64_t n4, ET* __restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  const float4 v = reinterpret_cast<const float4*>(x)[i];
  ET o[4] = {(ET)v.x, (ET)v.y, (ET)v.z, (ET)v.w};
  reinterpret_cast<uint2*>(y)[i] = *reinterpret_cast<const uint2*>(o);
}

// ------------------------------------------------------------------ shared pieces

struct MfmaArgs {
  const void* a_rows;     // gate/up: h as ET [T][d]; down: act as ET [T*k][f]
  int a_by_token;         // 1: A row = token of the pair (gate/up); 0: A row = pair (down)
  const int32_t* offsets;
  const int32_t* sorted_pair;
  const int32_t* slot_of_expert;
  int n_slots;
  const uint8_t* arena;
  int64_t slot_stride;
  int T, d, f, E, k;
  int K;                  // reduction length (d for gate/up, f for down)
  int64_t off_q0, off_q1, off_sb0, off_sb1;  // gate/up sections, or down in q0/sb0
  int NT;                 // N tiles
  const int2* work;
  const int* n_work;
  void* act_out;          // gate/up output [T*k][f] as ET
  float* pair_out;        // down output [T*k][d] fp32
};

// Dequantise 32 weights of one row (one 16-byte nibble chunk) with the row's
// (scale, bias) word into 4 x 16 bytes of ET, natural column order.
//  bf16: w = s*q + b in fp32 (exact for fp16 s, b), rounded to nearest-even bf16.
//  fp16: nibble pairs are masked into fp16 (1024 + q) (exact), 1024 is
//        subtracted (exact), then w = fma(q, s, b) rounds once; byte permutes
//        restore column order.  Packed 16-bit arithmetic: 19 ops per 8 weights.
template <typename ET>
__device__ __forceinline__ void dequant_chunk(uint4 q, uint32_t sb, uint4 out[4]);

template <>
__device__ __forceinline__ void dequant_chunk<_Float16>(uint4 q, uint32_t sb, uint4 out[4]) {
  const f16x2 s2 = __builtin_bit_cast(f16x2, (sb & 0xffffu) * 0x10001u);
  const f16x2 b2 = __builtin_bit_cast(f16x2, (sb >> 16) * 0x10001u);
  const f16x2 off = {(_Float16)1024.0f, (_Float16)1024.0f};
  const uint32_t m = 0x000F000Fu, M = 0x64006400u;
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t p[4];
    p[0] = (w[i] & m) | M;          // columns 0, 4 of the word
    p[1] = ((w[i] >> 4) & m) | M;   // 1, 5
    p[2] = ((w[i] >> 8) & m) | M;   // 2, 6
    p[3] = ((w[i] >> 12) & m) | M;  // 3, 7
    uint32_t v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f16x2 qq = __builtin_bit_cast(f16x2, p[j]) - off;
      v[j] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(qq, s2, b2));
    }
    // (c0,c4) (c1,c5) (c2,c6) (c3,c7) -> (c0,c1) (c2,c3) (c4,c5) (c6,c7)
    out[i] = make_uint4(__builtin_amdgcn_perm(v[1], v[0], 0x05040100u), __builtin_amdgcn_perm(v[3], v[2], 0x05040100u),
                        __builtin_amdgcn_perm(v[1], v[0], 0x07060302u), __builtin_amdgcn_perm(v[3], v[2], 0x07060302u));
  }
}

template <>
__device__ __forceinline__ void dequant_chunk<__bf16>(uint4 q, uint32_t sb, uint4 out[4]) {
  const float s = half_lo(sb), b = half_hi(sb);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    __bf16 v[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) v[n] = (__bf16)fmaf(s, (float)((w[i] >> (4 * n)) & 0xFu), b);
    out[i] = *reinterpret_cast<const uint4*>(v);
  }
}

// Row r of the B tile (128 weight rows) -> (matrix section, row index in the matrix)
struct BRow {
  int64_t q_off, sb_off;  // offsets of the row's tile start in the blob (row already added)
  bool valid;
};

// ------------------------------------------------------------------ the GEMM

// GATEUP = true: B rows 0..63 are gate rows of tile nt, 64..127 the same up rows;
// the epilogue writes bf16 gelu(gate) * up.  GATEUP = false: B rows are down rows
// nt*128 .. +127; the epilogue writes fp32 per-pair outputs.
template <typename ET, bool GATEUP>
__global__ __launch_bounds__(kThreads, 2) void k_grouped_mfma(MfmaArgs a) {
  typedef typename Elem<ET>::V8 V8;
  __shared__ __align__(16) ET sA[2][BM][LDK];
  __shared__ __align__(16) ET sB[2][BN][LDK];
  __shared__ int s_arow[BM];   // A row index (token or pair), -1 = padding
  __shared__ int s_pair[BM];
  const int t = threadIdx.x;
  const int wid = t / kWave, lane = t % kWave;
  const int nw = *a.n_work;
  const int wi = blockIdx.x / a.NT, nt = blockIdx.x % a.NT;
  if (wi >= nw) return;
  const int2 wk = a.work[wi];
  const int e = wk.x, m0 = wk.y;
  const int n_pairs = a.T * a.k;
  const int beg = max(0, min(a.offsets[e], n_pairs)), end = max(beg, min(a.offsets[e + 1], n_pairs));
  const int rows = max(0, min(BM, end - beg - m0));
  if (t < BM) {
    int p = -1;
    if (t < rows) {
      p = a.sorted_pair[beg + m0 + t];
      if (p < 0 || p >= n_pairs) p = -1;
    }
    s_pair[t] = p;
    s_arow[t] = p < 0 ? -1 : (a.a_by_token ? p / a.k : p);
  }
  // weights through the slot table; an absent expert gives NaN outputs
  const uint8_t* blob = nullptr;
  if (e >= 0 && e < a.E) {
    const int slot = a.slot_of_expert[e];
    if (slot >= 0 && slot < a.n_slots) blob = a.arena + (int64_t)slot * a.slot_stride;
  }
  const bool ok = blob != nullptr;
  if (!ok) blob = a.arena;
  __syncthreads();

  const int G = a.K / kGroup;  // K steps
  const int Nrows = GATEUP ? a.f : a.d;  // rows of the weight matrix
  // this thread's A load: row ar = t/2, 32 columns at (t%2)*32
  const int ar = t / 2, ah = t % 2;
  const int arow = s_arow[ar];
  const ET* a_src = reinterpret_cast<const ET*>(a.a_rows) + (int64_t)max(arow, 0) * a.K + ah * 32;
  // this thread's B load: row br = t%128 of the tile, chunk bc = t/128 of the step
  const int br = t % BN, bc = t / BN;
  int mrow;          // row in the weight matrix
  int64_t q_sec, sb_sec;
  if (GATEUP) {
    mrow = nt * 64 + (br % 64);
    q_sec = br < 64 ? a.off_q0 : a.off_q1;
    sb_sec = br < 64 ? a.off_sb0 : a.off_sb1;
  } else {
    mrow = nt * BN + br;
    q_sec = a.off_q0;
    sb_sec = a.off_sb0;
  }
  const bool brow_ok = mrow < Nrows;
  const int mrow_c = brow_ok ? mrow : Nrows - 1;
  const uint8_t* q_src = blob + q_sec + (int64_t)(mrow_c / kTileRows) * (kTileRows * a.K / 2) + (mrow_c % kTileRows) * 16;
  const uint8_t* sb_src = blob + sb_sec + (int64_t)(mrow_c / kTileRows) * (kTileRows * G * 4) + (mrow_c % kTileRows) * 4;

  uint4 ra[4], rq;
  uint32_t rsb;
  auto gload = [&](int ks) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ra[i] = arow >= 0 ? *reinterpret_cast<const uint4*>(a_src + ks * BK + i * 8) : make_uint4(0u, 0u, 0u, 0u);
    rq = *reinterpret_cast<const uint4*>(q_src + (int64_t)(2 * ks + bc) * 1024);
    rsb = *reinterpret_cast<const uint32_t*>(sb_src + (int64_t)ks * 256);
  };
  auto lstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(&sA[st][ar][ah * 32 + i * 8]) = ra[i];
    uint4 o[4];
    dequant_chunk<ET>(rq, brow_ok ? rsb : 0u, o);
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(&sB[st][br][bc * 32 + i * 8]) = o[i];
  };

  // wave tile: rows wm*64 .. +63 of the M tile; B rows per n-tile ni
  const int wm = wid % 2, wn = wid / 2;
  int brow_of[4];
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    if (GATEUP) brow_of[ni] = (ni < 2 ? 0 : 64) + wn * 32 + (ni % 2) * 16 + lane % 16;
    else brow_of[ni] = wn * 64 + ni * 16 + lane % 16;
  }
  floatx4 acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = floatx4{0.f, 0.f, 0.f, 0.f};

  gload(0);
  lstore(0);
  __syncthreads();
  for (int ks = 0; ks < G; ++ks) {
    const int st = ks & 1;
    if (ks + 1 < G) gload(ks + 1);
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      const int kc = kk * 32 + (lane / 16) * 8;
      V8 fa[4], fb[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        fa[mi] = *reinterpret_cast<const V8*>(&sA[st][wm * 64 + mi * 16 + lane % 16][kc]);
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) fb[ni] = *reinterpret_cast<const V8*>(&sB[st][brow_of[ni]][kc]);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = Elem<ET>::mfma(fa[mi], fb[ni], acc[mi][ni]);
    }
    if (ks + 1 < G) lstore(st ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds C[(lane/16)*4 + i][lane%16] of every 16x16 tile
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = wm * 64 + mi * 16 + (lane / 16) * 4 + i;
      const int p = s_pair[m];
      if (p < 0) continue;
      if (GATEUP) {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const int col = nt * 64 + wn * 32 + ni * 16 + lane % 16;
          float g = acc[mi][ni][i], u = acc[mi][ni + 2][i];
          float v = gelu_tanh(g) * u;
          if (!ok) v = f32_nan();
          reinterpret_cast<ET*>(a.act_out)[(int64_t)p * a.f + col] = (ET)v;
        }
      } else {
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const int col = nt * BN + wn * 64 + ni * 16 + lane % 16;
          if (col < a.d) a.pair_out[(int64_t)p * a.d + col] = ok ? acc[mi][ni][i] : f32_nan();
        }
      }
    }
  }
}

}  // namespace

// ------------------------------------------------------------------ host side

static int max_work(int T, int k, int E) { return (T * k + BM - 1) / BM + E; }

size_t mfma_workspace_bytes(int call, int T, int d, int f, int E, int k) {
  size_t b = 256 + round256((int64_t)max_work(T, k, E) * 8);
  if (call == MOE_CALL_GATEUP) b += round256((int64_t)T * d * 2);  // activations in 16-bit
  else b += round256((int64_t)T * k * d * 4);
  return b;
}

static void carve(void* ws, int T, int k, int E, int** n_work, int2** work, char** rest) {
  char* c = reinterpret_cast<char*>(ws);
  *n_work = reinterpret_cast<int*>(c);
  *work = reinterpret_cast<int2*>(c + 256);
  *rest = c + 256 + round256((int64_t)max_work(T, k, E) * 8);
}

hipError_t launch_gateup_mfma(bool f16, const float* h, const int32_t* offsets, const int32_t* sorted_pair,
                              const int32_t* slot_of_expert, int n_slots, const uint8_t* arena, int64_t slot_stride,
                              int T, int d, int f, int E, int k, int64_t off_q0, int64_t off_q1, int64_t off_sb0,
                              int64_t off_sb1, void* act_out, void* ws, hipStream_t s) {
  int* n_work;
  int2* work;
  char* rest;
  carve(ws, T, k, E, &n_work, &work, &rest);
  const int64_t n4 = (int64_t)T * d / 4;
  if (f16)
    hipLaunchKernelGGL(k_convert<_Float16>, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, h, n4,
                       reinterpret_cast<_Float16*>(rest));
  else
    hipLaunchKernelGGL(k_convert<__bf16>, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, h, n4,
                       reinterpret_cast<__bf16*>(rest));
  hipLaunchKernelGGL(k_mfma_schedule, dim3(1), dim3(256), 0, s, offsets, E, T * k, work, n_work);
  MfmaArgs a{};
  a.a_rows = rest;
  a.a_by_token = 1;
  a.offsets = offsets;
  a.sorted_pair = sorted_pair;
  a.slot_of_expert = slot_of_expert;
  a.n_slots = n_slots;
  a.arena = arena;
  a.slot_stride = slot_stride;
  a.T = T; a.d = d; a.f = f; a.E = E; a.k = k;
  a.K = d;
  a.off_q0 = off_q0; a.off_q1 = off_q1; a.off_sb0 = off_sb0; a.off_sb1 = off_sb1;
  a.NT = f / 64;
  a.work = work;
  a.n_work = n_work;
  a.act_out = act_out;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  take_profile_events(MOE_CALL_GATEUP, &ev0, &ev1);
  if (f16)
    launch_maybe_timed(k_grouped_mfma<_Float16, true>, max_work(T, k, E) * a.NT, kThreads, s, ev0, ev1, a);
  else
    launch_maybe_timed(k_grouped_mfma<__bf16, true>, max_work(T, k, E) * a.NT, kThreads, s, ev0, ev1, a);
  return hipGetLastError();
}

hipError_t launch_down_mfma(bool f16, const void* act_in, const int32_t* offsets, const int32_t* sorted_pair,
                            const int32_t* slot_of_expert, int n_slots, const uint8_t* arena, int64_t slot_stride,
                            int T, int d, int f, int E, int k, int64_t off_q, int64_t off_sb, void* ws,
                            float** pair_out, hipStream_t s) {
  int* n_work;
  int2* work;
  char* rest;
  carve(ws, T, k, E, &n_work, &work, &rest);
  *pair_out = reinterpret_cast<float*>(rest);
  hipLaunchKernelGGL(k_mfma_schedule, dim3(1), dim3(256), 0, s, offsets, E, T * k, work, n_work);
  MfmaArgs a{};
  a.a_rows = act_in;
  a.a_by_token = 0;
  a.offsets = offsets;
  a.sorted_pair = sorted_pair;
  a.slot_of_expert = slot_of_expert;
  a.n_slots = n_slots;
  a.arena = arena;
  a.slot_stride = slot_stride;
  a.T = T; a.d = d; a.f = f; a.E = E; a.k = k;
  a.K = f;
  a.off_q0 = off_q; a.off_sb0 = off_sb;
  a.NT = (d + BN - 1) / BN;
  a.work = work;
  a.n_work = n_work;
  a.pair_out = *pair_out;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  take_profile_events(MOE_CALL_DOWN_COMBINE, &ev0, &ev1);
  if (f16)
    launch_maybe_timed(k_grouped_mfma<_Float16, false>, max_work(T, k, E) * a.NT, kThreads, s, ev0, ev1, a);
  else
    launch_maybe_timed(k_grouped_mfma<__bf16, false>, max_work(T, k, E) * a.NT, kThreads, s, ev0, ev1, a);
  return hipGetLastError();
}

}  // namespace moe
