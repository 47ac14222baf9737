// Grouped int4 GEMM on MFMA for batched prefill.
//
// With many tokens the routed experts run as batched kernels over all the
// tokens routed to each expert ("Optimizing a 14.3 GB model for an 8 GB
// machine", section "Splitting the work improved attention and prefill":
// batched routed MoE), and the quantised weights reach the matrix hardware as
// small dequantised tiles that are used once and thrown away (same section:
// staged affine tiles).
//
// gfx950 design
//  * Work item = (expert, 128-pair M tile, N tile).  The list orders experts
//    by pair count, largest first, and within an expert M tile by M tile its N
//    tiles; it is cut into 8 stretches of equal cost, one per XCD, so an
//    expert's weights and an M tile's activation rows are shared in one L2.
//    Every persistent workgroup derives the list in its prologue; workgroup j
//    of XCD x runs items j, j + grid/8, ... of stretch x.
//  * Workgroup = 4 waves side by side along N.  A wave owns all 128 M rows x 64
//    weight rows: 8 x 4 tiles of v_mfma_f32_16x16x32_f16, fp32 accumulate.
//  * K step = one quantisation group (64 columns), three steps in flight: per
//    step each wave copies, with LDS-DMA (buffer_load ... lds), its share of
//    the activation tile (only the 32-row blocks the tile's rows need, rows
//    gathered through sorted_pair) and its 64 weight rows' nibble chunks and
//    (scale, bias) words.  Waves read the tile with explicit ds_read and
//    dequantise the nibbles in registers (exact fp16 via the 1024-exponent
//    trick).  The K order inside each 8-column block is
//    (0,4,1,5,2,6,3,7), the order in which nibbles come out of a 32-bit word;
//    activations are stored in that order.
//  * Gate/up: a wave's 64 weight rows are 32 gate rows and the same 32 up
//    rows, so gelu(gate) * up is formed from accumulators held by one lane.
//  * fp16 results are block-scaled: one power-of-two exponent per row and
//    64-column group keeps the group's largest magnitude in [2^14, 2^15), so
//    nothing overflows fp16 whatever the activations' range.
//  * Operands are fp16, not bf16: the MFMA rate is the same, and bf16's 8-bit
//    significand, on weights whose group means are far from zero, misses the
//    1e-2 output tolerance by the cancellation of 2816-term sums.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 128;               // pair rows per work item
constexpr int kItemFixedCost = 8;     // schedule cost of an item beyond its row groups of 16
constexpr int WN = 64;                // weight rows per wave
constexpr int kWaves = 4;             // waves per workgroup, side by side along N
constexpr int BN = WN * kWaves;       // weight rows per workgroup
constexpr int BK = 64;                // K step = one quantisation group
constexpr int kThreads = kWaves * kWave;
constexpr int kMaxExp = 100;          // block exponents are clamped to [-kMaxExp, kMaxExp]
constexpr int kRsrcWord3 = 0x00020000;  // buffer resource word 3: raw 32-bit data, no swizzle
// Split-K: when a launch has fewer items than workgroups, items of at most
// kSplitRows rows are cut into up to kMaxSplit K ranges of at least
// kMinSplitSteps steps.  Each range's workgroup writes its fp32 accumulators
// to the workspace; the last to arrive sums them in range order and runs the
// epilogue (so the result does not depend on which arrives last).
constexpr int kSplitRows = 32;
constexpr int kMaxSplit = 4;
constexpr int kMinSplitSteps = 6;
constexpr int kMaxSplitItems = 512;      // items of a launch that splits (bounds the partials)
constexpr int kPartF4 = 8 * kThreads;     // partials per split item, in floatx4: 2 row groups x 4 x the lanes
constexpr int64_t kCntBytes = 2048;      // arrival counters, one per split item group
static_assert(kCntBytes >= kMaxSplitItems * 4, "one 32-bit arrival counter per split item");
constexpr int kSc1 = 16;                 // buffer op cache policy: device-coherent (write-through store)

// Position p inside an 8-column block holds column kSlot[p].
__host__ __device__ constexpr int slot_col(int p) { return (p & 1) ? 4 + (p >> 1) : (p >> 1); }

// ------------------------------------------------------------------ operand types

template <typename ET>
struct Op;

template <>
struct Op<_Float16> {
  typedef f16x8 V8;
  static __device__ __forceinline__ floatx4 mfma(V8 a, V8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  // One nibble word (columns 0..7 of a block) -> 8 weights in slot order.
  // A nibble pair at bits 0-3 / 16-19 masked under the fp16 exponent of 1024
  // reads 1024 + q; a pair at bits 4-7 / 20-23 under the exponent of 64 reads
  // 64 + q (its mantissa step is 1/16).  So one shift by 8 serves all four
  // pairs.  The offset is subtracted (exact) and w = fma(q, s, b) rounds once.
  // k holds the masks 0x000F000F, 0x00F000F0 and the exponents 0x64006400,
  // 0x54005400 in registers (a gfx9 VOP3 takes no literal).
  struct Consts {
    uint32_t m0, m4, e10, e6;
  };
  static __device__ __forceinline__ uint4 dequant8(uint32_t w, f16x2 s2, f16x2 b2, const Consts& k) {
    const f16x2 o10 = {(_Float16)1024.0f, (_Float16)1024.0f}, o6 = {(_Float16)64.0f, (_Float16)64.0f};
    const uint32_t t = w >> 8;
    const uint32_t p0 = (w & k.m0) | k.e10, p1 = (w & k.m4) | k.e6, p2 = (t & k.m0) | k.e10, p3 = (t & k.m4) | k.e6;
    uint4 v;
    v.x = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(f16x2, p0) - o10, s2, b2));
    v.y = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(f16x2, p1) - o6, s2, b2));
    v.z = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(f16x2, p2) - o10, s2, b2));
    v.w = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(f16x2, p3) - o6, s2, b2));
    return v;
  }
  // (scale, scale) and (bias, bias) of one (scale, bias) word
  static __device__ __forceinline__ void split_sb(uint32_t sb, f16x2& s2, f16x2& b2) {
    s2 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(sb, sb, 0x01000100u));
    b2 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(sb, sb, 0x03020302u));
  }
  static constexpr bool kScaled = true;
};

// tanh-form GELU for the 16-bit act tiles, with tanh(y) = 1 - 2 / (1 + e^{2y})
// on the hardware exp2 and reciprocal: absolute error of the tanh ~1e-7,
// far below the 16-bit act's rounding; e^{2y} overflowing gives exactly 1,
// underflowing exactly -1, as tanh saturates (|z| >= 10 gives g or 0 exactly).
__device__ __forceinline__ float gelu_tanh_act16(float z) {
  const float k0 = 0.7978845608028654f;  // sqrt(2/pi)
  const float k1 = 0.044715f;
  const float y = k0 * (z + k1 * z * z * z);
  const float e = __builtin_amdgcn_exp2f(y * 2.8853900817779268f);  // e^{2y} = 2^{2y log2 e}
  const float t = 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + e);
  return 0.5f * z * (1.0f + t);
}

// Block exponent for a group whose largest magnitude is m: m * 2^-e in [2^14, 2^15).
__device__ __forceinline__ int block_exp(float m) {
  if (!(m > 0.0f) || !(m <= 3.0e38f)) return 0;  // zero, NaN or inf: leave as is
  const int ex = (int)((__builtin_bit_cast(uint32_t, m) >> 23) & 0xffu) - 127 - 14;
  return ex < -kMaxExp ? -kMaxExp : (ex > kMaxExp ? kMaxExp : ex);
}
__device__ __forceinline__ float exp2i(int e) { return __builtin_bit_cast(float, (uint32_t)(127 + e) << 23); }

// ------------------------------------------------------------------ schedule

// Work list: experts by size class (row groups of 16, descending, capped at
// kClasses - 1; ties by id); per expert, M tile by M tile, its N tiles in order
// (the N tiles of one M tile share the activation rows; the expert's weights
// stay in L2 across its M tiles).  Item = (expert, m0, n tile).  The list is
// cut into 8 stretches of about equal cost, one per XCD; an item costs
// kItemFixedCost + (row groups of 16 in its M tile).  Timed per item on the
// 2048-token layer, a K step costs about the same whatever the rows (the
// dequant, the step barrier, the DMA round trip), so a one-group tile takes a
// bit over half as long as a full one: about 7 (gate/up) to 9 (down) row
// groups of fixed cost.  Swept on the prefill step: 4 fixed units 147k, 6:
// 156k, 8: 157k, 10: 156k, 16: 155k, 32: 149k tokens/s.  What remains is the
// whole-item granularity, about 3 items per workgroup per launch.
//
// Every workgroup of the GEMM derives the same list from the expert offsets
// at its start (a separate scheduling launch cost more than this): ranks from
// wave ballots over the size classes, block scans of items and cost over the
// ranks, and each XCD boundary in closed form from the rank whose cost range
// holds it (3.7 us from launch to the first item, against 7.7 us with ranks by
// counting).  Items are not stored: an item index maps to its rank by binary
// search over the ranks' first items.
constexpr int kClasses = 32;
struct Plan {
  int ecnt[256];    // expert of each rank | its pair count << 8 (pair counts < 2^24)
  int beg[256];     // each rank's first position in sorted_pair (offsets, clamped)
  int ibase[256];   // first item of each rank (the item count W for ranks without items)
  int xstart[9];    // first item of each XCD's stretch; xstart[8] = W
  int split;        // K ranges of each item of at most kSplitRows rows (1: no split)
};

// Called by all 256 threads; `scratch` (176 ints of LDS) is free until the
// caller's next barrier.  G = K steps; cap = most items a split launch may have.
__device__ void plan_items(const int32_t* __restrict__ offsets, int E, int n_pairs, int NT, int G, int cap,
                           int min_rows, int* scratch, Plan& pl) {
  int* s_wc = scratch;             // [4][kClasses] experts of each class, per wave
  int* s_above = scratch + 128;    // [kClasses] experts in larger classes
  int* s_red = scratch + 160;      // [2][4] per-wave item totals
  int* s_wsum = scratch + 168;     // [2][4] per-wave scan totals
  int* s_start = pl.xstart;
  const int t = threadIdx.x, lane = t % kWave, wv = t / kWave;
  int cnt = 0, a = 0, cls = -1;
  if (t < E) {
    a = max(0, min(offsets[t], n_pairs));
    const int b = max(a, min(offsets[t + 1], n_pairs));
    cnt = b - a < min_rows ? 0 : b - a;
    cls = kClasses - 1 - min(kClasses - 1, (cnt + 15) / 16);  // 0 = largest
  }
  if (t < 9) s_start[t] = -1;
  // rank = experts of earlier classes + experts of this class with smaller ids
  const uint64_t below = (1ull << lane) - 1ull;
  int pos = 0;
#pragma unroll 8
  for (int c = 0; c < kClasses; ++c) {
    const uint64_t m = __ballot(cls == c);
    if (cls == c) pos = __popcll(m & below);
    if (lane == 0) s_wc[wv * kClasses + c] = __popcll(m);
  }
  __syncthreads();
  if (t < kClasses) {
    const int n = s_wc[t] + s_wc[kClasses + t] + s_wc[2 * kClasses + t] + s_wc[3 * kClasses + t];
    int inc = n;  // inclusive prefix over classes 0..t
#pragma unroll
    for (int o = 1; o < kClasses; o <<= 1) {
      const int v = __shfl_up(inc, o, kClasses);
      if (t >= o) inc += v;
    }
    s_above[t] = inc - n;
  }
  __syncthreads();
  if (cls >= 0) {
    int rank = s_above[cls] + pos;
    for (int w = 0; w < wv; ++w) rank += s_wc[w * kClasses + cls];
    pl.ecnt[rank] = t | (cnt << 8);
    pl.beg[rank] = a;
  }
  __syncthreads();
  // rank r = t: its items (M tiles x NT) and their cost
  const int r = t;
  const int rc = r < E ? pl.ecnt[r] >> 8 : 0;
  const int mt = (rc + BM - 1) / BM;
  // the split: as many K ranges as the workgroups left idle by the unsplit
  // items allow, the same for every small item
  const bool small = rc > 0 && rc <= kSplitRows;
  int red_w = mt * NT, red_s = small ? NT : 0;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    red_w += __shfl_xor(red_w, o, kWave);
    red_s += __shfl_xor(red_s, o, kWave);
  }
  if (lane == 0) {
    s_red[wv] = red_w;
    s_red[4 + wv] = red_s;
  }
  __syncthreads();
  const int W1 = s_red[0] + s_red[1] + s_red[2] + s_red[3], Ws = s_red[4] + s_red[5] + s_red[6] + s_red[7];
  int S = 1;
  if (Ws > 0) S = max(1, min(min(kMaxSplit, G / kMinSplitSteps), (cap - (W1 - Ws)) / Ws));
  const int sr = small ? S : 1;
  const int ipt = NT * sr;  // items per M tile
  const int n_items = mt * ipt;
  const int full = rc / BM, tail = rc % BM;
  const int c_full = kItemFixedCost + BM / 16, c_tail = (kItemFixedCost + (tail + 15) / 16 + sr - 1) / sr;
  const int cost = ipt * (full * c_full + (tail ? c_tail : 0));
  int inc_i = n_items, inc_c = cost;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int ui = __shfl_up(inc_i, o, kWave), uc = __shfl_up(inc_c, o, kWave);
    if (lane >= o) {
      inc_i += ui;
      inc_c += uc;
    }
  }
  if (lane == kWave - 1) {
    s_wsum[wv] = inc_i;
    s_wsum[4 + wv] = inc_c;
  }
  __syncthreads();
  int base_i = inc_i - n_items, base_c = inc_c - cost, W = 0, total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int si = s_wsum[w], sc = s_wsum[4 + w];
    if (w < wv) {
      base_i += si;
      base_c += sc;
    }
    W += si;
    total += sc;
  }
  pl.ibase[r] = base_i;
  // XCD x starts at the first item whose cost before it is >= ceil(x * total / 8)
  // (item i belongs to XCD min(7, cost_before_i * 8 / total)); the rank whose
  // cost range holds that target finds the item: its full tiles' items come
  // first, c_full each, then the tail tile's, c_tail each
  if (n_items > 0) {
    const int fc = full * ipt * c_full;
    for (int x = 1; x < 8; ++x) {
      const int target = (x * total + 7) / 8;
      if (target < base_c || target >= base_c + cost) continue;
      const int off = target - base_c;
      const int li = off < fc ? (off + c_full - 1) / c_full : full * ipt + (off - fc + c_tail - 1) / c_tail;
      s_start[x] = base_i + min(li, n_items);
    }
  }
  if (t == 0) {
    s_start[0] = 0;
    pl.split = S;
  }
  __syncthreads();
  if (t < kWave) {
    // XCDs past the last boundary get empty stretches: each unset start takes
    // the next set one (W past the last); the set starts rise with x
    int v = W;
    if (t < 8 && s_start[t] >= 0) v = s_start[t];
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int u = __shfl_down(v, o, 16);
      if (t + o < 16) v = min(v, u);
    }
    if (t < 9) s_start[t] = v;
  }
  __syncthreads();
}

// h (fp32 [n8 * 8]) -> 16-bit, slot order inside each 8-column block.
template <typename ET>
__global__ __launch_bounds__(256) void k_h_to_slots(const float* __restrict__ x, int64_t n8, ET* __restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const float4 lo = reinterpret_cast<const float4*>(x)[2 * i];
  const float4 hi = reinterpret_cast<const float4*>(x)[2 * i + 1];
  const float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  ET o[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) o[p] = (ET)v[slot_col(p)];
  reinterpret_cast<uint4*>(y)[i] = *reinterpret_cast<const uint4*>(o);
}

// ------------------------------------------------------------------ the GEMM

struct GemmArgs {
  const void* a_rows;     // gate/up: h [T][d] in slot order; down: act values [T*k][f], natural order
  int a_bytes;            // bytes of a_rows (buffer loads are 32-bit addressed)
  const int8_t* a_exp;    // down: act exponents [T*k][f/64]
  int a_by_token;         // 1: A row = token of the pair (gate/up); 0: A row = pair (down)
  const int32_t* offsets;
  const int32_t* sorted_pair;
  const int32_t* slot_of_expert;
  int n_slots;
  const uint8_t* arena;
  int64_t slot_stride;
  int T, d, f, E, k;
  int K;                  // reduction length (d for gate/up, f for down)
  int NT;                 // N tiles
  int64_t off_q0, off_q1, off_sb0, off_sb1;  // gate/up sections, or down in q0/sb0
  void* out;              // gate/up: act values [T*k][f] (ET); down: pair values [T*k][d] fp16
  int8_t* out_exp;        // exponents [T*k][cols/64]
  floatx4* part;          // split items' partial accumulators [split_cap][kPartF4]
  uint32_t* cnt;          // arrival counters [split_cap], zero between launches
  int split_cap;          // most items a split launch may have (also capped by the grid)
  int min_rows;           // experts with fewer pairs are left to the few-pairs kernel
};

// LDS of one pipeline stage (one K step).
struct StageLds {
  uint4 a[BM * 8];             // activation tile: 128 rows x 8 chunks of 16 bytes, swizzled
  uint4 q[kWaves][2][WN];      // per wave: 2 nibble chunks x 64 weight rows x 16 bytes
  uint32_t sb[kWaves][WN];     // per wave: (scale, bias) of 64 weight rows
};
constexpr int kStages = 3;        // K steps in flight: DMA runs two steps ahead
// per wave and step: 1..4 activation loads (as many as the tile's rows need)
// + 2 nibble + 1 scale/bias loads
constexpr int kMaxSteps = 128;    // K steps (groups) a down GEMM may have: f <= 8192

// Chunk position of 16-byte chunk c in activation row r: c ^ swz(r % 16).  Any
// 8 (or 16) consecutive rows read at one chunk index hit distinct LDS banks.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Wait until this wave's loads for step s have landed: with one more step in
// flight, at most that step's n_a + 3 loads may still be outstanding.
__device__ __forceinline__ void vm_wait_steps(bool one_more_in_flight, int n_a) {
  // s_waitcnt vmcnt(N), expcnt and lgkmcnt left unconstrained (gfx9 encoding)
  constexpr int kRest = (0x7 << 4) | (0xF << 8);
  if (!one_more_in_flight) __builtin_amdgcn_s_waitcnt(kRest);
  else if (n_a == 1) __builtin_amdgcn_s_waitcnt(4 | kRest);
  else if (n_a == 2) __builtin_amdgcn_s_waitcnt(5 | kRest);
  else if (n_a == 3) __builtin_amdgcn_s_waitcnt(6 | kRest);
  else __builtin_amdgcn_s_waitcnt(7 | kRest);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
__device__ __forceinline__ lds_ptr_t to_lds(void* p) { return (lds_ptr_t)(p); }
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)(p);
}

// The work-list GEMM's LDS-DMA is written as asm, so that the compiler does not
// see it: it would otherwise make every later LDS read wait for every DMA in
// flight (it cannot tell the stages apart), which empties the pipeline.  Each
// K step waits for its own DMA explicitly (vm_wait_steps, then the barrier),
// and the LDS reads are ordinary loads whose waits the compiler places.  The
// asm sets M0 to the LDS address itself; nothing else in the kernel uses M0.
// rs: buffer resource words (SGPRs); lane l's bytes land at lds + l * size.
__device__ __forceinline__ void dma_lds16(u32x4 rs, uint32_t lds, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rs), "s"(soff)
               : "memory");
}
__device__ __forceinline__ void dma_lds4(u32x4 rs, uint32_t lds, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rs), "s"(soff)
               : "memory");
}
// Raw buffer resource words for `bytes` bytes at p (stride 0, raw 32-bit data).
__device__ __forceinline__ u32x4 rsrc_words(const void* p, int bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)p;
  u32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((uint32_t)b);
  r.y = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32) & 0xFFFFu);
  r.z = __builtin_amdgcn_readfirstlane((uint32_t)bytes);
  r.w = (uint32_t)kRsrcWord3;
  return r;
}
// Keeps the compiler from moving LDS reads above a step barrier.
__device__ __forceinline__ void lds_fence() { asm volatile("" ::: "memory"); }

template <typename T>
__device__ __forceinline__ T lds_load(uint32_t addr) {
  return *(const __attribute__((address_space(3))) T*)(uintptr_t)addr;
}
template <int OFF>
__device__ __forceinline__ u32x4 lds_read128(uint32_t addr) {
  return lds_load<u32x4>(addr + OFF);
}
template <int OFF>
__device__ __forceinline__ u32x2 lds_read64(uint32_t addr) {
  return lds_load<u32x2>(addr + OFF);
}
template <int OFF>
__device__ __forceinline__ uint32_t lds_read32(uint32_t addr) {
  return lds_load<uint32_t>(addr + OFF);
}

// GATEUP: wave w of N tile nt owns act columns nt*128 + 32w .. +31 (gate rows
// and up rows of those indices).  Down: wave w owns output rows nt*256 + 64w .. +63.
// Persistent: workgroup j of XCD x runs items xstart[x] + j, + gridDim/8, ...
// DIRECT (the ablation of the staged tile): each lane loads its weight
// nibbles and (scale, bias) words from memory straight into registers, one
// K step ahead, instead of taking them from an LDS stage; activations are
// staged as before.
// Item timeline (a build option for measurement, off in the library): with
// MOE_GEMM_TIMELINE defined, thread 0 of every workgroup records the global
// 100 MHz clock (s_memrealtime) at its start, when its plan is ready and at its
// end, its compute unit (__smid) with its item count, and per item (the first
// kGtItems): the item's start, its (item, rows, K ranges, K range) word, the first K step's barrier and the end of its K
// loop; moe_debug_gemm_timeline() copies the table of the last launch of each
// GEMM (gate/up, down) to the host.  The few-pairs kernel writes the same
// table (per round of its wave 0's item: start, (item, rows) word, K loop
// start, K loop end).
#ifdef MOE_GEMM_TIMELINE
constexpr int kGtGroups = 1024, kGtItems = 24, kGtRow = 4 + 4 * kGtItems;
__device__ uint64_t g_gemm_timeline[2][kGtGroups][kGtRow];
#define GEMM_TL(slot, value)                                                        \
  do {                                                                               \
    if (threadIdx.x == 0 && blockIdx.x < kGtGroups)                                  \
      g_gemm_timeline[GATEUP ? 0 : 1][blockIdx.x][(slot)] = (uint64_t)(value);       \
  } while (0)
#define GEMM_TL_ITEM(j, k, value)                                                   \
  do {                                                                               \
    if ((j) < kGtItems) GEMM_TL(4 + 4 * (j) + (k), value);                           \
  } while (0)
#define GEMM_TL_ON 1
#else
#define GEMM_TL(slot, value) \
  do {                       \
  } while (0)
#define GEMM_TL_ITEM(j, k, value) \
  do {                            \
  } while (0)
#define GEMM_TL_ON 0
#endif

template <typename ET, bool GATEUP, bool DIRECT>
__global__ __launch_bounds__(kThreads, 2) void k_q4_gemm(GemmArgs a) {
  typedef Op<ET> O;
  typedef typename O::V8 V8;
  constexpr bool kScaledA = !GATEUP && O::kScaled;  // down: block-scaled fp16 activations
  __shared__ StageLds lds[kStages];
  __shared__ int s_pair[BM];
  __shared__ float s_wmax[kWaves];
  __shared__ int s_gexp[kMaxSteps];  // down: tile exponent of each K group
  __shared__ int s_fix;              // down: some row's exponents differ from its tile's
  __shared__ Plan s_plan;
  __shared__ uint32_t s_ticket;
  const int t = threadIdx.x;
  GEMM_TL(0, __builtin_amdgcn_s_memrealtime());
  int tl_j = 0;  // items this workgroup has started (timeline build)
  const int wid = __builtin_amdgcn_readfirstlane(t / kWave), lane = t % kWave;
  const int n = lane % 16, kq = lane / 16;  // MFMA lane coordinates
  const int G = a.K / kGroup;               // K steps
  const int n_pairs = a.T * a.k;
  const int Nrows = GATEUP ? a.f : a.d;
  const u32x4 rwA = rsrc_words(a.a_rows, a.a_bytes);
  typename O::Consts kc{0x000F000Fu, 0x00F000F0u, 0x64006400u, 0x54005400u};
  asm volatile("" : "+v"(kc.m0), "+v"(kc.m4), "+v"(kc.e10), "+v"(kc.e6));  // in VGPRs
  // per-lane LDS addresses inside stage 0 (stage st adds st * sizeof(StageLds))
  const uint32_t lds0 = lds_addr(&lds[0]);
  const uint32_t a_rd0 = lds0 + n * 128 + (((kq * 2) ^ swz(n)) * 16);
  const uint32_t a_rd1 = lds0 + n * 128 + (((kq * 2 + 1) ^ swz(n)) * 16);
  const uint32_t q_rd = lds_addr(&lds[0].q[wid][kq >> 1][n]) + (kq & 1) * 8;
  const uint32_t sb_rd = lds_addr(&lds[0].sb[wid][n]);

  // the work list, in LDS (stage 0 of the pipeline serves as scratch)
  plan_items(a.offsets, a.E, n_pairs, a.NT, G, min(a.split_cap, (int)gridDim.x), a.min_rows,
             reinterpret_cast<int*>(&lds[0]), s_plan);
  GEMM_TL(1, __builtin_amdgcn_s_memrealtime());
  const int xcd = (int)(blockIdx.x % 8), nper = (int)(gridDim.x / 8);
  const int i_end = __builtin_amdgcn_readfirstlane(s_plan.xstart[xcd + 1]);
  for (int item = __builtin_amdgcn_readfirstlane(s_plan.xstart[xcd]) + (int)(blockIdx.x / 8); item < i_end;
       item += nper) {
    __syncthreads();  // the previous item's LDS (or the plan's scratch) is no longer in use
    GEMM_TL_ITEM(tl_j, 0, __builtin_amdgcn_s_memrealtime());
    // values the whole workgroup shares, made wave-uniform for the compiler
    int rk = 0;
    {
      int hi = a.E - 1;  // last rank whose first item is <= item
      while (rk < hi) {
        const int mid = (rk + hi + 1) / 2;
        if (s_plan.ibase[mid] <= item) rk = mid;
        else hi = mid - 1;
      }
    }
    const int li = __builtin_amdgcn_readfirstlane(item - s_plan.ibase[rk]);
    // the expert, its pair count and first position come from the plan in
    // LDS (no global round trip before the item's first load)
    const int ec = __builtin_amdgcn_readfirstlane(s_plan.ecnt[rk]);
    const int e = ec & 255;
    // item = (M tile, N tile, K range): K steps s0 .. s1 - 1
    const int sr = __builtin_amdgcn_readfirstlane((ec >> 8) <= kSplitRows ? s_plan.split : 1);
    const int tile = __builtin_amdgcn_readfirstlane(li / sr), ks = __builtin_amdgcn_readfirstlane(li - tile * sr);
    const int s0 = __builtin_amdgcn_readfirstlane(ks * G / sr), s1 = __builtin_amdgcn_readfirstlane((ks + 1) * G / sr);
    const int m0 = __builtin_amdgcn_readfirstlane((tile / a.NT) * BM);
    const int nt = __builtin_amdgcn_readfirstlane(tile % a.NT);
    const int beg = __builtin_amdgcn_readfirstlane(s_plan.beg[rk]);
    const int end = beg + (ec >> 8);
    const int rows = max(0, min(BM, end - beg - m0));
    GEMM_TL_ITEM(tl_j, 1, ((uint64_t)item << 32) | ((uint64_t)rows << 16) | (uint64_t)(sr << 8) | (uint64_t)ks);
    // weights through the slot table; an absent expert gives NaN outputs.
    // The slot is requested before the tile's pair ids, so the two loads
    // share one memory round trip.
    const int slot_ld = (e >= 0 && e < a.E) ? a.slot_of_expert[e] : -1;
    if (t < BM) {
      int p = -1;
      if (t < rows) {
        p = a.sorted_pair[beg + m0 + t];
        if (p < 0 || p >= n_pairs) p = -1;
      }
      s_pair[t] = p;
    }
    if (kScaledA && t == 0) s_fix = 0;
    const int slot = __builtin_amdgcn_readfirstlane(slot_ld);
    const bool ok = slot >= 0 && slot < a.n_slots;
    const uint8_t* blob = a.arena + (ok ? (int64_t)slot * a.slot_stride : 0);
    __syncthreads();

    // ---- DMA sources.  Activations: load i of wave w fills slots (4i + w)*64 + lane
    // = row (4i + w)*8 + lane/8, chunk position lane%8, so every wave issues
    // n_a = ceil(rows / 32) loads and rows past 32 n_a are not fetched (no
    // MFMA reads them).  Padding rows read row 0.
    const int n_a = __builtin_amdgcn_readfirstlane(min(4, max(1, (rows + 31) / 32)));
    int a_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (i * 4 + wid) * 8 + lane / 8;
      const int p = s_pair[r];
      const int arow = p < 0 ? 0 : (a.a_by_token ? p / a.k : p);
      a_off[i] = (arow * a.K + ((lane % 8) ^ swz(r % 16)) * 8) * 2;
    }
    // Weights: lane = weight row of the wave (gate/up: lanes 0..31 gate rows,
    // 32..63 the same up rows); ragged tiles read row 0 and discard it.
    const int wave_base = GATEUP ? nt * (BN / 2) + wid * (WN / 2) : nt * BN + wid * WN;
    const bool wave_ok = wave_base < Nrows;
    const __amdgpu_buffer_rsrc_t rsB =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(blob), (short)0, (int)a.slot_stride, kRsrcWord3);
    int q_off, sb_off;
    {
      const bool up = GATEUP && lane >= 32;
      int r = GATEUP ? wave_base + (lane & 31) : wave_base + lane;
      r = wave_ok ? r : 0;
      q_off = (int)((up ? a.off_q1 : a.off_q0) + (int64_t)(r / kTileRows) * (kTileRows * a.K / 2) +
                    (r % kTileRows) * 16);
      sb_off = (int)((up ? a.off_sb1 : a.off_sb0) + (int64_t)(r / kTileRows) * (kTileRows * G * 4) +
                     (r % kTileRows) * 4);
    }
    const u32x4 rwB = rsrc_words(blob, (int)a.slot_stride);
    auto issue = [&](int s, int st) {
      const int so_a = __builtin_amdgcn_readfirstlane(s * BK * 2);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < n_a)
          dma_lds16(rwA, __builtin_amdgcn_readfirstlane(lds_addr(&lds[st].a[(i * 4 + wid) * kWave])), a_off[i], so_a);
      if (DIRECT) return;
      const int so_q = __builtin_amdgcn_readfirstlane(s * 2048);
#pragma unroll
      for (int c = 0; c < 2; ++c)
        dma_lds16(rwB, __builtin_amdgcn_readfirstlane(lds_addr(&lds[st].q[wid][c][0])), q_off + c * 1024, so_q);
      dma_lds4(rwB, __builtin_amdgcn_readfirstlane(lds_addr(&lds[st].sb[wid][0])), sb_off,
               __builtin_amdgcn_readfirstlane(s * 256));
    };
    // DIRECT: lane (n, kq) reads, for row group ng, 8 bytes (kq & 1) of chunk
    // 2s + kq/2 of wave row 16 ng + n, and that row's (scale, bias) word.
    // Rows 16 ng + n of one wave sit 256 bytes apart in their 64-row tile;
    // gate/up's up rows (ng >= 2) are the gate rows' offsets in the up section.
    int dq0 = 0, dsb0 = 0;
    if (DIRECT) {
      const int r = wave_ok ? wave_base + n : 0;
      dq0 = (int)(a.off_q0 + (int64_t)(r / kTileRows) * (kTileRows * a.K / 2) + (r % kTileRows) * 16) +
            (kq >> 1) * 1024 + (kq & 1) * 8;
      dsb0 = (int)(a.off_sb0 + (int64_t)(r / kTileRows) * (kTileRows * G * 4) + (r % kTileRows) * 4);
    }
    const int dq_up = GATEUP ? (int)(a.off_q1 - a.off_q0) - 512 : 0;   // ng 2, 3: up section, rows n, n + 16
    const int dsb_up = GATEUP ? (int)(a.off_sb1 - a.off_sb0) - 128 : 0;
    auto load_b = [&](int s, u32x2 (&q)[4], uint32_t (&sb)[4]) {
#pragma unroll
      for (int ng = 0; ng < 4; ++ng) {
        const int uq = __builtin_amdgcn_readfirstlane(s * 2048 + (ng >= 2 ? dq_up : 0));
        const int us = __builtin_amdgcn_readfirstlane(s * 256 + (ng >= 2 ? dsb_up : 0));
        q[ng] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rsB, dq0 + ng * 256, uq, 0));
        sb[ng] = __builtin_amdgcn_raw_buffer_load_b32(rsB, dsb0 + ng * 64, us, 0);
      }
    };
    u32x2 bq[4];
    uint32_t bsb[4];
    // the first two K steps go out before anything else (DIRECT: the
    // activations of step 0, the weights of step 0, the activations of step 1)
    issue(s0, 0);
    if (DIRECT) load_b(s0, bq, bsb);
    if (s1 - s0 > 1) issue(s0 + 1, 1);

    // down: each group's tile exponent.  Activations written by the gate/up
    // kernel share one exponent per tile and group, so the first row's are the
    // tile's; any row that differs switches on a rescale of its LDS slots.
    int tile_exp = 0;  // down: activation value = LDS value * 2^(tile_exp + (s_gexp[s] - tile_exp))
    bool fix_rows = false;
    if (kScaledA) {
      const int p = t < BM ? s_pair[t] : -1;
      const int8_t* ep = a.a_exp + (int64_t)max(p, 0) * G;
      const int8_t* e0 = a.a_exp + (int64_t)max(s_pair[0], 0) * G;  // row 0 of a tile is a pair
      bool differs = false;
      for (int g0 = 0; g0 < G; g0 += 16) {
        int v[16], v0[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          v[i] = (p >= 0 && g0 + i < G) ? (int)ep[g0 + i] : 0;
          v0[i] = (g0 + i < G) ? (int)e0[g0 + i] : 0;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          differs |= p >= 0 && v[i] != v0[i];
          if (t == 0 && g0 + i < G) s_gexp[g0 + i] = v0[i];
        }
      }
      if (differs) s_fix = 1;
      __syncthreads();
      fix_rows = s_fix != 0;
      if (fix_rows) {
        // rare: tile exponent = the largest of its rows
        __syncthreads();
        if (p >= 0)
          for (int g = 0; g < G; ++g) atomicMax(&s_gexp[g], (int)ep[g]);
        __syncthreads();
      }
      int te = -128;
      for (int g = 0; g < G; ++g) te = max(te, s_gexp[g]);
      tile_exp = te;
    }

    floatx4 acc[8][4];
#pragma unroll
    for (int mg = 0; mg < 8; ++mg)
#pragma unroll
      for (int ng = 0; ng < 4; ++ng) acc[mg][ng] = floatx4{0.f, 0.f, 0.f, 0.f};
    const int n_mg = __builtin_amdgcn_readfirstlane((rows + 15) / 16);
    const bool half1 = n_mg > 4;

    // Rows whose exponent for step s is below the tile's: rescale their slots in LDS.
    auto fix_step = [&](int s, int st) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int sl = t * 4 + i, r = sl / 8;
        const int p = s_pair[r];
        if (p < 0) continue;
        const int diff = (int)a.a_exp[(int64_t)p * G + s] - s_gexp[s];
        if (diff == 0) continue;
        const _Float16 c = diff < -24 ? (_Float16)0.0f : (_Float16)exp2i(diff);
        const f16x2 c2 = {c, c};
        uint4 v = lds[st].a[sl];
        uint32_t* w = reinterpret_cast<uint32_t*>(&v);
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, w[j]) * c2);
        lds[st].a[sl] = v;
      }
    };
    auto read_half = [&](u32x4 (&fa)[4], uint32_t base) {
      fa[0] = lds_read128<0>(base);
      fa[1] = lds_read128<2048>(base);
      fa[2] = lds_read128<4096>(base);
      fa[3] = lds_read128<6144>(base);
    };
    // gate/up: C[pair row][weight row]; down: C[weight row][pair row] (the
    // transposed product puts 4 consecutive output columns in one lane)
    auto mfma_half = [&](const u32x4 (&fa)[4], const V8 (&fb)[4], int h) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * h + i < n_mg) {
#pragma unroll
          for (int ng = 0; ng < 4; ++ng)
            acc[4 * h + i][ng] = GATEUP ? O::mfma(__builtin_bit_cast(V8, fa[i]), fb[ng], acc[4 * h + i][ng])
                                        : O::mfma(fb[ng], __builtin_bit_cast(V8, fa[i]), acc[4 * h + i][ng]);
        }
    };
    auto dequant = [&](V8 (&fb)[4], const u32x2 (&qv)[4], const f16x2 (&s2)[4], const f16x2 (&b2)[4], int j) {
#pragma unroll
      for (int ng = 0; ng < 4; ++ng)
        fb[ng] = __builtin_bit_cast(V8, O::dequant8(j == 0 ? qv[ng].x : qv[ng].y, s2[ng], b2[ng], kc));
    };
    auto compute = [&](int s, int st, const u32x2 (&dq)[4], const uint32_t (&dsb)[4]) {
      const uint32_t so = (uint32_t)st * (uint32_t)sizeof(StageLds);
      u32x4 fx[4], fy[4];
      u32x2 qv[4];
      uint32_t sbv[4];
      read_half(fx, a_rd0 + so);  // j = 0, rows 0..63
      if (DIRECT) {
#pragma unroll
        for (int ng = 0; ng < 4; ++ng) {
          qv[ng] = dq[ng];
          sbv[ng] = dsb[ng];
        }
      } else {
        qv[0] = lds_read64<0>(q_rd + so);
        qv[1] = lds_read64<256>(q_rd + so);
        qv[2] = lds_read64<512>(q_rd + so);
        qv[3] = lds_read64<768>(q_rd + so);
        sbv[0] = lds_read32<0>(sb_rd + so);
        sbv[1] = lds_read32<64>(sb_rd + so);
        sbv[2] = lds_read32<128>(sb_rd + so);
        sbv[3] = lds_read32<192>(sb_rd + so);
      }
      if (kScaledA) {
        // this group's activations carry 2^(s_gexp[s] - tile_exp) <= 1: fold it into s and b
        const int d = s_gexp[s] - tile_exp;
        if (d != 0) {
          const _Float16 c = d < -24 ? (_Float16)0.0f : (_Float16)exp2i(d);
          const f16x2 c2 = {c, c};
#pragma unroll
          for (int ng = 0; ng < 4; ++ng)
            sbv[ng] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, sbv[ng]) * c2);
        }
      }
      f16x2 s2[4], b2[4];
#pragma unroll
      for (int ng = 0; ng < 4; ++ng) O::split_sb(sbv[ng], s2[ng], b2[ng]);
      V8 fb[4];
      dequant(fb, qv, s2, b2, 0);
      if (half1) read_half(fy, a_rd0 + so + 8192);  // j = 0, rows 64..127
      mfma_half(fx, fb, 0);
      if (half1) {
        read_half(fx, a_rd1 + so);  // j = 1, rows 0..63
        mfma_half(fy, fb, 1);
      } else {
        read_half(fx, a_rd1 + so);
      }
      dequant(fb, qv, s2, b2, 1);
      if (half1) read_half(fy, a_rd1 + so + 8192);  // j = 1, rows 64..127
      mfma_half(fx, fb, 0);
      if (half1) mfma_half(fy, fb, 1);
    };
    for (int s = s0; s < s1; ++s) {
      const int st = (s - s0) % kStages;
      if (DIRECT) {
        // issue order per step: weights of s + 1, then activations of s + 2,
        // so only the activations of step s + 1 may still be in flight here
        constexpr int kRest = (0x7 << 4) | (0xF << 8);
        if (s + 1 < s1) {
          if (n_a == 1) __builtin_amdgcn_s_waitcnt(1 | kRest);
          else if (n_a == 2) __builtin_amdgcn_s_waitcnt(2 | kRest);
          else if (n_a == 3) __builtin_amdgcn_s_waitcnt(3 | kRest);
          else __builtin_amdgcn_s_waitcnt(4 | kRest);
        } else {
          __builtin_amdgcn_s_waitcnt(kRest);
        }
      } else {
        vm_wait_steps(s + 1 < s1, n_a);    // this wave's DMA for step s has landed
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // and its LDS accesses (lgkmcnt 0)
      __builtin_amdgcn_s_barrier();        // ... and every other wave's
      if (GEMM_TL_ON && s == s0) GEMM_TL_ITEM(tl_j, 2, __builtin_amdgcn_s_memrealtime());
      lds_fence();
      if (fix_rows) {
        fix_step(s, st);
        __syncthreads();
      }
      u32x2 nq[4];
      uint32_t nsb[4];
      if (DIRECT && s + 1 < s1) load_b(s + 1, nq, nsb);
      if (s + 2 < s1) issue(s + 2, (s - s0 + 2) % kStages);
      if (wave_ok) compute(s, st, bq, bsb);
      if (DIRECT && s + 1 < s1) {
#pragma unroll
        for (int ng = 0; ng < 4; ++ng) {
          bq[ng] = nq[ng];
          bsb[ng] = nsb[ng];
        }
      }
    }

    GEMM_TL_ITEM(tl_j, 3, __builtin_amdgcn_s_memrealtime());
    ++tl_j;
    // ---- split items: partials out; the last K range to arrive sums them
    // (in range order) and goes on to the epilogue, the others are done.
    // The partials are written through to memory and read back with
    // device-coherent loads, and each wave waits for its stores before the
    // workgroup's arrival, so no cache-wide release or acquire is needed (an
    // agent-scope acquire would drop the L2 lines every other workgroup of
    // the XCD is streaming).
    if (sr > 1) {
      const int first = item - ks;  // the item group's first item: its counter
      const __amdgpu_buffer_rsrc_t rsP = __builtin_amdgcn_make_buffer_rsrc(
          a.part + (int64_t)first * kPartF4, (short)0, sr * kPartF4 * (int)sizeof(floatx4), kRsrcWord3);
      const int lane_off = t * (int)sizeof(floatx4);
      if (wave_ok) {
        const int mine = __builtin_amdgcn_readfirstlane(ks * kPartF4 * (int)sizeof(floatx4));
#pragma unroll
        for (int mg = 0; mg < 2; ++mg)
          if (mg < n_mg)
#pragma unroll
            for (int ng = 0; ng < 4; ++ng)
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[mg][ng]), rsP,
                                                     lane_off + (mg * 4 + ng) * kThreads * (int)sizeof(floatx4),
                                                     mine, kSc1);
      }
      __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));  // vmcnt(0): this wave's partials are in memory
      __syncthreads();
      if (t == 0) s_ticket = __hip_atomic_fetch_add(a.cnt + first, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      if (s_ticket != (uint32_t)(sr - 1)) continue;
      if (wave_ok) {
#pragma unroll
        for (int mg = 0; mg < 2; ++mg)
          if (mg < n_mg)
#pragma unroll
            for (int ng = 0; ng < 4; ++ng) {
              const int off = lane_off + (mg * 4 + ng) * kThreads * (int)sizeof(floatx4);
              floatx4 v = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(rsP, off, 0, kSc1));
              for (int j = 1; j < sr; ++j)
                v += __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(
                                                     rsP, off, __builtin_amdgcn_readfirstlane(
                                                                   j * kPartF4 * (int)sizeof(floatx4)),
                                                     kSc1));
              acc[mg][ng] = v;
            }
      }
      if (t == 0) __hip_atomic_store(a.cnt + first, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- epilogue
    if (GATEUP) {
      // acc[mg][ng][i] = C[pair row mg*16 + kq*4 + i][weight row ng*16 + n of the wave];
      // act = gelu(gate) * up for wave columns c*16 + n, c = 0, 1.  The act
      // values go to an fp32 tile [128 rows][128 columns] in the stages' LDS
      // (free after the K loop), the block maximum on the way; then every
      // thread scales, converts and stores 16-byte runs of a row (each wave
      // stored single 16-bit values before, 64 store instructions a lane).
      float* tile = reinterpret_cast<float*>(&lds[0]);
      static_assert(sizeof(lds) >= (size_t)BM * 128 * sizeof(float), "the stages hold the act tile");
      float m = 0.0f;
      if (wave_ok) {
        // this lane's element of row kq * 4, column c * 16 + n of the wave, at
        // its slot position; the others lie at constant offsets from it (the
        // address is made opaque here, or the compiler builds all 64 at the
        // kernel's start and spills them)
        const int col = wid * (WN / 2) + n;
        uint32_t at = lds_addr(&lds[0]) + (uint32_t)(((kq * 4) * 128 + (col & ~7) + (col & 3) * 2 + ((col >> 2) & 1)) * 4);
        asm volatile("" : "+v"(at));
        typedef __attribute__((address_space(3))) float* lds_f32_t;
        const lds_f32_t tp = (lds_f32_t)(uintptr_t)at;
#pragma unroll
        for (int mg = 0; mg < 8; ++mg) {
          if (mg >= n_mg) continue;  // row groups past the tile's rows are not stored
#pragma unroll
          for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float g = acc[mg][c][i], u = acc[mg][c + 2][i];
              const float x = ok ? gelu_tanh_act16(g) * u : f32_nan();
              tp[(mg * 16 + i) * 128 + c * 16] = x;
              if (mg * 16 + kq * 4 + i < rows) m = fmaxf(m, fabsf(x));
            }
        }
      }
      // one exponent per M tile and 64-column group (waves 2g', 2g'+1)
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
      if (lane == 0) s_wmax[wid] = wave_ok ? m : 0.0f;
      __syncthreads();
      {
        const int Gf = a.f / kGroup, col0 = nt * (BN / 2);
        // chunk q: row q / 16, tile columns 8 (q % 16) .. + 7
#pragma unroll 2
        for (int k = 0; k < BM * 16 / kThreads; ++k) {
          const int q = k * kThreads + t, r = q / 16, cc = (q % 16) * 8;
          const int p = r < rows ? s_pair[r] : -1;
          if (p < 0 || col0 + cc >= a.f) continue;
          const int g2 = cc / kGroup;  // the tile's 64-column group: waves 2 g2, 2 g2 + 1
          const int ex = block_exp(fmaxf(s_wmax[2 * g2], s_wmax[2 * g2 + 1]));
          const float sc = exp2i(-ex);
          const float4 lo = *reinterpret_cast<const float4*>(tile + r * 128 + cc);
          const float4 hi = *reinterpret_cast<const float4*>(tile + r * 128 + cc + 4);
          ET o[8] = {(ET)(lo.x * sc), (ET)(lo.y * sc), (ET)(lo.z * sc), (ET)(lo.w * sc),
                     (ET)(hi.x * sc), (ET)(hi.y * sc), (ET)(hi.z * sc), (ET)(hi.w * sc)};
          *reinterpret_cast<uint4*>(reinterpret_cast<ET*>(a.out) + (int64_t)p * a.f + col0 + cc) =
              *reinterpret_cast<const uint4*>(o);
          if (cc % kGroup == 0) a.out_exp[(int64_t)p * Gf + (col0 + cc) / kGroup] = (int8_t)ex;
        }
      }
    } else if (wave_ok) {
      // acc[mg][ng][i] = C[output column ng*16 + kq*4 + i of the wave][pair row mg*16 + n]
      const int Gd = a.d / kGroup;
      const int grp = wave_base / kGroup;
#pragma unroll
      for (int mg = 0; mg < 8; ++mg) {
        float m = 0.0f;
#pragma unroll
        for (int ng = 0; ng < 4; ++ng)
#pragma unroll
          for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(acc[mg][ng][i]));
        m = fmaxf(m, __shfl_xor(m, 16, kWave));
        m = fmaxf(m, __shfl_xor(m, 32, kWave));
        const int p = s_pair[mg * 16 + n];
        if (p < 0) continue;
        const int ex = block_exp(m);
        const float sc = exp2i(-ex);
        _Float16* dst = reinterpret_cast<_Float16*>(a.out) + (int64_t)p * a.d + wave_base + kq * 4;
#pragma unroll
        for (int ng = 0; ng < 4; ++ng) {
          _Float16 h4[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) h4[i] = ok ? (_Float16)(acc[mg][ng][i] * sc) : (_Float16)f32_nan();
          *reinterpret_cast<uint2*>(dst + ng * 16) = *reinterpret_cast<const uint2*>(h4);
        }
        if (kq == 0) a.out_exp[(int64_t)p * Gd + grp] = (int8_t)max(-127, min(127, ex + tile_exp));
      }
    }
  }
  (void)tl_j;
  GEMM_TL(3, ((uint64_t)__smid() << 32) | (uint64_t)tl_j);
  GEMM_TL(2, __builtin_amdgcn_s_memrealtime());
}

// y[t] = residual[t] + sum_j w[t][j] * pair[t*k + j] in rank order, pair values
// fp16 block-scaled.  Thread = 8 columns of one token.
__global__ __launch_bounds__(256) void k_combine_scaled(const _Float16* __restrict__ pv, const int8_t* __restrict__ pe,
                                                        const float* __restrict__ topk_w,
                                                        const float* __restrict__ residual, float* __restrict__ y,
                                                        int T, int d, int k) {
  const int64_t n8 = (int64_t)T * d / 8;
  const int64_t i8 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i8 >= n8) return;
  const int t = (int)(i8 * 8 / d);
  const int col = (int)(i8 * 8 - (int64_t)t * d);
  const int Gd = d / kGroup;
  float acc[8];
  if (residual) {
    const float4 r0 = reinterpret_cast<const float4*>(residual)[2 * i8];
    const float4 r1 = reinterpret_cast<const float4*>(residual)[2 * i8 + 1];
    acc[0] = r0.x; acc[1] = r0.y; acc[2] = r0.z; acc[3] = r0.w;
    acc[4] = r1.x; acc[5] = r1.y; acc[6] = r1.z; acc[7] = r1.w;
  } else {
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
  }
  for (int j = 0; j < k; ++j) {
    const int64_t p = (int64_t)t * k + j;
    const float sc = topk_w[p] * exp2i(pe[p * Gd + col / kGroup]);
    const uint4 raw = *reinterpret_cast<const uint4*>(pv + p * d + col);
    const _Float16* h = reinterpret_cast<const _Float16*>(&raw);
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = fmaf(sc, (float)h[c], acc[c]);
  }
  reinterpret_cast<float4*>(y)[2 * i8] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  reinterpret_cast<float4*>(y)[2 * i8 + 1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

// ------------------------------------------------------------------ experts with few pairs
//
// An expert with at most 32 routed pairs (every expert when T <= 32, the many
// cold experts of a prefill batch) is bound by streaming its weights, not by
// the matrix cores.  The work-list GEMM above spends most of such an item on
// fixed costs (the shared activation tile, barrier-separated K steps, split-K
// partials through memory), and a workgroup runs one item at a time, so the
// memory round trips of an item's start (pair ids, slot, exponents) and of its
// K loop form one serial chain per workgroup.  Here every wave is on its own:
//  * Work item = (expert, 16 of its pairs, chunk of 64 outputs), one wave:
//    gate/up the 64 gate and 64 up rows of 64 act columns (one block exponent
//    group), down 64 output rows; an expert with 17..32 pairs has two items
//    per chunk, on the same XCD, whose second weight read hits L2 (two row
//    groups per wave would double the accumulator and operand registers and
//    spill).  Down: the four waves of a workgroup take four different items,
//    so many items' round trips overlap, with no barrier after the start.
//    Gate/up (44 K steps, and few items when T is small): two waves per item,
//    each half of the K steps, the halves summed through LDS (first plus
//    second: deterministic).
//    Items of expert rank r run on XCD r % 8, so an expert's activation rows
//    are fetched into one L2.
//  * The wave streams its weights through its own ring of K steps in LDS,
//    filled by LDS-DMA (buffer_load ... lds) kDepth steps ahead, and takes its
//    16-bit activation operand (h in slot order, or the block-scaled act) into
//    registers three steps ahead.
//  * The MFMA K order inside each 8-column block is the slot order
//    (0,4,1,5,2,6,3,7) in which dequant8 emits nibbles; the activations are
//    stored in that order.
//  * Outputs match the work-list GEMM's formats: gate/up act in slot order
//    with one exponent per (pair, 64-column group), here shared by the item's
//    rows; down fp16 pair values with one exponent per (pair, 64-row group).
constexpr int kSRows = 32;                // most pairs per expert on this path
constexpr int kSWaves = 4;
constexpr int kSThreads = kSWaves * kWave;
// activation steps in flight per wave: gate/up 2 (its ring of 2 steps lets
// three workgroups share a compute unit), down 3
template <bool GATEUP>
struct SAhead {
  static constexpr int value = GATEUP ? 2 : 3;
};

struct SmallArgs {
  const void* a_rows;     // gate/up: h fp16 [T][d] in slot order; down: act values fp16 [T*k][f]
  int a_bytes;
  const int8_t* a_exp;    // down: act exponents [T*k][f/64]
  const int32_t* offsets;
  const int32_t* sorted_pair;
  const int32_t* slot_of_expert;
  int n_slots;
  const uint8_t* arena;
  int64_t slot_stride;
  int T, d, f, E, k;
  int K;                  // reduction length: d (gate/up) or f (down)
  int NC;                 // chunks of 64 outputs
  int64_t off_q0, off_q1, off_sb0, off_sb1;
  void* out;              // gate/up: act values [T*k][f]; down: pair values [T*k][d] (fp16)
  int8_t* out_exp;
};

// One K step of one wave's weights in LDS, per matrix m (gate/up: gate, up;
// down: one): q[m][h][r] the 16 bytes of chunk 2s + h of tile row r, sb[m][r]
// the row's (scale, bias) word.  Each is one LDS-DMA load (lane = row).
template <bool GATEUP>
struct SStage {
  uint4 q[GATEUP ? 2 : 1][2][kWave];
  uint32_t sb[GATEUP ? 2 : 1][kWave];
};
template <bool GATEUP>
struct SDepth {
  static constexpr int value = GATEUP ? 2 : 5;  // weight steps in flight per wave (>= SAhead)
};
// Workgroups per compute unit: three (12 waves; the LDS rings of 2 gate/up or
// 5 down steps fit three times), so that a 32-token batch's ~530 gate/up and
// ~2,100 down items take one round, every gate/up item on four waves.
template <bool GATEUP>
struct SOcc {
  static constexpr int value = 3;
};
// Per-step activation operand of one lane: the 16 columns this lane
// multiplies (two MFMA K slices of 8) and (down) the row's exponent for the step.
struct SAct {
  u32x4 v[2];
  int ex;
};


template <bool GATEUP>
__global__ __launch_bounds__(kSThreads, SOcc<GATEUP>::value) void k_q4_small(SmallArgs a) {
  constexpr int NM = GATEUP ? 2 : 1;  // matrices
  constexpr int NG = 4 * NM;          // row groups of 16 per wave (gate/up: 4 gate, then the same 4 up)
  constexpr int D = SDepth<GATEUP>::value;
  constexpr int KS = GATEUP ? 2 : 1;        // waves per item (K parts)
  constexpr int IPW = kSWaves / KS;         // items per workgroup at a time
  constexpr int kSA = SAhead<GATEUP>::value;
  static_assert(D >= kSA, "a step's weights must be requested before its activations");
  typedef Op<_Float16> O;
  GEMM_TL(0, __builtin_amdgcn_s_memrealtime());
  int tl_j = 0;  // rounds this workgroup has started (timeline build)
  __shared__ SStage<GATEUP> s_ring[kSWaves][D];
  __shared__ int s_rank_e[256];             // expert of each small rank
  __shared__ int s_rank_beg[256];
  __shared__ int s_rank_cnt[256];
  __shared__ int s_wave_n[kSWaves];
  __shared__ int s_ppre[256 + 1];           // 16-pair parts of the ranks before each rank
  __shared__ int s_xb[2 * kSWaves];         // per wave: first rank of this XCD's stretch, of the next
  const int t = threadIdx.x;
  const int wid = __builtin_amdgcn_readfirstlane(t / kWave), lane = t % kWave;
  const int n = lane % 16, kq = lane / 16;
  const int G = a.K / kGroup;
  const int n_pairs = a.T * a.k;
  typename O::Consts kc{0x000F000Fu, 0x00F000F0u, 0x64006400u, 0x54005400u};
  asm volatile("" : "+v"(kc.m0), "+v"(kc.m4), "+v"(kc.e10), "+v"(kc.e6));

  // experts with 1..32 pairs, ranked by id (E <= 256: one thread each)
  {
    int cnt = 0, beg = 0;
    if (t < a.E) {
      beg = max(0, min(a.offsets[t], n_pairs));
      cnt = max(beg, min(a.offsets[t + 1], n_pairs)) - beg;
    }
    const bool small = cnt >= 1 && cnt <= kSRows;
    const uint64_t bal = __ballot(small);
    const int below = __builtin_popcountll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) s_wave_n[wid] = __builtin_popcountll(bal);
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wid; ++w) base += s_wave_n[w];
    if (small) {
      s_rank_e[base + below] = t;
      s_rank_beg[base + below] = beg;
      s_rank_cnt[base + below] = cnt;
    }
    __syncthreads();
  }
  const int n_small = s_wave_n[0] + s_wave_n[1] + s_wave_n[2] + s_wave_n[3];
  const int xcd = (int)(blockIdx.x % 8), nper = (int)(gridDim.x / 8);
  // XCD x runs the ranks whose first part falls in [x P / 8, (x + 1) P / 8)
  // of the P parts (whole experts, so an expert's parts share one L2; the
  // XCDs' part counts differ by at most one expert's).  Dealing the ranks
  // round-robin left one XCD with half again the average, and a second round.
  {
    const int np = t < n_small ? (s_rank_cnt[t] > 16 ? 2 : 1) : 0;
    int inc = np;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(inc, o, kWave);
      if (lane >= o) inc += v;
    }
    if (lane == kWave - 1) s_wave_n[wid] = inc;  // s_wave_n's counts are no longer needed
    __syncthreads();
    int before = inc - np;
    for (int w = 0; w < wid; ++w) before += s_wave_n[w];
    s_ppre[t] = before;
    if (t == 0) s_ppre[256] = s_wave_n[0] + s_wave_n[1] + s_wave_n[2] + s_wave_n[3];
    __syncthreads();
    const int P = s_ppre[256];
    const int lo = (xcd * P + 7) / 8, hi = ((xcd + 1) * P + 7) / 8;
    // first rank whose parts start at or past each bound (n_small past the last)
    const bool at_lo = t < n_small && s_ppre[t] >= lo, at_hi = t < n_small && s_ppre[t] >= hi;
    const uint64_t b_lo = __ballot(at_lo), b_hi = __ballot(at_hi);
    if (lane == 0) {
      s_xb[wid] = b_lo ? wid * kWave + __builtin_ctzll(b_lo) : 256;
      s_xb[kSWaves + wid] = b_hi ? wid * kWave + __builtin_ctzll(b_hi) : 256;
    }
    __syncthreads();
  }
  const int r_lo = min(n_small, min(min(s_xb[0], s_xb[1]), min(s_xb[2], s_xb[3])));
  const int r_hi = min(n_small, min(min(s_xb[4], s_xb[5]), min(s_xb[6], s_xb[7])));
  const int p_lo = s_ppre[r_lo];  // s_ppre[n_small] = P: ranks past n_small have no parts
  const int n_parts = s_ppre[r_hi] - p_lo;
  GEMM_TL(1, __builtin_amdgcn_s_memrealtime());
  const __amdgpu_buffer_rsrc_t rsA =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.a_rows), (short)0, a.a_bytes, kRsrcWord3);
  SStage<GATEUP>* ring = s_ring[wid];
  // LDS reads of this lane: row group ng = tile rows 16 (ng % 4) + n of matrix ng / 4
  const int rd_q = (kq >> 1) * (kWave * 16) + n * 16 + (kq & 1) * 8;
  // activation columns of this lane in a step: those of its two weight words
  const int colq = 32 * (kq >> 1) + 16 * (kq & 1);

  const int n_items = n_parts * a.NC;
  const int jw = (int)(blockIdx.x / 8);  // this workgroup's index in its XCD
  // every wave runs every round (the K parts meet at barriers); a wave without
  // an item skips its work.  A round's items go slot by slot over the XCD's
  // workgroups (item slot i of workgroup j runs item i * nper + j), so that a
  // round with fewer items than slots spreads them over all compute units
  // (workgroups j and j + nper / 2 share one) instead of doubling some up.
  // Gate/up: when the round's items number fewer than two per workgroup, the
  // first workgroups run one item on all four waves (K quarters) and the rest
  // two items (K halves), so that every wave has work.
  for (int base = 0; base < n_items;) {
    const int rem = n_items - base;
    const int n4 = GATEUP ? max(0, min(nper, 2 * nper - rem)) : 0;  // workgroups with one item
    const bool single = jw < n4;
    const int ks = GATEUP ? (single ? 4 : 2) : 1;  // waves per item
    const int is = wid / ks, kh = wid % ks;        // item slot of this wave, its K part
    const int q = single ? base + jw : base + n4 + is * (nper - n4) + (jw - n4);
    base += n4 + IPW * (nper - n4);
    const bool has = q < n_items;
    // K steps of this wave's part
    const int s0 = __builtin_amdgcn_readfirstlane(kh * G / ks), s1 = __builtin_amdgcn_readfirstlane((kh + 1) * G / ks);
    GEMM_TL_ITEM(tl_j, 0, __builtin_amdgcn_s_memrealtime());
    const int u = (has ? q : 0) / a.NC, c = (has ? q : 0) % a.NC;
    // the rank whose parts hold part p_lo + u: s_ppre[r] <= p_lo + u < s_ppre[r + 1]
    int rank = r_lo;
    for (int lo = r_lo, hi = r_hi - 1; lo <= hi;) {
      const int mid = (lo + hi) / 2;
      if (s_ppre[mid] <= p_lo + u) {
        rank = mid;
        lo = mid + 1;
      } else {
        hi = mid - 1;
      }
    }
    const int part = p_lo + u - s_ppre[rank];
    const int e = __builtin_amdgcn_readfirstlane(s_rank_e[rank]);
    const int beg = __builtin_amdgcn_readfirstlane(s_rank_beg[rank] + 16 * part);
    const int all_rows = s_rank_cnt[rank] - 16 * part;
    const int rows = __builtin_amdgcn_readfirstlane(all_rows < 16 ? all_rows : 16);
    // the item's pair ids (lane r holds row r's) and its slot, requested together
    int pr = -1;
    if (lane < rows) pr = a.sorted_pair[beg + lane];
    const int slot = __builtin_amdgcn_readfirstlane(a.slot_of_expert[e]);
    const bool ok = slot >= 0 && slot < a.n_slots;
    const uint8_t* blob = a.arena + (ok ? (int64_t)slot * a.slot_stride : 0);
    const u32x4 rwB = rsrc_words(blob, (int)a.slot_stride);
    const int tile_q = (int)(a.off_q0 + (int64_t)c * (kTileRows * a.K / 2)) + lane * 16;
    const int tile_sb = (int)(a.off_sb0 + (int64_t)c * (kTileRows * G * 4)) + lane * 4;
    const int up_q = GATEUP ? (int)(a.off_q1 - a.off_q0) : 0;
    const int up_sb = GATEUP ? (int)(a.off_sb1 - a.off_sb0) : 0;
    // weights of step s into ring slot s % D (asm LDS-DMA: the compiler would
    // otherwise drain every ring slot in flight before each step's LDS reads)
    auto dma = [&](int s) {
      SStage<GATEUP>& st = ring[(s - s0) % D];
      const int so_q = __builtin_amdgcn_readfirstlane(s * 2048), so_sb = __builtin_amdgcn_readfirstlane(s * 256);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        dma_lds16(rwB, __builtin_amdgcn_readfirstlane(lds_addr(&st.q[m][0][0])), tile_q + m * up_q, so_q);
        dma_lds16(rwB, __builtin_amdgcn_readfirstlane(lds_addr(&st.q[m][1][0])), tile_q + m * up_q + 1024, so_q);
        dma_lds4(rwB, __builtin_amdgcn_readfirstlane(lds_addr(&st.sb[m][0])), tile_sb + m * up_sb, so_sb);
      }
    };
    const int pre = s1 - s0 < D ? s1 - s0 : D;
    if (has)
      for (int i = 0; i < pre; ++i) dma(s0 + i);

    if (pr < 0 || pr >= n_pairs) pr = -1;
    // activation row of this lane (MFMA row n)
    const int prow = __shfl(pr, n, kWave);
    const int arow = prow < 0 ? 0 : (GATEUP ? prow / a.k : prow);
    // down: the item's largest act exponent over its rows and K groups
    int texp = 0;
    if (!GATEUP) {
      // 16 exponents per memory round trip (a loop of single loads paid one
      // round trip per K group before the item's first step)
      int m = -128;
      const int8_t* ep = a.a_exp + (int64_t)max(pr, 0) * G;
      for (int g0 = 0; g0 < G; g0 += 16) {
        int v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = (pr >= 0 && g0 + i < G) ? (int)ep[g0 + i] : -128;
#pragma unroll
        for (int i = 0; i < 16; ++i) m = max(m, v[i]);
      }
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) m = max(m, __shfl_xor(m, o, kWave));
      texp = m < -127 ? 0 : m;
    }
    // (a lane past the pairs reads at the buffer's end: zeros, no memory access)
    auto fetch_a = [&](int s, SAct& v) {
      const bool live = prow >= 0;
      const int off = live ? (arow * a.K + s * kGroup + colq) * 2 : a.a_bytes;
      v.v[0] = __builtin_amdgcn_raw_buffer_load_b128(rsA, off, 0, 0);
      v.v[1] = __builtin_amdgcn_raw_buffer_load_b128(rsA, off + 16, 0, 0);
      if (!GATEUP) {
        const int ev = (int)a.a_exp[(int64_t)arow * G + s];
        v.ex = live ? ev : texp;
      }
    };
    // the activation operand has landed: every load issued before it has too
    // (loads complete in order), among them the DMA of the same step
    auto landed = [&](const SAct& v) { asm volatile("" ::"v"(v.v[0]), "v"(v.v[1]) : "memory"); };
    floatx4 acc[NG];
#pragma unroll
    for (int ng = 0; ng < NG; ++ng) acc[ng] = floatx4{0.f, 0.f, 0.f, 0.f};
    // the A operand of K slice j (8 columns in slot order)
    auto a_slice = [&](const SAct& v, int j) -> f16x8 {
      f16x8 h = __builtin_bit_cast(f16x8, v.v[j]);
      if (!GATEUP) {
        // a row whose exponent for this group is below the item's: scale down
        const int dx = v.ex - texp;
        if (dx != 0) {
          const _Float16 cf = dx < -24 ? (_Float16)0.0f : (_Float16)exp2i(dx);
          h = h * cf;
        }
      }
      return h;
    };
    // step s: its weights from the ring (the slot is then refilled with step
    // s + D), the activations of step s + kSA, dequant and MFMAs
    auto one = [&](int s, const SAct& vc, SAct& vf) {
      landed(vc);
      const SStage<GATEUP>& st = ring[(s - s0) % D];
      u32x2 qv[NG];
      uint32_t sbv[NG];
#pragma unroll
      for (int ng = 0; ng < NG; ++ng) {
        const int m = ng / 4, rr = 16 * (ng % 4);
        qv[ng] = *reinterpret_cast<const u32x2*>(reinterpret_cast<const char*>(&st.q[m][0][0]) + rd_q + rr * 16);
        sbv[ng] = st.sb[m][rr + n];
      }
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(qv[0]), "+v"(sbv[0])::"memory");
      // the weights of step s + D, then the activations of step s + kSA
      // (the latter unconditional: no half-defined buffer)
      if (s + D < s1) dma(s + D);
      fetch_a(s + kSA < s1 ? s + kSA : s1 - 1, vf);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const f16x8 av = a_slice(vc, j);
#pragma unroll
        for (int ng = 0; ng < NG; ++ng) {
          f16x2 s2, b2;
          O::split_sb(sbv[ng], s2, b2);
          const f16x8 fb = __builtin_bit_cast(f16x8, O::dequant8(j == 0 ? qv[ng].x : qv[ng].y, s2, b2, kc));
          acc[ng] = O::mfma(av, fb, acc[ng]);
        }
      }
    };
    GEMM_TL_ITEM(tl_j, 1, ((uint64_t)q << 32) | ((uint64_t)rows << 16));
    GEMM_TL_ITEM(tl_j, 2, __builtin_amdgcn_s_memrealtime());
    if (has && s0 < s1) {
      if constexpr (kSA == 3) {
        SAct v0, v1, v2, v3;
        fetch_a(s0, v0);
        fetch_a(s0 + 1 < s1 ? s0 + 1 : s1 - 1, v1);
        fetch_a(s0 + 2 < s1 ? s0 + 2 : s1 - 1, v2);
        for (int s = s0; s < s1; s += 4) {
          one(s, v0, v3);
          if (s + 1 >= s1) break;
          one(s + 1, v1, v0);
          if (s + 2 >= s1) break;
          one(s + 2, v2, v1);
          if (s + 3 >= s1) break;
          one(s + 3, v3, v2);
        }
      } else {
        SAct v0, v1, v2;
        fetch_a(s0, v0);
        fetch_a(s0 + 1 < s1 ? s0 + 1 : s1 - 1, v1);
        for (int s = s0; s < s1; s += 3) {
          one(s, v0, v2);
          if (s + 1 >= s1) break;
          one(s + 1, v1, v0);
          if (s + 2 >= s1) break;
          one(s + 2, v2, v1);
        }
      }
    }
    GEMM_TL_ITEM(tl_j, 3, __builtin_amdgcn_s_memrealtime());
    ++tl_j;
    if (KS > 1) {
      // the other K parts' accumulators join the first's, in part order,
      // through the weight rings (free once every wave is past its K loop;
      // no ring DMA is in flight after a wave's last step)
      // partial (slot is, part kh > 0) at is * (ks - 1) + kh - 1: at most 3
      // (one item on four waves, or two items on two waves each)
      floatx4(*red)[NG][kWave] = reinterpret_cast<floatx4(*)[NG][kWave]>(&s_ring[0][0]);
      static_assert(sizeof(s_ring) >= 3 * NG * kWave * sizeof(floatx4), "the rings hold the partials");
      __syncthreads();
      if (has && kh != 0)
#pragma unroll
        for (int ng = 0; ng < NG; ++ng) red[is * (ks - 1) + kh - 1][ng][lane] = acc[ng];
      __syncthreads();
      if (has && kh == 0)
        for (int pk = 1; pk < ks; ++pk)
#pragma unroll
          for (int ng = 0; ng < NG; ++ng) acc[ng] += red[is * (ks - 1) + pk - 1][ng][lane];
      __syncthreads();  // the rings are free for the next round
    }
    if (!has || kh != 0) continue;
    if (GATEUP) {
      // acc[g][i] (g = 0..3) = C[pair row kq*4 + i][gate row 16 g + n], acc[g + 4][i] the
      // up row: act column 64 c + 16 g + n; act overwrites the gate accumulators.  The
      // exponent is the part's; the act of an expert's two parts may differ in it.
      float m = 0.0f;
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool live = kq * 4 + i < rows;
          const float x = live ? (ok ? gelu_tanh_act16(acc[g][i]) * acc[g + 4][i] : f32_nan()) : 0.0f;
          acc[g][i] = x;
          if (live) m = fmaxf(m, fabsf(x));
        }
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
      const int ex = block_exp(m);
      const float sc = exp2i(-ex);
      const int Gf = a.f / kGroup;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = kq * 4 + i;
        const int p = __shfl(pr, r, kWave);
        if (r >= rows || p < 0) continue;
        _Float16* dst = reinterpret_cast<_Float16*>(a.out) + (int64_t)p * a.f;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = c * kGroup + g * 16 + n;  // stored at its slot position
          dst[(col & ~7) + (col & 3) * 2 + ((col >> 2) & 1)] = (_Float16)(acc[g][i] * sc);
        }
        if (n == 0) a.out_exp[(int64_t)p * Gf + c] = (int8_t)ex;
      }
    } else {
      // acc[ng][i] = C[pair row kq*4 + i][output row 64 c + 16 ng + n] * 2^-texp;
      // one exponent per (pair row, 64 output rows)
      const int Gd = a.d / kGroup;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float m = 0.0f;
#pragma unroll
        for (int ng = 0; ng < NG; ++ng) m = fmaxf(m, fabsf(acc[ng][i]));
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
        const int r = kq * 4 + i;
        const int p = __shfl(pr, r, kWave);
        if (r >= rows || p < 0) continue;
        const int ex = block_exp(m);
        const float sc = exp2i(-ex);
        _Float16* dst = reinterpret_cast<_Float16*>(a.out) + (int64_t)p * a.d + c * kGroup + n;
#pragma unroll
        for (int ng = 0; ng < NG; ++ng) dst[ng * 16] = ok ? (_Float16)(acc[ng][i] * sc) : (_Float16)f32_nan();
        if (n == 0) a.out_exp[(int64_t)p * Gd + c] = (int8_t)max(-127, min(127, ex + texp));
      }
    }
  }
  (void)tl_j;
  GEMM_TL(3, ((uint64_t)__smid() << 32) | (uint64_t)tl_j);
  GEMM_TL(2, __builtin_amdgcn_s_memrealtime());
}

}  // namespace

// ------------------------------------------------------------------ host side

static int gemm_nt(bool gateup, int d, int f) { return gateup ? (f + BN / 2 - 1) / (BN / 2) : (d + BN - 1) / BN; }

// Upper bound of work items: sum over experts of ceil(c_e / BM) <= T*k/BM + E.
static int max_items(int T, int k, int E, int NT) { return ((T * k + BM - 1) / BM + E) * NT; }

// The down GEMM keeps one tile exponent per K group in LDS (s_gexp), so its K
// (= f) spans at most kMaxSteps groups; gate/up has no such bound.
bool mfma_supported(int d, int f) { return d % BK == 0 && f % BK == 0 && f / BK <= kMaxSteps; }

size_t mfma_act_bytes(int T, int f, int k) { return (size_t)T * k * f * 2 + (size_t)T * k * (f / kGroup); }

// Workspace: arrival counters, then h in 16-bit slot order (gate/up) or the
// pair outputs (down), then the split items' partials.
static int split_item_cap(int T, int k, int E, int NT) { return std::min(kMaxSplitItems, max_items(T, k, E, NT)); }
static int64_t part_bytes(int cap) { return (int64_t)cap * kPartF4 * (int64_t)sizeof(floatx4); }
static int64_t gateup_body_bytes(int T, int d) { return round256((int64_t)T * d * 2); }
static int64_t down_body_bytes(int T, int d, int k) {
  return round256((int64_t)T * k * d * 2) + round256((int64_t)T * k * (d / kGroup));
}

size_t mfma_workspace_bytes(int call, int T, int d, int f, int E, int k) {
  if (call == MOE_CALL_GATEUP)
    return kCntBytes + gateup_body_bytes(T, d) + part_bytes(split_item_cap(T, k, E, gemm_nt(true, d, f)));
  return kCntBytes + down_body_bytes(T, d, k) + part_bytes(split_item_cap(T, k, E, gemm_nt(false, d, f)));
}

// Persistent grid: per_cu workgroups per compute unit (the kernel's
// occupancy), a multiple of 8 so that every XCD has the same number of
// workgroups.
static int persistent_grid(int items, int per_cu = 2) {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8)
      cus = 256;
  }
  const int g = (cus * per_cu) / 8 * 8;
  return std::max(8, std::min(g, (items + 7) / 8 * 8));
}

template <typename ET, bool GATEUP, bool DIRECT = false>
static void launch_gemm(const GemmArgs& a, int items, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  launch_maybe_timed(k_q4_gemm<ET, GATEUP, DIRECT>, persistent_grid(items), kThreads, s, ev0, ev1, a);
}

// The few-pairs kernel's arguments from the work-list GEMM's.
static SmallArgs small_args(const GemmArgs& g, const void* a_rows, int a_bytes, int NC) {
  SmallArgs a{};
  a.a_rows = a_rows;
  a.a_bytes = a_bytes;
  a.a_exp = g.a_exp;
  a.offsets = g.offsets;
  a.sorted_pair = g.sorted_pair;
  a.slot_of_expert = g.slot_of_expert;
  a.n_slots = g.n_slots;
  a.arena = g.arena;
  a.slot_stride = g.slot_stride;
  a.T = g.T; a.d = g.d; a.f = g.f; a.E = g.E; a.k = g.k;
  a.K = g.K;
  a.NC = NC;
  a.off_q0 = g.off_q0; a.off_q1 = g.off_q1; a.off_sb0 = g.off_sb0; a.off_sb1 = g.off_sb1;
  a.out = g.out;
  a.out_exp = g.out_exp;
  return a;
}

// Batches of at most kSmallPathT tokens: experts with at most kSRows pairs go
// to k_q4_small, the others to the work-list GEMM (with T <= kSRows no expert
// has more, and the work-list GEMM is skipped).  Larger batches run every
// expert through the work-list GEMM: at 2048 prefill tokens moving the
// few-pairs experts to k_q4_small measured 4% slower for the step.
constexpr int kSmallPathT = 64;
template <bool GATEUP>
static void launch_small(const SmallArgs& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  const int items = std::min(a.E, a.T * a.k) * a.NC;
  const int per_wg = GATEUP ? 1 : kSWaves;  // items a workgroup runs at a time (gate/up: one on four waves)
  launch_maybe_timed(k_q4_small<GATEUP>, persistent_grid((items + per_wg - 1) / per_wg, SOcc<GATEUP>::value),
                     kSThreads, s, ev0, ev1, a);
}

hipError_t launch_gateup_mfma(bool direct, const float* h, const int32_t* offsets, const int32_t* sorted_pair,
                              const int32_t* slot_of_expert, int n_slots, const uint8_t* arena, int64_t slot_stride,
                              int T, int d, int f, int E, int k, int64_t off_q0, int64_t off_q1, int64_t off_sb0,
                              int64_t off_sb1, void* act_out, void* ws, hipStream_t s) {
  const int NT = gemm_nt(true, d, f);
  const int items = max_items(T, k, E, NT);
  char* rest = reinterpret_cast<char*>(ws) + kCntBytes;
  const int64_t n8 = (int64_t)T * d / 8;
  const bool use_small = T <= kSmallPathT, only_small = T <= kSRows;
  hipLaunchKernelGGL(k_h_to_slots<_Float16>, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, h, n8,
                     reinterpret_cast<_Float16*>(rest));
  GemmArgs a{};
  a.a_rows = rest;
  a.a_bytes = (int)((int64_t)T * d * 2);
  a.a_exp = nullptr;
  a.a_by_token = 1;
  a.offsets = offsets;
  a.sorted_pair = sorted_pair;
  a.slot_of_expert = slot_of_expert;
  a.n_slots = n_slots;
  a.arena = arena;
  a.slot_stride = slot_stride;
  a.T = T; a.d = d; a.f = f; a.E = E; a.k = k;
  a.K = d;
  a.NT = NT;
  a.off_q0 = off_q0; a.off_q1 = off_q1; a.off_sb0 = off_sb0; a.off_sb1 = off_sb1;
  a.out = act_out;
  a.out_exp = reinterpret_cast<int8_t*>(act_out) + (int64_t)T * k * f * 2;
  a.cnt = reinterpret_cast<uint32_t*>(ws);
  a.part = reinterpret_cast<floatx4*>(rest + gateup_body_bytes(T, d));
  a.split_cap = split_item_cap(T, k, E, NT);
  a.min_rows = use_small ? kSRows + 1 : 1;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  take_profile_events(MOE_CALL_GATEUP, &ev0, &ev1);
  if (!only_small) {
    if (direct) launch_gemm<_Float16, true, true>(a, items, s, ev0, use_small ? nullptr : ev1);
    else launch_gemm<_Float16, true>(a, items, s, ev0, use_small ? nullptr : ev1);
  }
  if (use_small) launch_small<true>(small_args(a, rest, a.a_bytes, f / kGroup), s, only_small ? ev0 : nullptr, ev1);
  return hipGetLastError();
}

hipError_t launch_down_mfma(bool direct, const void* act_in, const int32_t* offsets, const int32_t* sorted_pair,
                            const int32_t* slot_of_expert, int n_slots, const uint8_t* arena, int64_t slot_stride,
                            int T, int d, int f, int E, int k, int64_t off_q, int64_t off_sb, const float* topk_w,
                            const float* residual, float* y, void* ws, hipStream_t s) {
  const int NT = gemm_nt(false, d, f);
  const int items = max_items(T, k, E, NT);
  char* rest = reinterpret_cast<char*>(ws) + kCntBytes;
  _Float16* pair_val = reinterpret_cast<_Float16*>(rest);
  int8_t* pair_exp = reinterpret_cast<int8_t*>(rest + round256((int64_t)T * k * d * 2));
  GemmArgs a{};
  a.a_rows = act_in;
  a.a_bytes = (int)((int64_t)T * k * f * 2);
  a.a_exp = reinterpret_cast<const int8_t*>(act_in) + (int64_t)T * k * f * 2;
  a.a_by_token = 0;
  a.offsets = offsets;
  a.sorted_pair = sorted_pair;
  a.slot_of_expert = slot_of_expert;
  a.n_slots = n_slots;
  a.arena = arena;
  a.slot_stride = slot_stride;
  a.T = T; a.d = d; a.f = f; a.E = E; a.k = k;
  a.K = f;
  a.NT = NT;
  a.off_q0 = off_q; a.off_sb0 = off_sb;
  a.out = pair_val;
  a.out_exp = pair_exp;
  a.cnt = reinterpret_cast<uint32_t*>(ws);
  a.part = reinterpret_cast<floatx4*>(rest + down_body_bytes(T, d, k));
  a.split_cap = split_item_cap(T, k, E, NT);
  const bool use_small = T <= kSmallPathT, only_small = T <= kSRows;
  a.min_rows = use_small ? kSRows + 1 : 1;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  take_profile_events(MOE_CALL_DOWN_COMBINE, &ev0, &ev1);
  if (!only_small) {
    if (direct) launch_gemm<_Float16, false, true>(a, items, s, ev0, use_small ? nullptr : ev1);
    else launch_gemm<_Float16, false>(a, items, s, ev0, use_small ? nullptr : ev1);
  }
  if (use_small)
    launch_small<false>(small_args(a, act_in, a.a_bytes, d / kGroup), s, only_small ? ev0 : nullptr, ev1);
  const int64_t n8 = (int64_t)T * d / 8;
  hipLaunchKernelGGL(k_combine_scaled, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, pair_val, pair_exp,
                     topk_w, residual, y, T, d, k);
  return hipGetLastError();
}

}  // namespace moe

#ifdef MOE_GEMM_TIMELINE
// The item timeline of the last launch of each work-list GEMM: uint64
// [2][1024][100] (gate/up, down; workgroup; slots).  clear != 0 zero-fills it
// afterwards.
extern "C" int moe_debug_gemm_timeline(uint64_t* host_out, int clear) {
  hipError_t e = hipMemcpyFromSymbol(host_out, HIP_SYMBOL(moe::g_gemm_timeline), sizeof(moe::g_gemm_timeline), 0,
                                     hipMemcpyDeviceToHost);
  if (e == hipSuccess && clear) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(moe::g_gemm_timeline));
    if (e == hipSuccess) e = hipMemset(p, 0, sizeof(moe::g_gemm_timeline));
    if (e == hipSuccess) e = hipDeviceSynchronize();
  }
  return (int)e;
}
#endif
