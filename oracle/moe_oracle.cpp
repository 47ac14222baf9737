// Plain, slow CPU oracle of the routed int4 mixture-of-experts layer, in C++17.
//
// TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
// CPU-baseline leg load this library.  It shares no code with the HIP library
// (no kernels, headers, tables or helpers) and parses the expert byte format on
// its own from the format's definition.
//
// Arithmetic, step by step (fp32 unless stated; every sum runs sequentially in
// ascending index order, a multiply then an add, built with -ffp-contract=off):
//   dequant   w[r][c] = fp32(s) * q + fp32(b), q the unsigned nibble 0..15 and
//             (s, b) the fp16 scale and bias of the row's group of 64 columns.
//             INT4 weights in affine groups of 64 with a scale and a bias
//             ("Optimizing a 14.3 GB model for an 8 GB machine", section
//             "Vectorization helped when it respected the storage layout").
//             s has an 11-bit significand and q < 16, so s*q is exact in fp32,
//             and s*q + b spans at most 23 bits (fp16's smallest step is
//             2^-24, |s*q| < 2^-1), so the weight is exact in fp32 as well.
//   RMSNorm   h_i = x_i * (1 / sqrt(sum_i x_i^2 / d + eps)) * w_i.
//   router    l_e = sum_i Wr[e][i] h_i + bias_e; also the same sum in fp64, used
//             only to certify how far a decision is from a tie.  The router
//             names 8 of the 128 experts and only those run (TurboFieldfare
//             video transcript, paragraph on Gemma 4 as a mixture-of-experts
//             model).
//   top-k     a stable sort of the expert ids by fp32 logit, larger first, so
//             equal logits keep the lower id first; the first k in that order.
//   weights   w_j = exp(l_j - l_max) / sum_m exp(l_m - l_max) over the chosen,
//             in fp64 from the fp32 logits, rounded to fp32 (the softmax over
//             all experts renormalised over the chosen equals this).
//   gate/up   g_r = sum_c Wg[r][c] h_c, u_r = sum_c Wu[r][c] h_c, and
//             act_r = fp32(gelu_tanh(g_r) * u_r) with the tanh-form GELU in fp64.
//   down      o_i = sum_r Wd[i][r] act_r.
//   combine   y_i = x_i + sum_j w_j o_{j,i}, j in rank order (x omitted when no
//             residual is given).
//   permute   counts by expert, exclusive scan, pair ids grouped by expert with
//             ascending ids inside a group, and the inverse.
//   caches    the per-layer slot caches (LRU; LFU over all steps or a window),
//             rules stated at CacheState below.
// std::thread splits only independent work (rows, pairs, tokens); no sum is
// split or reordered.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <functional>
#include <thread>
#include <vector>

namespace {

constexpr int kGroup = 64;

int g_threads = 0;  // 0: every hardware thread

int n_threads() {
  if (g_threads > 0) return g_threads;
  const unsigned h = std::thread::hardware_concurrency();
  return h ? (int)h : 1;
}

// body(i) for every i in [0, n), items handed out one at a time from a shared
// counter; each item writes only its own outputs.
void parallel_for(int64_t n, const std::function<void(int64_t)>& body) {
  const int nt = (int)std::min<int64_t>(n_threads(), n);
  if (nt <= 1) {
    for (int64_t i = 0; i < n; ++i) body(i);
    return;
  }
  std::atomic<int64_t> next{0};
  std::vector<std::thread> pool;
  pool.reserve(nt);
  for (int w = 0; w < nt; ++w)
    pool.emplace_back([&] {
      for (int64_t i = next.fetch_add(1); i < n; i = next.fetch_add(1)) body(i);
    });
  for (auto& th : pool) th.join();
}

// IEEE binary16 -> binary32, from the format: sign, 5 exponent bits (bias 15),
// 10 fraction bits; exponent 0 is subnormal (fraction * 2^-24).
float half_to_float(uint16_t bits) {
  const int sign = bits >> 15, ex = (bits >> 10) & 0x1F, fr = bits & 0x3FF;
  double v;
  if (ex == 0)
    v = std::ldexp((double)fr, -24);
  else if (ex == 31)
    v = fr ? NAN : INFINITY;
  else
    v = std::ldexp(1024.0 + fr, ex - 25);
  return (float)(sign ? -v : v);
}

// bf16 is the upper half of an fp32 bit pattern.
float bf16_to_float(uint16_t bits) {
  const uint32_t u = (uint32_t)bits << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

// Byte offsets of the six sections of an expert blob, each on a 256-byte
// boundary: gate nibbles [f x d], up nibbles [f x d], down nibbles [d x f],
// gate pairs [f x d/64], up pairs, down pairs [d x f/64]; off[6] = total.
void sections(int d, int f, int64_t off[7]) {
  const int64_t size[6] = {(int64_t)f * d / 2, (int64_t)f * d / 2, (int64_t)d * f / 2,
                           (int64_t)f * (d / kGroup) * 4, (int64_t)f * (d / kGroup) * 4,
                           (int64_t)d * (f / kGroup) * 4};
  int64_t o = 0;
  for (int i = 0; i < 6; ++i) {
    o = (o + 255) / 256 * 256;
    off[i] = o;
    o += size[i];
  }
  off[6] = (o + 255) / 256 * 256;
}

// Element (r, c) of an R x C matrix stored in the blob format: rows tiled by
// 64; inside a tile the 16-byte column chunks of the 64 rows sit side by side.
//   nibble byte = (r/64)*(64*C/2) + (c/32)*1024 + (r%64)*16 + (c%32)/2, low 4 bits for even c
//   pair byte   = (r/64)*(64*(C/64)*4) + (c/64)*256 + (r%64)*4, fp16 scale then fp16 bias
float weight_at(const uint8_t* q, const uint8_t* sb, int C, int r, int c) {
  const int64_t nb = (int64_t)(r / 64) * (64LL * C / 2) + (c / 32) * 1024 + (r % 64) * 16 + (c % 32) / 2;
  const int nib = (c % 2 == 0) ? (q[nb] & 0xF) : (q[nb] >> 4);
  const int64_t pb = (int64_t)(r / 64) * (64LL * (C / kGroup) * 4) + (c / kGroup) * 256 + (r % 64) * 4;
  const float s = half_to_float(rd16(sb + pb));
  const float b = half_to_float(rd16(sb + pb + 2));
  return s * (float)nib + b;
}

// Dense fp32 copy of one matrix, rows split over threads.
std::vector<float> dequant_matrix(const uint8_t* q, const uint8_t* sb, int R, int C) {
  std::vector<float> w((size_t)R * C);
  parallel_for(R, [&](int64_t r) {
    for (int c = 0; c < C; ++c) w[(size_t)r * C + c] = weight_at(q, sb, C, (int)r, c);
  });
  return w;
}

struct Expert {
  std::vector<float> gate, up, down;  // [f][d], [f][d], [d][f]
};

Expert dequant_expert(const uint8_t* blob, int d, int f) {
  int64_t off[7];
  sections(d, f, off);
  Expert e;
  e.gate = dequant_matrix(blob + off[0], blob + off[3], f, d);
  e.up = dequant_matrix(blob + off[1], blob + off[4], f, d);
  e.down = dequant_matrix(blob + off[2], blob + off[5], d, f);
  return e;
}

// sum_c w[c] * v[c] in ascending c.
float dot(const float* w, const float* v, int n) {
  float acc = 0.0f;
  for (int c = 0; c < n; ++c) acc += w[c] * v[c];
  return acc;
}

// Four such sums over rows w, w + n, w + 2n, w + 3n, side by side: each is
// still its own sequential sum in ascending c (only the rows interleave).
void dot4(const float* w, const float* v, int n, float out[4]) {
  float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
  const float *w0 = w, *w1 = w + n, *w2 = w + 2 * n, *w3 = w + 3 * n;
  for (int c = 0; c < n; ++c) {
    a0 += w0[c] * v[c];
    a1 += w1[c] * v[c];
    a2 += w2[c] * v[c];
    a3 += w3[c] * v[c];
  }
  out[0] = a0;
  out[1] = a1;
  out[2] = a2;
  out[3] = a3;
}

// rows [r0, r1) of out = W v, W [R][n] row-major
void matvec_rows(const float* W, const float* v, int n, int r0, int r1, float* out) {
  int r = r0;
  for (; r + 4 <= r1; r += 4) dot4(W + (size_t)r * n, v, n, out + r);
  for (; r < r1; ++r) out[r] = dot(W + (size_t)r * n, v, n);
}

double gelu_tanh(double z) {
  const double k = std::sqrt(2.0 / 3.14159265358979323846);
  return 0.5 * z * (1.0 + std::tanh(k * (z + 0.044715 * z * z * z)));
}

constexpr int kRowBlock = 64;

// act[m] = fp32(gelu(Wg h[m]) * (Wu h[m])) for M rows of h; work split over
// (row of h, block of 64 act columns).
void gateup_rows(const Expert& e, int d, int f, const float* h, int M, float* act) {
  const int nb = (f + kRowBlock - 1) / kRowBlock;
  parallel_for((int64_t)M * nb, [&](int64_t it) {
    const int m = (int)(it / nb), b = (int)(it % nb);
    const int r0 = b * kRowBlock, r1 = std::min(f, r0 + kRowBlock);
    float g[kRowBlock], u[kRowBlock];
    matvec_rows(e.gate.data() + (size_t)r0 * d, h + (size_t)m * d, d, 0, r1 - r0, g);
    matvec_rows(e.up.data() + (size_t)r0 * d, h + (size_t)m * d, d, 0, r1 - r0, u);
    for (int r = r0; r < r1; ++r) act[(size_t)m * f + r] = (float)(gelu_tanh(g[r - r0]) * (double)u[r - r0]);
  });
}

// out[m] = Wd act[m]; work split over (row of act, block of 64 output rows).
void down_rows(const Expert& e, int d, int f, const float* act, int M, float* out) {
  const int nb = (d + kRowBlock - 1) / kRowBlock;
  parallel_for((int64_t)M * nb, [&](int64_t it) {
    const int m = (int)(it / nb), b = (int)(it % nb);
    const int r0 = b * kRowBlock, r1 = std::min(d, r0 + kRowBlock);
    matvec_rows(e.down.data(), act + (size_t)m * f, f, r0, r1, out + (size_t)m * d);
  });
}

// ---------------------------------------------------------------- caches
// State of one layer's slot cache: the expert in each slot (-1 empty) and the
// step it was last used (-1 never).  A step with selection S:
//   1. every hit gets stamp = t;
//   2. each miss, in ascending expert id, takes a victim slot and stamp t.
// LRU victim: the slot with the smallest (stamp, slot index); empty slots have
//   stamp -1 and so fill lowest first; a slot stamped t is never chosen
//   because k <= slots.
// LFU victim: the lowest empty slot if any; else, among slots not stamped t,
//   the one whose expert has the smallest (use count, stamp, slot index).
//   Use count of e = the steps counted (all so far, or the last W, the current
//   one included) whose selection holds e, resident or not.
// Bounded per-layer cache, LRU then LFU with a 64-token window tried
// ("Optimizing a 14.3 GB model for an 8 GB machine", section "MoE needed
// parallel work, reuse, and coarse overlap"; goinfer "When the model doesn't
// fit": LRU over resident slots).
struct CacheState {
  int policy = 0;  // 0 LRU, 1 LFU whole run, 2 LFU window
  int window = 0;
  int n_slots = 0, n_experts = 0;
  std::vector<int32_t> slot_expert;
  std::vector<int64_t> stamp;
  std::vector<std::vector<int32_t>> history;  // every step's selection, oldest first
  std::vector<int64_t> count;                 // use counts over the counted steps

  void rebuild_counts() {
    count.assign(n_experts, 0);
    const size_t h0 = (policy == 2 && (int64_t)history.size() > window) ? history.size() - window : 0;
    for (size_t s = h0; s < history.size(); ++s)
      for (int32_t e : history[s]) count[e] += 1;
  }
};

}  // namespace

extern "C" {

void oro_set_threads(int n) { g_threads = n; }
int oro_threads(void) { return n_threads(); }

int oro_blob_offsets(int d, int f, int64_t* off7) {
  if (d <= 0 || f <= 0 || d % kGroup || f % kGroup) return 1;
  sections(d, f, off7);
  return 0;
}

void oro_dequant(const uint8_t* blob, int64_t q_off, int64_t sb_off, int R, int C, float* w) {
  const std::vector<float> v = dequant_matrix(blob + q_off, blob + sb_off, R, C);
  std::memcpy(w, v.data(), v.size() * sizeof(float));
}

double oro_gelu_tanh(double z) { return gelu_tanh(z); }

void oro_rmsnorm(const float* x, int T, int d, const float* nw, float eps, float* h) {
  for (int t = 0; t < T; ++t) {
    const float* xr = x + (size_t)t * d;
    float ss = 0.0f;
    for (int i = 0; i < d; ++i) ss += xr[i] * xr[i];
    const float inv = 1.0f / std::sqrt(ss / (float)d + eps);
    for (int i = 0; i < d; ++i) h[(size_t)t * d + i] = xr[i] * inv * (nw ? nw[i] : 1.0f);
  }
}

// out = x / sqrt(mean(x^2) + eps): the unit-RMS rescale between decode steps.
void oro_rms_rescale(const float* x, int T, int d, float eps, float* out) {
  oro_rmsnorm(x, T, d, nullptr, eps, out);
}

void oro_router(const float* h, int T, int d, int E, const float* rw, const float* bias, float* lg32,
                double* lg64) {
  parallel_for((int64_t)T * E, [&](int64_t it) {
    const int t = (int)(it / E), e = (int)(it % E);
    const float* hr = h + (size_t)t * d;
    const float* wr = rw + (size_t)e * d;
    float s = 0.0f;
    double s64 = 0.0;
    for (int i = 0; i < d; ++i) {
      s += wr[i] * hr[i];
      s64 += (double)wr[i] * (double)hr[i];
    }
    lg32[it] = bias ? s + bias[e] : s;
    lg64[it] = bias ? s64 + (double)bias[e] : s64;
  });
}

// The k experts with the largest logits, in descending order; equal logits:
// the lower id first (a stable sort of the ids by logit).
void oro_select_topk(const float* lg, int E, int k, int32_t* idx) {
  std::vector<int32_t> ids(E);
  for (int e = 0; e < E; ++e) ids[e] = e;
  std::stable_sort(ids.begin(), ids.end(), [&](int32_t a, int32_t b) { return lg[a] > lg[b]; });
  for (int j = 0; j < k; ++j) idx[j] = ids[j];
}

// Softmax over the chosen experts' logits (fp64, rounded to fp32).
void oro_weights(const float* lg, int k, const int32_t* idx, float* w) {
  double m = (double)lg[idx[0]];
  for (int j = 1; j < k; ++j) m = std::max(m, (double)lg[idx[j]]);
  std::vector<double> z(k);
  double sum = 0.0;
  for (int j = 0; j < k; ++j) {
    z[j] = std::exp((double)lg[idx[j]] - m);
    sum += z[j];
  }
  for (int j = 0; j < k; ++j) w[j] = (float)(z[j] / sum);
}

void oro_expert_gateup(const uint8_t* blob, int d, int f, const float* h, int M, float* act) {
  const Expert e = dequant_expert(blob, d, f);
  gateup_rows(e, d, f, h, M, act);
}

void oro_expert_down(const uint8_t* blob, int d, int f, const float* act, int M, float* out) {
  const Expert e = dequant_expert(blob, d, f);
  down_rows(e, d, f, act, M, out);
}

// The selected experts and the combine for T tokens: blobs[e] is expert e's
// blob (only the experts idx names are read); out_pairs [T*k][d] receives
// each pair's expert output when not null.  Experts run one after another;
// inside one, its pairs' rows are split over threads.
void oro_experts_combine(const float* x, const float* h, int T, int d, int f, int E, int k, const int32_t* idx,
                         const float* w, const uint8_t* const* blobs, int residual, float* y, float* out_pairs) {
  std::vector<float> outs((size_t)T * k * d, 0.0f);
  for (int e = 0; e < E; ++e) {
    std::vector<int> pairs;
    for (int p = 0; p < T * k; ++p)
      if (idx[p] == e) pairs.push_back(p);
    if (pairs.empty()) continue;
    const Expert ex = dequant_expert(blobs[e], d, f);
    const int M = (int)pairs.size();
    std::vector<float> hs((size_t)M * d), act((size_t)M * f), o((size_t)M * d);
    for (int m = 0; m < M; ++m)
      std::memcpy(&hs[(size_t)m * d], h + (size_t)(pairs[m] / k) * d, sizeof(float) * d);
    gateup_rows(ex, d, f, hs.data(), M, act.data());
    down_rows(ex, d, f, act.data(), M, o.data());
    for (int m = 0; m < M; ++m) std::memcpy(&outs[(size_t)pairs[m] * d], &o[(size_t)m * d], sizeof(float) * d);
  }
  parallel_for(T, [&](int64_t t) {
    for (int i = 0; i < d; ++i) {
      float acc = residual ? x[(size_t)t * d + i] : 0.0f;
      for (int j = 0; j < k; ++j) acc += w[(size_t)t * k + j] * outs[((size_t)t * k + j) * d + i];
      y[(size_t)t * d + i] = acc;
    }
  });
  if (out_pairs) std::memcpy(out_pairs, outs.data(), outs.size() * sizeof(float));
}

void oro_permute(const int32_t* idx, int T, int k, int E, int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                 int32_t* pair_pos) {
  const int P = T * k;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int p = 0; p < P; ++p) counts[idx[p]] += 1;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  std::vector<int32_t> ids(P);
  for (int p = 0; p < P; ++p) ids[p] = p;
  std::stable_sort(ids.begin(), ids.end(), [&](int32_t a, int32_t b) { return idx[a] < idx[b]; });
  for (int n = 0; n < P; ++n) {
    sorted_pair[n] = ids[n];
    pair_pos[ids[n]] = n;
  }
}

void oro_shared_gemv_bf16(const uint16_t* w, const float* h, int T, int rows, int cols, float* out) {
  std::vector<float> W((size_t)rows * cols);
  parallel_for(rows, [&](int64_t r) {
    for (int c = 0; c < cols; ++c) W[(size_t)r * cols + c] = bf16_to_float(w[(size_t)r * cols + c]);
  });
  const int nb = (rows + kRowBlock - 1) / kRowBlock;
  parallel_for((int64_t)T * nb, [&](int64_t it) {
    const int t = (int)(it / nb), b = (int)(it % nb);
    const int r0 = b * kRowBlock, r1 = std::min(rows, r0 + kRowBlock);
    matvec_rows(W.data(), h + (size_t)t * cols, cols, r0, r1, out + (size_t)t * rows);
  });
}

// out = residual + W_down (gelu_tanh(W_gate h) * (W_up h)), bf16 weights:
// w_gu [2 f_sh][d] (gate rows, then up rows), w_down [d][f_sh].
void oro_shared_expert_bf16(const uint16_t* w_gu, const uint16_t* w_down, const float* h, const float* residual,
                            int T, int d, int f_sh, float* out) {
  std::vector<float> gu((size_t)T * 2 * f_sh), act((size_t)T * f_sh), o((size_t)T * d);
  oro_shared_gemv_bf16(w_gu, h, T, 2 * f_sh, d, gu.data());
  for (int t = 0; t < T; ++t)
    for (int r = 0; r < f_sh; ++r) {
      const float g = gu[(size_t)t * 2 * f_sh + r], u = gu[(size_t)t * 2 * f_sh + f_sh + r];
      act[(size_t)t * f_sh + r] = (float)(gelu_tanh(g) * (double)u);
    }
  oro_shared_gemv_bf16(w_down, act.data(), T, d, f_sh, o.data());
  for (int t = 0; t < T; ++t)
    for (int i = 0; i < d; ++i)
      out[(size_t)t * d + i] = residual ? residual[(size_t)t * d + i] + o[(size_t)t * d + i] : o[(size_t)t * d + i];
}

// ---------------------------------------------------------------- caches
void* oro_cache_new(int policy, int window, int n_slots, int n_experts) {
  if (policy < 0 || policy > 2 || n_slots < 1 || n_experts < 1 || (policy == 2 && window < 1)) return nullptr;
  CacheState* c = new CacheState;
  c->policy = policy;
  c->window = window;
  c->n_slots = n_slots;
  c->n_experts = n_experts;
  c->slot_expert.assign(n_slots, -1);
  c->stamp.assign(n_slots, -1);
  c->count.assign(n_experts, 0);
  return c;
}

void oro_cache_free(void* h) { delete static_cast<CacheState*>(h); }

// One step: hit[j] for sel[j]; installs [k][3] = (expert, slot, evicted
// expert or -1) in the order they were made; returns the number of installs.
int oro_cache_step(void* h, int64_t t, const int32_t* sel, int k, uint8_t* hit, int32_t* installs) {
  CacheState& c = *static_cast<CacheState*>(h);
  std::vector<int32_t> cur(sel, sel + k);
  c.history.push_back(cur);
  if (c.policy != 0) {
    for (int32_t e : cur) c.count[e] += 1;
    if (c.policy == 2 && (int64_t)c.history.size() > c.window)
      for (int32_t e : c.history[c.history.size() - 1 - c.window]) c.count[e] -= 1;
  }
  std::vector<int32_t> slot_of(c.n_experts, -1);
  for (int s = 0; s < c.n_slots; ++s)
    if (c.slot_expert[s] >= 0) slot_of[c.slot_expert[s]] = s;
  std::vector<int32_t> misses;
  for (int j = 0; j < k; ++j) {
    hit[j] = slot_of[sel[j]] >= 0 ? 1 : 0;
    if (hit[j])
      c.stamp[slot_of[sel[j]]] = t;
    else
      misses.push_back(sel[j]);
  }
  std::sort(misses.begin(), misses.end());
  int n = 0;
  for (int32_t e : misses) {
    int victim = -1;
    if (c.policy == 0) {
      for (int s = 0; s < c.n_slots; ++s)
        if (victim < 0 || c.stamp[s] < c.stamp[victim]) victim = s;  // ties: the lower slot, met first
    } else {
      for (int s = 0; s < c.n_slots && victim < 0; ++s)
        if (c.slot_expert[s] < 0) victim = s;
      if (victim < 0) {
        for (int s = 0; s < c.n_slots; ++s) {
          if (c.stamp[s] == t) continue;
          if (victim < 0) {
            victim = s;
            continue;
          }
          const int64_t cs = c.count[c.slot_expert[s]], cv = c.count[c.slot_expert[victim]];
          if (cs < cv || (cs == cv && c.stamp[s] < c.stamp[victim])) victim = s;
        }
      }
    }
    installs[3 * n + 0] = e;
    installs[3 * n + 1] = victim;
    installs[3 * n + 2] = c.slot_expert[victim];
    ++n;
    c.slot_expert[victim] = e;
    c.stamp[victim] = t;
  }
  return n;
}

void oro_cache_get(void* h, int32_t* slot_expert, int64_t* stamp, int64_t* counts) {
  const CacheState& c = *static_cast<const CacheState*>(h);
  std::copy(c.slot_expert.begin(), c.slot_expert.end(), slot_expert);
  std::copy(c.stamp.begin(), c.stamp.end(), stamp);
  if (counts) std::copy(c.count.begin(), c.count.end(), counts);
}

int oro_cache_history_len(void* h) { return (int)static_cast<CacheState*>(h)->history.size(); }

// history [n][k], oldest first
void oro_cache_get_history(void* h, int k, int32_t* out) {
  const CacheState& c = *static_cast<const CacheState*>(h);
  for (size_t s = 0; s < c.history.size(); ++s)
    for (int j = 0; j < k; ++j) out[s * k + j] = j < (int)c.history[s].size() ? c.history[s][j] : -1;
}

// Restore (slot_expert, stamp, history [n][k]); counts are recomputed from
// the history.
void oro_cache_set(void* h, const int32_t* slot_expert, const int64_t* stamp, int n_hist, int k,
                   const int32_t* hist) {
  CacheState& c = *static_cast<CacheState*>(h);
  c.slot_expert.assign(slot_expert, slot_expert + c.n_slots);
  c.stamp.assign(stamp, stamp + c.n_slots);
  c.history.clear();
  for (int s = 0; s < n_hist; ++s) {
    std::vector<int32_t> sel;
    for (int j = 0; j < k; ++j)
      if (hist[s * k + j] >= 0) sel.push_back(hist[s * k + j]);
    c.history.push_back(sel);
  }
  c.rebuild_counts();
}

}  // extern "C"
