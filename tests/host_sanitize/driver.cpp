// Host checks of the library's C ABI and expert cache, built with
// AddressSanitizer and UndefinedBehaviorSanitizer against the stand-ins in
// stub_runtime.cpp and stub_kernels.cpp (no GPU: "device" memory is host
// memory and copies happen at the time of the call).
//   1. Argument checks of every entry point: refusals give the documented
//      status and valid calls reach the (stubbed) launch.
//   2. The expert cache over many steps, in each staging mode and eviction
//      policy: after every step each resident expert's slot holds that
//      expert's blob, the slot table on the host and in "device" memory
//      agree with the exported slot -> expert map, and the statistics add up.
//   3. A HIP failure injected at every runtime call of every staged step:
//      the step reports MOE_ERR_HIP and leaves the cache as it was, or with
//      the slots of already-enqueued copies emptied, or (failure of the
//      hit-mask copy only) committed; the retried step then gives exactly the
//      state a cache without the failure reaches from the same start.
//   4. Failures injected into cache creation, split staging set-up and the
//      device-state set-up release everything they made (the sanitizer's leak
//      check and the stub's live-handle count).
// Exit status 0 when every check passed; a failed check prints its line.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/libmoe.h"

extern "C" void stub_fail_at(long n);
extern "C" long stub_calls(void);
extern "C" long stub_live_handles(void);

namespace {

int g_checks = 0;
#define EXPECT(cond)                                                                \
  do {                                                                              \
    ++g_checks;                                                                     \
    if (!(cond)) {                                                                  \
      std::fprintf(stderr, "check failed at %s:%d: %s (last error: %s)\n", __FILE__, \
                   __LINE__, #cond, moe_last_error());                              \
      std::exit(1);                                                                 \
    }                                                                               \
  } while (0)
#define EXPECT_STATUS(call, want) EXPECT((call) == (want))

// 256-byte aligned zeroed host memory standing in for device buffers.
struct Buf {
  void* p = nullptr;
  explicit Buf(size_t n) {
    p = std::aligned_alloc(256, (n + 255) / 256 * 256);
    std::memset(p, 0, (n + 255) / 256 * 256);
  }
  ~Buf() { std::free(p); }
  Buf(const Buf&) = delete;
  Buf& operator=(const Buf&) = delete;
  template <class T>
  T* as() const {
    return static_cast<T*>(p);
  }
};

uint64_t g_rng = 0x9e3779b97f4a7c15ull;
uint32_t next_u32() {
  g_rng ^= g_rng << 13;
  g_rng ^= g_rng >> 7;
  g_rng ^= g_rng << 17;
  return (uint32_t)(g_rng >> 11);
}

// ---------------------------------------------------------------- 1. the ABI
void check_abi() {
  const moe_dims dims{256, 128, 8, 2};
  const int T = 5;
  hipStream_t s = nullptr;
  EXPECT_STATUS(hipStreamCreateWithFlags(&s, hipStreamNonBlocking), hipSuccess);

  EXPECT(moe_expert_blob_bytes(moe_dims{100, 128, 8, 2}) == -1);
  EXPECT(moe_expert_blob_bytes(dims) > 0);
  int64_t off[6];
  EXPECT_STATUS(moe_expert_blob_offsets(dims, off), MOE_OK);
  EXPECT(off[0] == 0 && off[5] < moe_expert_blob_bytes(dims));
  EXPECT_STATUS(moe_expert_blob_offsets(dims, nullptr), MOE_ERR_ARG);
  EXPECT(moe_workspace_size(MOE_CALL_ROUTE, 0, dims, MOE_PREC_FP32) == SIZE_MAX);
  EXPECT(moe_workspace_size(MOE_CALL_GATEUP, T, dims, MOE_PREC_BF16_MFMA) == SIZE_MAX);
  EXPECT(moe_workspace_size((moe_call)7, T, dims, MOE_PREC_FP32) == SIZE_MAX);
  EXPECT(moe_act_bytes(T, moe_dims{256, 128, 300, 2}, MOE_PREC_FP32) == SIZE_MAX);
  for (int st = 0; st <= 7; ++st) EXPECT(moe_status_string((moe_status)st) != nullptr);

  const int d = dims.d, f = dims.f, E = dims.n_experts, k = dims.top_k;
  const int64_t blob = moe_expert_blob_bytes(dims), stride = (blob + 255) / 256 * 256;
  Buf x(sizeof(float) * T * d), nw(sizeof(float) * d), rw(sizeof(float) * E * d), rb(sizeof(float) * E);
  Buf h(sizeof(float) * T * d), idx(sizeof(int32_t) * T * k), w(sizeof(float) * T * k);
  const size_t ws_route = moe_workspace_size(MOE_CALL_ROUTE, T, dims, MOE_PREC_FP32);
  Buf ws(1 << 20);

  // moe_route
  EXPECT_STATUS(moe_route(x.as<float>(), nw.as<float>(), 1e-6f, rw.as<float>(), rb.as<float>(), T, dims,
                          h.as<float>(), idx.as<int32_t>(), w.as<float>(), ws.p, ws_route, s),
                MOE_OK);
  EXPECT_STATUS(moe_route(nullptr, nw.as<float>(), 1e-6f, rw.as<float>(), rb.as<float>(), T, dims, h.as<float>(),
                          idx.as<int32_t>(), w.as<float>(), ws.p, ws_route, s),
                MOE_ERR_ARG);
  EXPECT_STATUS(moe_route(x.as<float>() + 1, nw.as<float>(), 1e-6f, rw.as<float>(), rb.as<float>(), T, dims,
                          h.as<float>(), idx.as<int32_t>(), w.as<float>(), ws.p, ws_route, s),
                MOE_ERR_ALIGN);
  EXPECT_STATUS(moe_route(x.as<float>(), nw.as<float>(), 1e-6f, rw.as<float>(), rb.as<float>(), T, dims,
                          h.as<float>(), idx.as<int32_t>(), w.as<float>(), ws.p, ws_route - 1, s),
                MOE_ERR_CAPACITY);
  EXPECT_STATUS(moe_route(x.as<float>(), nw.as<float>(), -1.0f, rw.as<float>(), rb.as<float>(), T, dims,
                          h.as<float>(), idx.as<int32_t>(), w.as<float>(), ws.p, ws_route, s),
                MOE_ERR_ARG);
  EXPECT_STATUS(moe_route(x.as<float>(), nw.as<float>(), 1e-6f, rw.as<float>(), rb.as<float>(), T,
                          moe_dims{256, 128, 8, 9}, h.as<float>(), idx.as<int32_t>(), w.as<float>(), ws.p, ws_route,
                          s),
                MOE_ERR_ARG);
  EXPECT_STATUS(moe_route_noalloc(x.as<float>(), nw.as<float>(), 1e-6f, rw.as<float>(), rb.as<float>(), T, dims,
                                  h.as<float>(), idx.as<int32_t>(), w.as<float>(), s),
                MOE_OK);
  // a launch failure surfaces as MOE_ERR_HIP with the runtime's text
  stub_fail_at(0);
  EXPECT_STATUS(moe_route(x.as<float>(), nw.as<float>(), 1e-6f, rw.as<float>(), rb.as<float>(), T, dims,
                          h.as<float>(), idx.as<int32_t>(), w.as<float>(), ws.p, ws_route, s),
                MOE_ERR_HIP);
  EXPECT(std::strstr(moe_last_error(), "moe_route") != nullptr);

  // moe_permute
  Buf counts(sizeof(int32_t) * E), offs(sizeof(int32_t) * (E + 1)), sorted(sizeof(int32_t) * T * k),
      pos(sizeof(int32_t) * T * k);
  EXPECT_STATUS(moe_permute(idx.as<int32_t>(), T, dims, counts.as<int32_t>(), offs.as<int32_t>(),
                            sorted.as<int32_t>(), pos.as<int32_t>(), nullptr, 0, s),
                MOE_OK);
  EXPECT_STATUS(moe_permute(idx.as<int32_t>(), 40000, dims, counts.as<int32_t>(), offs.as<int32_t>(),
                            sorted.as<int32_t>(), pos.as<int32_t>(), nullptr, 0, s),
                MOE_ERR_ARG);

  // gate/up and down, both precisions
  const int S = 4;
  Buf arena((size_t)S * stride), table(sizeof(int32_t) * E);
  const size_t act_fp32 = moe_act_bytes(T, dims, MOE_PREC_FP32), act_f16 = moe_act_bytes(T, dims, MOE_PREC_F16_MFMA);
  Buf act(act_fp32 > act_f16 ? act_fp32 : act_f16), y(sizeof(float) * T * d);
  for (moe_precision p : {MOE_PREC_FP32, MOE_PREC_F16_MFMA, MOE_PREC_F16_MFMA_DIRECT}) {
    const size_t wg = moe_workspace_size(MOE_CALL_GATEUP, T, dims, p);
    const size_t wd = moe_workspace_size(MOE_CALL_DOWN_COMBINE, T, dims, p);
    EXPECT(wg <= (1 << 20) && wd <= (1 << 20));
    EXPECT_STATUS(moe_expert_q4_gateup(h.as<float>(), idx.as<int32_t>(), table.as<int32_t>(), S, arena.as<uint8_t>(),
                                       stride, offs.as<int32_t>(), sorted.as<int32_t>(), nullptr, 0, T, dims, p,
                                       act.p, ws.p, wg, s),
                  MOE_OK);
    EXPECT_STATUS(moe_expert_q4_down_combine(act.p, idx.as<int32_t>(), w.as<float>(), table.as<int32_t>(), S,
                                             arena.as<uint8_t>(), stride, offs.as<int32_t>(), sorted.as<int32_t>(),
                                             pos.as<int32_t>(), x.as<float>(), T, dims, p, y.as<float>(), ws.p, wd, s),
                  MOE_OK);
    // a slot stride below the blob, a misaligned arena
    EXPECT_STATUS(moe_expert_q4_gateup(h.as<float>(), idx.as<int32_t>(), table.as<int32_t>(), S, arena.as<uint8_t>(),
                                       stride - 256, offs.as<int32_t>(), sorted.as<int32_t>(), nullptr, 0, T, dims, p,
                                       act.p, ws.p, wg, s),
                  MOE_ERR_ARG);
    EXPECT_STATUS(moe_expert_q4_down_combine(act.p, idx.as<int32_t>(), w.as<float>(), table.as<int32_t>(), S,
                                             arena.as<uint8_t>() + 16, stride, offs.as<int32_t>(), sorted.as<int32_t>(),
                                             pos.as<int32_t>(), x.as<float>(), T, dims, p, y.as<float>(), ws.p, wd, s),
                  MOE_ERR_ALIGN);
    if (wd > 0)
      EXPECT_STATUS(moe_expert_q4_down_combine(act.p, idx.as<int32_t>(), w.as<float>(), table.as<int32_t>(), S,
                                               arena.as<uint8_t>(), stride, offs.as<int32_t>(), sorted.as<int32_t>(),
                                               pos.as<int32_t>(), x.as<float>(), T, dims, p, y.as<float>(), ws.p,
                                               wd - 1, s),
                    MOE_ERR_CAPACITY);
  }
  // the MFMA path needs the grouping; bf16 operands are refused
  EXPECT_STATUS(moe_expert_q4_gateup(h.as<float>(), idx.as<int32_t>(), table.as<int32_t>(), S, arena.as<uint8_t>(),
                                     stride, nullptr, nullptr, nullptr, 0, T, dims, MOE_PREC_F16_MFMA, act.p, ws.p,
                                     1 << 20, s),
                MOE_ERR_UNSUPPORTED);
  EXPECT_STATUS(moe_expert_q4_gateup(h.as<float>(), idx.as<int32_t>(), table.as<int32_t>(), S, arena.as<uint8_t>(),
                                     stride, offs.as<int32_t>(), sorted.as<int32_t>(), nullptr, 0, T, dims,
                                     MOE_PREC_BF16_MFMA, act.p, ws.p, 1 << 20, s),
                MOE_ERR_UNSUPPORTED);
  EXPECT_STATUS(moe_expert_q4_gateup(h.as<float>(), idx.as<int32_t>(), table.as<int32_t>(), S, arena.as<uint8_t>(),
                                     stride, offs.as<int32_t>(), nullptr, nullptr, 0, T, dims, MOE_PREC_FP32, act.p,
                                     ws.p, 1 << 20, s),
                MOE_ERR_ARG);
  Buf pmask(T * k);
  EXPECT_STATUS(moe_expert_q4_gateup(h.as<float>(), idx.as<int32_t>(), table.as<int32_t>(), S, arena.as<uint8_t>(),
                                     stride, nullptr, nullptr, pmask.as<uint8_t>(), 1, T, dims, MOE_PREC_FP32, act.p,
                                     ws.p, 1 << 20, s),
                MOE_OK);

  // fused decode
  const int L = 3;
  Buf xio(sizeof(float) * (L + 1) * d), nwl(sizeof(float) * L * d), rwl(sizeof(float) * L * E * d);
  Buf tables(sizeof(int32_t) * L * E), arenaL((size_t)L * S * stride), ti(sizeof(int32_t) * L * k),
      tw(sizeof(float) * L * k);
  const size_t wdec = moe_workspace_size(MOE_CALL_DECODE_LAYERS, L, dims, MOE_PREC_FP32);
  Buf wsd(wdec);
  EXPECT_STATUS(moe_decode_layers(xio.as<float>(), L, nwl.as<float>(), 1e-6f, rwl.as<float>(), nullptr,
                                  tables.as<int32_t>(), S, arenaL.as<uint8_t>(), S * stride, stride, dims,
                                  ti.as<int32_t>(), tw.as<float>(), xio.as<float>(), wsd.p, wdec, s),
                MOE_OK);
  EXPECT_STATUS(moe_decode_layers(xio.as<float>(), L, nwl.as<float>(), 1e-6f, rwl.as<float>(), nullptr,
                                  tables.as<int32_t>(), S, arenaL.as<uint8_t>(), S * stride - 256, stride, dims,
                                  ti.as<int32_t>(), tw.as<float>(), nullptr, wsd.p, wdec, s),
                MOE_ERR_ARG);
  EXPECT_STATUS(moe_decode_layers(xio.as<float>(), L, nwl.as<float>(), 1e-6f, rwl.as<float>(), nullptr,
                                  tables.as<int32_t>(), S, arenaL.as<uint8_t>(), S * stride, stride, dims,
                                  ti.as<int32_t>(), tw.as<float>(), nullptr, wsd.as<uint8_t>() + 16, wdec, s),
                MOE_ERR_ALIGN);
  // d beyond the fused kernel (slot sizes that fit it, never dereferenced)
  const moe_dims wide{4096, 128, 8, 2};
  const int64_t stride_w = (moe_expert_blob_bytes(wide) + 255) / 256 * 256;
  EXPECT_STATUS(moe_decode_layers(xio.as<float>(), L, nwl.as<float>(), 1e-6f, rwl.as<float>(), nullptr,
                                  tables.as<int32_t>(), S, arenaL.as<uint8_t>(), S * stride_w, stride_w, wide,
                                  ti.as<int32_t>(), tw.as<float>(), nullptr, wsd.p, wdec, s),
                MOE_ERR_UNSUPPORTED);
  EXPECT_STATUS(moe_decode_layers(xio.as<float>(), L, nwl.as<float>(), 1e-6f, rwl.as<float>(), nullptr,
                                  tables.as<int32_t>(), S, arenaL.as<uint8_t>(), S * stride, stride, dims,
                                  ti.as<int32_t>(), tw.as<float>(), nullptr, wsd.p, wdec - 1, s),
                MOE_ERR_CAPACITY);
  // the error word: clear, timed out, other shapes
  EXPECT_STATUS(moe_decode_check(wsd.p, s), MOE_OK);
  wsd.as<uint8_t>()[384] = 1;
  EXPECT_STATUS(moe_decode_check(wsd.p, s), MOE_ERR_STATE);
  wsd.as<uint8_t>()[384] = 2;
  EXPECT_STATUS(moe_decode_check(wsd.p, s), MOE_ERR_STATE);
  EXPECT(std::strstr(moe_last_error(), "other shapes") != nullptr);

  // shared expert and rescale
  Buf wgu(2 * 2 * 64 * d), wdn(2 * d * 64), sh_out(sizeof(float) * T * d);
  const size_t wsh = moe_shared_expert_workspace_size(T, 64);
  EXPECT(moe_shared_expert_workspace_size(T, 60) == SIZE_MAX);
  EXPECT_STATUS(moe_shared_expert_bf16(wgu.as<uint16_t>(), wdn.as<uint16_t>(), h.as<float>(), x.as<float>(), T, d, 64,
                                       sh_out.as<float>(), ws.p, wsh, s),
                MOE_OK);
  EXPECT_STATUS(moe_shared_expert_bf16(wgu.as<uint16_t>(), wdn.as<uint16_t>(), h.as<float>(), x.as<float>() + 1, T, d,
                                       64, sh_out.as<float>(), ws.p, wsh, s),
                MOE_ERR_ALIGN);
  EXPECT_STATUS(moe_shared_gemv_bf16(wgu.as<uint16_t>(), h.as<float>(), T, 128, d, sh_out.as<float>(), s), MOE_OK);
  EXPECT_STATUS(moe_shared_gemv_bf16(wgu.as<uint16_t>(), h.as<float>(), T, 128, 12, sh_out.as<float>(), s),
                MOE_ERR_ARG);
  EXPECT_STATUS(moe_rms_rescale(x.as<float>(), T, d, 1e-6f, h.as<float>(), s), MOE_OK);
  EXPECT_STATUS(moe_rms_rescale(x.as<float>(), T, 6, 1e-6f, h.as<float>(), s), MOE_ERR_ARG);
  EXPECT_STATUS(moe_profile_next_launch((moe_call)7, nullptr, nullptr), MOE_ERR_ARG);
  EXPECT_STATUS(hipStreamDestroy(s), hipSuccess);
}

// -------------------------------------------------------- 2. and 3. the cache
struct Rig {
  int L, E, S, k;
  int64_t blob, stride;
  uint8_t* pool = nullptr;  // "pinned" host pool [L][E][blob]
  Buf* arena = nullptr;
  Buf* tables = nullptr;

  Rig(int L_, int E_, int S_, int k_, int64_t blob_) : L(L_), E(E_), S(S_), k(k_), blob(blob_) {
    stride = (blob + 255) / 256 * 256;
    EXPECT_STATUS(hipHostMalloc((void**)&pool, (size_t)L * E * blob, 0), hipSuccess);
    for (int l = 0; l < L; ++l)
      for (int e = 0; e < E; ++e)
        for (int64_t i = 0; i < blob; ++i)
          pool[((int64_t)l * E + e) * blob + i] = (uint8_t)(l * 131 + e * 29 + i * 7 + (i >> 8) * 13 + 1);
    arena = new Buf((size_t)L * S * stride);
    tables = new Buf(sizeof(int32_t) * L * E);
    std::memset(arena->p, 0xEE, (size_t)L * S * stride);
  }
  ~Rig() {
    delete arena;
    delete tables;
    (void)hipHostFree(pool);
  }
  Rig(const Rig&) = delete;
  Rig& operator=(const Rig&) = delete;

  moe_cache* create(int policy, int window, int staging, int streams) {
    moe_cache* c = nullptr;
    EXPECT_STATUS(moe_cache_create(L, E, S, k, pool, blob, arena->as<uint8_t>(), stride, tables->as<int32_t>(), &c),
                  MOE_OK);
    EXPECT_STATUS(moe_cache_set_policy(c, policy, window), MOE_OK);
    EXPECT_STATUS(moe_cache_set_staging(c, staging, streams), MOE_OK);
    return c;
  }
};

// The exported state of a cache.
struct State {
  std::vector<int32_t> se;
  std::vector<int64_t> stamp, counts;
  std::vector<int32_t> recent;
  moe_stage_stats stats{};
  bool operator==(const State& o) const {
    return se == o.se && stamp == o.stamp && counts == o.counts && recent == o.recent &&
           stats.hits == o.stats.hits && stats.misses == o.stats.misses && stats.bytes_staged == o.stats.bytes_staged;
  }
};

State snapshot(const moe_cache* c, const Rig& r, int window) {
  State s;
  s.se.resize((size_t)r.L * r.S);
  s.stamp.resize((size_t)r.L * r.S);
  s.counts.resize((size_t)r.L * r.E);
  s.recent.resize((size_t)r.L * (window > 0 ? window : 1) * r.k);
  EXPECT_STATUS(moe_cache_export(c, s.se.data(), s.stamp.data()), MOE_OK);
  EXPECT_STATUS(moe_cache_export_usage(c, s.counts.data(), s.recent.data()), MOE_OK);
  EXPECT_STATUS(moe_cache_stats(c, &s.stats), MOE_OK);
  return s;
}

// Every resident expert's slot holds its blob; tables agree with the map.
// device_ok[l]: layer l's "device" table must already match (it may lag one
// call behind after a failed step).
void check_cache(const moe_cache* c, const Rig& r, const std::vector<char>& device_ok) {
  std::vector<int32_t> se((size_t)r.L * r.S), tbl(r.E);
  std::vector<int64_t> stamp((size_t)r.L * r.S);
  EXPECT_STATUS(moe_cache_export(c, se.data(), stamp.data()), MOE_OK);
  for (int l = 0; l < r.L; ++l) {
    EXPECT_STATUS(moe_cache_slot_table(c, l, tbl.data()), MOE_OK);
    std::vector<int32_t> want(r.E, -1);
    for (int s = 0; s < r.S; ++s) {
      const int e = se[(size_t)l * r.S + s];
      EXPECT(e >= -1 && e < r.E);
      if (e < 0) {
        EXPECT(stamp[(size_t)l * r.S + s] == -1);
        continue;
      }
      EXPECT(want[e] == -1);  // an expert sits in one slot at most
      want[e] = s;
      EXPECT(std::memcmp(r.arena->as<uint8_t>() + ((int64_t)l * r.S + s) * r.stride,
                         r.pool + ((int64_t)l * r.E + e) * r.blob, r.blob) == 0);
    }
    EXPECT(tbl == want);
    if (device_ok[l])
      EXPECT(std::memcmp(r.tables->as<int32_t>() + (int64_t)l * r.E, want.data(), sizeof(int32_t) * r.E) == 0);
  }
}

// k distinct experts, skewed towards the low ids so that hits and misses mix.
std::vector<int32_t> pick(int E, int k) {
  std::vector<int32_t> sel;
  while ((int)sel.size() < k) {
    const uint32_t u = next_u32();
    const int e = (u & 3) ? (int)((u >> 2) % (uint32_t)(E / 2 + 1)) : (int)((u >> 2) % (uint32_t)E);
    bool dup = false;
    for (int v : sel) dup |= v == e;
    if (!dup) sel.push_back(e);
  }
  return sel;
}

// A cache holding `st` (and the arena bytes of `from`), for the reference step.
moe_cache* clone(const Rig& from, Rig& to, const State& st, int policy, int window) {
  std::memcpy(to.arena->p, from.arena->p, (size_t)from.L * from.S * from.stride);
  moe_cache* c = to.create(policy, window, MOE_STAGE_COPY, 0);
  EXPECT_STATUS(moe_cache_import(c, st.se.data(), st.stamp.data()), MOE_OK);
  EXPECT_STATUS(moe_cache_import_usage(c, st.counts.data(), st.recent.data()), MOE_OK);
  return c;
}

int g_failures_injected = 0, g_emptied = 0, g_committed = 0;

void run_cache(int policy, int window, int staging, int streams, bool inject) {
  Rig r(2, 12, 5, 3, 16 * 67);  // blob a multiple of 16 (kernel staging), stride padded to 256
  Rig twin(2, 12, 5, 3, 16 * 67);
  moe_cache* c = r.create(policy, window, staging, streams);
  std::vector<char> device_ok(r.L, 1);
  hipStream_t side = nullptr, compute = nullptr;
  EXPECT_STATUS(hipStreamCreateWithFlags(&side, hipStreamNonBlocking), hipSuccess);
  EXPECT_STATUS(hipStreamCreateWithFlags(&compute, hipStreamNonBlocking), hipSuccess);
  Buf mask_dev(r.k);
  std::vector<uint8_t> mask(r.k);
  const int steps = 14;
  for (int step = 0; step < steps; ++step)
    for (int l = 0; l < r.L; ++l) {
      const std::vector<int32_t> sel = pick(r.E, r.k);
      const State before = snapshot(c, r, window);
      // the reference: the same step on a cache that does not fail
      moe_cache* ref = clone(r, twin, before, policy, window);
      EXPECT_STATUS(moe_slot_stage(ref, l, step, sel.data(), side, compute, mask_dev.as<uint8_t>(), mask.data(),
                                   nullptr),
                    MOE_OK);
      State want = snapshot(ref, twin, window);
      // the clone's statistics start at zero: they hold this step alone
      want.stats.hits += before.stats.hits;
      want.stats.misses += before.stats.misses;
      want.stats.bytes_staged += before.stats.bytes_staged;
      const std::vector<uint8_t> want_mask = mask;
      EXPECT_STATUS(moe_cache_destroy(ref), MOE_OK);
      bool diverged = false;  // a failed attempt changed the state
      for (long n = 0;; ++n) {
        if (!inject) n = -1;
        const State pre = snapshot(c, r, window);
        stub_fail_at(n);
        const moe_status st =
            moe_slot_stage(c, l, step, sel.data(), side, compute, mask_dev.as<uint8_t>(), mask.data(), nullptr);
        stub_fail_at(-1);
        if (st == MOE_OK) break;
        EXPECT(inject && st == MOE_ERR_HIP);
        ++g_failures_injected;
        const State post = snapshot(c, r, window);
        if (post.stats.hits + post.stats.misses == pre.stats.hits + pre.stats.misses + r.k) {
          // the hit-mask copy failed after the step was committed
          if (!diverged) EXPECT(post == want);
          ++g_committed;
          diverged = true;
          break;
        }
        // not committed: unchanged, or some slots emptied
        EXPECT(post.counts == pre.counts && post.recent == pre.recent && post.stats.hits == pre.stats.hits);
        bool emptied = false;
        for (size_t i = 0; i < pre.se.size(); ++i) {
          if (post.se[i] == pre.se[i] && post.stamp[i] == pre.stamp[i]) continue;
          EXPECT(post.se[i] == -1 && post.stamp[i] == -1);
          EXPECT(i / r.S == (size_t)l);  // only this layer's slots
          emptied = true;
        }
        if (emptied) {
          ++g_emptied;
          diverged = true;
        }
        // after a failed step the device table is only promised again once
        // the layer's next call has succeeded
        device_ok[l] = 0;
        check_cache(c, r, device_ok);
      }
      device_ok[l] = 1;
      check_cache(c, r, device_ok);
      if (!diverged) {
        EXPECT(snapshot(c, r, window) == want);
        EXPECT(mask == want_mask);
        EXPECT(std::memcmp(mask_dev.p, mask.data(), r.k) == 0);
      }
      // hits are the experts resident before the step
      if (!diverged)
        for (int j = 0; j < r.k; ++j) {
          bool resident = false;
          for (int s = 0; s < r.S; ++s) resident |= before.se[(size_t)l * r.S + s] == sel[j];
          EXPECT(mask[j] == (resident ? 1 : 0));
        }
      EXPECT_STATUS(moe_cache_wait(c, l, compute), MOE_OK);
      for (int j = 0; j < r.k; ++j) EXPECT_STATUS(moe_cache_wait_expert(c, l, j, compute), MOE_OK);
      EXPECT_STATUS(moe_cache_wait_expert(c, l, r.k, compute), MOE_ERR_ARG);
      EXPECT_STATUS(moe_cache_wait_expert(c, l, -1, compute), MOE_ERR_ARG);
    }
  // the cache refuses a policy or staging change now
  EXPECT_STATUS(moe_cache_set_policy(c, MOE_CACHE_LRU, 0), MOE_ERR_STATE);
  EXPECT_STATUS(moe_cache_set_staging(c, MOE_STAGE_COPY, 0), MOE_ERR_STATE);
  // bad selections change nothing
  const State before = snapshot(c, r, window);
  const int32_t repeat[3] = {1, 1, 2}, range[3] = {0, 1, 12};
  EXPECT_STATUS(moe_slot_stage(c, 0, 99, repeat, side, compute, mask_dev.as<uint8_t>(), nullptr, nullptr),
                MOE_ERR_ARG);
  EXPECT_STATUS(moe_slot_stage(c, 0, 99, range, side, compute, mask_dev.as<uint8_t>(), nullptr, nullptr), MOE_ERR_ARG);
  EXPECT_STATUS(moe_slot_stage(c, 2, 99, range, side, compute, mask_dev.as<uint8_t>(), nullptr, nullptr), MOE_ERR_ARG);
  EXPECT(snapshot(c, r, window) == before);
  EXPECT_STATUS(moe_cache_destroy(c), MOE_OK);
  EXPECT_STATUS(hipStreamDestroy(side), hipSuccess);
  EXPECT_STATUS(hipStreamDestroy(compute), hipSuccess);
}

// ------------------------------------------------ 4. failures while setting up
void check_setup_failures() {
  Rig r(2, 8, 4, 2, 512);
  const long live0 = stub_live_handles();
  int failed = 0;
  for (long n = 0;; ++n) {
    moe_cache* c = reinterpret_cast<moe_cache*>(&failed);  // must be cleared on failure
    stub_fail_at(n);
    const moe_status st =
        moe_cache_create(r.L, r.E, r.S, r.k, r.pool, r.blob, r.arena->as<uint8_t>(), r.stride, r.tables->as<int32_t>(), &c);
    stub_fail_at(-1);
    if (st == MOE_OK) {
      EXPECT(c != nullptr);
      // split staging: every part-way failure releases what it made
      for (long m = 0;; ++m) {
        stub_fail_at(m);
        const moe_status s2 = moe_cache_set_staging(c, MOE_STAGE_COPY_SPLIT, 4);
        stub_fail_at(-1);
        if (s2 == MOE_OK) break;
        EXPECT(s2 == MOE_ERR_HIP);
        ++failed;
      }
      // the device copy of the state: the same
      for (long m = 0;; ++m) {
        stub_fail_at(m);
        const moe_status s3 = moe_cache_enable_device(c);
        stub_fail_at(-1);
        if (s3 == MOE_OK) break;
        // a failed device-pointer query reads as a pool the device cannot address
        EXPECT(s3 == MOE_ERR_HIP || s3 == MOE_ERR_UNSUPPORTED);
        ++failed;
      }
      EXPECT_STATUS(moe_cache_enable_device(c), MOE_OK);  // idempotent
      EXPECT_STATUS(moe_slot_stage(c, 0, 0, std::vector<int32_t>{0, 1}.data(), nullptr, nullptr,
                                   r.arena->as<uint8_t>(), nullptr, nullptr),
                    MOE_ERR_STATE);
      EXPECT_STATUS(moe_cache_destroy(c), MOE_OK);
      break;
    }
    EXPECT(st == MOE_ERR_HIP && c == nullptr);
    ++failed;
  }
  EXPECT(failed > 10);
  EXPECT(stub_live_handles() == live0);
  // argument refusals of creation
  moe_cache* c = nullptr;
  EXPECT_STATUS(moe_cache_create(r.L, r.E, r.S, r.k, r.pool, r.blob, r.arena->as<uint8_t>() + 16, r.stride,
                                 r.tables->as<int32_t>(), &c),
                MOE_ERR_ALIGN);
  EXPECT_STATUS(moe_cache_create(r.L, r.E, r.E + 1, r.k, r.pool, r.blob, r.arena->as<uint8_t>(), r.stride,
                                 r.tables->as<int32_t>(), &c),
                MOE_ERR_ARG);
  EXPECT_STATUS(moe_cache_create(r.L, r.E, r.S, r.k, r.pool, r.blob, r.arena->as<uint8_t>(), r.stride - 256,
                                 r.tables->as<int32_t>(), &c),
                MOE_ERR_ARG);
  EXPECT(c == nullptr);
  EXPECT_STATUS(moe_cache_destroy(nullptr), MOE_OK);
}

}  // namespace

int main() {
  check_abi();
  check_setup_failures();
  const int policies[3][2] = {{MOE_CACHE_LRU, 0}, {MOE_CACHE_LFU, 0}, {MOE_CACHE_LFU_WINDOW, 4}};
  const int stagings[3][2] = {{MOE_STAGE_COPY, 0}, {MOE_STAGE_COPY_SPLIT, 3}, {MOE_STAGE_KERNEL, 0}};
  for (const auto& p : policies)
    for (const auto& s : stagings) {
      run_cache(p[0], p[1], s[0], s[1], false);
      run_cache(p[0], p[1], s[0], s[1], true);
    }
  EXPECT(stub_live_handles() == 0);
  EXPECT(g_emptied > 0 && g_committed > 0);
  std::printf("host checks passed: %d checks, %d injected step failures (%d emptied slots, %d after commit)\n",
              g_checks, g_failures_injected, g_emptied, g_committed);
  return 0;
}
