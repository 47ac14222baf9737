// C ABI of libmoe: argument checks, workspace carving and kernel launches.
// Every check runs on the host before anything is enqueued.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "common.h"
#include "kernels.h"

namespace {

constexpr int kMaxMfmaPairs = 1 << 22;  // T*k bound of the MFMA path (int32 item and row indices)

// The MFMA kernels address h, act and one slot with 32-bit buffer offsets.
bool mfma_fits_32bit(int32_t T, const moe_dims& d, int64_t slot_stride) {
  const int64_t lim = INT32_MAX;
  return (int64_t)T * d.d * 2 < lim && (int64_t)T * d.top_k * d.f * 2 < lim && slot_stride < lim;
}

thread_local std::string g_last_error;

moe_status fail(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

moe_status hip_fail(hipError_t e, const char* where) {
  return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

moe_status check_dims(const moe_dims& d) {
  if (d.d <= 0 || d.f <= 0 || d.d % 64 || d.f % 64)
    return fail(MOE_ERR_ARG, "dims: d=%d f=%d must be positive multiples of 64", d.d, d.f);
  if (d.top_k < 1 || d.top_k > 16 || d.n_experts < d.top_k || d.n_experts > 256)
    return fail(MOE_ERR_ARG, "dims: need 1 <= k <= 16 and k <= E <= 256 (k=%d E=%d)", d.top_k,
                d.n_experts);
  return MOE_OK;
}

#define CHECK_PTR(p)                                                   \
  do {                                                                 \
    if (!(p)) return fail(MOE_ERR_ARG, "%s: %s is null", fn, #p);      \
  } while (0)
#define CHECK_ALIGN(p)                                                                   \
  do {                                                                                   \
    if ((p) && !aligned16(p)) return fail(MOE_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, #p); \
  } while (0)

moe_status check_slots(const char* fn, const int32_t* slot_of_expert, int32_t n_slots,
                       const uint8_t* arena, int64_t slot_stride, const moe_dims& dims) {
  CHECK_PTR(slot_of_expert);
  CHECK_PTR(arena);
  CHECK_ALIGN(slot_of_expert);
  if (n_slots < 1) return fail(MOE_ERR_ARG, "%s: n_slots=%d", fn, n_slots);
  if (reinterpret_cast<uintptr_t>(arena) % 256) return fail(MOE_ERR_ALIGN, "%s: arena not 256-byte aligned", fn);
  const int64_t blob = moe_expert_blob_bytes(dims);
  if (slot_stride % 256 || slot_stride < blob)
    return fail(MOE_ERR_ARG, "%s: slot_stride=%lld must be a multiple of 256 and >= %lld", fn,
                (long long)slot_stride, (long long)blob);
  return MOE_OK;
}

}  // namespace

namespace {
struct ProfileArm {
  int call = -1;
  hipEvent_t start = nullptr, stop = nullptr;
};
thread_local ProfileArm g_profile;
}  // namespace

bool moe::take_profile_events(int call, hipEvent_t* start, hipEvent_t* stop) {
  if (g_profile.call != call || !g_profile.start || !g_profile.stop) return false;
  *start = g_profile.start;
  *stop = g_profile.stop;
  g_profile = ProfileArm{};
  return true;
}

namespace moe_bridge {
void set_error(const std::string& s) { g_last_error = s; }
}  // namespace moe_bridge

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_ARG: return "invalid argument";
    case MOE_ERR_ALIGN: return "misaligned buffer";
    case MOE_ERR_UNSUPPORTED: return "unsupported combination";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_STATE: return "invalid state";
    case MOE_ERR_CAPACITY: return "workspace too small";
  }
  return "unknown status";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

int64_t moe_expert_blob_bytes(moe_dims dims) {
  if (dims.d <= 0 || dims.f <= 0 || dims.d % 64 || dims.f % 64) return -1;
  return moe::blob_layout(dims.d, dims.f).total;
}

moe_status moe_expert_blob_offsets(moe_dims dims, int64_t offsets[6]) {
  const char* fn = "moe_expert_blob_offsets";
  CHECK_PTR(offsets);
  if (dims.d <= 0 || dims.f <= 0 || dims.d % 64 || dims.f % 64)
    return fail(MOE_ERR_ARG, "dims: d=%d f=%d must be positive multiples of 64", dims.d, dims.f);
  const moe::BlobLayout b = moe::blob_layout(dims.d, dims.f);
  offsets[0] = b.gate_q;
  offsets[1] = b.up_q;
  offsets[2] = b.down_q;
  offsets[3] = b.gate_sb;
  offsets[4] = b.up_sb;
  offsets[5] = b.down_sb;
  return MOE_OK;
}

size_t moe_act_bytes(int32_t T, moe_dims dims, moe_precision prec) {
  if (T < 1 || check_dims(dims) != MOE_OK) return SIZE_MAX;
  switch (prec) {
    case MOE_PREC_FP32: return (size_t)T * dims.top_k * dims.f * 4;
    case MOE_PREC_F16_MFMA:
    case MOE_PREC_F16_MFMA_DIRECT: return moe::mfma_act_bytes(T, dims.f, dims.top_k);
    case MOE_PREC_BF16_MFMA: return SIZE_MAX;  // refused: see moe_precision
  }
  return SIZE_MAX;
}

size_t moe_workspace_size(moe_call call, int32_t T, moe_dims dims, moe_precision prec) {
  if (T < 1 || check_dims(dims) != MOE_OK) return SIZE_MAX;
  switch (call) {
    case MOE_CALL_ROUTE: return moe::route_workspace_bytes(T, dims.d, dims.n_experts);
    case MOE_CALL_PERMUTE: return moe::permute_workspace_bytes(T * dims.top_k, dims.n_experts);
    case MOE_CALL_GATEUP:
    case MOE_CALL_DOWN_COMBINE:
      if (prec == MOE_PREC_BF16_MFMA) return SIZE_MAX;  // refused: see moe_precision
      if (prec == MOE_PREC_F16_MFMA || prec == MOE_PREC_F16_MFMA_DIRECT)
        return moe::mfma_workspace_bytes((int)call, T, dims.d, dims.f, dims.n_experts, dims.top_k);
      return moe::gemv_workspace_bytes((int)call, T, dims.d, dims.top_k, true);
    case MOE_CALL_DECODE_LAYERS:  // T = number of layers
      return moe::decode_fused_workspace_bytes(T, dims.d, dims.f, dims.n_experts, dims.top_k);
  }
  return SIZE_MAX;
}

moe_status moe_route(const float* x, const float* norm_w, float eps, const float* router_w,
                     const float* router_bias, int32_t T, moe_dims dims, float* h_out,
                     int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* fn = "moe_route";
  if (moe_status s = check_dims(dims)) return s;
  if (T < 1) return fail(MOE_ERR_ARG, "%s: T=%d", fn, T);
  CHECK_PTR(x); CHECK_PTR(router_w); CHECK_PTR(h_out); CHECK_PTR(topk_idx); CHECK_PTR(topk_w); CHECK_PTR(ws);
  CHECK_ALIGN(x); CHECK_ALIGN(norm_w); CHECK_ALIGN(router_w); CHECK_ALIGN(router_bias);
  CHECK_ALIGN(h_out); CHECK_ALIGN(topk_idx); CHECK_ALIGN(topk_w); CHECK_ALIGN(ws);
  if (!(eps >= 0.0f)) return fail(MOE_ERR_ARG, "%s: eps must be >= 0", fn);
  const size_t need = moe::route_workspace_bytes(T, dims.d, dims.n_experts);
  if (ws_bytes < need) return fail(MOE_ERR_CAPACITY, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  hipError_t e = moe::launch_route(x, norm_w, eps, router_w, router_bias, T, dims.d, dims.n_experts,
                                   dims.top_k, h_out, topk_idx, topk_w, ws, stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, fn);
}

moe_status moe_route_noalloc(const float* x, const float* norm_w, float eps, const float* router_w,
                             const float* router_bias, int32_t T, moe_dims dims, float* h_out,
                             int32_t* topk_idx, float* topk_w, hipStream_t stream) {
  const char* fn = "moe_route_noalloc";
  if (moe_status s = check_dims(dims)) return s;
  if (T < 1) return fail(MOE_ERR_ARG, "%s: T=%d", fn, T);
  CHECK_PTR(x); CHECK_PTR(router_w); CHECK_PTR(h_out); CHECK_PTR(topk_idx); CHECK_PTR(topk_w);
  CHECK_ALIGN(x); CHECK_ALIGN(norm_w); CHECK_ALIGN(router_w); CHECK_ALIGN(router_bias);
  CHECK_ALIGN(h_out); CHECK_ALIGN(topk_idx); CHECK_ALIGN(topk_w);
  if (!(eps >= 0.0f)) return fail(MOE_ERR_ARG, "%s: eps must be >= 0", fn);
  const size_t need = moe::route_workspace_bytes(T, dims.d, dims.n_experts);
  if (need > moe::kRouteScratchBytes)
    return fail(MOE_ERR_CAPACITY, "%s: T=%d E=%d needs %zu bytes of scratch; this entry point holds %zu per device",
                fn, T, dims.n_experts, need, moe::kRouteScratchBytes);
  void* scratch = nullptr;
  hipError_t e = moe::route_scratch(&scratch);
  if (e != hipSuccess) return hip_fail(e, fn);
  e = moe::launch_route(x, norm_w, eps, router_w, router_bias, T, dims.d, dims.n_experts, dims.top_k, h_out,
                        topk_idx, topk_w, scratch, stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, fn);
}

moe_status moe_permute(const int32_t* topk_idx, int32_t T, moe_dims dims, int32_t* counts,
                       int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
  const char* fn = "moe_permute";
  if (moe_status s = check_dims(dims)) return s;
  if (T < 1 || (int64_t)T * dims.top_k > 65536) return fail(MOE_ERR_ARG, "%s: T=%d (T*k <= 65536)", fn, T);
  CHECK_PTR(topk_idx); CHECK_PTR(counts); CHECK_PTR(offsets); CHECK_PTR(sorted_pair); CHECK_PTR(pair_pos);
  CHECK_ALIGN(topk_idx); CHECK_ALIGN(counts); CHECK_ALIGN(offsets); CHECK_ALIGN(sorted_pair); CHECK_ALIGN(pair_pos);
  CHECK_ALIGN(ws);
  hipError_t e = moe::launch_permute(topk_idx, T * dims.top_k, dims.n_experts, counts, offsets,
                                     sorted_pair, pair_pos, ws, ws ? ws_bytes : 0, stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, fn);
}

moe_status moe_expert_q4_gateup(const float* h, const int32_t* topk_idx, const int32_t* slot_of_expert,
                                int32_t n_slots, const uint8_t* arena, int64_t slot_stride,
                                const int32_t* offsets, const int32_t* sorted_pair,
                                const uint8_t* pair_mask, int32_t mask_value, int32_t T, moe_dims dims,
                                moe_precision prec, void* act, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  const char* fn = "moe_expert_q4_gateup";
  if (moe_status s = check_dims(dims)) return s;
  if (T < 1) return fail(MOE_ERR_ARG, "%s: T=%d", fn, T);
  CHECK_PTR(h); CHECK_PTR(topk_idx); CHECK_PTR(act);
  CHECK_ALIGN(h); CHECK_ALIGN(topk_idx); CHECK_ALIGN(act); CHECK_ALIGN(ws); CHECK_ALIGN(offsets);
  CHECK_ALIGN(sorted_pair);
  if (moe_status s = check_slots(fn, slot_of_expert, n_slots, arena, slot_stride, dims)) return s;
  if ((offsets == nullptr) != (sorted_pair == nullptr))
    return fail(MOE_ERR_ARG, "%s: offsets and sorted_pair must both be given or both be null", fn);
  if (pair_mask && offsets)
    return fail(MOE_ERR_UNSUPPORTED, "%s: pair_mask works only on the ungrouped path", fn);
  const bool grouped = offsets != nullptr;
  const moe::BlobLayout L = moe::blob_layout(dims.d, dims.f);
  if (prec == MOE_PREC_FP32) {
    if (!moe::gemv_supported(dims.d, dims.f, dims.top_k))
      return fail(MOE_ERR_UNSUPPORTED, "%s: dims d=%d f=%d outside the fp32 kernels' range", fn, dims.d, dims.f);
    const size_t need = moe::gemv_workspace_bytes(MOE_CALL_GATEUP, T, dims.d, dims.top_k, grouped);
    if (ws_bytes < need) return fail(MOE_ERR_CAPACITY, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
    moe::GateupArgs a{};
    a.h = h; a.topk_idx = topk_idx; a.slot_of_expert = slot_of_expert; a.n_slots = n_slots;
    a.arena = arena; a.slot_stride = slot_stride; a.offsets = offsets; a.sorted_pair = sorted_pair;
    a.pair_mask = pair_mask; a.mask_value = mask_value;
    a.T = T; a.d = dims.d; a.f = dims.f; a.E = dims.n_experts; a.k = dims.top_k;
    a.off_q0 = L.gate_q; a.off_q1 = L.up_q; a.off_sb0 = L.gate_sb; a.off_sb1 = L.up_sb;
    a.act = reinterpret_cast<float*>(act);
    hipError_t e = moe::launch_gateup_fp32(a, stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, fn);
  }
  if (prec == MOE_PREC_BF16_MFMA)
    return fail(MOE_ERR_UNSUPPORTED,
                "%s: bf16 operands (8-bit significand) can miss the 1e-2 output tolerance on offset weights; "
                "MOE_PREC_F16_MFMA runs at the same MFMA rate with 3 more bits", fn);
  if (prec == MOE_PREC_F16_MFMA || prec == MOE_PREC_F16_MFMA_DIRECT) {
    if (!grouped)
      return fail(MOE_ERR_UNSUPPORTED, "%s: the MFMA path needs offsets and sorted_pair (moe_permute)", fn);
    if (!moe::mfma_supported(dims.d, dims.f))
      return fail(MOE_ERR_UNSUPPORTED, "%s: f=%d beyond the MFMA path's 8192 (128 groups of 64)", fn, dims.f);
    if ((int64_t)T * dims.top_k > kMaxMfmaPairs)
      return fail(MOE_ERR_ARG, "%s: T*k must be <= %d on the MFMA path", fn, kMaxMfmaPairs);
    if (!mfma_fits_32bit(T, dims, slot_stride))
      return fail(MOE_ERR_ARG, "%s: h, act and a slot must each stay below 2 GiB on the MFMA path", fn);
    const size_t need = moe::mfma_workspace_bytes(MOE_CALL_GATEUP, T, dims.d, dims.f, dims.n_experts, dims.top_k);
    if (!ws) return fail(MOE_ERR_ARG, "%s: ws is null", fn);
    if (ws_bytes < need) return fail(MOE_ERR_CAPACITY, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
    hipError_t e = moe::launch_gateup_mfma(prec == MOE_PREC_F16_MFMA_DIRECT, h, offsets, sorted_pair, slot_of_expert,
                                           n_slots, arena, slot_stride, T, dims.d, dims.f, dims.n_experts,
                                           dims.top_k, L.gate_q, L.up_q, L.gate_sb, L.up_sb, act, ws, stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, fn);
  }
  return fail(MOE_ERR_UNSUPPORTED, "%s: precision %d not available", fn, (int)prec);
}

moe_status moe_expert_q4_down_combine(const void* act, const int32_t* topk_idx, const float* topk_w,
                                      const int32_t* slot_of_expert, int32_t n_slots,
                                      const uint8_t* arena, int64_t slot_stride, const int32_t* offsets,
                                      const int32_t* sorted_pair, const int32_t* pair_pos,
                                      const float* residual, int32_t T, moe_dims dims,
                                      moe_precision prec, float* y, void* ws, size_t ws_bytes,
                                      hipStream_t stream) {
  const char* fn = "moe_expert_q4_down_combine";
  (void)pair_pos;
  if (moe_status s = check_dims(dims)) return s;
  if (T < 1) return fail(MOE_ERR_ARG, "%s: T=%d", fn, T);
  CHECK_PTR(act); CHECK_PTR(topk_idx); CHECK_PTR(topk_w); CHECK_PTR(y);
  CHECK_ALIGN(act); CHECK_ALIGN(topk_idx); CHECK_ALIGN(topk_w); CHECK_ALIGN(y); CHECK_ALIGN(ws);
  CHECK_ALIGN(offsets); CHECK_ALIGN(sorted_pair); CHECK_ALIGN(pair_pos); CHECK_ALIGN(residual);
  if (moe_status s = check_slots(fn, slot_of_expert, n_slots, arena, slot_stride, dims)) return s;
  if ((offsets == nullptr) != (sorted_pair == nullptr))
    return fail(MOE_ERR_ARG, "%s: offsets and sorted_pair must both be given or both be null", fn);
  const bool grouped = offsets != nullptr;
  const moe::BlobLayout L = moe::blob_layout(dims.d, dims.f);
  if (prec == MOE_PREC_FP32) {
    if (!moe::gemv_supported(dims.d, dims.f, dims.top_k))
      return fail(MOE_ERR_UNSUPPORTED, "%s: dims d=%d f=%d outside the fp32 kernels' range", fn, dims.d, dims.f);
    const size_t need = moe::gemv_workspace_bytes(MOE_CALL_DOWN_COMBINE, T, dims.d, dims.top_k, grouped);
    if (ws_bytes < need) return fail(MOE_ERR_CAPACITY, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
    moe::DownArgs a{};
    a.act = reinterpret_cast<const float*>(act); a.topk_idx = topk_idx; a.topk_w = topk_w;
    a.slot_of_expert = slot_of_expert; a.n_slots = n_slots; a.arena = arena; a.slot_stride = slot_stride;
    a.offsets = offsets; a.sorted_pair = sorted_pair; a.residual = residual; a.y = y;
    a.T = T; a.d = dims.d; a.f = dims.f; a.E = dims.n_experts; a.k = dims.top_k;
    a.off_q = L.down_q; a.off_sb = L.down_sb;
    hipError_t e = moe::launch_down_fp32(a, ws, stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, fn);
  }
  if (prec == MOE_PREC_BF16_MFMA)
    return fail(MOE_ERR_UNSUPPORTED,
                "%s: bf16 operands (8-bit significand) can miss the 1e-2 output tolerance on offset weights; "
                "MOE_PREC_F16_MFMA runs at the same MFMA rate with 3 more bits", fn);
  if (prec == MOE_PREC_F16_MFMA || prec == MOE_PREC_F16_MFMA_DIRECT) {
    if (!grouped)
      return fail(MOE_ERR_UNSUPPORTED, "%s: the MFMA path needs offsets and sorted_pair (moe_permute)", fn);
    if (!moe::mfma_supported(dims.d, dims.f))
      return fail(MOE_ERR_UNSUPPORTED, "%s: f=%d beyond the MFMA path's 8192 (128 groups of 64)", fn, dims.f);
    if ((int64_t)T * dims.top_k > kMaxMfmaPairs)
      return fail(MOE_ERR_ARG, "%s: T*k must be <= %d on the MFMA path", fn, kMaxMfmaPairs);
    if (!mfma_fits_32bit(T, dims, slot_stride))
      return fail(MOE_ERR_ARG, "%s: h, act and a slot must each stay below 2 GiB on the MFMA path", fn);
    const size_t need =
        moe::mfma_workspace_bytes(MOE_CALL_DOWN_COMBINE, T, dims.d, dims.f, dims.n_experts, dims.top_k);
    if (!ws) return fail(MOE_ERR_ARG, "%s: ws is null", fn);
    if (ws_bytes < need) return fail(MOE_ERR_CAPACITY, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
    hipError_t e = moe::launch_down_mfma(prec == MOE_PREC_F16_MFMA_DIRECT, act, offsets, sorted_pair, slot_of_expert,
                                         n_slots, arena, slot_stride, T, dims.d, dims.f, dims.n_experts,
                                         dims.top_k, L.down_q, L.down_sb, topk_w, residual, y, ws, stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, fn);
  }
  return fail(MOE_ERR_UNSUPPORTED, "%s: precision %d not available", fn, (int)prec);
}

moe_status moe_shared_gemv_bf16(const uint16_t* w, const float* h, int32_t T, int32_t rows,
                                int32_t cols, float* out, hipStream_t stream) {
  const char* fn = "moe_shared_gemv_bf16";
  CHECK_PTR(w); CHECK_PTR(h); CHECK_PTR(out);
  CHECK_ALIGN(w); CHECK_ALIGN(h); CHECK_ALIGN(out);
  if (T < 1 || rows < 1 || cols < 8 || cols % 8)
    return fail(MOE_ERR_ARG, "%s: T=%d rows=%d cols=%d (cols %% 8 == 0)", fn, T, rows, cols);
  hipError_t e = moe::launch_shared_gemv_bf16(w, h, T, rows, cols, out, stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, fn);
}

size_t moe_shared_expert_workspace_size(int32_t T, int32_t f_sh) {
  if (T < 1 || f_sh < 8 || f_sh % 8) return SIZE_MAX;
  return moe::shared_expert_workspace_bytes(T, f_sh);
}

moe_status moe_shared_expert_bf16(const uint16_t* w_gu, const uint16_t* w_down, const float* h,
                                  const float* residual, int32_t T, int32_t d, int32_t f_sh, float* out,
                                  void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* fn = "moe_shared_expert_bf16";
  CHECK_PTR(w_gu); CHECK_PTR(w_down); CHECK_PTR(h); CHECK_PTR(out); CHECK_PTR(ws);
  CHECK_ALIGN(w_gu); CHECK_ALIGN(w_down); CHECK_ALIGN(h); CHECK_ALIGN(out); CHECK_ALIGN(ws);
  if (residual) CHECK_ALIGN(residual);
  if (T < 1 || d < 8 || d % 8 || f_sh < 8 || f_sh % 8)
    return fail(MOE_ERR_ARG, "%s: T=%d d=%d f_sh=%d (d, f_sh multiples of 8)", fn, T, d, f_sh);
  if (ws_bytes < moe::shared_expert_workspace_bytes(T, f_sh))
    return fail(MOE_ERR_CAPACITY, "%s: workspace of %zu bytes, need %zu", fn, ws_bytes,
                moe::shared_expert_workspace_bytes(T, f_sh));
  hipError_t e = moe::launch_shared_expert_bf16(w_gu, w_down, h, residual, T, d, f_sh, out, ws, stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, fn);
}

static int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return cus;
}

moe_status moe_decode_layers(float* x_io, int32_t n_layers, const float* norm_w, float eps,
                             const float* router_w, const float* router_bias,
                             const int32_t* slot_tables, int32_t n_slots, const uint8_t* arena,
                             int64_t layer_stride, int64_t slot_stride, moe_dims dims,
                             int32_t* topk_idx, float* topk_w, float* x_next,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* fn = "moe_decode_layers";
  if (moe_status s = check_dims(dims)) return s;
  if (n_layers < 1) return fail(MOE_ERR_ARG, "%s: n_layers=%d", fn, n_layers);
  CHECK_PTR(x_io); CHECK_PTR(router_w); CHECK_PTR(topk_idx); CHECK_PTR(topk_w); CHECK_PTR(ws);
  CHECK_ALIGN(x_io); CHECK_ALIGN(norm_w); CHECK_ALIGN(router_w); CHECK_ALIGN(router_bias);
  CHECK_ALIGN(topk_idx); CHECK_ALIGN(topk_w); CHECK_ALIGN(x_next); CHECK_ALIGN(ws);
  if (!(eps >= 0.0f)) return fail(MOE_ERR_ARG, "%s: eps must be >= 0", fn);
  if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(MOE_ERR_ALIGN, "%s: ws must be 256-byte aligned", fn);
  if (moe_status s = check_slots(fn, slot_tables, n_slots, arena, slot_stride, dims)) return s;
  if (layer_stride % 256 || layer_stride < (int64_t)n_slots * slot_stride)
    return fail(MOE_ERR_ARG, "%s: layer_stride=%lld must be a multiple of 256 and >= n_slots * slot_stride", fn,
                (long long)layer_stride);
  int G = 0, rpw = 0;
  if (!moe::decode_fused_supported(dims.d, dims.f, dims.n_experts, dims.top_k, device_cus(), &G, &rpw))
    return fail(MOE_ERR_UNSUPPORTED, "%s: dims d=%d f=%d E=%d k=%d outside the fused kernel's range", fn, dims.d,
                dims.f, dims.n_experts, dims.top_k);
  const size_t need = moe::decode_fused_workspace_bytes(n_layers, dims.d, dims.f, dims.n_experts, dims.top_k);
  if (ws_bytes < need) return fail(MOE_ERR_CAPACITY, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  const moe::BlobLayout L = moe::blob_layout(dims.d, dims.f);
  hipError_t e = moe::launch_decode_fused(x_io, n_layers, norm_w, eps, router_w, router_bias, slot_tables, n_slots,
                                          arena, layer_stride, slot_stride, dims.d, dims.f, dims.n_experts,
                                          dims.top_k, L.gate_q, L.up_q, L.down_q, L.gate_sb, L.up_sb, L.down_sb,
                                          topk_idx, topk_w, x_next, ws, G, rpw, stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, fn);
}

moe_status moe_decode_check(const void* ws, hipStream_t stream) {
  const char* fn = "moe_decode_check";
  CHECK_PTR(ws);
  uint32_t flag = 0;
  hipError_t e = hipMemcpyAsync(&flag, reinterpret_cast<const char*>(ws) + moe::kDecodeErrOffset, 4,
                                hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, fn);
  if (flag == 2u) return fail(MOE_ERR_STATE, "%s: the workspace was laid out for other shapes (zero-fill it)", fn);
  if (flag) return fail(MOE_ERR_STATE, "%s: a wait for another workgroup's values timed out", fn);
  return MOE_OK;
}

moe_status moe_profile_next_launch(moe_call call, hipEvent_t start, hipEvent_t stop) {
  if ((int)call < 0 || (int)call > MOE_CALL_DECODE_LAYERS)
    return fail(MOE_ERR_ARG, "moe_profile_next_launch: unknown call %d", (int)call);
  g_profile.call = (start && stop) ? (int)call : -1;
  g_profile.start = start;
  g_profile.stop = stop;
  return MOE_OK;
}

moe_status moe_rms_rescale(const float* x, int32_t T, int32_t d, float eps, float* out,
                           hipStream_t stream) {
  const char* fn = "moe_rms_rescale";
  CHECK_PTR(x); CHECK_PTR(out);
  CHECK_ALIGN(x); CHECK_ALIGN(out);
  if (T < 1 || d < 4 || d % 4) return fail(MOE_ERR_ARG, "%s: T=%d d=%d", fn, T, d);
  hipError_t e = moe::launch_rms_rescale(x, T, d, eps, out, stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, fn);
}

}  // extern "C"
