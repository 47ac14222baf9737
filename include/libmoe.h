/*
 * libmoe — routed int4 mixture-of-experts layer for AMD Instinct MI355X (gfx950).
 *
 * One MoE layer as the pages describe it: a small router picks 8 of 128
 * feed-forward experts per token and only those run (TurboFieldfare video
 * transcript, paragraph on Gemma 4 as a mixture-of-experts model); the experts'
 * projections are INT4 in affine groups of 64 with a scale and a bias per group
 * ("Optimizing a 14.3 GB model for an 8 GB machine", section "Vectorization
 * helped when it respected the storage layout"); expert weights are read through
 * preallocated per-layer cache slots kept by a bounded cache (same page, sections
 * "Explicit reads made expert streaming work" and "MoE needed parallel work,
 * reuse, and coarse overlap").
 *
 * Conventions shared by every call
 *  - Every pointer named *_dev or documented as "device" is device memory the
 *    caller allocated (hipMalloc or a torch tensor); *_host is host memory.
 *    The library keeps no pointer after a call returns, except those registered
 *    with moe_cache_create.  It allocates no device memory on any compute call;
 *    the only set-up calls that do are moe_cache_enable_device (the cache's
 *    device state) and moe_cache_set_staging (its copy streams).
 *  - Every compute call is asynchronous and ordered on the stream it is given
 *    (0 = the null stream).  Argument checks run on the host before anything is
 *    enqueued; a failed check enqueues nothing and returns an error code.
 *    Faults inside kernels surface at the next synchronisation as HIP errors.
 *  - Float and int32 buffers must be 16-byte aligned (MOE_ERR_ALIGN otherwise):
 *    kernels use 128-bit loads and the pages show what a wider load does to a
 *    sub-tensor that is only 2-byte aligned (same page, section
 *    "Vectorization helped when it respected the storage layout").
 *  - Workspaces ("ws") are caller-owned device buffers of moe_workspace_size()
 *    bytes.  A workspace must be zero-filled before its first use; every call
 *    leaves the counters it uses at zero again, so it can be reused by later
 *    calls on the same stream without clearing.  Two calls in flight at the same
 *    time must not share a workspace.
 *  - moe_last_error() returns a thread-local text for the last failing call.
 *
 * Dimensions (moe_dims): d = hidden size, f = expert width, n_experts = E,
 * top_k = k.  Requirements: d % 64 == 0, f % 64 == 0, 1 <= k <= 16,
 * k <= E <= 256.  The layer the pages describe has d = 2816, f = 704, E = 128,
 * k = 8.  Token t's j-th routed expert forms the pair p = t * k + j.
 *
 * Expert blob format (one expert; byte offsets from moe_expert_blob_offsets):
 *   six sections, each starting on a 256-byte boundary, in this order:
 *   gate nibbles [f x d], up nibbles [f x d], down nibbles [d x f],
 *   gate (scale, bias) [f x d/64], up (scale, bias) [f x d/64],
 *   down (scale, bias) [d x f/64].
 *   A matrix of R rows (outputs) and C columns (inputs) stores element (r, c):
 *     nibble byte = (r/64)*(64*C/2) + (c/32)*1024 + (r%64)*16 + (c%32)/2,
 *                   low 4 bits for even c, high 4 bits for odd c;
 *     pair byte   = (r/64)*(64*(C/64)*4) + (c/64)*256 + (r%64)*4,
 *                   fp16 scale at +0 and fp16 bias at +2 (little-endian);
 *   and w[r][c] = scale * q + bias with q in 0..15.  Rows are tiled by 64 and,
 *   inside a tile, the 16-byte column chunks of the 64 rows sit side by side, so
 *   that one 64-lane wavefront reads 1 KiB contiguous per load with one row per
 *   lane.  Staging an expert copies its blob verbatim: the stored layout is the
 *   layout the kernels read (TurboFieldfare video transcript, paragraph on the
 *   installer storing weights in the kernel's layout).
 *
 * Expert FFN: act = gelu_tanh(W_gate h) * (W_up h);  out = W_down act, with
 * gelu_tanh(z) = 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))).
 * Routing: logits = W_router h (+ bias); the k largest logits are chosen (equal
 * logits: the lower expert id wins), in descending order; their weights are the
 * softmax over all E renormalised over the k chosen.
 * Combine: y[t] = residual[t] + sum_j w[t][j] * out[t*k+j], j in rank order.
 */
#ifndef LIBMOE_H
#define LIBMOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_ARG = 1,         /* null pointer, bad size or dimension */
  MOE_ERR_ALIGN = 2,       /* a buffer violates the alignment contract */
  MOE_ERR_UNSUPPORTED = 3, /* a valid combination this build does not implement */
  MOE_ERR_HIP = 4,         /* a HIP runtime call failed */
  MOE_ERR_STATE = 5,       /* a cache call in the wrong state */
  MOE_ERR_CAPACITY = 6     /* workspace too small */
} moe_status;

typedef struct moe_dims {
  int32_t d;         /* hidden size (router input, expert input and output) */
  int32_t f;         /* expert FFN width */
  int32_t n_experts; /* experts per layer, E */
  int32_t top_k;     /* experts chosen per token, k */
} moe_dims;

typedef enum moe_precision {
  MOE_PREC_FP32 = 0,      /* int4 weights, activations kept to ~fp32 accuracy, fp32 accumulate (decode) */
  MOE_PREC_BF16_MFMA = 1, /* refused (MOE_ERR_UNSUPPORTED): bf16 operands (8-bit significand) on
                             weights whose per-group means sit far from zero lose 1-6% per output
                             row to the cancellation of 2816-term sums, beyond the 1e-2 tolerance,
                             and fp16 runs at the same rate; the value is kept so that the codes
                             stay stable */
  MOE_PREC_F16_MFMA = 2,  /* grouped GEMM: int4 -> fp16 weights, fp16 activations, fp16 MFMA, fp32
                             accumulate: the same MFMA rate as bf16 with 3 more significand bits;
                             intermediate values are block-scaled, so fp16's range does not bind */
  MOE_PREC_F16_MFMA_DIRECT = 3  /* the same results as MOE_PREC_F16_MFMA, with the int4 weights loaded
                             straight into registers instead of through a staged LDS tile: the
                             ablation of the staged dequant tile ("Optimizing a 14.3 GB model for
                             an 8 GB machine", section "Splitting the work improved attention and
                             prefill": staged tiles against direct UInt4 reads) */
} moe_precision;

typedef enum moe_call {
  MOE_CALL_ROUTE = 0,
  MOE_CALL_PERMUTE = 1,
  MOE_CALL_GATEUP = 2,
  MOE_CALL_DOWN_COMBINE = 3,
  MOE_CALL_DECODE_LAYERS = 4
} moe_call;

/* Text of a status code, and the thread-local detail of the last failure. */
const char* moe_status_string(moe_status s);
const char* moe_last_error(void);

/* Bytes of one expert blob (format above), or -1 for invalid dims. */
int64_t moe_expert_blob_bytes(moe_dims dims);

/* Byte offsets of the six blob sections: gate_q, up_q, down_q, gate_sb, up_sb,
 * down_sb, written to offsets[0..5]. */
moe_status moe_expert_blob_offsets(moe_dims dims, int64_t offsets[6]);

/* Workspace bytes a call needs for T tokens (0 when it needs none; SIZE_MAX
 * for invalid dims). */
size_t moe_workspace_size(moe_call call, int32_t T, moe_dims dims, moe_precision prec);

/* Bytes of the act buffer that moe_expert_q4_gateup writes and
 * moe_expert_q4_down_combine reads, for T tokens at precision prec:
 *   MOE_PREC_FP32       fp32 [T*k][f].
 *   MOE_PREC_F16_MFMA*  block-scaled: fp16 values [T*k][f],
 *                       then int8 exponents [T*k][f/64] at byte offset
 *                       T*k*f*2.  Inside each block of 8 columns the values
 *                       are stored in the order 0,4,1,5,2,6,3,7 (the order the
 *                       matrix cores consume them): element (p, 8b + j) is
 *                       value[p][8b + pos(j)] * 2^exp[p][(8b + j) / 64] with
 *                       pos(j) = 2*(j%4) + j/4.  fp16 exponents are shared by
 *                       the pairs an expert processes together and put the
 *                       group's largest magnitude in [2^14, 2^15).
 * SIZE_MAX for invalid dims. */
size_t moe_act_bytes(int32_t T, moe_dims dims, moe_precision prec);

/* ---------------------------------------------------------------------------
 * moe_route — RMSNorm, router matvec, softmax, top-k, renormalisation.
 * The router picks 8 of 128 experts from the layer's input (TurboFieldfare
 * video transcript, paragraphs on the router naming the experts it wants).
 *   x        device fp32 [T][d]      layer input (residual stream)
 *   norm_w   device fp32 [d] or NULL RMSNorm weight; NULL: h = x (no norm)
 *   eps      RMSNorm epsilon: h = x / sqrt(mean(x^2) + eps) * norm_w
 *   router_w device fp32 [E][d]      router matrix, row-major
 *   router_bias device fp32 [E] or NULL   added to the logits
 *   h_out    device fp32 [T][d]      the normalised input the experts read
 *   topk_idx device int32 [T][k]     chosen experts, descending logit order
 *   topk_w   device fp32 [T][k]      their renormalised softmax weights
 *   ws       workspace of moe_workspace_size(MOE_CALL_ROUTE, T, ...) bytes
 * Errors: MOE_ERR_ARG (null/bad dims/T < 1), MOE_ERR_ALIGN, MOE_ERR_CAPACITY.
 * NaN logits are outside the contract.
 * ------------------------------------------------------------------------- */
moe_status moe_route(const float* x, const float* norm_w, float eps,
                     const float* router_w, const float* router_bias,
                     int32_t T, moe_dims dims,
                     float* h_out, int32_t* topk_idx, float* topk_w,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_route_noalloc — moe_route without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, results and
 * errors as moe_route, bit for bit.  Its scratch is a static device array of
 * 16 MiB per GPU (held until the process ends; looked up once per device on
 * the first call there), so the call allocates nothing.  Calls needing more
 * scratch than that (moe_workspace_size(MOE_CALL_ROUTE, T, ...) > 16 MiB,
 * e.g. more than about 4000 tokens at E = 256) return MOE_ERR_CAPACITY.
 * Every call on one GPU shares the array: calls that overlap in time on one
 * GPU (on different streams, or from different threads) race and must not be
 * issued.  A HIP failure to find the array gives MOE_ERR_HIP.
 * ------------------------------------------------------------------------- */
moe_status moe_route_noalloc(const float* x, const float* norm_w, float eps,
                             const float* router_w, const float* router_bias,
                             int32_t T, moe_dims dims,
                             float* h_out, int32_t* topk_idx, float* topk_w,
                             hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_permute — group the T*k (token, rank) pairs by expert so that all tokens
 * routed to one expert run against one read of its weights (the batched routed
 * MoE of "Optimizing a 14.3 GB model for an 8 GB machine", section "Splitting
 * the work improved attention and prefill").
 *   topk_idx    device int32 [T][k]   from moe_route (values in 0..E-1)
 *   counts      device int32 [E]      pairs per expert
 *   offsets     device int32 [E+1]    exclusive prefix sum of counts; offsets[E] = T*k
 *   sorted_pair device int32 [T*k]    pair ids grouped by expert, ascending inside a group
 *   pair_pos    device int32 [T*k]    inverse: sorted_pair[pair_pos[p]] = p
 *   ws          device, moe_workspace_size(MOE_CALL_PERMUTE) bytes (non-zero
 *               past 1024 pairs), or NULL.  Given: chunks of 1024 pairs are
 *               ranked by one workgroup each and placed by a second launch.
 *               NULL (or too small): one workgroup walks every pair (slower
 *               for many pairs).  The outputs are the same either way.
 * Deterministic; no atomics whose order reaches the output.  T*k <= 65536.
 * Errors: MOE_ERR_ARG, MOE_ERR_ALIGN.
 * ------------------------------------------------------------------------- */
moe_status moe_permute(const int32_t* topk_idx, int32_t T, moe_dims dims,
                       int32_t* counts, int32_t* offsets,
                       int32_t* sorted_pair, int32_t* pair_pos,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_expert_q4_gateup — act[p] = gelu_tanh(W_gate[e] h[t]) * (W_up[e] h[t])
 * for every pair p = t*k + j with e = topk_idx[p]; the expert's blob is found
 * through the layer's slot table: arena + slot_of_expert[e] * slot_stride
 * (preallocated per-layer cache slots, "Optimizing a 14.3 GB model for an 8 GB
 * machine", section "Explicit reads made expert streaming work").
 *   h              device fp32 [T][d]     from moe_route
 *   topk_idx       device int32 [T][k]
 *   slot_of_expert device int32 [E]       this layer's slot per expert (-1 = absent)
 *   n_slots        slots in the arena; a pair whose slot is outside 0..n_slots-1
 *                  gets NaN outputs instead of a read
 *   arena          device, n_slots * slot_stride bytes, 256-byte aligned
 *   slot_stride    bytes between slots, a multiple of 256, >= blob bytes
 *   offsets, sorted_pair  device, from moe_permute, or both NULL.  Given: each
 *                  expert's weights are read once for all its pairs.  NULL:
 *                  every pair reads its expert on its own (batch-1 decode).
 *   pair_mask      device uint8 [T*k] or NULL: only pairs with
 *                  pair_mask[p] == mask_value are computed, the others are left
 *                  untouched (cache hits first, then the misses, "Optimizing a
 *                  14.3 GB model for an 8 GB machine", section "MoE needed
 *                  parallel work, reuse, and coarse overlap").  Only with
 *                  offsets == NULL.
 *   prec           MOE_PREC_FP32: act is fp32 [T*k][f];
 *                  MOE_PREC_F16_MFMA(_DIRECT): grouped GEMM on MFMA
 *                  (needs offsets, T*k <= 2^22); act is block-scaled 16-bit
 *                  (layout and size: moe_act_bytes).  With few tokens, experts
 *                  of at most 32 routed rows are split along K over several
 *                  workgroups; their partial sums and arrival counters live in
 *                  ws, and the result is the same bits whichever arrives last.
 *   act            device, moe_act_bytes(T, dims, prec) bytes
 * Errors: MOE_ERR_ARG, MOE_ERR_ALIGN, MOE_ERR_CAPACITY, MOE_ERR_UNSUPPORTED.
 * ------------------------------------------------------------------------- */
moe_status moe_expert_q4_gateup(const float* h, const int32_t* topk_idx,
                                const int32_t* slot_of_expert, int32_t n_slots,
                                const uint8_t* arena, int64_t slot_stride,
                                const int32_t* offsets, const int32_t* sorted_pair,
                                const uint8_t* pair_mask, int32_t mask_value,
                                int32_t T, moe_dims dims, moe_precision prec,
                                void* act, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_expert_q4_down_combine — out[p] = W_down[e] act[p], then
 * y[t] = residual[t] + sum_j topk_w[t][j] * out[t*k+j], summed in rank order
 * (deterministic).  The token's output mixes only the experts its router
 * named, weighted by the router (TurboFieldfare video transcript, paragraph
 * on Gemma 4 as a mixture-of-experts model; "Optimizing a 14.3 GB model for an
 * 8 GB machine", section "MoE needed parallel work, reuse, and coarse
 * overlap": the routed MoE of each layer).  Same slot-table, offsets and
 * precision rules as gateup.
 *   act       device, from moe_expert_q4_gateup at the same prec (layout: moe_act_bytes)
 *   topk_w    device fp32 [T][k]
 *   pair_pos  device int32 [T*k] from moe_permute, or NULL with offsets NULL
 *   residual  device fp32 [T][d] or NULL (then y is the expert mix alone);
 *             may equal y (in place)
 *   y         device fp32 [T][d]
 * Errors: MOE_ERR_ARG, MOE_ERR_ALIGN, MOE_ERR_CAPACITY, MOE_ERR_UNSUPPORTED.
 * ------------------------------------------------------------------------- */
moe_status moe_expert_q4_down_combine(const void* act, const int32_t* topk_idx, const float* topk_w,
                                      const int32_t* slot_of_expert, int32_t n_slots,
                                      const uint8_t* arena, int64_t slot_stride,
                                      const int32_t* offsets, const int32_t* sorted_pair,
                                      const int32_t* pair_pos, const float* residual,
                                      int32_t T, moe_dims dims, moe_precision prec,
                                      float* y, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Bounded per-layer expert cache with side-stream staging.
 * A cache keeps, for each of n_layers layers, n_slots device slots of an arena
 * and the expert each holds; misses are copied from a pinned host pool into the
 * least-recently-used slot on a side stream while the compute stream runs other
 * work (bounded per-layer cache: "Optimizing a 14.3 GB model for an 8 GB
 * machine", section "MoE needed parallel work, reuse, and coarse overlap";
 * LRU over resident slots: goinfer "When the model doesn't fit").
 * LRU rule per layer, step t, selection S: first every hit is stamped t; then
 * each miss, in ascending expert id, takes the slot with the smallest
 * (stamp, slot index); empty slots have stamp -1 and so fill lowest first.
 * ------------------------------------------------------------------------- */
typedef struct moe_cache moe_cache;

typedef struct moe_stage_stats {
  int64_t hits;         /* cumulative over the cache's life */
  int64_t misses;
  int64_t bytes_staged;
} moe_stage_stats;

/* host_pool: pinned host memory, n_layers * n_experts * blob_bytes, expert
 *   (l, e) at ((l * n_experts) + e) * blob_bytes (registered, not copied).
 * arena: device, n_layers * n_slots * slot_stride bytes; slot s of layer l at
 *   ((l * n_slots) + s) * slot_stride.
 * slot_tables: device int32 [n_layers][n_experts]; the cache writes it (-1 =
 *   not resident) and kernels read it as slot_of_expert = slot_tables + l * E.
 *   The cache fills it with -1 on creation (synchronously).
 * Requires top_k <= n_slots <= n_experts. */
moe_status moe_cache_create(int32_t n_layers, int32_t n_experts, int32_t n_slots, int32_t top_k,
                            const uint8_t* host_pool, int64_t blob_bytes,
                            uint8_t* arena, int64_t slot_stride,
                            int32_t* slot_tables, moe_cache** out);
moe_status moe_cache_destroy(moe_cache* c);

/* One step of one layer.  sel_host: the k chosen experts (host int32, rank
 * order).  Runs the LRU rule on the host, then enqueues on `side`: a wait for
 * all work already enqueued on `compute` (so no kernel still reads a victim
 * slot), the copy of the layer's new slot table, then one hipMemcpyAsync per
 * miss (pinned pool -> its slot).  hit_mask_dev (device uint8 [k]) receives 1 for
 * hits and 0 for misses through a copy enqueued on `compute`; hit_mask_host
 * (may be NULL) gets the same on return.  Entries of hit experts keep their
 * slot, so kernels for hits may run on `compute` before moe_cache_wait.
 * `step` is the stamp the rule records (callers pass a step counter; it
 * orders LRU choices), and the hit mask is how the caller runs cache hits
 * first and misses after moe_cache_wait ("Optimizing a 14.3 GB model for an
 * 8 GB machine", section "MoE needed parallel work, reuse, and coarse
 * overlap": cached hits first, then the experts that needed a read).
 * Failure: a HIP error (MOE_ERR_HIP) before the step's copies are enqueued
 * leaves the cache exactly as it was.  A failure after some were enqueued
 * leaves the rest as it was but empties the slots those copies target (they
 * may be overwritten): on the host at once, in the device table at the
 * layer's next call (until that call succeeds, kernels must not read the
 * layer's device table).  Once the step's copies, table copy and event are
 * enqueued the step is committed; if only the hit-mask copy then fails, the
 * call returns MOE_ERR_HIP with the step committed. */
moe_status moe_slot_stage(moe_cache* c, int32_t layer, int32_t step, const int32_t* sel_host,
                          hipStream_t side, hipStream_t compute,
                          uint8_t* hit_mask_dev, uint8_t* hit_mask_host,
                          moe_stage_stats* stats);
/* Eviction policy of a cache (default MOE_CACHE_LRU).  The pages replace LRU
 * by LFU, pushing out the expert used least, and try a 64-token LFU window
 * beside the whole-run count ("Optimizing a 14.3 GB model for an 8 GB
 * machine", section "MoE needed parallel work, reuse, and coarse overlap";
 * TurboFieldfare video transcript, paragraph on the expert cache).
 * Use count of expert e of a layer = the number of counted steps of that layer
 * (moe_slot_stage calls, the current one included) whose selection holds e:
 * every step so far for MOE_CACHE_LFU (resident or not), the last `window`
 * steps for MOE_CACHE_LFU_WINDOW.  A step stamps its hits first; then each
 * miss, in ascending expert id, takes the lowest empty slot, else the slot not
 * used in this step whose expert has the smallest (use count, stamp, slot).
 * window: 1..MOE_CACHE_MAX_WINDOW for MOE_CACHE_LFU_WINDOW, ignored otherwise.
 * Errors: MOE_ERR_ARG (unknown policy, window out of range), MOE_ERR_STATE
 * (called after the cache staged a step or imported usage). */
enum {
  MOE_CACHE_LRU = 0,
  MOE_CACHE_LFU = 1,
  MOE_CACHE_LFU_WINDOW = 2,
  MOE_CACHE_MAX_WINDOW = 4096
};
moe_status moe_cache_set_policy(moe_cache* c, int32_t policy, int32_t window);
/* Checkpoint of the use counts: counts_host int64 [n_layers][n_experts];
 * recent_host int32 [n_layers][window][top_k], the selections of each layer's
 * last `window` steps, oldest first, -1 before the first steps (required for
 * MOE_CACHE_LFU_WINDOW, unused otherwise).  Import checks that windowed counts
 * equal those of recent_host (else MOE_ERR_STATE); with moe_cache_export /
 * moe_cache_import it resumes a run exactly. */
moe_status moe_cache_export_usage(const moe_cache* c, int64_t* counts_host, int32_t* recent_host);
moe_status moe_cache_import_usage(moe_cache* c, const int64_t* counts_host, const int32_t* recent_host);
/* How misses are copied into their slots (default MOE_STAGE_COPY).  The pages
 * read misses explicitly into slots and keep several reads in flight
 * ("Optimizing a 14.3 GB model for an 8 GB machine", sections "Explicit reads
 * made expert streaming work" and "MoE needed parallel work, reuse, and coarse
 * overlap": bounded parallel reads).
 *   MOE_STAGE_COPY        one hipMemcpyAsync per miss on the side stream.
 *   MOE_STAGE_COPY_SPLIT  each blob cut into n_streams pieces (4 KiB
 *                         multiples), piece i copied on library-owned stream
 *                         i (2..MOE_STAGE_MAX_STREAMS), joined back into the
 *                         side stream.
 *   MOE_STAGE_KERNEL      one kernel launch on the side stream per step copies
 *                         all misses, the GPU reading the pinned pool through
 *                         its device mapping (checked here: a pool the device
 *                         cannot address, or blob_bytes % 16 != 0, gives
 *                         MOE_ERR_UNSUPPORTED).
 * Slot tables, hit masks and ordering against the compute stream are the same
 * in every mode.  Set once, before the first staged step (else MOE_ERR_STATE). */
enum {
  MOE_STAGE_COPY = 0,
  MOE_STAGE_COPY_SPLIT = 1,
  MOE_STAGE_KERNEL = 2,
  MOE_STAGE_MAX_STREAMS = 8
};
moe_status moe_cache_set_staging(moe_cache* c, int32_t mode, int32_t n_streams);
/* The cache on the device, for decode steps that never wait for the host.
 * After moe_cache_enable_device (which allocates the device copy of the cache
 * state and copies the current state there; LRU or whole-run LFU; the pool
 * must be device-mapped pinned memory, as for MOE_STAGE_KERNEL), each step of
 * a layer is moe_slot_stage_device instead of moe_slot_stage:
 *   sel_dev       device int32 [k]: the layer's chosen experts (a row of
 *                 moe_route's topk_idx), read on `compute`;
 *   on `compute`  one wave runs the same eviction rule as the host cache,
 *                 updates the device slot table and writes hit_mask_dev;
 *   on `side`     after that, one copy kernel pulls the misses' blobs from the
 *                 pinned pool into their slots (moe_cache_wait as before).
 * Nothing is copied to or waited for on the host.  moe_cache_slot_table,
 * moe_cache_export, moe_cache_export_usage and moe_cache_stats bring the host
 * view up to date first (they wait for the device).  In device mode
 * moe_slot_stage and moe_cache_import give MOE_ERR_STATE.  A selection out of
 * range or repeating an expert changes nothing and is reported as MOE_ERR_ARG
 * by the next call that reads the state back.  The ordering is the pages':
 * kernels of hits may run on `compute` before moe_cache_wait. */
moe_status moe_cache_enable_device(moe_cache* c);
moe_status moe_slot_stage_device(moe_cache* c, int32_t layer, int32_t step, const int32_t* sel_dev,
                                 hipStream_t side, hipStream_t compute, uint8_t* hit_mask_dev);
/* Cumulative hits, misses and staged bytes (device mode: waits for the device). */
moe_status moe_cache_stats(const moe_cache* c, moe_stage_stats* out);
/* Make `compute` wait until the layer's last staging has landed. */
moe_status moe_cache_wait(moe_cache* c, int32_t layer, hipStream_t compute);
/* Finer overlap: make `compute` wait only until the expert at rank `rank`
 * (0..top_k-1) of the layer's last moe_slot_stage step is in its slot, so that
 * its kernels can start while later misses are still being copied (the pages
 * try launching each routed expert as soon as its own read lands and measure
 * it against hits-first: "Optimizing a 14.3 GB model for an 8 GB machine",
 * section "MoE needed parallel work, reuse, and coarse overlap").  A hit
 * returns at once; in MOE_STAGE_COPY mode each miss has its own event (the
 * slot table is copied before the misses, so it is covered too); in the other
 * staging modes this waits for the whole step, as moe_cache_wait does.
 * Errors: MOE_ERR_ARG, MOE_ERR_STATE (device mode), MOE_ERR_HIP. */
moe_status moe_cache_wait_expert(moe_cache* c, int32_t layer, int32_t rank, hipStream_t compute);
/* Host copy of a layer's slot table (expert -> slot, -1 absent), int32 [E]. */
moe_status moe_cache_slot_table(const moe_cache* c, int32_t layer, int32_t* out_host);
/* Checkpoint: per layer the expert of each slot [L][S] and its stamp [L][S]. */
moe_status moe_cache_export(const moe_cache* c, int32_t* slot_expert_host, int64_t* stamp_host);
/* Restore exported state; rewrites the device slot tables synchronously.  The
 * arena contents are the caller's business (restage or keep). */
moe_status moe_cache_import(moe_cache* c, const int32_t* slot_expert_host, const int64_t* stamp_host);

/* ---------------------------------------------------------------------------
 * moe_decode_layers — batch-1 decode of one token through n_layers routed MoE
 * layers in one launch: per layer RMSNorm, router, softmax, top-k,
 * renormalised weights, the selected experts' int4 gate/up, GELU, down and the
 * rank-ordered combine with the residual, exactly as moe_route +
 * moe_expert_q4_gateup + moe_expert_q4_down_combine (MOE_PREC_FP32) compute
 * them, layer after layer (the routed MoE of "Optimizing a 14.3 GB model for an
 * 8 GB machine" and the router of the TurboFieldfare video transcript).  The
 * workgroups of the launch hand values to each other through the workspace
 * (written once per launch, read by polling until written) instead of kernel
 * boundaries or device-wide barriers.
 *   x_io         device fp32 [n_layers + 1][d]: x_io[0] is the input token;
 *                layer l writes its output (with the residual) to x_io[l + 1]
 *   norm_w       device fp32 [n_layers][d] or NULL (no RMSNorm)
 *   router_w     device fp32 [n_layers][E][d];  router_bias [n_layers][E] or NULL
 *   slot_tables  device int32 [n_layers][E]: layer l's slot per expert (-1 absent)
 *   arena        layer l's slot s at arena + l*layer_stride + s*slot_stride
 *                (256-byte aligned; layer_stride >= n_slots * slot_stride)
 *   topk_idx, topk_w  device [n_layers][k] (out): each layer's choice and weights
 *   x_next       device fp32 [d] or NULL: x_io[n_layers] rescaled to unit RMS
 *                (the next decode step's input; may be x_io itself)
 *   ws           256-byte aligned workspace of
 *                moe_workspace_size(MOE_CALL_DECODE_LAYERS, n_layers, ...)
 *                bytes (the T argument counts layers for this call),
 *                zero-filled before its first use and then passed
 *                unchanged to every call with the same n_layers and dims (it
 *                carries a launch count and two sets of exchange regions that
 *                alternate between launches); calls that share a workspace
 *                must be stream-ordered.  A call with other shapes on a used
 *                workspace writes nothing and sets the error word.
 * Requires the device to run all k*f/32 workgroups at once (one per compute
 * unit is enough); a value that does not arrive within ~0.25 s sets an error
 * word instead of hanging: moe_decode_check reports it.
 * Supported: d <= 3072, f <= 768, E <= 256, k <= 8, k * f / 32 <= 256 and
 * d <= 16 * k * f / 32; otherwise MOE_ERR_UNSUPPORTED.
 * Errors: MOE_ERR_ARG, MOE_ERR_ALIGN, MOE_ERR_CAPACITY, MOE_ERR_UNSUPPORTED.
 * ------------------------------------------------------------------------- */
moe_status moe_decode_layers(float* x_io, int32_t n_layers, const float* norm_w, float eps,
                             const float* router_w, const float* router_bias,
                             const int32_t* slot_tables, int32_t n_slots, const uint8_t* arena,
                             int64_t layer_stride, int64_t slot_stride, moe_dims dims,
                             int32_t* topk_idx, float* topk_w, float* x_next,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/* Waits for `stream` and reports MOE_ERR_STATE if a moe_decode_layers call on
 * this workspace hit its wait time limit or found the workspace laid out for
 * other shapes (its outputs are then invalid and the workspace must be
 * zero-filled again). */
moe_status moe_decode_check(const void* ws, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Shared-path GEMV with bf16 weights: out[t][r] = sum_c W[r][c] * h[t][c].
 * The always-resident work the GPU runs while expert misses are being copied
 * (coarse overlap: "Optimizing a 14.3 GB model for an 8 GB machine", section
 * "MoE needed parallel work, reuse, and coarse overlap").
 *   w   device bf16 bits [rows][cols] row-major, 16-byte aligned; cols % 8 == 0
 *   h   device fp32 [T][cols];  out device fp32 [T][rows]
 * ------------------------------------------------------------------------- */
moe_status moe_shared_gemv_bf16(const uint16_t* w, const float* h, int32_t T,
                                int32_t rows, int32_t cols, float* out, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * The always-resident shared expert, bf16 weights, in the routed experts'
 * gated form: out = residual + W_down (gelu_tanh(W_gate h) * (W_up h)).  One
 * shared expert runs for every token (TurboFieldfare video transcript,
 * paragraph on the two weight piles), and it is the work the GPU does while
 * expert misses are read ("Optimizing a 14.3 GB model for an 8 GB machine",
 * section "MoE needed parallel work, reuse, and coarse overlap").  Passing
 * `out` as the residual of moe_expert_q4_down_combine adds the routed experts
 * to it: y = (x + shared(h)) + sum_j w_j o_j.
 *   w_gu      device bf16 bits [2*f_sh][d]: the f_sh gate rows, then the f_sh up rows
 *   w_down    device bf16 bits [d][f_sh]
 *   h         device fp32 [T][d];  residual device fp32 [T][d] or NULL
 *   out       device fp32 [T][d] (may be the residual)
 *   ws        device, moe_shared_expert_workspace_size(T, f_sh) bytes (the fp32 act)
 * d and f_sh multiples of 8; 16-byte aligned pointers.
 * Errors: MOE_ERR_ARG, MOE_ERR_ALIGN, MOE_ERR_CAPACITY.
 * ------------------------------------------------------------------------- */
size_t moe_shared_expert_workspace_size(int32_t T, int32_t f_sh);
moe_status moe_shared_expert_bf16(const uint16_t* w_gu, const uint16_t* w_down, const float* h,
                                  const float* residual, int32_t T, int32_t d, int32_t f_sh, float* out,
                                  void* ws, size_t ws_bytes, hipStream_t stream);

/* Kernel timing: the next launch of `call`'s main kernel (the dequant-GEMV of
 * gate/up or down, or the router kernel) records `start` and `stop` at the
 * kernel's own begin and end (hipExtLaunchKernelGGL events), so the caller
 * can measure one kernel's duration on its stream without the launch gap.
 * One-shot and per calling thread; NULL events disarm. */
moe_status moe_profile_next_launch(moe_call call, hipEvent_t start, hipEvent_t stop);

/* Unit-RMS rescale out[t] = x[t] / sqrt(mean(x[t]^2) + eps), used to feed one
 * decode step's output back as the next step's input.  out may equal x. */
moe_status moe_rms_rescale(const float* x, int32_t T, int32_t d, float eps,
                           float* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBMOE_H */
