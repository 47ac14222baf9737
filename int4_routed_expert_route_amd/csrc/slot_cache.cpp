// Bounded per-layer expert cache: host LRU bookkeeping, pinned-host -> HBM
// staging of misses on a side stream, device slot tables.
//
// The pages keep a bounded number of routed experts per layer in preallocated
// slots, read misses explicitly into them, and run cached hits first while the
// misses are still arriving ("Optimizing a 14.3 GB model for an 8 GB machine",
// sections "Explicit reads made expert streaming work" and "MoE needed parallel
// work, reuse, and coarse overlap"); goinfer ("When the model doesn't fit")
// keeps an LRU over resident slots.  The first page then replaces LRU by LFU
// (the expert used least is pushed out) and tries a 64-token LFU window beside
// the whole-run count; both are policies here.  On MI355X the pool sits in
// pinned host memory and a miss is one DMA copy of the expert blob, verbatim,
// over PCIe.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/libmoe.h"
#include "kernels.h"

struct moe_cache {
  int L = 0, E = 0, S = 0, k = 0;
  const uint8_t* pool = nullptr;
  int64_t blob = 0;
  uint8_t* arena = nullptr;
  int64_t stride = 0;
  int32_t* tables_dev = nullptr;
  std::vector<int32_t> slot_expert;  // [L][S], -1 empty
  std::vector<int64_t> stamp;        // [L][S], -1 never used
  int32_t* table_host = nullptr;     // pinned [L][E]: source of the slot-table copies
  uint8_t* mask_host = nullptr;      // pinned [L][k]: source of the hit-mask copies
  std::vector<hipEvent_t> staged;    // per layer: last staging on the side stream
  std::vector<hipEvent_t> masked;    // per layer: last hit-mask copy on the compute stream
  std::vector<hipEvent_t> landed;    // [L][k]: MOE_STAGE_COPY, after the copy of the step's i-th miss
  std::vector<int32_t> rank_miss;    // [L][k]: miss index of the expert at rank j of the last step, -1 hit
  std::vector<char> staged_used, masked_used;
  std::vector<char> table_stale;     // per layer: a failed step left the device table behind the host state
  hipEvent_t compute_mark = nullptr;
  moe_stage_stats stats{0, 0, 0};
  // eviction policy (moe_cache_set_policy) and, for LFU, the use counts
  int policy = MOE_CACHE_LRU;
  int window = 0;                    // MOE_CACHE_LFU_WINDOW: steps counted
  std::vector<int64_t> count;        // [L][E] selections within the counted steps
  std::vector<int32_t> recent;       // [L][window][k] ring of the last selections, -1 = none
  std::vector<int64_t> steps_seen;   // [L] moe_slot_stage calls so far
  bool staged_any = false;
  // how misses are copied (moe_cache_set_staging)
  int staging = MOE_STAGE_COPY;
  std::vector<hipStream_t> helpers;  // MOE_STAGE_COPY_SPLIT: library-owned copy streams
  std::vector<hipEvent_t> joins;     // one per helper stream
  hipEvent_t fork = nullptr;
  const uint8_t* pool_dev = nullptr; // MOE_STAGE_KERNEL: the pool as the device addresses it
  // device mode (moe_cache_enable_device): the state lives in device memory
  bool device = false;
  int32_t* d_slot_expert = nullptr;  // [L][S]
  int64_t* d_stamp = nullptr;        // [L][S]
  int64_t* d_count = nullptr;        // [L][E]
  int32_t* d_miss = nullptr;         // [L][k][2]
  int32_t* d_nmiss = nullptr;        // [L]
  int64_t* d_stats = nullptr;        // [3]
  uint32_t* d_err = nullptr;         // [1]
  std::vector<hipEvent_t> routed;    // per layer: the rule has run on the compute stream
};

// Failures are reported through the library's thread-local error text (api.cpp).
namespace moe_bridge {
void set_error(const std::string& s);
}

namespace {

moe_status cfail(moe_status s, const std::string& msg) {
  moe_bridge::set_error(msg);
  return s;
}

moe_status hipcheck(hipError_t e, const char* what) {
  if (e == hipSuccess) return MOE_OK;
  return cfail(MOE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// The pinned source of a layer's slot-table copy, from a slot -> expert array.
void fill_table(moe_cache* c, int layer, const int32_t* se) {
  int32_t* t = c->table_host + (int64_t)layer * c->E;
  for (int e = 0; e < c->E; ++e) t[e] = -1;
  for (int s = 0; s < c->S; ++s)
    if (se[s] >= 0) t[se[s]] = s;
}

void rebuild_table(moe_cache* c, int layer) { fill_table(c, layer, c->slot_expert.data() + (int64_t)layer * c->S); }

// The device copy of the state (moe_cache_enable_device), also after a
// part-way failure of that call.
void release_device_state(moe_cache* c) {
  for (hipEvent_t& e : c->routed)
    if (e) { hipEventDestroy(e); e = nullptr; }
  c->routed.clear();
  for (void** p : {(void**)&c->d_slot_expert, (void**)&c->d_stamp, (void**)&c->d_count, (void**)&c->d_miss,
                   (void**)&c->d_nmiss, (void**)&c->d_stats, (void**)&c->d_err})
    if (*p) { hipFree(*p); *p = nullptr; }
}

// The helper streams of split staging, also after a part-way failure of
// moe_cache_set_staging.
void release_split_streams(moe_cache* c) {
  for (size_t i = 0; i < c->helpers.size(); ++i) {
    if (c->helpers[i]) { hipStreamSynchronize(c->helpers[i]); hipStreamDestroy(c->helpers[i]); }
    if (c->joins[i]) hipEventDestroy(c->joins[i]);
  }
  c->helpers.clear();
  c->joins.clear();
  if (c->fork) hipEventDestroy(c->fork);
  c->fork = nullptr;
}

// Device mode: bring the host mirror up to date (waits for the device).
moe_status pull_device_state(const moe_cache* cc) {
  moe_cache* c = const_cast<moe_cache*>(cc);
  if (!c->device) return MOE_OK;
  moe_status st;
  if ((st = hipcheck(hipDeviceSynchronize(), "hipDeviceSynchronize")) ||
      (st = hipcheck(hipMemcpy(c->slot_expert.data(), c->d_slot_expert, sizeof(int32_t) * c->slot_expert.size(),
                               hipMemcpyDeviceToHost), "hipMemcpy")) ||
      (st = hipcheck(hipMemcpy(c->stamp.data(), c->d_stamp, sizeof(int64_t) * c->stamp.size(), hipMemcpyDeviceToHost),
                     "hipMemcpy")) ||
      (st = hipcheck(hipMemcpy(c->count.data(), c->d_count, sizeof(int64_t) * c->count.size(), hipMemcpyDeviceToHost),
                     "hipMemcpy")))
    return st;
  int64_t stats[3];
  uint32_t err = 0;
  if ((st = hipcheck(hipMemcpy(stats, c->d_stats, sizeof(stats), hipMemcpyDeviceToHost), "hipMemcpy")) ||
      (st = hipcheck(hipMemcpy(&err, c->d_err, 4, hipMemcpyDeviceToHost), "hipMemcpy")))
    return st;
  c->stats = moe_stage_stats{stats[0], stats[1], stats[2]};
  if (err) return cfail(MOE_ERR_ARG, "device cache: a selection was out of range or repeated an expert");
  return MOE_OK;
}
}  // namespace

extern "C" {

moe_status moe_cache_create(int32_t n_layers, int32_t n_experts, int32_t n_slots, int32_t top_k,
                            const uint8_t* host_pool, int64_t blob_bytes, uint8_t* arena,
                            int64_t slot_stride, int32_t* slot_tables, moe_cache** out) {
  if (!out || !host_pool || !arena || !slot_tables)
    return cfail(MOE_ERR_ARG, "moe_cache_create: null pointer");
  *out = nullptr;
  if (n_layers < 1 || n_experts < 1 || n_experts > 256 || top_k < 1 || n_slots < top_k ||
      n_slots > n_experts || blob_bytes < 1 || slot_stride < blob_bytes || slot_stride % 256)
    return cfail(MOE_ERR_ARG, "moe_cache_create: bad sizes (need k <= slots <= experts <= 256, "
                              "slot_stride % 256 == 0 and >= blob_bytes)");
  if (reinterpret_cast<uintptr_t>(arena) % 256 || reinterpret_cast<uintptr_t>(slot_tables) % 16)
    return cfail(MOE_ERR_ALIGN, "moe_cache_create: arena must be 256-byte and tables 16-byte aligned");
  moe_cache* c = new moe_cache();
  c->L = n_layers; c->E = n_experts; c->S = n_slots; c->k = top_k;
  c->pool = host_pool; c->blob = blob_bytes; c->arena = arena; c->stride = slot_stride;
  c->tables_dev = slot_tables;
  c->slot_expert.assign((size_t)n_layers * n_slots, -1);
  c->stamp.assign((size_t)n_layers * n_slots, -1);
  c->staged.assign(n_layers, nullptr);
  c->landed.assign((size_t)n_layers * top_k, nullptr);
  c->rank_miss.assign((size_t)n_layers * top_k, -1);
  c->masked.assign(n_layers, nullptr);
  c->staged_used.assign(n_layers, 0);
  c->table_stale.assign(n_layers, 0);
  c->masked_used.assign(n_layers, 0);
  c->count.assign((size_t)n_layers * n_experts, 0);
  c->steps_seen.assign(n_layers, 0);
  moe_status st = MOE_OK;
  if ((st = hipcheck(hipHostMalloc((void**)&c->table_host, sizeof(int32_t) * n_layers * n_experts,
                                   hipHostMallocDefault), "hipHostMalloc")) ||
      (st = hipcheck(hipHostMalloc((void**)&c->mask_host, (size_t)n_layers * top_k, hipHostMallocDefault),
                     "hipHostMalloc")) ||
      (st = hipcheck(hipEventCreateWithFlags(&c->compute_mark, hipEventDisableTiming), "hipEventCreate"))) {
    moe_cache_destroy(c);
    return st;
  }
  for (int l = 0; l < n_layers; ++l) {
    if ((st = hipcheck(hipEventCreateWithFlags(&c->staged[l], hipEventDisableTiming), "hipEventCreate")) ||
        (st = hipcheck(hipEventCreateWithFlags(&c->masked[l], hipEventDisableTiming), "hipEventCreate"))) {
      moe_cache_destroy(c);
      return st;
    }
    for (int j = 0; j < top_k; ++j)
      if ((st = hipcheck(hipEventCreateWithFlags(&c->landed[(size_t)l * top_k + j], hipEventDisableTiming),
                         "hipEventCreate"))) {
        moe_cache_destroy(c);
        return st;
      }
    rebuild_table(c, l);
  }
  if ((st = hipcheck(hipMemcpy(slot_tables, c->table_host, sizeof(int32_t) * n_layers * n_experts,
                               hipMemcpyHostToDevice), "hipMemcpy"))) {
    moe_cache_destroy(c);
    return st;
  }
  *out = c;
  return MOE_OK;
}

moe_status moe_cache_destroy(moe_cache* c) {
  if (!c) return MOE_OK;
  if (c->device) hipDeviceSynchronize();
  release_device_state(c);
  release_split_streams(c);
  for (size_t l = 0; l < c->staged.size(); ++l) {
    if (c->staged[l]) { hipEventSynchronize(c->staged[l]); hipEventDestroy(c->staged[l]); }
    if (c->masked[l]) { hipEventSynchronize(c->masked[l]); hipEventDestroy(c->masked[l]); }
  }
  for (hipEvent_t e : c->landed)
    if (e) hipEventDestroy(e);
  if (c->compute_mark) hipEventDestroy(c->compute_mark);
  if (c->table_host) hipHostFree(c->table_host);
  if (c->mask_host) hipHostFree(c->mask_host);
  delete c;
  return MOE_OK;
}

moe_status moe_slot_stage(moe_cache* c, int32_t layer, int32_t step, const int32_t* sel_host,
                          hipStream_t side, hipStream_t compute, uint8_t* hit_mask_dev,
                          uint8_t* hit_mask_host, moe_stage_stats* stats) {
  if (!c || !sel_host || !hit_mask_dev) return cfail(MOE_ERR_ARG, "moe_slot_stage: null pointer");
  if (c->device) return cfail(MOE_ERR_STATE, "moe_slot_stage: the cache runs on the device (moe_slot_stage_device)");
  if (layer < 0 || layer >= c->L) return cfail(MOE_ERR_ARG, "moe_slot_stage: layer out of range");
  for (int j = 0; j < c->k; ++j) {
    if (sel_host[j] < 0 || sel_host[j] >= c->E)
      return cfail(MOE_ERR_ARG, "moe_slot_stage: expert id out of range");
    for (int i = 0; i < j; ++i)
      if (sel_host[i] == sel_host[j]) return cfail(MOE_ERR_ARG, "moe_slot_stage: repeated expert");
  }
  // The pinned sources of this layer's previous copies must have been consumed.
  moe_status st;
  if (c->staged_used[layer] && (st = hipcheck(hipEventSynchronize(c->staged[layer]), "hipEventSynchronize")))
    return st;
  if (c->masked_used[layer] && (st = hipcheck(hipEventSynchronize(c->masked[layer]), "hipEventSynchronize")))
    return st;
  // An earlier step of this layer failed after some of its copies were
  // enqueued: its victim slots were emptied on the host; the device table
  // follows before anything else is staged.
  if (c->table_stale[layer]) {
    rebuild_table(c, layer);
    if ((st = hipcheck(hipMemcpy(c->tables_dev + (int64_t)layer * c->E, c->table_host + (int64_t)layer * c->E,
                                 sizeof(int32_t) * c->E, hipMemcpyHostToDevice), "hipMemcpy")))
      return st;
    c->table_stale[layer] = 0;
  }

  // The step is worked out on copies of the layer's state and committed only
  // once every copy of it is enqueued; a failure before that leaves the state
  // as it was.
  std::vector<int32_t> se(c->slot_expert.begin() + (int64_t)layer * c->S,
                          c->slot_expert.begin() + (int64_t)(layer + 1) * c->S);
  std::vector<int64_t> sp(c->stamp.begin() + (int64_t)layer * c->S, c->stamp.begin() + (int64_t)(layer + 1) * c->S);
  std::vector<int64_t> cnt(c->count.begin() + (int64_t)layer * c->E, c->count.begin() + (int64_t)(layer + 1) * c->E);
  std::vector<int32_t> ring;
  int32_t* ring_at = nullptr;
  // expert -> slot for this layer
  std::vector<int> where(c->E, -1);
  for (int s = 0; s < c->S; ++s)
    if (se[s] >= 0) where[se[s]] = s;
  // use counts: this step's selection enters, and with a window the step
  // that falls out of it leaves
  if (c->policy == MOE_CACHE_LFU_WINDOW) {
    ring_at = c->recent.data() + ((int64_t)layer * c->window + c->steps_seen[layer] % c->window) * c->k;
    ring.assign(ring_at, ring_at + c->k);
    for (int j = 0; j < c->k; ++j) {
      if (ring[j] >= 0) --cnt[ring[j]];
      ring[j] = sel_host[j];
    }
  }
  for (int j = 0; j < c->k; ++j) ++cnt[sel_host[j]];
  // phase 1: stamp the hits
  std::vector<uint8_t> mask(c->k);
  std::vector<int> misses;
  for (int j = 0; j < c->k; ++j) {
    const int e = sel_host[j];
    mask[j] = where[e] >= 0 ? 1 : 0;
    if (where[e] >= 0) sp[where[e]] = step;
    else misses.push_back(e);
  }
  // phase 2: misses in ascending expert id take the (stamp, slot)-smallest slot
  std::vector<int> sorted = misses;
  for (size_t i = 1; i < sorted.size(); ++i)
    for (size_t j = i; j > 0 && sorted[j - 1] > sorted[j]; --j) std::swap(sorted[j - 1], sorted[j]);
  std::vector<std::pair<int, int>> installs;  // (expert, slot)
  for (int e : sorted) {
    int victim = 0;
    if (c->policy == MOE_CACHE_LRU) {
      // smallest (stamp, slot): empty slots (stamp -1) first
      for (int s = 1; s < c->S; ++s)
        if (sp[s] < sp[victim]) victim = s;
    } else {
      // lowest empty slot, else among slots not used in this step the
      // smallest (use count of its expert, stamp, slot)
      victim = -1;
      for (int s = 0; s < c->S && victim < 0; ++s)
        if (se[s] < 0) victim = s;
      if (victim < 0)
        for (int s = 0; s < c->S; ++s) {
          if (sp[s] == step) continue;
          if (victim < 0 || cnt[se[s]] < cnt[se[victim]] ||
              (cnt[se[s]] == cnt[se[victim]] && sp[s] < sp[victim]))
            victim = s;
        }
    }
    se[victim] = e;
    sp[victim] = step;
    installs.emplace_back(e, victim);
  }

  bool table_enqueued = false, copies_enqueued = false;
  auto failed = [&](moe_status err) {
    // Copies already enqueued may overwrite their victim slots: those slots no
    // longer hold the expert the old state names, so they become empty, on
    // the host now and on the device at the layer's next step.  The side
    // stream is drained first: its enqueued table copy reads the pinned table
    // this rewrites.
    if (table_enqueued || copies_enqueued) (void)hipStreamSynchronize(side);
    if (copies_enqueued)
      for (const auto& in : installs) {
        c->slot_expert[(int64_t)layer * c->S + in.second] = -1;
        c->stamp[(int64_t)layer * c->S + in.second] = -1;
      }
    if (table_enqueued) c->table_stale[layer] = 1;
    rebuild_table(c, layer);
    return err;
  };
  // enqueue: side waits for everything already on compute, then copies
  if ((st = hipcheck(hipEventRecord(c->compute_mark, compute), "hipEventRecord")) ||
      (st = hipcheck(hipStreamWaitEvent(side, c->compute_mark, 0), "hipStreamWaitEvent")))
    return failed(st);
  if (!installs.empty()) {
    // the layer's new slot table first: a wait on one miss's copy
    // (moe_cache_wait_expert) then also covers the table that names its slot
    fill_table(c, layer, se.data());
    table_enqueued = true;
    if ((st = hipcheck(hipMemcpyAsync(c->tables_dev + (int64_t)layer * c->E,
                                      c->table_host + (int64_t)layer * c->E, sizeof(int32_t) * c->E,
                                      hipMemcpyHostToDevice, side), "hipMemcpyAsync")))
      return failed(st);
    if (c->staging == MOE_STAGE_KERNEL) {
      // one launch per kMaxStageCopies misses; the GPU reads the pool itself
      for (size_t i0 = 0; i0 < installs.size(); i0 += moe::kMaxStageCopies) {
        moe::StageCopyArgs a{};
        a.bytes = c->blob;
        a.n = (int)std::min(installs.size() - i0, (size_t)moe::kMaxStageCopies);
        for (int i = 0; i < a.n; ++i) {
          a.src[i] = c->pool_dev + ((int64_t)layer * c->E + installs[i0 + i].first) * c->blob;
          a.dst[i] = c->arena + ((int64_t)layer * c->S + installs[i0 + i].second) * c->stride;
        }
        copies_enqueued = true;
        if ((st = hipcheck(moe::launch_stage_copy(a, side), "stage copy kernel"))) return failed(st);
      }
    } else if (c->staging == MOE_STAGE_COPY_SPLIT) {
      // each blob in as many pieces as helper streams, one piece per stream
      // (each stream can drive its own copy engine); `side` joins them
      const int n = (int)c->helpers.size();
      const int64_t piece = ((c->blob + n - 1) / n + 4095) / 4096 * 4096;
      if ((st = hipcheck(hipEventRecord(c->fork, side), "hipEventRecord"))) return failed(st);
      for (int i = 0; i < n; ++i) {
        if ((st = hipcheck(hipStreamWaitEvent(c->helpers[i], c->fork, 0), "hipStreamWaitEvent"))) return failed(st);
        for (const auto& in : installs) {
          const int64_t o = (int64_t)i * piece, len = std::min(piece, c->blob - o);
          if (len <= 0) continue;
          const uint8_t* src = c->pool + ((int64_t)layer * c->E + in.first) * c->blob + o;
          uint8_t* dst = c->arena + ((int64_t)layer * c->S + in.second) * c->stride + o;
          copies_enqueued = true;
          if ((st = hipcheck(hipMemcpyAsync(dst, src, len, hipMemcpyHostToDevice, c->helpers[i]), "hipMemcpyAsync")))
            return failed(st);
        }
        if ((st = hipcheck(hipEventRecord(c->joins[i], c->helpers[i]), "hipEventRecord")) ||
            (st = hipcheck(hipStreamWaitEvent(side, c->joins[i], 0), "hipStreamWaitEvent")))
          return failed(st);
      }
    } else {
      // one copy per miss, each followed by its own event (moe_cache_wait_expert)
      for (size_t i = 0; i < installs.size(); ++i) {
        const auto& in = installs[i];
        const uint8_t* src = c->pool + ((int64_t)layer * c->E + in.first) * c->blob;
        uint8_t* dst = c->arena + ((int64_t)layer * c->S + in.second) * c->stride;
        copies_enqueued = true;
        if ((st = hipcheck(hipMemcpyAsync(dst, src, c->blob, hipMemcpyHostToDevice, side), "hipMemcpyAsync")) ||
            (st = hipcheck(hipEventRecord(c->landed[(size_t)layer * c->k + i], side), "hipEventRecord")))
          return failed(st);
      }
    }
  }
  if ((st = hipcheck(hipEventRecord(c->staged[layer], side), "hipEventRecord"))) return failed(st);
  c->staged_used[layer] = 1;
  // commit: the copies, the table and the event are all enqueued
  std::copy(se.begin(), se.end(), c->slot_expert.begin() + (int64_t)layer * c->S);
  std::copy(sp.begin(), sp.end(), c->stamp.begin() + (int64_t)layer * c->S);
  std::copy(cnt.begin(), cnt.end(), c->count.begin() + (int64_t)layer * c->E);
  if (ring_at) std::copy(ring.begin(), ring.end(), ring_at);
  for (int j = 0; j < c->k; ++j) {
    int32_t& m = c->rank_miss[(size_t)layer * c->k + j];
    m = -1;
    for (size_t i = 0; i < installs.size(); ++i)
      if (installs[i].first == sel_host[j]) m = (int32_t)i;
  }
  ++c->steps_seen[layer];
  c->staged_any = true;
  c->stats.hits += c->k - (int64_t)misses.size();
  c->stats.misses += (int64_t)misses.size();
  c->stats.bytes_staged += (int64_t)misses.size() * c->blob;
  if (stats) *stats = c->stats;
  // the hit mask follows on the compute stream; if it cannot be enqueued the
  // staging above still stands (the state is committed) and the call fails
  uint8_t* pinned_mask = c->mask_host + (int64_t)layer * c->k;
  std::memcpy(pinned_mask, mask.data(), c->k);
  if ((st = hipcheck(hipMemcpyAsync(hit_mask_dev, pinned_mask, c->k, hipMemcpyHostToDevice, compute),
                     "hipMemcpyAsync")) ||
      (st = hipcheck(hipEventRecord(c->masked[layer], compute), "hipEventRecord")))
    return st;
  c->masked_used[layer] = 1;
  if (hit_mask_host) std::memcpy(hit_mask_host, mask.data(), c->k);
  return MOE_OK;
}

moe_status moe_cache_set_policy(moe_cache* c, int32_t policy, int32_t window) {
  if (!c) return cfail(MOE_ERR_ARG, "moe_cache_set_policy: null cache");
  if (policy != MOE_CACHE_LRU && policy != MOE_CACHE_LFU && policy != MOE_CACHE_LFU_WINDOW)
    return cfail(MOE_ERR_ARG, "moe_cache_set_policy: unknown policy");
  if (policy == MOE_CACHE_LFU_WINDOW && (window < 1 || window > MOE_CACHE_MAX_WINDOW))
    return cfail(MOE_ERR_ARG, "moe_cache_set_policy: window must be in 1..4096 steps");
  if (c->staged_any) return cfail(MOE_ERR_STATE, "moe_cache_set_policy: the cache has already staged a step");
  c->policy = policy;
  c->window = policy == MOE_CACHE_LFU_WINDOW ? window : 0;
  c->recent.assign((size_t)c->L * c->window * c->k, -1);
  return MOE_OK;
}

moe_status moe_cache_set_staging(moe_cache* c, int32_t mode, int32_t n_streams) {
  if (!c) return cfail(MOE_ERR_ARG, "moe_cache_set_staging: null cache");
  if (mode != MOE_STAGE_COPY && mode != MOE_STAGE_COPY_SPLIT && mode != MOE_STAGE_KERNEL)
    return cfail(MOE_ERR_ARG, "moe_cache_set_staging: unknown mode");
  if (mode == MOE_STAGE_COPY_SPLIT && (n_streams < 2 || n_streams > MOE_STAGE_MAX_STREAMS))
    return cfail(MOE_ERR_ARG, "moe_cache_set_staging: split staging needs 2..8 streams");
  if (c->staged_any || c->staging != MOE_STAGE_COPY)
    return cfail(MOE_ERR_STATE, "moe_cache_set_staging: set once, before the first staged step");
  moe_status st = MOE_OK;
  if (mode == MOE_STAGE_KERNEL) {
    // the kernel reads the pool through its device mapping; refuse a pool
    // the device cannot address instead of letting the kernel fault
    void* d = nullptr;
    if (c->blob % 16 || hipHostGetDevicePointer(&d, const_cast<uint8_t*>(c->pool), 0) != hipSuccess || !d ||
        reinterpret_cast<uintptr_t>(d) % 16) {
      (void)hipGetLastError();
      return cfail(MOE_ERR_UNSUPPORTED, "moe_cache_set_staging: the host pool is not device-mapped pinned memory "
                                        "(or blob_bytes % 16 != 0)");
    }
    c->pool_dev = static_cast<const uint8_t*>(d);
  } else if (mode == MOE_STAGE_COPY_SPLIT) {
    // a failure part-way releases what was made: the mode stays unset
    c->helpers.assign(n_streams, nullptr);
    c->joins.assign(n_streams, nullptr);
    if ((st = hipcheck(hipEventCreateWithFlags(&c->fork, hipEventDisableTiming), "hipEventCreate"))) {
      release_split_streams(c);
      return st;
    }
    for (int i = 0; i < n_streams; ++i)
      if ((st = hipcheck(hipStreamCreateWithFlags(&c->helpers[i], hipStreamNonBlocking), "hipStreamCreate")) ||
          (st = hipcheck(hipEventCreateWithFlags(&c->joins[i], hipEventDisableTiming), "hipEventCreate"))) {
        release_split_streams(c);
        return st;
      }
  }
  c->staging = mode;
  return MOE_OK;
}

moe_status moe_cache_export_usage(const moe_cache* c, int64_t* counts_host, int32_t* recent_host) {
  if (!c || !counts_host) return cfail(MOE_ERR_ARG, "moe_cache_export_usage: null pointer");
  moe_status pst = pull_device_state(c);
  if (pst) return pst;
  if (c->policy == MOE_CACHE_LFU_WINDOW && !recent_host)
    return cfail(MOE_ERR_ARG, "moe_cache_export_usage: the windowed policy needs recent_host");
  std::memcpy(counts_host, c->count.data(), sizeof(int64_t) * c->count.size());
  if (c->policy == MOE_CACHE_LFU_WINDOW)
    for (int l = 0; l < c->L; ++l)
      for (int i = 0; i < c->window; ++i) {
        // oldest first: the ring position the next step overwrites
        const int64_t pos = (c->steps_seen[l] + i) % c->window;
        std::memcpy(recent_host + ((int64_t)l * c->window + i) * c->k,
                    c->recent.data() + ((int64_t)l * c->window + pos) * c->k, sizeof(int32_t) * c->k);
      }
  return MOE_OK;
}

moe_status moe_cache_import_usage(moe_cache* c, const int64_t* counts_host, const int32_t* recent_host) {
  if (!c || !counts_host) return cfail(MOE_ERR_ARG, "moe_cache_import_usage: null pointer");
  if (c->policy == MOE_CACHE_LFU_WINDOW && !recent_host)
    return cfail(MOE_ERR_ARG, "moe_cache_import_usage: the windowed policy needs recent_host");
  for (size_t i = 0; i < c->count.size(); ++i)
    if (counts_host[i] < 0) return cfail(MOE_ERR_STATE, "moe_cache_import_usage: negative use count");
  if (c->policy == MOE_CACHE_LFU_WINDOW) {
    // the counts must be those of the window's selections
    std::vector<int64_t> want((size_t)c->L * c->E, 0);
    for (int l = 0; l < c->L; ++l)
      for (int i = 0; i < c->window * c->k; ++i) {
        const int e = recent_host[(int64_t)l * c->window * c->k + i];
        if (e < -1 || e >= c->E) return cfail(MOE_ERR_STATE, "moe_cache_import_usage: bad expert id");
        if (e >= 0) ++want[(int64_t)l * c->E + e];
      }
    for (size_t i = 0; i < want.size(); ++i)
      if (want[i] != counts_host[i])
        return cfail(MOE_ERR_STATE, "moe_cache_import_usage: counts differ from the window's selections");
    std::memcpy(c->recent.data(), recent_host, sizeof(int32_t) * c->recent.size());
    // the ring restarts at position 0 holding the oldest step
    for (int l = 0; l < c->L; ++l) c->steps_seen[l] = 0;
  }
  std::memcpy(c->count.data(), counts_host, sizeof(int64_t) * c->count.size());
  c->staged_any = true;
  return MOE_OK;
}

moe_status moe_cache_enable_device(moe_cache* c) {
  if (!c) return cfail(MOE_ERR_ARG, "moe_cache_enable_device: null cache");
  if (c->device) return MOE_OK;
  if (c->policy == MOE_CACHE_LFU_WINDOW)
    return cfail(MOE_ERR_UNSUPPORTED, "moe_cache_enable_device: LRU or whole-run LFU only");
  if (c->E > 256 || c->S > 256) return cfail(MOE_ERR_UNSUPPORTED, "moe_cache_enable_device: at most 256 experts");
  void* d = nullptr;
  if (c->blob % 16 || hipHostGetDevicePointer(&d, const_cast<uint8_t*>(c->pool), 0) != hipSuccess || !d ||
      reinterpret_cast<uintptr_t>(d) % 16) {
    (void)hipGetLastError();
    return cfail(MOE_ERR_UNSUPPORTED, "moe_cache_enable_device: the host pool is not device-mapped pinned memory "
                                      "(or blob_bytes % 16 != 0)");
  }
  c->pool_dev = static_cast<const uint8_t*>(d);
  // finish every host-side staging first
  for (int l = 0; l < c->L; ++l) {
    if (c->staged_used[l]) hipEventSynchronize(c->staged[l]);
    if (c->masked_used[l]) hipEventSynchronize(c->masked[l]);
  }
  const size_t nLS = (size_t)c->L * c->S, nLE = (size_t)c->L * c->E;
  moe_status st;
  if ((st = hipcheck(hipMalloc(&c->d_slot_expert, sizeof(int32_t) * nLS), "hipMalloc")) ||
      (st = hipcheck(hipMalloc(&c->d_stamp, sizeof(int64_t) * nLS), "hipMalloc")) ||
      (st = hipcheck(hipMalloc(&c->d_count, sizeof(int64_t) * nLE), "hipMalloc")) ||
      (st = hipcheck(hipMalloc(&c->d_miss, sizeof(int32_t) * 2 * c->L * c->k), "hipMalloc")) ||
      (st = hipcheck(hipMalloc(&c->d_nmiss, sizeof(int32_t) * c->L), "hipMalloc")) ||
      (st = hipcheck(hipMalloc(&c->d_stats, sizeof(int64_t) * 3), "hipMalloc")) ||
      (st = hipcheck(hipMalloc(&c->d_err, sizeof(uint32_t)), "hipMalloc")))
    return release_device_state(c), st;
  const int64_t stats[3] = {c->stats.hits, c->stats.misses, c->stats.bytes_staged};
  const uint32_t zero = 0;
  if ((st = hipcheck(hipMemcpy(c->d_slot_expert, c->slot_expert.data(), sizeof(int32_t) * nLS, hipMemcpyHostToDevice),
                     "hipMemcpy")) ||
      (st = hipcheck(hipMemcpy(c->d_stamp, c->stamp.data(), sizeof(int64_t) * nLS, hipMemcpyHostToDevice),
                     "hipMemcpy")) ||
      (st = hipcheck(hipMemcpy(c->d_count, c->count.data(), sizeof(int64_t) * nLE, hipMemcpyHostToDevice),
                     "hipMemcpy")) ||
      (st = hipcheck(hipMemcpy(c->d_stats, stats, sizeof(stats), hipMemcpyHostToDevice), "hipMemcpy")) ||
      (st = hipcheck(hipMemcpy(c->d_err, &zero, 4, hipMemcpyHostToDevice), "hipMemcpy")))
    return release_device_state(c), st;
  c->routed.assign(c->L, nullptr);
  for (int l = 0; l < c->L; ++l)
    if ((st = hipcheck(hipEventCreateWithFlags(&c->routed[l], hipEventDisableTiming), "hipEventCreate")))
      return release_device_state(c), st;
  c->device = true;
  c->staged_any = true;
  return MOE_OK;
}

moe_status moe_slot_stage_device(moe_cache* c, int32_t layer, int32_t step, const int32_t* sel_dev,
                                 hipStream_t side, hipStream_t compute, uint8_t* hit_mask_dev) {
  if (!c || !sel_dev || !hit_mask_dev) return cfail(MOE_ERR_ARG, "moe_slot_stage_device: null pointer");
  if (!c->device) return cfail(MOE_ERR_STATE, "moe_slot_stage_device: call moe_cache_enable_device first");
  if (layer < 0 || layer >= c->L || step < 0) return cfail(MOE_ERR_ARG, "moe_slot_stage_device: bad layer or step");
  moe::CacheStepArgs a{};
  a.E = c->E; a.S = c->S; a.k = c->k;
  a.policy = c->policy == MOE_CACHE_LFU ? 1 : 0;
  a.step = step;
  a.blob = c->blob;
  a.sel = sel_dev;
  a.table = c->tables_dev + (int64_t)layer * c->E;
  a.slot_expert = c->d_slot_expert + (int64_t)layer * c->S;
  a.stamp = c->d_stamp + (int64_t)layer * c->S;
  a.count = c->d_count + (int64_t)layer * c->E;
  a.hit_mask = hit_mask_dev;
  a.miss = c->d_miss + (int64_t)layer * 2 * c->k;
  a.n_miss = c->d_nmiss + layer;
  a.stats = c->d_stats;
  a.err = c->d_err;
  moe_status st;
  // the rule on the compute stream, after the router and after every kernel
  // that still reads this layer's slots; the copies then on the side stream
  if ((st = hipcheck(moe::launch_cache_step(a, compute), "cache step kernel")) ||
      (st = hipcheck(hipEventRecord(c->routed[layer], compute), "hipEventRecord")) ||
      (st = hipcheck(hipStreamWaitEvent(side, c->routed[layer], 0), "hipStreamWaitEvent")) ||
      (st = hipcheck(moe::launch_stage_misses(c->pool_dev + (int64_t)layer * c->E * c->blob,
                                              c->arena + (int64_t)layer * c->S * c->stride, c->E, c->S, c->k, c->blob,
                                              c->stride, a.miss, a.n_miss, side), "stage kernel")) ||
      (st = hipcheck(hipEventRecord(c->staged[layer], side), "hipEventRecord")))
    return st;
  c->staged_used[layer] = 1;
  return MOE_OK;
}

moe_status moe_cache_stats(const moe_cache* c, moe_stage_stats* out) {
  if (!c || !out) return cfail(MOE_ERR_ARG, "moe_cache_stats: null pointer");
  moe_status st = pull_device_state(c);
  *out = c->stats;
  return st;
}

moe_status moe_cache_wait(moe_cache* c, int32_t layer, hipStream_t compute) {
  if (!c || layer < 0 || layer >= c->L) return cfail(MOE_ERR_ARG, "moe_cache_wait: bad cache or layer");
  if (!c->staged_used[layer]) return MOE_OK;
  return hipcheck(hipStreamWaitEvent(compute, c->staged[layer], 0), "hipStreamWaitEvent");
}

moe_status moe_cache_wait_expert(moe_cache* c, int32_t layer, int32_t rank, hipStream_t compute) {
  if (!c || layer < 0 || layer >= c->L || rank < 0 || rank >= c->k)
    return cfail(MOE_ERR_ARG, "moe_cache_wait_expert: bad cache, layer or rank");
  if (c->device) return cfail(MOE_ERR_STATE, "moe_cache_wait_expert: the cache runs on the device");
  if (!c->staged_used[layer]) return MOE_OK;
  const int32_t m = c->rank_miss[(size_t)layer * c->k + rank];
  if (m < 0) return MOE_OK;  // a hit: resident before the step
  hipEvent_t ev = c->staging == MOE_STAGE_COPY ? c->landed[(size_t)layer * c->k + m] : c->staged[layer];
  return hipcheck(hipStreamWaitEvent(compute, ev, 0), "hipStreamWaitEvent");
}

moe_status moe_cache_slot_table(const moe_cache* c, int32_t layer, int32_t* out_host) {
  if (!c || !out_host || layer < 0 || layer >= c->L)
    return cfail(MOE_ERR_ARG, "moe_cache_slot_table: bad argument");
  moe_status pst = pull_device_state(c);
  if (pst) return pst;
  for (int e = 0; e < c->E; ++e) out_host[e] = -1;
  for (int s = 0; s < c->S; ++s) {
    const int e = c->slot_expert[(int64_t)layer * c->S + s];
    if (e >= 0) out_host[e] = s;
  }
  return MOE_OK;
}

moe_status moe_cache_export(const moe_cache* c, int32_t* slot_expert_host, int64_t* stamp_host) {
  if (!c || !slot_expert_host || !stamp_host) return cfail(MOE_ERR_ARG, "moe_cache_export: null pointer");
  moe_status pst = pull_device_state(c);
  if (pst) return pst;
  std::memcpy(slot_expert_host, c->slot_expert.data(), sizeof(int32_t) * c->slot_expert.size());
  std::memcpy(stamp_host, c->stamp.data(), sizeof(int64_t) * c->stamp.size());
  return MOE_OK;
}

moe_status moe_cache_import(moe_cache* c, const int32_t* slot_expert_host, const int64_t* stamp_host) {
  if (!c || !slot_expert_host || !stamp_host) return cfail(MOE_ERR_ARG, "moe_cache_import: null pointer");
  if (c->device) return cfail(MOE_ERR_STATE, "moe_cache_import: import before moe_cache_enable_device");
  for (int l = 0; l < c->L; ++l) {
    std::vector<char> seen(c->E, 0);
    for (int s = 0; s < c->S; ++s) {
      const int e = slot_expert_host[(int64_t)l * c->S + s];
      if (e < -1 || e >= c->E || (e >= 0 && seen[e]))
        return cfail(MOE_ERR_STATE, "moe_cache_import: invalid slot assignment");
      if (e >= 0) seen[e] = 1;
    }
  }
  for (int l = 0; l < c->L; ++l) {
    if (c->staged_used[l]) hipEventSynchronize(c->staged[l]);
    if (c->masked_used[l]) hipEventSynchronize(c->masked[l]);
  }
  std::memcpy(c->slot_expert.data(), slot_expert_host, sizeof(int32_t) * c->slot_expert.size());
  std::memcpy(c->stamp.data(), stamp_host, sizeof(int64_t) * c->stamp.size());
  for (int l = 0; l < c->L; ++l) rebuild_table(c, l);
  std::fill(c->rank_miss.begin(), c->rank_miss.end(), -1);
  const moe_status st = hipcheck(hipMemcpy(c->tables_dev, c->table_host, sizeof(int32_t) * c->L * c->E,
                                           hipMemcpyHostToDevice), "hipMemcpy");
  // a failed rewrite leaves the device tables to each layer's next step
  std::fill(c->table_stale.begin(), c->table_stale.end(), st == MOE_OK ? 0 : 1);
  return st;
}

}  // extern "C"
