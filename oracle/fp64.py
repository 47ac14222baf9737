"""Float64 textbook form of the routed int4 MoE layer, in numpy.

TEST INFRASTRUCTURE.  This is the cross-check of the oracle proper (the plain
C++ fp32 oracle in ``moe_oracle.cpp``, loaded through ``oracle.cpp``): the same
steps written from the same definitions, in another language and in float64,
with dense dequantised matrices and library matrix products.  The pins hold
for both, and the two agree to fp32 rounding on random layers.  Only
``tests/``, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this module.  It shares no code with
the HIP library (no kernels, headers, tables or helpers) and parses the expert
byte format on its own from the format's definition.  All floating point is
float64 except where a float decides an integer (the top-k choice), which is
taken on float32-rounded logits because that is the precision the GPU decides in.

What the pages fix, and what they leave open
--------------------------------------------
* A layer holds 128 small feed-forward experts and a small router; the router
  names 8 experts per token and only those run (TurboFieldfare video transcript,
  paragraph on Gemma 4 as a mixture-of-experts model).  30 such layers, experts
  of about 3.36 MB each (same transcript, paragraph on the two weight piles).
* Expert projections are INT4 with affine groups of 64 carrying a scale and a
  bias per group ("Optimizing a 14.3 GB model for an 8 GB machine", section
  "Vectorization helped when it respected the storage layout").  The pages'
  scale/bias are BF16; this library's workload uses fp16 scale and bias.
* Expert weights are read through preallocated per-layer cache slots; a bounded
  cache keeps recently used experts ("Optimizing ...", section "MoE needed
  parallel work, reuse, and coarse overlap"; goinfer "When the model doesn't
  fit": LRU over resident slots).
* Left open by the pages, taken here as: the expert is the gated FFN
  out = down(gelu_tanh(gate h) * up h); routing is softmax over all experts,
  top-k by logit with ties to the lowest expert id, weights renormalised over
  the k chosen; the combine is y = residual + sum_j w_j * out_j in rank order;
  w = s*q + b with unsigned q in 0..15 (no zero point); the even input column is
  the low nibble of its byte; matrices are stored [out, in] with groups along
  the input dimension; RMSNorm multiplies by its weight (not 1 + weight) with
  eps = 1e-6.

Expert blob format (one expert, d = hidden, f = expert width)
-------------------------------------------------------------
Six sections, in this order, each starting on a 256-byte boundary:
gate nibbles [f x d], up nibbles [f x d], down nibbles [d x f],
gate (scale, bias) [f x d/64], up (scale, bias) [f x d/64], down (scale, bias) [d x f/64].
For a matrix of R rows and C columns (R, C multiples of 64), element (r, c):
  nibble byte = (r // 64) * (64 * C / 2) + (c // 32) * 1024 + (r % 64) * 16 + (c % 32) // 2
  nibble      = low four bits if c is even, high four bits if c is odd
  pair byte   = (r // 64) * (64 * (C/64) * 4) + (c // 64) * 256 + (r % 64) * 4
                (fp16 scale at +0, fp16 bias at +2, little-endian)
i.e. rows are tiled by 64; inside a tile, the 16-byte column chunks of the 64
rows are stored chunk-major so one row's chunk sits next to its neighbours'.
"""
from __future__ import annotations

import itertools
import math
from functools import lru_cache

import numpy as np

GROUP = 64
TILE_ROWS = 64
EPS = 1e-6

# --------------------------------------------------------------------------------------
# expert blob format
# --------------------------------------------------------------------------------------

SECTION_NAMES = ("gate_q", "up_q", "down_q", "gate_sb", "up_sb", "down_sb")


def blob_sections(d: int, f: int) -> dict:
    """Byte (offset, size) of each section of an expert blob, and the total."""
    sizes = {
        "gate_q": f * d // 2,
        "up_q": f * d // 2,
        "down_q": d * f // 2,
        "gate_sb": f * (d // GROUP) * 4,
        "up_sb": f * (d // GROUP) * 4,
        "down_sb": d * (f // GROUP) * 4,
    }
    out, off = {}, 0
    for name in SECTION_NAMES:
        off = (off + 255) // 256 * 256
        out[name] = (off, sizes[name])
        off += sizes[name]
    out["total"] = (off + 255) // 256 * 256
    return out


def blob_bytes(d: int, f: int) -> int:
    return blob_sections(d, f)["total"]


@lru_cache(maxsize=8)
def _element_indices(R: int, C: int):
    """Byte index of each element's nibble, its shift, and the byte index of
    each (row, group) scale/bias pair, straight from the format definition."""
    r = np.arange(R, dtype=np.int64)[:, None]
    c = np.arange(C, dtype=np.int64)[None, :]
    nib_byte = (r // 64) * (64 * C // 2) + (c // 32) * 1024 + (r % 64) * 16 + (c % 32) // 2
    shift = 4 * (c % 2)
    g = np.arange(C // GROUP, dtype=np.int64)[None, :]
    pair_byte = (r // 64) * (64 * (C // GROUP) * 4) + g * 256 + (r % 64) * 4
    return nib_byte, np.broadcast_to(shift, (R, C)), pair_byte


def dequant(blob: np.ndarray, q_off: int, sb_off: int, R: int, C: int) -> np.ndarray:
    """Dense float64 matrix w[r, c] = s[r, c//64] * q[r, c] + b[r, c//64].

    The product and sum are exact in float64 (fp16 scale times a 4-bit integer
    plus an fp16 bias), so the dequantised weight is uniquely defined."""
    blob = np.asarray(blob, dtype=np.uint8)
    nib_byte, shift, pair_byte = _element_indices(R, C)
    q = ((blob[q_off + nib_byte] >> shift.astype(np.uint8)) & 0xF).astype(np.float64)
    halves = blob.view("<f2")
    s = halves[(sb_off + pair_byte) // 2].astype(np.float64)
    b = halves[(sb_off + pair_byte) // 2 + 1].astype(np.float64)
    cols_group = np.arange(C) // GROUP
    return s[:, cols_group] * q + b[:, cols_group]


def expert_matrices(blob: np.ndarray, d: int, f: int):
    """(W_gate [f,d], W_up [f,d], W_down [d,f]) of one expert, float64."""
    sec = blob_sections(d, f)
    wg = dequant(blob, sec["gate_q"][0], sec["gate_sb"][0], f, d)
    wu = dequant(blob, sec["up_q"][0], sec["up_sb"][0], f, d)
    wd = dequant(blob, sec["down_q"][0], sec["down_sb"][0], d, f)
    return wg, wu, wd


def encode_matrix(q: np.ndarray, s: np.ndarray, b: np.ndarray):
    """Inverse of ``dequant``'s parsing: integer nibbles q [R, C] (0..15) and fp16
    s, b [R, C/64] -> (nibble bytes, pair bytes) in the blob format."""
    R, C = q.shape
    nib_byte, shift, pair_byte = _element_indices(R, C)
    nib = np.zeros(R * C // 2, dtype=np.uint8)
    np.bitwise_or.at(nib, nib_byte.ravel(), (q.astype(np.uint8) << shift.astype(np.uint8)).ravel())
    pairs = np.zeros(R * (C // GROUP) * 2, dtype=np.float16)
    pairs[(pair_byte // 2).ravel()] = s.astype(np.float16).ravel()
    pairs[(pair_byte // 2 + 1).ravel()] = b.astype(np.float16).ravel()
    return nib, pairs.view(np.uint8)


def encode_expert(qs: dict, d: int, f: int) -> np.ndarray:
    """Build an expert blob from {"gate": (q, s, b), "up": ..., "down": ...}."""
    sec = blob_sections(d, f)
    blob = np.zeros(sec["total"], dtype=np.uint8)
    for m in ("gate", "up", "down"):
        nib, pairs = encode_matrix(*qs[m])
        o, n = sec[m + "_q"]
        blob[o:o + n] = nib
        o, n = sec[m + "_sb"]
        blob[o:o + n] = pairs
    return blob


def quantize_group_affine(w: np.ndarray, s: np.ndarray, b: np.ndarray) -> np.ndarray:
    """q = round((w - b) / s) per element, with s, b per group of 64 columns."""
    cols_group = np.arange(w.shape[1]) // GROUP
    return np.rint((w - b[:, cols_group]) / s[:, cols_group]).astype(np.int64)


# --------------------------------------------------------------------------------------
# the layer, step by step
# --------------------------------------------------------------------------------------

def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float = EPS) -> np.ndarray:
    """h = x / sqrt(mean(x^2) + eps) * w, per token row."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=np.float64)


def rms_rescale(x: np.ndarray, eps: float = EPS) -> np.ndarray:
    """Unit-RMS rescale used as decode step feedback: x / sqrt(mean(x^2) + eps)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def router_logits(h: np.ndarray, router_w: np.ndarray, bias=None) -> np.ndarray:
    """logits[t, e] = sum_i Wr[e, i] * h[t, i] (+ bias[e]), float64."""
    lg = np.asarray(h, dtype=np.float64) @ np.asarray(router_w, dtype=np.float64).T
    if bias is not None:
        lg = lg + np.asarray(bias, dtype=np.float64)
    return lg


def select_topk(logits_row, k: int) -> list:
    """The k experts with the largest logits, in descending order; equal logits
    go to the lower expert id.  Explicit sort on (-logit, id)."""
    order = sorted(range(len(logits_row)), key=lambda e: (-float(logits_row[e]), e))
    return order[:k]


def softmax(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    z = np.exp(v - v.max())
    return z / z.sum()


def routing_weights(logits_row, selected) -> np.ndarray:
    """Softmax over all experts, then renormalised over the selected ones."""
    p = softmax(logits_row)
    sel = p[list(selected)]
    return sel / sel.sum()


def route(x, norm_w, router_w, bias, k: int, eps: float = EPS):
    """Routing of T tokens.  Returns (h, logits64, idx [T,k], w [T,k]).

    h is the RMSNorm output (x itself when norm_w is None).  The choice is made
    on the float32-rounded logits; weights come from the float64 logits."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    h = rmsnorm(x, norm_w, eps) if norm_w is not None else x.copy()
    lg = router_logits(h, router_w, bias)
    lg32 = lg.astype(np.float32)
    T = x.shape[0]
    idx = np.zeros((T, k), dtype=np.int32)
    w = np.zeros((T, k), dtype=np.float64)
    for t in range(T):
        sel = select_topk(lg32[t], k)
        idx[t] = sel
        w[t] = routing_weights(lg[t], sel)
    return h, lg, idx, w


def gelu_tanh(z):
    """GELU, tanh approximation: 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3)))."""
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z ** 3)))


def expert_gateup(blob, h, d: int, f: int) -> np.ndarray:
    """act = gelu_tanh(W_gate h) * (W_up h) for rows of h [M, d] -> [M, f]."""
    wg, wu, _ = expert_matrices(blob, d, f)
    h = np.atleast_2d(np.asarray(h, dtype=np.float64))
    return gelu_tanh(h @ wg.T) * (h @ wu.T)


def expert_down(blob, act, d: int, f: int) -> np.ndarray:
    """o = W_down act for rows of act [M, f] -> [M, d]."""
    _, _, wd = expert_matrices(blob, d, f)
    return np.atleast_2d(np.asarray(act, dtype=np.float64)) @ wd.T


def combine(residual, w, outs) -> np.ndarray:
    """y[t] = residual[t] + sum_j w[t, j] * outs[t, j] (outs [T, k, d]); the
    residual is skipped when None."""
    w = np.asarray(w, dtype=np.float64)
    outs = np.asarray(outs, dtype=np.float64)
    T, k = w.shape
    y = np.zeros((T, outs.shape[-1])) if residual is None else np.array(residual, dtype=np.float64)
    for t in range(T):
        for j in range(k):
            y[t] = y[t] + w[t, j] * outs[t, j]
    return y


def moe_layer(x, norm_w, router_w, bias, blob_of, d: int, f: int, k: int,
              eps: float = EPS, residual: bool = True, idx_override=None):
    """One routed MoE layer on T tokens: route, run the selected experts, combine.

    ``blob_of(e)`` returns expert e's blob (for instance through a slot table).
    ``idx_override`` replaces the oracle's own choice (used when an uncertified
    near-tie was decided differently by the GPU).  Returns (y, idx, w, h, logits)."""
    h, lg, idx, w = route(x, norm_w, router_w, bias, k, eps)
    if idx_override is not None:
        idx = np.asarray(idx_override, dtype=np.int32).reshape(idx.shape)
        w = np.stack([routing_weights(lg[t], idx[t]) for t in range(len(idx))])
    T = h.shape[0]
    outs = np.zeros((T, k, d))
    for e in sorted(set(idx.ravel().tolist())):
        rows = [(t, j) for t in range(T) for j in range(k) if idx[t, j] == e]
        blob = blob_of(e)
        hs = np.stack([h[t] for t, _ in rows])
        o = expert_down(blob, expert_gateup(blob, hs, d, f), d, f)
        for n, (t, j) in enumerate(rows):
            outs[t, j] = o[n]
    y = combine(np.atleast_2d(x) if residual else None, w, outs)
    return y, idx, w, h, lg


# --------------------------------------------------------------------------------------
# grouping pairs by expert
# --------------------------------------------------------------------------------------

def permute(idx, n_experts: int):
    """Group the T*k (token, rank) pairs by expert.  Pair p = t*k + j.

    counts[e] = number of pairs routed to e; offsets = exclusive prefix sum of
    counts (offsets[E] = T*k); sorted_pair lists the pairs of each expert in
    ascending pair id, expert after expert; pair_pos is its inverse."""
    flat = np.asarray(idx, dtype=np.int64).ravel()
    counts = np.zeros(n_experts, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    for e in range(n_experts):
        offsets[e + 1] = offsets[e] + counts[e]
    sorted_pair = np.argsort(flat, kind="stable")
    pair_pos = np.empty_like(sorted_pair)
    pair_pos[sorted_pair] = np.arange(len(flat))
    return (counts.astype(np.int32), offsets.astype(np.int32),
            sorted_pair.astype(np.int32), pair_pos.astype(np.int32))


# --------------------------------------------------------------------------------------
# bounded per-layer expert cache
# --------------------------------------------------------------------------------------

class LruSlotCache:
    """Least-recently-used expert cache of one layer with ``n_slots`` slots.

    State: the expert in each slot (-1 = empty) and the step it was last used
    (-1 = never).  A step with selection S first stamps every hit with the
    step number, then places each miss, in ascending expert id, into the slot
    with the smallest (stamp, slot index): empty slots fill lowest first and a
    slot used in this step is never evicted in the same step (k <= slots)."""

    def __init__(self, n_slots: int, n_experts: int):
        self.n_slots, self.n_experts = n_slots, n_experts
        self.slot_expert = [-1] * n_slots
        self.stamp = [-1] * n_slots

    def slot_of_expert(self) -> list:
        table = [-1] * self.n_experts
        for s, e in enumerate(self.slot_expert):
            if e >= 0:
                table[e] = s
        return table

    def step(self, t: int, selection):
        """Returns (hit mask in selection order, [(expert, slot, evicted)] installs)."""
        table = self.slot_of_expert()
        hit = [table[e] >= 0 for e in selection]
        for e, h in zip(selection, hit):
            if h:
                self.stamp[table[e]] = t
        installs = []
        for e in sorted(e for e, h in zip(selection, hit) if not h):
            victim = min(range(self.n_slots), key=lambda s: (self.stamp[s], s))
            installs.append((e, victim, self.slot_expert[victim]))
            self.slot_expert[victim] = e
            self.stamp[victim] = t
        return hit, installs

    def export_state(self):
        return list(self.slot_expert), list(self.stamp)

    def import_state(self, state):
        self.slot_expert, self.stamp = list(state[0]), list(state[1])


class LfuSlotCache:
    """Least-frequently-used expert cache of one layer with ``n_slots`` slots.

    The pages replace LRU by LFU: the expert pushed out is the one used least,
    because a few experts are picked again and again ("Optimizing a 14.3 GB
    model for an 8 GB machine", section "MoE needed parallel work, reuse, and
    coarse overlap": LRU -> LFU, and a 64-token LFU window tried beside the
    whole-run count; TurboFieldfare video transcript, paragraph on the expert
    cache).  Left open by the pages, taken here as:

    * use count of expert e at step t = the number of steps, among those the
      count covers, whose selection contains e, the current step included.
      ``window=None`` counts every step since the cache was created (whether
      or not e was resident then); ``window=W`` counts the last W steps.
    * a step first stamps every hit with the step number; then each miss, in
      ascending expert id, takes an empty slot if there is one (lowest index
      first), else the slot, among those not used in this step, whose expert
      has the smallest (use count, stamp, slot index).

    The counts are recomputed from the kept selection history at every victim
    choice (no running totals), so the rule can be read off directly."""

    def __init__(self, n_slots: int, n_experts: int, window=None):
        self.n_slots, self.n_experts, self.window = n_slots, n_experts, window
        self.slot_expert = [-1] * n_slots
        self.stamp = [-1] * n_slots
        self.history = []  # selections of the steps so far, oldest first

    def slot_of_expert(self) -> list:
        table = [-1] * self.n_experts
        for s, e in enumerate(self.slot_expert):
            if e >= 0:
                table[e] = s
        return table

    def use_count(self, e: int) -> int:
        steps = self.history if self.window is None else self.history[-self.window:]
        return sum(1 for sel in steps if e in sel)

    def step(self, t: int, selection):
        """Returns (hit mask in selection order, [(expert, slot, evicted)] installs)."""
        self.history.append(set(int(e) for e in selection))
        table = self.slot_of_expert()
        hit = [table[e] >= 0 for e in selection]
        for e, h in zip(selection, hit):
            if h:
                self.stamp[table[e]] = t
        installs = []
        for e in sorted(e for e, h in zip(selection, hit) if not h):
            empty = [s for s in range(self.n_slots) if self.slot_expert[s] < 0]
            if empty:
                victim = empty[0]
            else:
                free = [s for s in range(self.n_slots) if self.stamp[s] != t]
                victim = min(free, key=lambda s: (self.use_count(self.slot_expert[s]), self.stamp[s], s))
            installs.append((e, victim, self.slot_expert[victim]))
            self.slot_expert[victim] = e
            self.stamp[victim] = t
        return hit, installs

    def counts(self) -> list:
        return [self.use_count(e) for e in range(self.n_experts)]

    def export_state(self):
        return list(self.slot_expert), list(self.stamp), [set(sel) for sel in self.history]

    def import_state(self, state):
        self.slot_expert, self.stamp = list(state[0]), list(state[1])
        self.history = [set(sel) for sel in state[2]]


# --------------------------------------------------------------------------------------
# shared path: the filler GEMV and the shared expert (bf16 weights)
# --------------------------------------------------------------------------------------

def bf16_bits_to_float(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 values (bf16 is the top half of fp32)."""
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def shared_gemv(w_bits: np.ndarray, h) -> np.ndarray:
    """s = W h with W given as bf16 bits [rows, cols]; h [T, cols] -> [T, rows]."""
    return np.atleast_2d(np.asarray(h, dtype=np.float64)) @ bf16_bits_to_float(w_bits).T


def shared_expert(h, w_gu_bits: np.ndarray, w_down_bits: np.ndarray, residual=None) -> np.ndarray:
    """The always-resident shared expert (TurboFieldfare video transcript,
    paragraph on the two weight piles: one shared expert runs for every token;
    "Optimizing a 14.3 GB model for an 8 GB machine", section "MoE needed
    parallel work, reuse, and coarse overlap": the shared MLP is the work that
    hides expert reads).  Taken here in the routed experts' gated form with
    bf16 weights: w_gu [2 f_sh, d] holds the gate rows, then the up rows;
    w_down [d, f_sh]; out = residual + W_down (gelu_tanh(W_gate h) * (W_up h))."""
    h = np.atleast_2d(np.asarray(h, dtype=np.float64))
    gu = h @ bf16_bits_to_float(w_gu_bits).T
    f_sh = gu.shape[1] // 2
    act = gelu_tanh(gu[:, :f_sh]) * gu[:, f_sh:]
    out = act @ bf16_bits_to_float(w_down_bits).T
    if residual is not None:
        out = out + np.atleast_2d(np.asarray(residual, dtype=np.float64))
    return out


# --------------------------------------------------------------------------------------
# brute-force helpers used by the pins
# --------------------------------------------------------------------------------------

def topk_bruteforce(logits_row, k: int) -> list:
    """Best k-subset by sum of logits (ties: lexicographically smallest ids),
    returned in descending logit order (ties: lower id first)."""
    best, best_key = None, None
    for comb in itertools.combinations(range(len(logits_row)), k):
        key = (math.fsum(float(logits_row[e]) for e in comb), tuple(-e for e in comb))
        if best_key is None or key > best_key:
            best, best_key = comb, key
    return sorted(best, key=lambda e: (-float(logits_row[e]), e))
