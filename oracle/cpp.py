"""Python face of the plain C++17 CPU oracle (``oracle/moe_oracle.cpp``).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this module.  It shares no code
with the HIP library.  The functions keep the names and signatures of the
float64 numpy oracle (``oracle.fp64``), so a test can run either; this one is
the oracle the GPU results are compared against: fp32 arithmetic with every
sum sequential in ascending index order, scalar dequant from the blob bytes,
top-k by an explicit stable sort, ``std::thread`` across independent rows,
pairs and tokens only.  The arithmetic of each step, and the passage of the
pages it follows, is stated at the top of ``moe_oracle.cpp``.

Values come back as float32 arrays (the oracle's own precision); router
logits also come back in float64, computed beside the fp32 sums, to certify
how far a routing decision is from a tie.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import fp64 as _fmt  # byte-format encoders for building test blobs, and the brute-force checker

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.cpp")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(BUILD, "libmoe_oracle.so")

GROUP = 64
TILE_ROWS = 64
EPS = 1e-6
SECTION_NAMES = ("gate_q", "up_q", "down_q", "gate_sb", "up_sb", "down_sb")

encode_matrix = _fmt.encode_matrix
encode_expert = _fmt.encode_expert
quantize_group_affine = _fmt.quantize_group_affine
topk_bruteforce = _fmt.topk_bruteforce
bf16_bits_to_float = _fmt.bf16_bits_to_float


def build(verbose: bool = False) -> str:
    """Compile the oracle with g++ (plain C++17, no contraction of a*b+c)."""
    os.makedirs(BUILD, exist_ok=True)
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread", "-ffp-contract=off", "-Wall",
           SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"oracle build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", flush=True)
    return LIB


_lib = None

_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_vp = ctypes.c_void_p
_i = ctypes.c_int


def lib():
    """The loaded oracle library, built first if missing or older than its source."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        L = ctypes.CDLL(LIB)
        sig = {
            "oro_set_threads": (None, [_i]),
            "oro_threads": (_i, []),
            "oro_blob_offsets": (_i, [_i, _i, _i64p]),
            "oro_dequant": (None, [_u8p, ctypes.c_int64, ctypes.c_int64, _i, _i, _f32p]),
            "oro_gelu_tanh": (ctypes.c_double, [ctypes.c_double]),
            "oro_rmsnorm": (None, [_f32p, _i, _i, _f32p, ctypes.c_float, _f32p]),
            "oro_rms_rescale": (None, [_f32p, _i, _i, ctypes.c_float, _f32p]),
            "oro_router": (None, [_f32p, _i, _i, _i, _f32p, _f32p, _f32p, _f64p]),
            "oro_select_topk": (None, [_f32p, _i, _i, _i32p]),
            "oro_weights": (None, [_f32p, _i, _i32p, _f32p]),
            "oro_expert_gateup": (None, [_u8p, _i, _i, _f32p, _i, _f32p]),
            "oro_expert_down": (None, [_u8p, _i, _i, _f32p, _i, _f32p]),
            "oro_experts_combine": (None, [_f32p, _f32p, _i, _i, _i, _i, _i, _i32p, _f32p,
                                           ctypes.POINTER(_u8p), _i, _f32p, _f32p]),
            "oro_permute": (None, [_i32p, _i, _i, _i, _i32p, _i32p, _i32p, _i32p]),
            "oro_shared_gemv_bf16": (None, [_u16p, _f32p, _i, _i, _i, _f32p]),
            "oro_shared_expert_bf16": (None, [_u16p, _u16p, _f32p, _f32p, _i, _i, _i, _f32p]),
            "oro_cache_new": (_vp, [_i, _i, _i, _i]),
            "oro_cache_free": (None, [_vp]),
            "oro_cache_step": (_i, [_vp, ctypes.c_int64, _i32p, _i, _u8p, _i32p]),
            "oro_cache_get": (None, [_vp, _i32p, _i64p, _i64p]),
            "oro_cache_history_len": (_i, [_vp]),
            "oro_cache_get_history": (None, [_vp, _i, _i32p]),
            "oro_cache_set": (None, [_vp, _i32p, _i64p, _i, _i, _i32p]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
        L.oro_set_threads(default_threads())
    return _lib


def default_threads() -> int:
    """The CPUs this process may run on, capped by OMP_NUM_THREADS when set."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    omp = os.environ.get("OMP_NUM_THREADS", "")
    return min(n, int(omp)) if omp.isdigit() and int(omp) > 0 else n


def set_threads(n: int) -> None:
    """Threads the oracle uses (0: every hardware thread)."""
    lib().oro_set_threads(int(n))


def threads() -> int:
    return int(lib().oro_threads())


def _p(a: np.ndarray, ptype):
    return a.ctypes.data_as(ptype)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _u8(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.uint8))


# --------------------------------------------------------------------------- format

def blob_sections(d: int, f: int) -> dict:
    """Byte (offset, size) of each section of an expert blob, and the total."""
    off = np.zeros(7, dtype=np.int64)
    if lib().oro_blob_offsets(d, f, _p(off, _i64p)) != 0:
        raise ValueError(f"d={d} f={f}: not multiples of {GROUP}")
    sizes = (f * d // 2, f * d // 2, d * f // 2, f * (d // GROUP) * 4, f * (d // GROUP) * 4, d * (f // GROUP) * 4)
    out = {n: (int(off[i]), sizes[i]) for i, n in enumerate(SECTION_NAMES)}
    out["total"] = int(off[6])
    return out


def blob_bytes(d: int, f: int) -> int:
    return blob_sections(d, f)["total"]


def dequant(blob, q_off: int, sb_off: int, R: int, C: int) -> np.ndarray:
    """Dense fp32 matrix w[r, c] = s * q + b of one blob section pair."""
    b = _u8(blob)
    w = np.empty((R, C), dtype=np.float32)
    lib().oro_dequant(_p(b, _u8p), int(q_off), int(sb_off), R, C, _p(w, _f32p))
    return w


def expert_matrices(blob, d: int, f: int):
    """(W_gate [f,d], W_up [f,d], W_down [d,f]) of one expert, fp32."""
    sec = blob_sections(d, f)
    return (dequant(blob, sec["gate_q"][0], sec["gate_sb"][0], f, d),
            dequant(blob, sec["up_q"][0], sec["up_sb"][0], f, d),
            dequant(blob, sec["down_q"][0], sec["down_sb"][0], d, f))


# --------------------------------------------------------------------------- layer steps

def rmsnorm(x, w, eps: float = EPS) -> np.ndarray:
    x = np.atleast_2d(_f32(x))
    h = np.empty_like(x)
    ww = None if w is None else _f32(w)
    lib().oro_rmsnorm(_p(x, _f32p), x.shape[0], x.shape[1], None if ww is None else _p(ww, _f32p),
                      float(eps), _p(h, _f32p))
    return h


def rms_rescale(x, eps: float = EPS) -> np.ndarray:
    x = np.atleast_2d(_f32(x))
    out = np.empty_like(x)
    lib().oro_rms_rescale(_p(x, _f32p), x.shape[0], x.shape[1], float(eps), _p(out, _f32p))
    return out


def router_logits2(h, router_w, bias=None):
    """(fp32 logits, fp64 logits) [T, E]."""
    h = np.atleast_2d(_f32(h))
    rw = _f32(router_w)
    E = rw.shape[0]
    T, d = h.shape
    lg32 = np.empty((T, E), dtype=np.float32)
    lg64 = np.empty((T, E), dtype=np.float64)
    bb = None if bias is None else _f32(bias)
    lib().oro_router(_p(h, _f32p), T, d, E, _p(rw, _f32p), None if bb is None else _p(bb, _f32p),
                     _p(lg32, _f32p), _p(lg64, _f64p))
    return lg32, lg64


def router_logits(h, router_w, bias=None) -> np.ndarray:
    return router_logits2(h, router_w, bias)[1]


def select_topk(logits_row, k: int) -> list:
    """The k largest (fp32) logits' experts, descending; equal: lower id first."""
    lg = _f32(logits_row).ravel()
    out = np.empty(k, dtype=np.int32)
    lib().oro_select_topk(_p(lg, _f32p), lg.size, k, _p(out, _i32p))
    return out.tolist()


def routing_weights(logits_row, selected) -> np.ndarray:
    """Softmax over the selected experts' fp32 logits (fp64 inside, fp32 out)."""
    lg = _f32(logits_row).ravel()
    sel = np.ascontiguousarray(np.asarray(selected, dtype=np.int32))
    w = np.empty(sel.size, dtype=np.float32)
    lib().oro_weights(_p(lg, _f32p), sel.size, _p(sel, _i32p), _p(w, _f32p))
    return w


def route(x, norm_w, router_w, bias, k: int, eps: float = EPS):
    """Routing of T tokens: (h fp32, logits fp64 [T,E], idx int32 [T,k], w fp32 [T,k])."""
    x = np.atleast_2d(_f32(x))
    h = rmsnorm(x, norm_w, eps) if norm_w is not None else x.copy()
    lg32, lg64 = router_logits2(h, router_w, bias)
    T = x.shape[0]
    idx = np.zeros((T, k), dtype=np.int32)
    w = np.zeros((T, k), dtype=np.float32)
    for t in range(T):
        idx[t] = select_topk(lg32[t], k)
        w[t] = routing_weights(lg32[t], idx[t])
    return h, lg64, idx, w


def route32(x, norm_w, router_w, bias, k: int, eps: float = EPS):
    """As ``route``, plus the fp32 logits the decisions were taken on."""
    x = np.atleast_2d(_f32(x))
    h = rmsnorm(x, norm_w, eps) if norm_w is not None else x.copy()
    lg32, lg64 = router_logits2(h, router_w, bias)
    idx = np.stack([select_topk(lg32[t], k) for t in range(x.shape[0])]).astype(np.int32)
    w = np.stack([routing_weights(lg32[t], idx[t]) for t in range(x.shape[0])]).astype(np.float32)
    return h, lg32, lg64, idx, w


def gelu_tanh(z):
    """GELU, tanh form, evaluated in fp64 by the oracle library."""
    z = np.asarray(z, dtype=np.float64)
    f = lib().oro_gelu_tanh
    out = np.array([f(float(v)) for v in z.ravel()], dtype=np.float64).reshape(z.shape)
    return out if out.shape else float(out)


def expert_gateup(blob, h, d: int, f: int) -> np.ndarray:
    """act = fp32(gelu_tanh(W_gate h) * (W_up h)) for rows of h [M, d] -> [M, f]."""
    b = _u8(blob)
    h = np.atleast_2d(_f32(h))
    act = np.empty((h.shape[0], f), dtype=np.float32)
    lib().oro_expert_gateup(_p(b, _u8p), d, f, _p(h, _f32p), h.shape[0], _p(act, _f32p))
    return act


def expert_down(blob, act, d: int, f: int) -> np.ndarray:
    """o = W_down act for rows of act [M, f] -> [M, d]."""
    b = _u8(blob)
    a = np.atleast_2d(_f32(act))
    out = np.empty((a.shape[0], d), dtype=np.float32)
    lib().oro_expert_down(_p(b, _u8p), d, f, _p(a, _f32p), a.shape[0], _p(out, _f32p))
    return out


def experts_combine(x, h, idx, w, blob_of, d: int, f: int, E: int, residual: bool = True, pair_outputs=False):
    """The experts idx names, run on h, and the rank-ordered combine with x."""
    x = np.atleast_2d(_f32(x))
    h = np.atleast_2d(_f32(h))
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int32))
    w = _f32(w)
    T, k = idx.shape
    keep = {}
    ptrs = (_u8p * E)()
    for e in sorted(set(idx.ravel().tolist())):
        keep[e] = _u8(blob_of(e))
        ptrs[e] = _p(keep[e], _u8p)
    y = np.empty((T, d), dtype=np.float32)
    outs = np.empty((T * k, d), dtype=np.float32) if pair_outputs else None
    lib().oro_experts_combine(_p(x, _f32p), _p(h, _f32p), T, d, f, E, k, _p(idx, _i32p), _p(w, _f32p), ptrs,
                              1 if residual else 0, _p(y, _f32p), None if outs is None else _p(outs, _f32p))
    return (y, outs) if pair_outputs else y


def moe_layer(x, norm_w, router_w, bias, blob_of, d: int, f: int, k: int,
              eps: float = EPS, residual: bool = True, idx_override=None):
    """One routed MoE layer on T tokens: route, run the selected experts, combine.

    ``idx_override`` replaces the oracle's own choice (an uncertified near-tie
    the GPU decided the other way); the weights are then those of the given
    experts.  Returns (y fp32, idx, w fp32, h fp32, logits fp64)."""
    h, lg32, lg64, idx, w = route32(x, norm_w, router_w, bias, k, eps)
    if idx_override is not None:
        idx = np.asarray(idx_override, dtype=np.int32).reshape(idx.shape)
        w = np.stack([routing_weights(lg32[t], idx[t]) for t in range(idx.shape[0])]).astype(np.float32)
    E = np.asarray(router_w).shape[0]
    y = experts_combine(x, h, idx, w, blob_of, d, f, E, residual)
    return y, idx, w, h, lg64


# --------------------------------------------------------------------------- permute

def permute(idx, n_experts: int):
    """(counts [E], offsets [E+1], sorted_pair [T*k], pair_pos [T*k]), int32."""
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int32))
    T, k = idx.reshape(idx.shape[0], -1).shape
    P = T * k
    counts = np.empty(n_experts, dtype=np.int32)
    offsets = np.empty(n_experts + 1, dtype=np.int32)
    sp = np.empty(P, dtype=np.int32)
    pp = np.empty(P, dtype=np.int32)
    lib().oro_permute(_p(idx, _i32p), T, k, n_experts, _p(counts, _i32p), _p(offsets, _i32p), _p(sp, _i32p),
                      _p(pp, _i32p))
    return counts, offsets, sp, pp


# --------------------------------------------------------------------------- caches

class _Cache:
    def __init__(self, policy: int, window: int, n_slots: int, n_experts: int):
        self.n_slots, self.n_experts = n_slots, n_experts
        self._h = lib().oro_cache_new(policy, window, n_slots, n_experts)
        if not self._h:
            raise ValueError("bad cache arguments")
        self._k = 0

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            _lib.oro_cache_free(h)
            self._h = None

    def _get(self):
        se = np.empty(self.n_slots, dtype=np.int32)
        st = np.empty(self.n_slots, dtype=np.int64)
        cn = np.empty(self.n_experts, dtype=np.int64)
        lib().oro_cache_get(self._h, _p(se, _i32p), _p(st, _i64p), _p(cn, _i64p))
        return se, st, cn

    @property
    def slot_expert(self) -> list:
        return self._get()[0].tolist()

    @property
    def stamp(self) -> list:
        return self._get()[1].tolist()

    def slot_of_expert(self) -> list:
        table = [-1] * self.n_experts
        for s, e in enumerate(self.slot_expert):
            if e >= 0:
                table[e] = s
        return table

    def step(self, t: int, selection):
        """Returns (hit mask in selection order, [(expert, slot, evicted)] installs)."""
        sel = np.ascontiguousarray(np.asarray(selection, dtype=np.int32).ravel())
        k = sel.size
        self._k = max(self._k, k)
        hit = np.empty(k, dtype=np.uint8)
        inst = np.empty(3 * k, dtype=np.int32)
        n = lib().oro_cache_step(self._h, int(t), _p(sel, _i32p), k, _p(hit, _u8p), _p(inst, _i32p))
        return [bool(v) for v in hit], [tuple(int(v) for v in inst[3 * i:3 * i + 3]) for i in range(n)]

    def _history(self):
        n = lib().oro_cache_history_len(self._h)
        k = max(self._k, 1)
        out = np.empty((n, k), dtype=np.int32)
        lib().oro_cache_get_history(self._h, k, _p(out, _i32p))
        return [set(int(e) for e in row if e >= 0) for row in out]

    def _set(self, slot_expert, stamp, history):
        se = np.ascontiguousarray(np.asarray(slot_expert, dtype=np.int32))
        st = np.ascontiguousarray(np.asarray(stamp, dtype=np.int64))
        k = max([len(s) for s in history] + [1])
        self._k = max(self._k, k)
        hist = np.full((len(history), k), -1, dtype=np.int32)
        for i, s in enumerate(history):
            v = sorted(s)
            hist[i, :len(v)] = v
        lib().oro_cache_set(self._h, _p(se, _i32p), _p(st, _i64p), len(history), k, _p(hist, _i32p))


class LruSlotCache(_Cache):
    """LRU expert cache of one layer: hits stamped first, then each miss in
    ascending expert id takes the slot with the smallest (stamp, slot index)."""

    def __init__(self, n_slots: int, n_experts: int):
        super().__init__(0, 0, n_slots, n_experts)

    def export_state(self):
        se, st, _ = self._get()
        return se.tolist(), st.tolist()

    def import_state(self, state):
        self._set(state[0], state[1], [])


class LfuSlotCache(_Cache):
    """LFU expert cache of one layer, use counts over every step so far
    (``window=None``) or the last ``window`` steps; rule as in moe_oracle.cpp."""

    def __init__(self, n_slots: int, n_experts: int, window=None):
        super().__init__(1 if window is None else 2, 0 if window is None else int(window), n_slots, n_experts)
        self.window = window

    def counts(self) -> list:
        return self._get()[2].tolist()

    def use_count(self, e: int) -> int:
        return self.counts()[e]

    def export_state(self):
        se, st, _ = self._get()
        return se.tolist(), st.tolist(), self._history()

    def import_state(self, state):
        self._set(state[0], state[1], state[2])


# --------------------------------------------------------------------------- shared path

def _u16(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.uint16))


def shared_gemv(w_bits, h) -> np.ndarray:
    """s = W h with W given as bf16 bits [rows, cols]; h [T, cols] -> fp32 [T, rows]."""
    w = _u16(w_bits)
    h = np.atleast_2d(_f32(h))
    rows, cols = w.shape
    out = np.empty((h.shape[0], rows), dtype=np.float32)
    lib().oro_shared_gemv_bf16(_p(w, _u16p), _p(h, _f32p), h.shape[0], rows, cols, _p(out, _f32p))
    return out


def shared_expert(h, w_gu_bits, w_down_bits, residual=None) -> np.ndarray:
    """residual + W_down (gelu_tanh(W_gate h) * (W_up h)), bf16 weights (fp32 out)."""
    wgu = _u16(w_gu_bits)
    wdn = _u16(w_down_bits)
    h = np.atleast_2d(_f32(h))
    T, d = h.shape
    f_sh = wgu.shape[0] // 2
    res = None if residual is None else np.atleast_2d(_f32(residual))
    out = np.empty((T, d), dtype=np.float32)
    lib().oro_shared_expert_bf16(_p(wgu, _u16p), _p(wdn, _u16p), _p(h, _f32p),
                                 None if res is None else _p(res, _f32p), T, d, f_sh, _p(out, _f32p))
    return out
