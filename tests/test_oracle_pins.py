"""Pins of the CPU oracle against facts that do not come from the oracle itself:
hand-worked fixtures, closed forms, exact integer arithmetic, brute force on
tiny inputs and invariants.  CPU only.

Every pin runs on both forms of the oracle: the plain C++ fp32 oracle the GPU
is checked against (``oracle``, id "cpp") and the float64 numpy form
(``oracle.fp64``, id "fp64").  Where a pin compares against a float64
textbook value, the fp32 oracle is held to 1e-5 (its own rounding), the
float64 form to 1e-10 or tighter; exact-arithmetic pins are exact for both."""
import json
import math
import os
import random

import numpy as np
import pytest

import oracle
import oracle.fp64
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(params=["cpp", "fp64"])
def orc(request):
    return oracle if request.param == "cpp" else oracle.fp64


def _tol(orc, fp32_tol, fp64_tol):
    return fp32_tol if orc is oracle else fp64_tol


def _load(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


# ----------------------------------------------------------------------------- format

def test_blob_size_matches_pages(orc):
    # ~3.36 MB per expert, 30 x 128 experts ~ 12.9 GB (TurboFieldfare video transcript,
    # paragraph on the two weight piles)
    nbytes = orc.blob_bytes(2816, 704)
    assert nbytes == 3_345_408
    assert abs(nbytes / 3.36e6 - 1) < 0.01
    assert abs(30 * 128 * nbytes / 12.9e9 - 1) < 0.01
    sec = orc.blob_sections(2816, 704)
    assert [sec[n][0] for n in orc.SECTION_NAMES] == [0, 991_232, 1_982_464, 2_973_696, 3_097_600, 3_221_504]
    # the generator's payload split agrees with the format's sections
    nib, pairs = synth.blob_payload_sizes(2816, 704)
    assert nib == sec["gate_sb"][0] and nib + 4 * pairs == nbytes


def test_layout_worked_example(orc):
    g = _load("layout_worked_example.json")
    R, C = g["R"], g["C"]
    nib = np.zeros(R * C // 2, dtype=np.uint8)
    for n in g["nibbles"]:
        nib[n["byte"]] |= np.uint8(n["q"] << (4 if n["high"] else 0))
    pairs = np.zeros(R * (C // 64) * 2, dtype=np.float16)
    pairs[0::2] = g["default_scale"]
    pairs[1::2] = g["default_bias"]
    for p in g["pairs"]:
        pairs[p["byte"] // 2] = p["scale"]
        pairs[p["byte"] // 2 + 1] = p["bias"]
    blob = np.concatenate([nib, pairs.view(np.uint8)])
    w = orc.dequant(blob, 0, nib.size, R, C)
    special = {(e["r"], e["c"]): e["w"] for e in g["expect"]}
    for (r, c), v in special.items():
        assert w[r, c] == v, (r, c, w[r, c], v)
    # every element not named by a nibble or pair entry is scale*0 + bias of its group
    named_rows_groups = {(p["r"], p["g"]) for p in g["pairs"]}
    named_elems = {(n["r"], n["c"]) for n in g["nibbles"]}
    for r in range(R):
        for c in range(C):
            if (r, c) in named_elems or (r, c // 64) in named_rows_groups:
                continue
            assert w[r, c] == 0.0


def test_known_bytes(orc):
    # byte 0x21 holds column 0 = 1 (low nibble) and column 1 = 2 (high nibble)
    R, C = 64, 64
    nib = np.zeros(R * C // 2, dtype=np.uint8)
    nib[0] = 0x21
    pairs = np.zeros(R * 2, dtype=np.float16)
    pairs[0::2] = 1.0
    w = orc.dequant(np.concatenate([nib, pairs.view(np.uint8)]), 0, nib.size, R, C)
    assert w[0, 0] == 1.0 and w[0, 1] == 2.0 and np.count_nonzero(w) == 2


def test_quant_roundtrip_exact(orc):
    rs = np.random.default_rng(1)
    R, C = 128, 192
    q = rs.integers(0, 16, (R, C))
    s = rs.uniform(0.005, 0.02, (R, C // 64)).astype(np.float16).astype(np.float64)
    b = rs.uniform(-0.1, 0.1, (R, C // 64)).astype(np.float16).astype(np.float64)
    nib, pairs = orc.encode_matrix(q, s, b)
    w = orc.dequant(np.concatenate([nib, pairs]), 0, nib.size, R, C)
    g = np.arange(C) // 64
    assert np.array_equal(w, s[:, g] * q + b[:, g])
    assert np.array_equal(orc.quantize_group_affine(w, s, b), q)


def test_unit_scale_integer_matvec_exact(orc):
    # unit scale, zero bias: weights are the nibbles; with x in {-1,0,1} every
    # partial sum is a small integer, so the float result equals integer arithmetic
    rs = np.random.default_rng(2)
    R, C = 128, 256
    q = rs.integers(0, 16, (R, C))
    nib, pairs = orc.encode_matrix(q, np.ones((R, C // 64)), np.zeros((R, C // 64)))
    w = orc.dequant(np.concatenate([nib, pairs]), 0, nib.size, R, C)
    x = rs.integers(-1, 2, C)
    assert np.array_equal(w @ x.astype(np.float64), (q @ x).astype(np.float64))


# ----------------------------------------------------------------------------- GELU

def test_gelu_closed_forms(orc):
    assert orc.gelu_tanh(0.0) == 0.0
    for z in (10.0, 12.5, 40.0):
        assert orc.gelu_tanh(z) == z
        assert orc.gelu_tanh(-z) == 0.0
    assert abs(float(orc.gelu_tanh(1.0)) - 0.8411919906) < 1e-9


def test_gelu_close_to_erf_gelu(orc):
    # the tanh form approximates x * Phi(x) to within about 4.7e-4 everywhere
    z = np.linspace(-8, 8, 4001)
    exact = np.array([0.5 * v * (1 + math.erf(v / math.sqrt(2))) for v in z])
    err = np.abs(orc.gelu_tanh(z) - exact)
    assert err.max() < 5e-4
    assert err.max() > 4e-4  # it is the tanh approximation, not erf itself


# ----------------------------------------------------------------------------- routing

def test_router_zero_weights_equal_bias(orc):
    E, d, k = 128, 64, 8
    h, lg, idx, w = orc.route(np.ones((1, d)), None, np.zeros((E, d)), np.full(E, 0.25), k)
    assert idx.tolist() == [list(range(8))]
    assert np.all(w == 1.0 / 8)


def test_router_planted_ties_lowest_id(orc):
    E, d, k = 16, 8, 4
    bias = np.zeros(E)
    bias[[3, 9, 12]] = 2.0       # three tied at the top
    bias[[1, 5, 7]] = 1.0        # ties across the k boundary: 1 wins over 5 and 7
    _, _, idx, _ = orc.route(np.ones((1, d)), None, np.zeros((E, d)), bias, k)
    assert idx.tolist() == [[3, 9, 12, 1]]


def test_topk_matches_bruteforce_subsets(orc):
    rs = random.Random(3)
    for trial in range(300):
        E, k = rs.randint(3, 10), 0
        k = rs.randint(1, E)
        # small integers to force ties often
        row = [float(rs.randint(-3, 3)) / 4 for _ in range(E)]
        assert orc.select_topk(row, k) == orc.topk_bruteforce(row, k), (row, k)


def test_weights_sum_to_one_and_closed_form(orc):
    rs = np.random.default_rng(4)
    lg = rs.normal(0, 2, 128)
    sel = orc.select_topk(lg, 8)
    w = orc.routing_weights(lg, sel)
    eps = np.finfo(np.float32 if orc is oracle else np.float64).eps
    assert abs(float(np.sum(w, dtype=np.float64)) - 1.0) < 8 * eps
    # softmax over 128 then renormalise == softmax over the selected logits
    z = np.exp(lg[sel] - lg[sel].max())
    assert np.allclose(w, z / z.sum(), rtol=_tol(orc, 1e-6, 1e-14), atol=0)
    assert np.all(np.diff(w) <= 0)


# ----------------------------------------------------------------------------- layer

def _tiny_model(seed, d=128, f=64, E=8):
    """Random tiny experts built with Python's own RNG as dense (q, s, b)."""
    rs = random.Random(seed)
    experts = []
    for _ in range(E):
        mats = {}
        for name, (R, C) in (("gate", (f, d)), ("up", (f, d)), ("down", (d, f))):
            q = [[rs.randint(0, 15) for _ in range(C)] for _ in range(R)]
            s = [[float(np.float16(rs.uniform(0.005, 0.02))) for _ in range(C // 64)] for _ in range(R)]
            b = [[float(np.float16(rs.uniform(-0.1, 0.1))) for _ in range(C // 64)] for _ in range(R)]
            mats[name] = (q, s, b)
        experts.append(mats)
    return experts


def _loops_ffn(mats, h, act=None):
    """Expert FFN with Python loops over the dense (q, s, b) lists (float64).
    ``act`` given: the down projection of that act instead of the computed one."""
    def dense_row(m, r, c):
        q, s, b = m
        return s[r][c // 64] * q[r][c] + b[r][c // 64]
    given = act
    gq = mats["gate"]
    f, d = len(gq[0]), len(gq[0][0])
    act = []
    for r in range(f):
        g = 0.0
        u = 0.0
        for c in range(d):
            g += dense_row(mats["gate"], r, c) * h[c]
            u += dense_row(mats["up"], r, c) * h[c]
        gl = 0.5 * g * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (g + 0.044715 * g * g * g)))
        act.append(gl * u)
    if given is not None:
        act = list(given)
    out = []
    for i in range(d):
        acc = 0.0
        for r in range(f):
            acc += dense_row(mats["down"], i, r) * act[r]
        out.append(acc)
    return np.array(act), np.array(out)


def _blob_of_tiny(mats, d, f, orc=oracle):
    enc = {n: (np.array(m[0]), np.array(m[1]), np.array(m[2])) for n, m in mats.items()}
    return orc.encode_expert(enc, d, f)


def test_expert_ffn_bruteforce_tiny(orc):
    d, f = 128, 64
    experts = _tiny_model(5, d, f, E=2)
    h = np.random.default_rng(5).normal(0, 1, d)
    for mats in experts:
        blob = _blob_of_tiny(mats, d, f)
        act_ref, out_ref = _loops_ffn(mats, h)
        act = orc.expert_gateup(blob, h, d, f)[0]
        out = orc.expert_down(blob, act, d, f)[0]
        tol = _tol(orc, 1e-5, 1e-12)
        assert np.abs(act - act_ref).max() <= tol * np.abs(act_ref).max()
        # down from the oracle's own act: the check is of the down step alone
        _, out_ref = _loops_ffn(mats, h, act=np.asarray(act, dtype=np.float64))
        assert np.abs(out - out_ref).max() <= tol * np.abs(out_ref).max()


def test_moe_layer_bruteforce_tiny(orc):
    # E=8, k=2, d=128, f=64, T=3 through textbook loops: softmax over 8, top-2 by
    # sort, renormalise, sum of the two experts' outputs plus the residual.
    d, f, E, k, T = 128, 64, 8, 2, 3
    experts = _tiny_model(6, d, f, E)
    blobs = [_blob_of_tiny(m, d, f) for m in experts]
    rs = np.random.default_rng(6)
    x = rs.normal(0, 1, (T, d))
    nw = rs.normal(1, 0.1, d)
    rw = rs.normal(0, 0.1, (E, d))
    bias = rs.normal(0, 0.5, E)
    y, idx, w, h, lg = orc.moe_layer(x, nw, rw, bias, lambda e: blobs[e], d, f, k)
    for t in range(T):
        ms = sum(v * v for v in x[t]) / d
        hh = [x[t][i] / math.sqrt(ms + 1e-6) * nw[i] for i in range(d)]
        logits = [sum(rw[e][i] * hh[i] for i in range(d)) + bias[e] for e in range(E)]
        mx = max(logits)
        p = [math.exp(v - mx) for v in logits]
        p = [v / sum(p) for v in p]
        order = sorted(range(E), key=lambda e: (-logits[e], e))[:k]
        assert idx[t].tolist() == order
        ws = [p[e] / sum(p[o] for o in order) for e in order]
        acc = list(x[t])
        for j, e in enumerate(order):
            _, out = _loops_ffn(experts[e], hh)
            acc = [a + ws[j] * o for a, o in zip(acc, out)]
        tol = _tol(orc, 1e-5, 1e-10)
        assert np.abs(y[t] - np.array(acc)).max() <= tol * np.abs(acc).max()


def test_one_hot_routing_is_single_expert(orc):
    d, f, E, k = 128, 64, 8, 8
    experts = _tiny_model(7, d, f, E)
    blobs = [_blob_of_tiny(m, d, f) for m in experts]
    x = np.random.default_rng(7).normal(0, 1, (1, d))
    for star in (0, 5):
        bias = np.zeros(E)
        bias[star] = 1000.0
        y, idx, w, h, _ = orc.moe_layer(x, None, np.zeros((E, d)), bias, lambda e: blobs[e], d, f, k)
        assert idx[0, 0] == star and w[0, 0] == 1.0 and np.all(w[0, 1:] == 0.0)
        single = orc.expert_down(blobs[star], orc.expert_gateup(blobs[star], x, d, f), d, f)
        if orc is oracle:  # fp32 throughout: y = fp32(x) + fp32(single), one fp32 add
            assert np.array_equal(y, x.astype(np.float32) + single)
        else:
            assert np.array_equal(y, x + single)


def test_slot_permutation_invariance(orc):
    d, f, E, k = 128, 64, 8, 3
    experts = _tiny_model(8, d, f, E)
    blobs = [_blob_of_tiny(m, d, f) for m in experts]
    stride = blobs[0].size
    rs = np.random.default_rng(8)
    x = rs.normal(0, 1, (4, d))
    rw = rs.normal(0, 0.1, (E, d))
    outs = []
    for perm in (np.arange(E), rs.permutation(E), rs.permutation(E)):
        arena = np.zeros(E * stride, dtype=np.uint8)
        for e in range(E):
            arena[perm[e] * stride:(perm[e] + 1) * stride] = blobs[e]
        blob_of = lambda e, perm=perm, arena=arena: arena[perm[e] * stride:(perm[e] + 1) * stride]
        outs.append(orc.moe_layer(x, None, rw, None, blob_of, d, f, k)[0])
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_rms_rescale_unit_rms(orc):
    x = np.random.default_rng(9).normal(3, 7, (5, 2816))
    y = orc.rms_rescale(x)
    y = np.asarray(y, dtype=np.float64)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=_tol(orc, 1e-6, 1e-9))


# ----------------------------------------------------------------------------- permute

@pytest.mark.parametrize("T,k,E", [(1, 8, 128), (3, 2, 8), (32, 8, 128), (257, 8, 128), (2048, 8, 128)])
def test_permute_invariants_and_bruteforce(orc, T, k, E):
    rs = np.random.default_rng(T)
    idx = np.stack([rs.choice(E, k, replace=False) for _ in range(T)])
    counts, offsets, sorted_pair, pair_pos = orc.permute(idx, E)
    assert counts.sum() == T * k and offsets[0] == 0 and offsets[-1] == T * k
    assert np.array_equal(np.diff(offsets), counts)
    assert sorted(sorted_pair.tolist()) == list(range(T * k))
    assert np.array_equal(sorted_pair[pair_pos], np.arange(T * k))
    flat = idx.ravel()
    buckets = [[p for p in range(T * k) if flat[p] == e] for e in range(E)]
    assert sorted_pair.tolist() == [p for b in buckets for p in b]


# ----------------------------------------------------------------------------- LRU

def test_lru_hand_worked_trace(orc):
    g = _load("lru_trace_4slots.json")
    c = orc.LruSlotCache(g["n_slots"], g["n_experts"])
    for t, st in enumerate(g["steps"]):
        hit, installs = c.step(t, st["sel"])
        assert hit == st["hit"], t
        assert [list(i) for i in installs] == st["installs"], t
        assert c.slot_expert == st["slots"], t
        assert c.stamp == st["stamps"], t


def test_lru_invariants_and_resume(orc):
    E, S, k, steps = 128, 64, 8, 512
    sel = synth.markov_selections(E, k, steps, seed=0, layer=3)
    a = orc.LruSlotCache(S, E)
    hits = 0
    for t in range(steps):
        before = set(e for e in a.slot_expert if e >= 0)
        hit, installs = a.step(t, sel[t].tolist())
        after = set(e for e in a.slot_expert if e >= 0)
        assert set(sel[t].tolist()) <= after
        assert sum(not h for h in hit) == len(set(sel[t].tolist()) - before) == len(installs)
        hits += sum(hit)
        if t == 255:
            state = a.export_state()
    # resume from the exported state reproduces the straight run
    b = orc.LruSlotCache(S, E)
    b.import_state(state)
    for t in range(256, steps):
        b.step(t, sel[t].tolist())
    assert b.export_state() == a.export_state()
    # with as many slots as experts every expert hits after its first use
    full = orc.LruSlotCache(E, E)
    seen = set()
    for t in range(steps):
        hit, _ = full.step(t, sel[t].tolist())
        assert hit == [e in seen for e in sel[t].tolist()]
        seen |= set(sel[t].tolist())


# ----------------------------------------------------------------------------- LFU

@pytest.mark.parametrize("key", ["whole_run", "window_2"])
def test_lfu_hand_worked_trace(orc, key):
    g = _load("lfu_trace_3slots.json")
    c = orc.LfuSlotCache(g["n_slots"], g["n_experts"], window=g[key]["window"])
    for t, st in enumerate(g[key]["steps"]):
        hit, installs = c.step(t, st["sel"])
        assert hit == st["hit"], t
        assert [list(i) for i in installs] == st["installs"], t
        assert c.slot_expert == st["slots"], t
        assert c.stamp == st["stamps"], t


def test_lfu_window_one_is_lru(orc):
    # a one-step window gives every resident expert not chosen now a count of
    # zero, so the choice falls to (stamp, slot): exactly the LRU rule
    for S, k, layer in ((64, 8, 0), (12, 4, 5)):
        E = 128 if S == 64 else 32
        sel = synth.markov_selections(E, k, 300, seed=1, layer=layer)
        a, b = orc.LruSlotCache(S, E), orc.LfuSlotCache(S, E, window=1)
        for t in range(300):
            assert a.step(t, sel[t].tolist()) == b.step(t, sel[t].tolist()), (S, t)
            assert a.slot_expert == b.slot_expert and a.stamp == b.stamp


@pytest.mark.parametrize("window", [None, 16])
def test_lfu_invariants_and_resume(orc, window):
    E, S, k, steps = 64, 16, 4, 240
    sel = synth.markov_selections(E, k, steps, seed=2, layer=1)
    a = orc.LfuSlotCache(S, E, window=window)
    for t in range(steps):
        before = list(a.slot_expert)
        hit, installs = a.step(t, sel[t].tolist())
        after = set(e for e in a.slot_expert if e >= 0)
        assert set(sel[t].tolist()) <= after
        assert sum(not h for h in hit) == len(set(sel[t].tolist()) - set(e for e in before if e >= 0))
        # an evicted expert was not chosen in this step, and every unchosen
        # resident that stayed is used at least as often as any evicted one
        chosen = set(sel[t].tolist())
        evicted = [ev for _, _, ev in installs if ev >= 0]
        kept = [e for e in before if e >= 0 and e not in chosen and e not in evicted]
        assert not (set(evicted) & chosen)
        if evicted and kept:
            cnt = a.counts()
            assert max(cnt[e] for e in evicted) <= min(cnt[e] for e in kept), t
        if t == 119:
            state = a.export_state()
    b = orc.LfuSlotCache(S, E, window=window)
    b.import_state(state)
    for t in range(120, steps):
        b.step(t, sel[t].tolist())
    assert b.export_state() == a.export_state()


def test_lfu_whole_run_keeps_the_popular_expert(orc):
    # two slots, one choice per step: once expert 0 has been chosen twice it
    # outlives the experts seen once (hits at steps 6 and 9), where LRU
    # evicts it every time
    E, S, k = 8, 2, 1
    seq = [[0], [1], [2], [0], [3], [4], [0], [5], [6], [0]]
    lfu, lru = orc.LfuSlotCache(S, E), orc.LruSlotCache(S, E)
    lfu_hits = sum(lfu.step(t, s)[0][0] for t, s in enumerate(seq))
    lru_hits = sum(lru.step(t, s)[0][0] for t, s in enumerate(seq))
    assert lfu_hits == 2 and lru_hits == 0


# ----------------------------------------------------------------------------- shared expert

def _bf16_bits_exact(w: np.ndarray) -> np.ndarray:
    """bf16 bits of values that bf16 holds exactly (small integers)."""
    bits = np.asarray(w, dtype=np.float32).view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0)
    return (bits >> 16).astype(np.uint16)


def test_shared_expert_is_the_routed_expert_ffn(orc):
    # an int4 expert with unit scale and zero bias has integer weights 0..15,
    # which bf16 holds exactly: the shared expert on those weights must be the
    # routed oracle's gate/up + down of that expert (independent code paths)
    d, f = 128, 64
    rs = np.random.default_rng(4)
    m = {name: (rs.integers(0, 16, (R, C)), np.ones((R, C // 64)), np.zeros((R, C // 64)))
         for name, (R, C) in (("gate", (f, d)), ("up", (f, d)), ("down", (d, f)))}
    blob = orc.encode_expert(m, d, f)
    h = rs.normal(0.0, 0.05, (3, d))
    x = rs.normal(0.0, 1.0, (3, d))
    w_gu = _bf16_bits_exact(np.concatenate([m["gate"][0], m["up"][0]]))
    w_dn = _bf16_bits_exact(m["down"][0])
    got = orc.shared_expert(h, w_gu, w_dn, residual=x)
    for t in range(3):
        act = orc.expert_gateup(blob, h[t], d, f)
        want = x[t] + orc.expert_down(blob, act, d, f)
        assert np.allclose(got[t], want, rtol=_tol(orc, 1e-6, 1e-12), atol=_tol(orc, 1e-5, 1e-9))


def test_shared_expert_zero_up_gives_the_residual(orc):
    d, f_sh = 64, 32
    rs = np.random.default_rng(5)
    w_gu = _bf16_bits_exact(np.concatenate([rs.integers(-3, 4, (f_sh, d)), np.zeros((f_sh, d))]))
    w_dn = _bf16_bits_exact(rs.integers(-3, 4, (d, f_sh)))
    x = rs.normal(0.0, 1.0, (2, d))
    want = x.astype(np.float32) if orc is oracle else x
    assert np.array_equal(orc.shared_expert(rs.normal(0, 1, (2, d)), w_gu, w_dn, residual=x), want)


# ----------------------------------------------------------------------------- shared GEMV

def test_shared_gemv_integer_exact(orc):
    # small-integer bf16 weights (exact in bf16) against small-integer inputs:
    # every partial sum is an integer below 2^24, so the result must equal the
    # integer matrix product exactly, in any summation order
    rs = np.random.default_rng(11)
    rows, cols, T = 96, 320, 3
    wi = rs.integers(-7, 8, (rows, cols))
    hi = rs.integers(-4, 5, (T, cols))
    got = np.asarray(orc.shared_gemv(_bf16_bits_exact(wi), hi.astype(np.float64)), dtype=np.float64)
    assert np.array_equal(got, (hi @ wi.T).astype(np.float64))


def test_shared_gemv_bf16_decoding(orc):
    # one-hot inputs read single weights back: bf16 bits 0x3F80 = 1.0, 0xC040 = -3.0,
    # 0x4049 = 3.140625, 0x0001 = 2^-133 (the smallest subnormal), 0x7F7F = max finite
    bits = np.array([[0x3F80, 0xC040, 0x4049, 0x0001, 0x7F7F, 0x0000, 0x8000, 0x3E80]], dtype=np.uint16)
    want = [1.0, -3.0, 3.140625, 2.0 ** -133, float(np.float32(3.3895313892515355e38)), 0.0, -0.0, 0.25]
    for c in range(8):
        h = np.zeros((1, 8))
        h[0, c] = 1.0
        assert float(np.asarray(orc.shared_gemv(bits, h))[0, 0]) == want[c], c


# ----------------------------------------------------------------------------- fp16 parse

def test_dequant_every_fp16_scale(orc):
    # nibble 1 and bias 0 give w = scale: every finite fp16 bit pattern as a
    # scale must read back as numpy's float16 value of those bits
    pat = np.arange(0, 1 << 16, dtype=np.uint32)
    finite = ((pat >> 10) & 0x1F) != 0x1F
    vals = pat[finite].astype(np.uint16).view(np.float16)
    n = vals.size
    R = (n + 63) // 64 * 64
    scale = np.zeros(R, dtype=np.float16)
    scale[:n] = vals
    q = np.zeros((R, 64), dtype=np.int64)
    q[:, 0] = 1
    nib, pairs = orc.encode_matrix(q, scale.astype(np.float64)[:, None], np.zeros((R, 1)))
    # encode_matrix rounds scale to fp16 again: identity for fp16 values
    w = np.asarray(orc.dequant(np.concatenate([nib, pairs]), 0, nib.size, R, 64), dtype=np.float64)
    assert np.array_equal(w[:n, 0], vals.astype(np.float64))
    assert np.all(w[:, 1:] == 0.0)


# ----------------------------------------------------------------------------- the two forms agree

@pytest.mark.parametrize("T,norm,zipf", [(3, True, True), (5, False, False)])
def test_cpp_oracle_matches_fp64_form_tiny(T, norm, zipf):
    # E=8, k=2, d=128, f=64 layers: the fp32 C++ oracle against the float64
    # numpy form of the same definitions, routing identical where the fp64
    # logit gap at the k boundary is above fp32 rounding
    d, f, E, k = 128, 64, 8, 2
    for seed in range(4):
        experts = _tiny_model(20 + seed, d, f, E)
        blobs = [_blob_of_tiny(m, d, f) for m in experts]
        rs = np.random.default_rng(20 + seed)
        x = rs.normal(0, 1, (T, d))
        nw = rs.normal(1, 0.1, d) if norm else None
        rw = rs.normal(0, 0.1, (E, d))
        bias = rs.normal(0, 0.5, E) if zipf else None
        y64, idx64, w64, h64, lg64 = oracle.fp64.moe_layer(x, nw, rw, bias, lambda e: blobs[e], d, f, k)
        y32, idx32, w32, h32, _ = oracle.moe_layer(x, nw, rw, bias, lambda e: blobs[e], d, f, k,
                                                   idx_override=idx64)
        assert np.abs(np.asarray(h32, np.float64) - h64).max() <= 1e-6 * np.abs(h64).max()
        assert np.abs(np.asarray(w32, np.float64) - w64).max() <= 1e-6
        for t in range(T):
            srt = np.sort(lg64[t])[::-1]
            if srt[k - 1] - srt[k] > 1e-4 * max(1.0, abs(srt[k - 1])):
                assert oracle.moe_layer(x[t:t + 1], nw, rw, bias, lambda e: blobs[e], d, f, k)[1][0].tolist() \
                    == idx64[t].tolist()
            err = np.abs(np.asarray(y32[t], np.float64) - y64[t]).max() / np.abs(y64[t]).max()
            assert err <= 1e-5, (seed, t, err)


def test_cpp_oracle_matches_fp64_form_full_size():
    # one token through one layer of the full shape (d=2816, f=704, E=128, k=8)
    d, f, E, k = synth.D_MODEL, synth.D_FF, synth.N_EXPERTS, synth.TOP_K
    rw = synth.router_weight(d, E, 3, 0)
    nw = synth.norm_weight(d, 3, 0)
    bias = synth.zipf_bias(E, 3, 0)
    x = synth.tokens(1, d, 3)
    cache = {}

    def blob_of(e):
        if e not in cache:
            cache[e] = synth.expert_blob(d, f, 3, 0, e)
        return cache[e]
    y64, idx64, w64, _, lg64 = oracle.fp64.moe_layer(x, nw, rw, bias, blob_of, d, f, k)
    y32, idx32, w32, _, _ = oracle.moe_layer(x, nw, rw, bias, blob_of, d, f, k)
    assert idx32.tolist() == idx64.tolist()
    assert np.abs(np.asarray(y32, np.float64) - y64).max() <= 1e-5 * np.abs(y64).max()
