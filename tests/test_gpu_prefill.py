"""GPU parity of the batched (prefill) path: route -> permute -> grouped MFMA
gate/up -> grouped MFMA down + rank-ordered combine, against the CPU oracle.
The fp16-operand path (staged tiles, and direct loads) is held to 1e-2 per
output row; bf16 operands are refused by the library."""
import numpy as np
import pytest
import torch

import oracle as orc
import synth
from helpers import D, E, F, K, TOL_BF16, LayerData, check_topk, decode_scaled_act, row_rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int4_routed_expert_route_amd.api as api
    api.lib()
    return api


def _np(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


PRECS = {"f16": ("MOE_PREC_F16_MFMA", torch.float16, TOL_BF16),
         "f16direct": ("MOE_PREC_F16_MFMA_DIRECT", torch.float16, TOL_BF16)}


def run_prefill(api, x_np, layer, blobs_dev, d, f, E_, k, slots=None, n_slots=None, prec="f16"):
    """route, permute, MFMA gate/up and down; returns dict of device tensors."""
    T = x_np.shape[0]
    dm = api.dims(d, f, E_, k)
    stride = api.moe_expert_blob_bytes(dm)
    slots = torch.arange(E_, dtype=torch.int32, device="cuda") if slots is None else slots
    n_slots = E_ if n_slots is None else n_slots
    x = torch.from_numpy(x_np).cuda()
    h = torch.empty(T, d, device="cuda")
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, device="cuda")
    ws = lambda c, p=0: torch.zeros(max(api.moe_workspace_size(c, T, dm, p), 256), dtype=torch.uint8, device="cuda")
    api.moe_route(x, None if layer.norm_w is None else torch.from_numpy(layer.norm_w).cuda(), 1e-6,
                  torch.from_numpy(layer.router_w).cuda(),
                  None if layer.bias is None else torch.from_numpy(layer.bias).cuda(), T, dm, h, idx, w, ws(0))
    counts = torch.empty(E_, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E_ + 1, dtype=torch.int32, device="cuda")
    sp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    pp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    api.moe_permute(idx, T, dm, counts, offsets, sp, pp)
    pname, pdtype, _ = PRECS[prec]
    pcode = getattr(api, pname)
    act = torch.zeros(api.moe_act_bytes(T, dm, pcode), dtype=torch.uint8, device="cuda")
    api.moe_expert_q4_gateup(h, idx, slots, n_slots, blobs_dev, stride, offsets, sp, None, 0, T, dm,
                             pcode, act, ws(2, pcode))
    y = torch.empty(T, d, device="cuda")
    api.moe_expert_q4_down_combine(act, idx, w, slots, n_slots, blobs_dev, stride, offsets, sp, pp, x, T, dm,
                                   pcode, y, ws(3, pcode))
    return dict(x=x, h=h, idx=idx, w=w, act=decode_scaled_act(act, T * k, f, pdtype), y=y, counts=counts)


class SmallLayer:
    def __init__(self, d, f, E_, seed):
        self.router_w = synth.router_weight(d, E_, seed, 0)
        self.norm_w = synth.norm_weight(d, seed, 0)
        self.bias = synth.zipf_bias(E_, seed, 0)
        self.blobs = {e: synth.expert_blob(d, f, seed, 0, e) for e in range(E_)}

    def blob_of(self, e):
        return self.blobs[e]


@pytest.mark.parametrize("prec", ["f16", "f16direct"])
@pytest.mark.parametrize("d,f,E_,k,T", [(256, 128, 16, 4, 40), (320, 192, 8, 2, 7), (2816, 704, 128, 8, 1),
                                        (2816, 704, 128, 8, 48), (384, 256, 4, 2, 300), (1088, 576, 16, 4, 40),
                                        (1600, 768, 16, 4, 40)])
def test_prefill_parity_small(api, d, f, E_, k, T, prec):
    """Several M tiles per expert (T=300 over 4 experts) with ragged tails,
    N tiles with a partial last tile (f=192, d=320), and single tokens.  With
    few items the small ones are split along K (at least 6 steps a range):
    T=1 (one row each; gate/up in 4 ranges of 11 K steps, down's 11 steps not
    split); d=1088, f=576 (gate/up's 17 steps in 8 + 9, a partial N tile);
    d=1600, f=768 (gate/up's 25 steps in 6, 6, 6, 7, down's 12 in 6 + 6 with a
    partial N tile).  The last two have experts of more than 32 rows, which
    are not split, beside split ones."""
    tol = PRECS[prec][2]
    layer = SmallLayer(d, f, E_, seed=4)
    arena = torch.from_numpy(np.concatenate([layer.blobs[e] for e in range(E_)])).cuda()
    x_np = synth.tokens(T, d, seed=4, stream=T)
    out = run_prefill(api, x_np, layer, arena, d, f, E_, k, prec=prec)
    gi = _np(out["idx"])
    _, lg, ridx, _ = orc.route(x_np, layer.norm_w, layer.router_w, layer.bias, k)
    check_topk(gi, ridx, lg)
    ry, _, _, rh, _ = orc.moe_layer(x_np, layer.norm_w, layer.router_w, layer.bias, layer.blob_of, d, f, k,
                                    idx_override=gi)
    act = out["act"]
    ract = np.stack([orc.expert_gateup(layer.blobs[int(gi[t, j])], rh[t], d, f)[0]
                     for t in range(T) for j in range(k)])
    e_act = row_rel_err(act, ract)
    e_y = row_rel_err(_np(out["y"]) - x_np, ry - x_np)
    print(f"[{prec}] act {e_act:.3e}  moe-out {e_y:.3e}", flush=True)
    assert e_act < tol
    assert row_rel_err(_np(out["y"]), ry) < tol
    assert e_y < tol


class UniformLayer(SmallLayer):
    """No router bias: the choice spreads nearly evenly over the experts."""

    def __init__(self, d, f, E_, seed):
        super().__init__(d, f, E_, seed)
        self.bias = None


@pytest.mark.parametrize("d,f,E_,k,T", [(2816, 704, 128, 8, 64), (1024, 1408, 128, 8, 64)])
def test_few_pairs_multi_item_rounds(api, d, f, E_, k, T):
    """Batches of up to 64 tokens send experts of at most 32 pairs to the
    few-pairs kernel.  Spread evenly, 512 pairs over 128 experts give every
    XCD about 16 expert parts: with f=704 that is more gate/up items than the
    XCD's 96 workgroups, so a round mixes workgroups running one item on four
    waves with ones running two on K halves; with f=1408 a round of two items
    per workgroup comes first.  d=2816 gives down two rounds of four items per
    workgroup.  The premise is checked on the oracle's routing."""
    tol = TOL_BF16
    layer = UniformLayer(d, f, E_, seed=11)
    x_np = synth.tokens(T, d, seed=11, stream=T)
    _, lg, ridx, _ = orc.route(x_np, layer.norm_w, layer.router_w, layer.bias, k)
    cnt = np.bincount(np.asarray(ridx).ravel(), minlength=E_)
    parts = int(np.sum((cnt > 0) & (cnt <= 16)) + 2 * np.sum((cnt > 16) & (cnt <= 32)))
    assert parts * (f // 64) > 8 * 96, f"only {parts} expert parts: no multi-item gate/up round"
    arena = torch.from_numpy(np.concatenate([layer.blobs[e] for e in range(E_)])).cuda()
    out = run_prefill(api, x_np, layer, arena, d, f, E_, k)
    gi = _np(out["idx"])
    check_topk(gi, ridx, lg)
    ry, _, _, rh, _ = orc.moe_layer(x_np, layer.norm_w, layer.router_w, layer.bias, layer.blob_of, d, f, k,
                                    idx_override=gi)
    ract = np.stack([orc.expert_gateup(layer.blobs[int(gi[t, j])], rh[t], d, f)[0]
                     for t in range(T) for j in range(k)])
    e_act = row_rel_err(out["act"], ract)
    e_y = row_rel_err(_np(out["y"]) - x_np, ry - x_np)
    print(f"parts {parts}  act {e_act:.3e}  moe-out {e_y:.3e}", flush=True)
    assert e_act < tol
    assert e_y < tol


@pytest.mark.parametrize("prec", ["f16", "f16direct"])
def test_prefill_large_activations(api, prec):
    """On weights with a positive mean offset, inputs close to a constant
    vector make every gate/up sum coherent (g, u ~ 260), so gelu(g) * u ~ 7e4
    exceeds fp16's largest value: the block-scaled intermediates must still
    match the oracle."""
    T = 24
    layer = LayerData(seed=0, layer=1, offset_weights=True)
    arena = torch.from_numpy(np.concatenate([layer.blobs[e] for e in range(E)])).cuda()
    x_np = (1.0 + 0.01 * synth.tokens(T, D, seed=0, stream=5)).astype(np.float32)
    out = run_prefill(api, x_np, layer, arena, D, F, E, K, prec=prec)
    gi = _np(out["idx"])
    ry, _, _, rh, _ = orc.moe_layer(x_np, layer.norm_w, layer.router_w, layer.bias, layer.blob_of, D, F, K,
                                    idx_override=gi)
    ract = np.stack([orc.expert_gateup(layer.blobs[int(gi[t, j])], rh[t], D, F)[0]
                     for t in range(T) for j in range(K)])
    assert np.abs(ract).max() > 65504.0
    tol = PRECS[prec][2]
    e_act = row_rel_err(out["act"], ract)
    e_y = row_rel_err(_np(out["y"]) - x_np, ry - x_np)
    print(f"[{prec}] large: act {e_act:.3e}  moe-out {e_y:.3e}", flush=True)
    assert e_act < tol and e_y < tol


@pytest.mark.parametrize("prec", ["f16", "f16direct"])
def test_prefill_exact_gateup(api, prec):
    """Unit scale, zero bias, h in {0,1} with 8 ones per token, gate nibbles in
    8..15: 16-bit operands are exact, fp32 sums of integers are exact and GELU
    saturates (g >= 64), so act decodes to the round-to-nearest-even 16-bit
    value of g*u exactly (power-of-two block scaling commutes with rounding)."""
    d, f, E_, k, T = 256, 128, 8, 2, 20
    rs = np.random.default_rng(21)
    qs = []
    blobs = []
    for _ in range(E_):
        m = {}
        for name, (R, C) in (("gate", (f, d)), ("up", (f, d)), ("down", (d, f))):
            lo = 8 if name == "gate" else 0
            m[name] = (rs.integers(lo, 16, (R, C)), np.ones((R, C // 64)), np.zeros((R, C // 64)))
        qs.append(m)
        blobs.append(orc.encode_expert(m, d, f))
    arena = torch.from_numpy(np.concatenate(blobs)).cuda()
    dm = api.dims(d, f, E_, k)
    stride = api.moe_expert_blob_bytes(dm)
    slots = torch.arange(E_, dtype=torch.int32, device="cuda")
    h_np = np.zeros((T, d), np.float32)
    for t in range(T):
        h_np[t, rs.choice(d, 8, replace=False)] = 1.0
    idx_np = np.stack([rs.choice(E_, k, replace=False) for _ in range(T)]).astype(np.int32)
    h = torch.from_numpy(h_np).cuda()
    idx = torch.from_numpy(idx_np).cuda()
    counts = torch.empty(E_, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E_ + 1, dtype=torch.int32, device="cuda")
    sp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    pp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    api.moe_permute(idx, T, dm, counts, offsets, sp, pp)
    pname, pdtype, _ = PRECS[prec]
    pcode = getattr(api, pname)
    act = torch.zeros(api.moe_act_bytes(T, dm, pcode), dtype=torch.uint8, device="cuda")
    ws = torch.zeros(api.moe_workspace_size(2, T, dm, pcode), dtype=torch.uint8, device="cuda")
    api.moe_expert_q4_gateup(h, idx, slots, E_, arena, stride, offsets, sp, None, 0, T, dm, pcode, act, ws)
    torch.cuda.synchronize()
    got = decode_scaled_act(act, T * k, f, pdtype)
    for t in range(T):
        for j in range(k):
            e = idx_np[t, j]
            g = qs[e]["gate"][0] @ h_np[t].astype(np.int64)
            u = qs[e]["up"][0] @ h_np[t].astype(np.int64)
            assert g.min() >= 64 and (g * u).max() <= 14400
            ref = torch.from_numpy((g.astype(np.float64) * u).astype(np.float32)).to(pdtype).double().numpy()
            assert np.array_equal(got[t * k + j], ref), (t, j)


@pytest.mark.parametrize("prec", ["f16", "f16direct"])
def test_prefill_full_size_sampled(api, prec):
    """One layer at the full prefill shape (2048 tokens, Zipf routing), in the
    bench's launch configuration; the oracle recomputes a sample of tokens."""
    T = 2048
    layer = LayerData(seed=0, layer=0)
    arena = torch.from_numpy(np.concatenate([layer.blobs[e] for e in range(E)])).cuda()
    x_np = synth.tokens(T, D, seed=0, stream=99)
    out = run_prefill(api, x_np, layer, arena, D, F, E, K, prec=prec)
    gi = _np(out["idx"])
    counts = _np(out["counts"])
    assert counts.sum() == T * K and counts.max() > 500  # Zipf-skewed load
    sample = np.random.default_rng(0).choice(T, 12, replace=False)
    _, lg, ridx, _ = orc.route(x_np[sample], layer.norm_w, layer.router_w, layer.bias, K)
    check_topk(gi[sample], ridx, lg)
    ry, *_ = orc.moe_layer(x_np[sample], layer.norm_w, layer.router_w, layer.bias, layer.blob_of, D, F, K,
                           idx_override=gi[sample])
    e_y = row_rel_err(_np(out["y"])[sample] - x_np[sample], ry - x_np[sample])
    print(f"[{prec}] full-size moe-out {e_y:.3e}", flush=True)
    assert row_rel_err(_np(out["y"])[sample], ry) < PRECS[prec][2]
    assert e_y < PRECS[prec][2]
    assert np.all(np.isfinite(_np(out["y"])))


@pytest.mark.parametrize("d,f,E_,k,T", [(256, 128, 16, 4, 40), (2816, 704, 128, 8, 300), (1600, 768, 16, 4, 40)])
def test_prefill_direct_loads_match_staged_tiles(api, d, f, E_, k, T):
    """Weights loaded straight into registers give bit for bit the staged-tile
    path's act and output: the same dequantised values meet the same MFMAs in
    the same order; only where the nibbles come from differs."""
    layer = SmallLayer(d, f, E_, seed=31)
    arena = torch.from_numpy(np.concatenate([layer.blobs[e] for e in range(E_)])).cuda()
    x_np = synth.tokens(T, d, seed=31, stream=5)
    a = run_prefill(api, x_np, layer, arena, d, f, E_, k, prec="f16")
    b = run_prefill(api, x_np, layer, arena, d, f, E_, k, prec="f16direct")
    assert np.array_equal(_np(a["idx"]), _np(b["idx"]))
    assert np.array_equal(a["act"], b["act"])
    assert np.array_equal(_np(a["y"]), _np(b["y"]))


@pytest.mark.parametrize("d,f,E_,k,T", [(2816, 704, 128, 8, 1), (2816, 704, 128, 8, 32), (1600, 768, 16, 4, 40),
                                        (2816, 704, 128, 8, 200), (1600, 768, 16, 4, 120)])
def test_split_k_deterministic_and_counters_reset(api, d, f, E_, k, T):
    """Every call gives the same bits and leaves the workspace's arrival
    counters at zero, so one workspace serves call after call.  Up to 64
    tokens the experts with few pairs run on the few-pairs kernel (K parts
    summed through LDS in a fixed order; 32 tokens is the batched-decode
    shape); beyond, the work-list GEMM splits their items along K and the last
    K range to arrive sums the partials in range order (the last case splits
    the down GEMM too)."""
    layer = SmallLayer(d, f, E_, seed=12)
    arena = torch.from_numpy(np.concatenate([layer.blobs[e] for e in range(E_)])).cuda()
    x_np = synth.tokens(T, d, seed=12, stream=T)
    ref = run_prefill(api, x_np, layer, arena, d, f, E_, k)
    dm = api.dims(d, f, E_, k)
    stride = api.moe_expert_blob_bytes(dm)
    slots = torch.arange(E_, dtype=torch.int32, device="cuda")
    counts = torch.empty(E_, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E_ + 1, dtype=torch.int32, device="cuda")
    sp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    pp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    api.moe_permute(ref["idx"], T, dm, counts, offsets, sp, pp)
    pc = api.MOE_PREC_F16_MFMA
    wsg = torch.zeros(api.moe_workspace_size(api.MOE_CALL_GATEUP, T, dm, pc), dtype=torch.uint8, device="cuda")
    wsd = torch.zeros(api.moe_workspace_size(api.MOE_CALL_DOWN_COMBINE, T, dm, pc), dtype=torch.uint8,
                      device="cuda")
    for _ in range(3):
        act = torch.zeros(api.moe_act_bytes(T, dm, pc), dtype=torch.uint8, device="cuda")
        api.moe_expert_q4_gateup(ref["h"], ref["idx"], slots, E_, arena, stride, offsets, sp, None, 0, T, dm, pc,
                                 act, wsg)
        y = torch.empty(T, d, device="cuda")
        api.moe_expert_q4_down_combine(act, ref["idx"], ref["w"], slots, E_, arena, stride, offsets, sp, pp,
                                       ref["x"], T, dm, pc, y, wsd)
        assert np.array_equal(decode_scaled_act(act, T * k, f, torch.float16), ref["act"])
        assert np.array_equal(_np(y), _np(ref["y"]))
        assert not _np(wsg[:2048]).any() and not _np(wsd[:2048]).any()
    ry, *_ = orc.moe_layer(x_np, layer.norm_w, layer.router_w, layer.bias, layer.blob_of, d, f, k,
                           idx_override=_np(ref["idx"]))
    assert row_rel_err(_np(ref["y"]) - x_np, ry - x_np) < TOL_BF16
