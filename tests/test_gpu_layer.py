"""GPU parity of every libmoe call against the CPU oracle (one layer, small T).

Runs on an MI355X through the C ABI (ctypes binding).  Inputs are seeded and
synthetic (synth/); expected values come from oracle/ only."""
import numpy as np
import pytest
import torch

import oracle as orc
import synth
from helpers import D, E, F, K, TOL_FP32, LayerData, check_topk, row_rel_err

pytestmark = pytest.mark.gpu

L = None
DM = None


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global L, DM
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int4_routed_expert_route_amd.api as api
    api.lib()
    L = api
    DM = api.dims(D, F, E, K)
    yield


@pytest.fixture(scope="module")
def layer0():
    return LayerData(seed=0, layer=0)


@pytest.fixture(scope="module")
def dev_layer(layer0):
    stride = orc.blob_bytes(D, F)
    host = np.concatenate([layer0.blobs[e] for e in range(E)])
    arena = torch.from_numpy(host).cuda()
    slots = torch.arange(E, dtype=torch.int32, device="cuda")
    return dict(arena=arena, stride=stride, slots=slots,
                router_w=torch.from_numpy(layer0.router_w).cuda(),
                bias=torch.from_numpy(layer0.bias).cuda(),
                norm_w=torch.from_numpy(layer0.norm_w).cuda())


def _ws(call, T, prec=0):
    n = max(L.moe_workspace_size(call, T, DM, prec), 256)
    return torch.zeros(n, dtype=torch.uint8, device="cuda")


def _route(x, dl, T, norm=True, bias=True):
    h = torch.empty(T, D, dtype=torch.float32, device="cuda")
    idx = torch.empty(T, K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, K, dtype=torch.float32, device="cuda")
    L.moe_route(x, dl["norm_w"] if norm else None, 1e-6, dl["router_w"], dl["bias"] if bias else None, T, DM,
                h, idx, w, _ws(L.MOE_CALL_ROUTE, T))
    return h, idx, w


def _gateup(h, idx, dl, T, slots=None, offsets=None, sorted_pair=None, mask=None, mask_value=1, act=None):
    if act is None:
        act = torch.zeros(T * K, F, dtype=torch.float32, device="cuda")
    L.moe_expert_q4_gateup(h, idx, dl["slots"] if slots is None else slots, dl.get("n_slots", E), dl["arena"],
                           dl["stride"],
                           offsets, sorted_pair, mask, mask_value, T, DM, L.MOE_PREC_FP32, act,
                           _ws(L.MOE_CALL_GATEUP, T))
    return act


def _down(act, idx, w, dl, T, residual, slots=None, offsets=None, sorted_pair=None, pair_pos=None):
    y = torch.empty(T, D, dtype=torch.float32, device="cuda")
    L.moe_expert_q4_down_combine(act, idx, w, dl["slots"] if slots is None else slots, dl.get("n_slots", E),
                                 dl["arena"],
                                 dl["stride"], offsets, sorted_pair, pair_pos, residual, T, DM,
                                 L.MOE_PREC_FP32, y, _ws(L.MOE_CALL_DOWN_COMBINE, T))
    return y


def _np(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


# ----------------------------------------------------------------------------- route

@pytest.mark.parametrize("T,norm,bias", [(1, False, False), (1, True, True), (3, True, True),
                                         (8, True, True), (9, True, True), (32, True, True),
                                         (32, False, True), (40, False, False), (257, True, False),
                                         (600, True, True), (1024, True, True), (2048, False, True)])
def test_route_parity(layer0, dev_layer, T, norm, bias):
    x = synth.tokens(T, D, seed=0, stream=T)
    h, idx, w = _route(torch.from_numpy(x).cuda(), dev_layer, T, norm, bias)
    rh, lg, ridx, rw = orc.route(x, layer0.norm_w if norm else None, layer0.router_w,
                                 layer0.bias if bias else None, K)
    assert row_rel_err(_np(h), rh) < 1e-5
    gi = _np(idx)
    check_topk(gi, ridx, lg)
    rw_g = np.stack([orc.routing_weights(lg[t], gi[t]) for t in range(T)])
    assert row_rel_err(_np(w), rw_g) < TOL_FP32
    assert np.allclose(_np(w).sum(axis=1), 1.0, atol=1e-5)


def test_route_equal_logits_and_ties(dev_layer):
    # one token (fused small path), 20 (one 16-token router tile) and 300
    # (two tiles per workgroup, ragged last tile)
    for T in (1, 20, 300):
        x = torch.from_numpy(synth.tokens(T, D, seed=1)).cuda()
        zero_w = torch.zeros(E, D, dtype=torch.float32, device="cuda")
        bias = torch.full((E,), 0.5, dtype=torch.float32, device="cuda")
        h = torch.empty(T, D, device="cuda")
        idx = torch.empty(T, K, dtype=torch.int32, device="cuda")
        w = torch.empty(T, K, device="cuda")
        L.moe_route(x, None, 1e-6, zero_w, bias, T, DM, h, idx, w, _ws(L.MOE_CALL_ROUTE, T))
        assert (_np(idx) == np.arange(8)).all()
        assert (_np(w) == np.float32(0.125)).all()
        b = np.zeros(E, dtype=np.float32)
        b[[100, 7, 64]] = 3.0
        b[[5, 90, 2, 77, 31, 6]] = 2.0
        L.moe_route(x, None, 1e-6, zero_w, torch.from_numpy(b).cuda(), T, DM, h, idx, w, _ws(L.MOE_CALL_ROUTE, T))
        assert (_np(idx) == np.array([7, 64, 100, 2, 5, 6, 31, 77])).all()


# ----------------------------------------------------------------------------- experts

def test_layer_c0_parity(layer0, dev_layer):
    """Single MoE layer, 1 token, no norm: route -> gate/up -> down + combine."""
    x = synth.tokens(1, D, seed=0)
    xd = torch.from_numpy(x).cuda()
    h, idx, w = _route(xd, dev_layer, 1, norm=False, bias=False)
    act = _gateup(h, idx, dev_layer, 1)
    y = _down(act, idx, w, dev_layer, 1, xd)
    y0 = _down(act, idx, w, dev_layer, 1, None)
    gi = _np(idx)
    ry, ridx, rw, rh, lg = orc.moe_layer(x, None, layer0.router_w, None, layer0.blob_of, D, F, K)
    check_topk(gi, ridx, lg)
    ry, _, rw, rh, _ = orc.moe_layer(x, None, layer0.router_w, None, layer0.blob_of, D, F, K, idx_override=gi)
    racts = np.stack([orc.expert_gateup(layer0.blobs[int(e)], rh[0], D, F)[0] for e in gi[0]])
    assert row_rel_err(_np(act), racts) < TOL_FP32
    assert row_rel_err(_np(y), ry) < TOL_FP32
    assert row_rel_err(_np(y0), ry - x) < TOL_FP32


@pytest.mark.parametrize("T", [1, 2, 5])
def test_layer_decode_parity_with_norm(layer0, dev_layer, T):
    x = synth.tokens(T, D, seed=2, stream=T)
    xd = torch.from_numpy(x).cuda()
    h, idx, w = _route(xd, dev_layer, T)
    act = _gateup(h, idx, dev_layer, T)
    y = _down(act, idx, w, dev_layer, T, xd)
    gi = _np(idx)
    _, _, _, _, lg = orc.moe_layer(x, layer0.norm_w, layer0.router_w, layer0.bias, layer0.blob_of, D, F, K)
    ry, ridx, rw, rh, lg = orc.moe_layer(x, layer0.norm_w, layer0.router_w, layer0.bias, layer0.blob_of, D, F, K,
                                         idx_override=gi)
    assert row_rel_err(_np(y), ry) < TOL_FP32
    assert row_rel_err(_np(y) - x, ry - x) < TOL_FP32


def _unit_blob(rs, with_bias=False):
    """Expert with unit scale and zero bias: the weights are the nibbles."""
    qs = {}
    for m, (R, C) in (("gate", (F, D)), ("up", (F, D)), ("down", (D, F))):
        q = rs.integers(0, 16, (R, C))
        qs[m] = (q, np.ones((R, C // 64)), np.zeros((R, C // 64)))
    return orc.encode_expert(qs, D, F), qs


def test_exact_integer_expert():
    """Unit scale, zero bias, x in {0,1}: gate, up and down sums are exact
    integers and GELU saturates exactly, so GPU and oracle agree bit for bit."""
    rs = np.random.default_rng(11)
    blobs, qs = zip(*[_unit_blob(rs) for _ in range(K)])
    stride = orc.blob_bytes(D, F)
    arena = torch.from_numpy(np.concatenate(blobs)).cuda()
    slots = torch.full((E,), -1, dtype=torch.int32)
    sel = np.array([3, 17, 40, 41, 99, 100, 126, 127], dtype=np.int32)
    slots[sel] = torch.arange(K, dtype=torch.int32)
    dl = dict(arena=arena, stride=stride, slots=slots.cuda(), n_slots=K)
    x = (rs.random((1, D)) < 0.05).astype(np.float32)
    h = torch.from_numpy(x).cuda()
    idx = torch.from_numpy(sel[None, :]).cuda()
    act = _gateup(h, idx, dl, 1)
    a = _np(act)
    ref = []
    for j in range(K):
        g = qs[j]["gate"][0] @ x[0].astype(np.int64)
        u = qs[j]["up"][0] @ x[0].astype(np.int64)
        assert g.min() >= 10
        ref.append((g.astype(np.float64) * u).astype(np.float32))
    assert np.array_equal(a, np.stack(ref))
    # down with small integer activations and power-of-two weights: exact
    act_i = rs.integers(-2, 3, (K, F)).astype(np.float32)
    wts = np.array([[1, 0.5, 0.25, 0.125, 2, 4, 1, 1]], dtype=np.float32)
    y = _down(torch.from_numpy(act_i).cuda(), idx, torch.from_numpy(wts).cuda(), dl, 1, None)
    ref_y = sum(wts[0, j] * (qs[j]["down"][0] @ act_i[j].astype(np.int64)) for j in range(K))
    assert np.array_equal(_np(y)[0], ref_y.astype(np.float32))


def test_slot_permutation_invariance(layer0, dev_layer):
    x = torch.from_numpy(synth.tokens(2, D, seed=3)).cuda()
    h, idx, w = _route(x, dev_layer, 2)
    y_ref = _np(_down(_gateup(h, idx, dev_layer, 2), idx, w, dev_layer, 2, x))
    perm = synth.slot_permutation(E, seed=0, layer=0)
    host = np.zeros(E * dev_layer["stride"], dtype=np.uint8)
    for e in range(E):
        host[perm[e] * dev_layer["stride"]:(perm[e] + 1) * dev_layer["stride"]] = layer0.blobs[e]
    dl = dict(arena=torch.from_numpy(host).cuda(), stride=dev_layer["stride"],
              slots=torch.from_numpy(perm).cuda())
    y = _np(_down(_gateup(h, idx, dl, 2), idx, w, dl, 2, x))
    assert np.array_equal(y, y_ref)


def test_unaligned_views_and_determinism(layer0, dev_layer):
    """Buffers at 16-byte (not 256-byte) offsets inside larger allocations; two
    runs give identical bits."""
    T = 3
    x_np = synth.tokens(T, D, seed=4)
    big = torch.zeros(T * D + 4, dtype=torch.float32, device="cuda")
    x = big[4:].view(T, D)
    x.copy_(torch.from_numpy(x_np))
    hb = torch.zeros(T * D + 12, device="cuda")
    h = hb[12:].view(T, D)
    ib = torch.zeros(T * K + 4, dtype=torch.int32, device="cuda")
    idx = ib[4:].view(T, K)
    wb = torch.zeros(T * K + 4, device="cuda")
    w = wb[4:].view(T, K)
    L.moe_route(x, dev_layer["norm_w"], 1e-6, dev_layer["router_w"], dev_layer["bias"], T, DM, h, idx, w,
                _ws(L.MOE_CALL_ROUTE, T))
    ab = torch.zeros(T * K * F + 4, device="cuda")
    act = ab[4:].view(T * K, F)
    _gateup(h, idx, dev_layer, T, act=act)
    y1 = _np(_down(act, idx, w, dev_layer, T, x))
    y2 = _np(_down(_gateup(h, idx, dev_layer, T), idx, w, dev_layer, T, x))
    assert np.array_equal(y1, y2)
    gi = _np(idx)
    ry, *_ = orc.moe_layer(x_np, layer0.norm_w, layer0.router_w, layer0.bias, layer0.blob_of, D, F, K,
                           idx_override=gi)
    assert row_rel_err(y1, ry) < TOL_FP32
    # a 4-byte offset is refused before anything runs
    with pytest.raises(L.MoeError) as ei:
        L.moe_route(big[1:1 + D].view(1, D), None, 1e-6, dev_layer["router_w"], None, 1, DM, h[:1], idx[:1],
                    w[:1], _ws(L.MOE_CALL_ROUTE, 1))
    assert ei.value.status == L.MOE_ERR_ALIGN


def test_absent_slot_gives_nan(dev_layer):
    x = torch.from_numpy(synth.tokens(1, D, seed=5)).cuda()
    h, idx, w = _route(x, dev_layer, 1)
    slots = dev_layer["slots"].clone()
    missing = int(_np(idx)[0, 2])
    slots[missing] = -1
    act = _np(_gateup(h, idx, dev_layer, 1, slots=slots))
    assert np.isnan(act[2]).all() and np.isfinite(np.delete(act, 2, axis=0)).all()


def test_pair_mask_hits_then_misses(layer0, dev_layer):
    x = torch.from_numpy(synth.tokens(1, D, seed=6)).cuda()
    h, idx, w = _route(x, dev_layer, 1)
    full = _np(_gateup(h, idx, dev_layer, 1))
    mask = torch.tensor([1, 0, 1, 1, 0, 0, 1, 0], dtype=torch.uint8, device="cuda")
    act = torch.full((K, F), 7.0, device="cuda")
    _gateup(h, idx, dev_layer, 1, mask=mask, mask_value=1, act=act)
    part = _np(act)
    m = mask.cpu().numpy().astype(bool)
    assert np.array_equal(part[m], full[m]) and (part[~m] == 7.0).all()
    _gateup(h, idx, dev_layer, 1, mask=mask, mask_value=0, act=act)
    assert np.array_equal(_np(act), full)


# ----------------------------------------------------------------------------- permute + grouped

@pytest.mark.parametrize("with_ws", [False, True])
@pytest.mark.parametrize("T", [1, 3, 32, 257, 2048, 8192])
def test_permute_exact(T, with_ws):
    """Both permute paths against the oracle: one workgroup walking every pair
    (no workspace), and, past 1024 pairs with a workspace, the two launches over
    chunks of 1024 pairs (257 tokens: a ragged last chunk; 8192: the 64-chunk
    maximum)."""
    rs = np.random.default_rng(T)
    p = synth.zipf_probs(E, 0, 0)
    idx_np = np.stack([rs.choice(E, K, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    idx = torch.from_numpy(idx_np).cuda()
    counts = torch.full((E,), -5, dtype=torch.int32, device="cuda")
    offsets = torch.full((E + 1,), -5, dtype=torch.int32, device="cuda")
    sp = torch.full((T * K,), -5, dtype=torch.int32, device="cuda")
    pp = torch.full((T * K,), -5, dtype=torch.int32, device="cuda")
    nb = L.moe_workspace_size(L.MOE_CALL_PERMUTE, T, DM)
    assert (nb > 0) == (T * K > 1024)
    ws = torch.full((max(nb, 256),), 0x5A, dtype=torch.uint8, device="cuda") if with_ws else None
    L.moe_permute(idx, T, DM, counts, offsets, sp, pp, ws)
    rc, ro, rsp, rpp = orc.permute(idx_np, E)
    assert np.array_equal(_np(counts), rc) and np.array_equal(_np(offsets), ro)
    assert np.array_equal(_np(sp), rsp) and np.array_equal(_np(pp), rpp)


@pytest.mark.parametrize("T", [4, 32])
def test_grouped_batch_parity(layer0, dev_layer, T):
    x_np = synth.tokens(T, D, seed=7, stream=T)
    x = torch.from_numpy(x_np).cuda()
    h, idx, w = _route(x, dev_layer, T)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    sp = torch.empty(T * K, dtype=torch.int32, device="cuda")
    pp = torch.empty(T * K, dtype=torch.int32, device="cuda")
    L.moe_permute(idx, T, DM, counts, offsets, sp, pp)
    act = _gateup(h, idx, dev_layer, T, offsets=offsets, sorted_pair=sp)
    y = _down(act, idx, w, dev_layer, T, x, offsets=offsets, sorted_pair=sp, pair_pos=pp)
    # the ungrouped path on the same inputs
    act_u = _gateup(h, idx, dev_layer, T)
    y_u = _down(act_u, idx, w, dev_layer, T, x)
    gi = _np(idx)
    ry, *_ = orc.moe_layer(x_np, layer0.norm_w, layer0.router_w, layer0.bias, layer0.blob_of, D, F, K,
                           idx_override=gi)
    assert row_rel_err(_np(y), ry) < TOL_FP32
    assert row_rel_err(_np(y_u), ry) < TOL_FP32
    assert row_rel_err(_np(act), _np(act_u)) < 1e-5


# ----------------------------------------------------------------------------- small helpers

def test_shared_gemv_bf16():
    rows, cols, T = 1024, D, 3
    wb = synth.shared_weight_bf16(rows, cols, seed=0, layer=0)
    h_np = synth.tokens(T, cols, seed=8)
    out = torch.empty(T, rows, device="cuda")
    L.moe_shared_gemv_bf16(torch.from_numpy(wb.view(np.int16)).cuda(), torch.from_numpy(h_np).cuda(), T, rows,
                           cols, out)
    assert row_rel_err(_np(out), orc.shared_gemv(wb, h_np)) < TOL_FP32


@pytest.mark.parametrize("d,f_sh,T,resid", [(256, 96, 1, True), (256, 96, 5, False), (256, 104, 9, True),
                                           (2816, 3776, 1, True)])
def test_shared_expert_bf16(d, f_sh, T, resid):
    """The shared expert (bf16 gated FFN plus residual) against the oracle, and
    as the residual of the routed combine: y = (x + shared(h)) + sum_j w_j o_j."""
    w_gu = synth.shared_weight_bf16(2 * f_sh, d, 3, 0)
    w_dn = synth.shared_weight_bf16(d, f_sh, 3, 1)
    h_np = synth.tokens(T, d, 3)
    x_np = synth.tokens(T, d, 4)
    dev = lambda a: torch.from_numpy(a).cuda()
    out = torch.empty(T, d, device="cuda")
    ws = torch.zeros(L.moe_shared_expert_workspace_size(T, f_sh), dtype=torch.uint8, device="cuda")
    L.moe_shared_expert_bf16(dev(w_gu.view(np.int16)), dev(w_dn.view(np.int16)), dev(h_np),
                             dev(x_np) if resid else None, T, d, f_sh, out, ws)
    want = orc.shared_expert(h_np, w_gu, w_dn, residual=x_np if resid else None)
    if resid:  # the shared expert's own contribution, not hidden under the residual
        assert row_rel_err(_np(out) - x_np, want - x_np) < TOL_FP32
    assert row_rel_err(_np(out), want) < TOL_FP32


def test_shared_expert_into_routed_combine(layer0, dev_layer):
    """One decode token: shared expert into the residual, then the routed
    layer's down + combine on top, against the oracle's layer plus the
    oracle's shared expert."""
    d, f_sh, T = D, 512, 1
    w_gu = synth.shared_weight_bf16(2 * f_sh, d, 5, 0)
    w_dn = synth.shared_weight_bf16(d, f_sh, 5, 1)
    x_np = synth.tokens(T, d, 6)
    dev = lambda a: torch.from_numpy(a).cuda()
    dm = L.dims(D, F, E, K)
    ws = lambda c: torch.zeros(max(L.moe_workspace_size(c, T, dm), 256), dtype=torch.uint8, device="cuda")
    x = dev(x_np)
    h = torch.empty(T, d, device="cuda")
    idx = torch.empty(T, K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, K, device="cuda")
    L.moe_route(x, dev_layer["norm_w"], 1e-6, dev_layer["router_w"], dev_layer["bias"], T, dm, h, idx, w, ws(0))
    res = torch.empty(T, d, device="cuda")
    sws = torch.zeros(L.moe_shared_expert_workspace_size(T, f_sh), dtype=torch.uint8, device="cuda")
    L.moe_shared_expert_bf16(dev(w_gu.view(np.int16)), dev(w_dn.view(np.int16)), h, x, T, d, f_sh, res, sws)
    act = torch.empty(T * K, F, device="cuda")
    L.moe_expert_q4_gateup(h, idx, dev_layer["slots"], E, dev_layer["arena"], dev_layer["stride"], None, None, None,
                           0, T, dm, L.MOE_PREC_FP32, act, ws(2))
    y = torch.empty(T, d, device="cuda")
    L.moe_expert_q4_down_combine(act, idx, w, dev_layer["slots"], E, dev_layer["arena"], dev_layer["stride"], None,
                                 None, None, res, T, dm, L.MOE_PREC_FP32, y, ws(3))
    gi = _np(idx)
    ry, *_ = orc.moe_layer(x_np, layer0.norm_w, layer0.router_w, layer0.bias, layer0.blob_of, D, F, K,
                           idx_override=gi)
    hh = orc.rmsnorm(x_np, layer0.norm_w)
    want = ry + orc.shared_expert(hh, w_gu, w_dn)
    assert row_rel_err(_np(y) - x_np, want - x_np) < TOL_FP32


def test_rms_rescale():
    x_np = synth.tokens(5, D, seed=9) * 13.0
    x = torch.from_numpy(x_np).cuda()
    L.moe_rms_rescale(x, 5, D, 1e-6, x)
    assert row_rel_err(_np(x), orc.rms_rescale(x_np)) < 1e-5


@pytest.mark.parametrize("d,f,E,k,T", [(256, 128, 16, 4, 2), (128, 64, 8, 2, 3), (640, 192, 32, 8, 1),
                                       (2816, 704, 128, 8, 1), (256, 2048, 16, 4, 2), (128, 1792, 16, 16, 1)])
def test_other_shapes_parity(d, f, E, k, T):
    """Shapes whose groups do not fill every K-part (and the full shape again),
    ungrouped and grouped; f of 28 and 32 groups take the down kernels' widest
    lane slice (8 groups per K-part), with 16 waves per workgroup at k = 16."""
    dm = L.dims(d, f, E, k)
    stride = L.moe_expert_blob_bytes(dm)
    blobs = [synth.expert_blob(d, f, 3, 0, e) for e in range(E)]
    arena = torch.from_numpy(np.concatenate(blobs)).cuda()
    slots = torch.arange(E, dtype=torch.int32, device="cuda")
    rw = synth.router_weight(d, E, 3, 0)
    nw = synth.norm_weight(d, 3, 0)
    x_np = synth.tokens(T, d, 3, stream=d)
    x = torch.from_numpy(x_np).cuda()
    h = torch.empty(T, d, device="cuda")
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, device="cuda")
    ws = lambda c: torch.zeros(max(L.moe_workspace_size(c, T, dm), 256), dtype=torch.uint8, device="cuda")
    L.moe_route(x, torch.from_numpy(nw).cuda(), 1e-6, torch.from_numpy(rw).cuda(), None, T, dm, h, idx, w, ws(0))
    gi = _np(idx)
    ry, *_ = orc.moe_layer(x_np, nw, rw, None, lambda e: blobs[e], d, f, k, idx_override=gi)
    act = torch.empty(T * k, f, device="cuda")
    y = torch.empty(T, d, device="cuda")
    L.moe_expert_q4_gateup(h, idx, slots, E, arena, stride, None, None, None, 0, T, dm, L.MOE_PREC_FP32, act, ws(2))
    L.moe_expert_q4_down_combine(act, idx, w, slots, E, arena, stride, None, None, None, x, T, dm, L.MOE_PREC_FP32,
                                 y, ws(3))
    assert row_rel_err(_np(y), ry) < TOL_FP32
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    sp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    pp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    L.moe_permute(idx, T, dm, counts, offsets, sp, pp)
    act2 = torch.empty(T * k, f, device="cuda")
    y2 = torch.empty(T, d, device="cuda")
    L.moe_expert_q4_gateup(h, idx, slots, E, arena, stride, offsets, sp, None, 0, T, dm, L.MOE_PREC_FP32, act2,
                           ws(2))
    L.moe_expert_q4_down_combine(act2, idx, w, slots, E, arena, stride, offsets, sp, pp, x, T, dm,
                                 L.MOE_PREC_FP32, y2, ws(3))
    assert row_rel_err(_np(y2), ry) < TOL_FP32
