"""GPU parity of moe_decode_layers (batch-1 decode through many layers in one
launch) against the CPU oracle, layer by layer (each layer's oracle input is
the GPU's output of the previous layer), and against the per-call path."""
import numpy as np
import pytest
import torch

import oracle as orc
import synth
from helpers import TOL_FP32, check_topk, row_rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int4_routed_expert_route_amd.api as api
    api.lib()
    return api


class Stack:
    """n_layers seeded layers on the device, slots per layer permuted."""

    def __init__(self, api, d, f, E, k, n_layers, seed, norm=True, bias=True, permute=True):
        self.d, self.f, self.E, self.k, self.L = d, f, E, k, n_layers
        self.dm = api.dims(d, f, E, k)
        self.stride = api.moe_expert_blob_bytes(self.dm)
        self.blobs = [[synth.expert_blob(d, f, seed, l, e) for e in range(E)] for l in range(n_layers)]
        self.rw = np.stack([synth.router_weight(d, E, seed, l) for l in range(n_layers)])
        self.nw = np.stack([synth.norm_weight(d, seed, l) for l in range(n_layers)]) if norm else None
        self.bias = np.stack([synth.zipf_bias(E, seed, l) for l in range(n_layers)]) if bias else None
        # slot s of layer l holds expert perm[l][s]
        perms = [synth.slot_permutation(E, seed, l) if permute else np.arange(E, dtype=np.int32)
                 for l in range(n_layers)]
        host = np.concatenate([np.concatenate([self.blobs[l][e] for e in perms[l]]) for l in range(n_layers)])
        self.arena = torch.from_numpy(host).cuda()
        tables = np.zeros((n_layers, E), dtype=np.int32)
        for l in range(n_layers):
            tables[l, perms[l]] = np.arange(E, dtype=np.int32)
        self.tables = torch.from_numpy(tables).cuda()
        self.rw_d = torch.from_numpy(self.rw).cuda()
        self.nw_d = None if self.nw is None else torch.from_numpy(self.nw).cuda()
        self.bias_d = None if self.bias is None else torch.from_numpy(self.bias).cuda()
        self.ws = torch.zeros(api.moe_workspace_size(api.MOE_CALL_DECODE_LAYERS, n_layers, self.dm), dtype=torch.uint8,
                              device="cuda")

    def run(self, api, x0, x_next=None):
        x_io = torch.zeros(self.L + 1, self.d, device="cuda")
        x_io[0].copy_(torch.from_numpy(np.asarray(x0, dtype=np.float32).reshape(-1)))
        idx = torch.zeros(self.L, self.k, dtype=torch.int32, device="cuda")
        w = torch.zeros(self.L, self.k, device="cuda")
        api.moe_decode_layers(x_io, self.L, self.nw_d, 1e-6, self.rw_d, self.bias_d, self.tables, self.E, self.arena,
                              self.E * self.stride, self.stride, self.dm, idx, w, x_next, self.ws)
        api.moe_decode_check(self.ws)
        return x_io.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()

    def oracle_layer(self, l, x, idx_override):
        nw = None if self.nw is None else self.nw[l]
        bias = None if self.bias is None else self.bias[l]
        return orc.moe_layer(x[None, :], nw, self.rw[l], bias, lambda e: self.blobs[l][e], self.d, self.f, self.k,
                             idx_override=idx_override[None, :])


def _check_layers(st, x_io, idx, w, tol=TOL_FP32):
    for l in range(st.L):
        xin = x_io[l].astype(np.float64)
        nw = None if st.nw is None else st.nw[l]
        bias = None if st.bias is None else st.bias[l]
        _, lg, ridx, rw_ = orc.route(xin[None, :], nw, st.rw[l], bias, st.k)
        check_topk(idx[l][None, :], ridx, lg)
        ry, _, rw2, _, _ = st.oracle_layer(l, xin, idx[l])
        assert np.allclose(w[l], rw2[0], rtol=1e-5, atol=1e-6), (l, w[l], rw2[0])
        err = row_rel_err(x_io[l + 1] - x_io[l], ry[0] - xin)
        assert err < tol, (l, err)


@pytest.mark.parametrize("d,f,E,k,L", [(256, 128, 16, 4, 3), (640, 192, 32, 8, 3), (2816, 704, 128, 8, 3)])
def test_decode_layers_parity(api, d, f, E, k, L):
    st = Stack(api, d, f, E, k, L, seed=11)
    x0 = synth.tokens(1, d, 11)[0]
    x_io, idx, w = st.run(api, x0)
    assert np.all(np.isfinite(x_io))
    _check_layers(st, x_io, idx, w)


def test_decode_layers_ragged_shape(api):
    """E not a multiple of 4 or 32 (padded partial rows and rank keys), odd k, and
    rows that do not divide over the workgroups (a short last block and
    workgroups with no down rows)."""
    d, f, E, k, L = 128, 128, 20, 3, 3
    st = Stack(api, d, f, E, k, L, seed=17)
    x_io, idx, w = st.run(api, synth.tokens(1, d, 17)[0])
    assert np.all(np.isfinite(x_io))
    _check_layers(st, x_io, idx, w)


def test_decode_layers_absent_slot_gives_nan(api):
    """A chosen expert whose slot table entry is -1 is never read: that layer's
    output is NaN (which the next layer's waits still see as written), and the
    launch completes without a wait error."""
    d, f, E, k, L = 256, 128, 16, 4, 2
    st = Stack(api, d, f, E, k, L, seed=18)
    x0 = synth.tokens(1, d, 18)[0]
    _, idx, _ = st.run(api, x0)
    tables = st.tables.cpu().numpy()
    tables[0, idx[0][0]] = -1  # layer 0's first choice becomes absent
    st.tables = torch.from_numpy(tables).cuda()
    x_io, idx2, _ = st.run(api, x0)
    assert np.array_equal(idx2[0], idx[0])
    assert np.all(np.isnan(x_io[1]))


def test_decode_layers_without_norm_or_bias(api):
    st = Stack(api, 256, 128, 16, 4, 2, seed=12, norm=False, bias=False, permute=False)
    x_io, idx, w = st.run(api, synth.tokens(1, 256, 12)[0])
    _check_layers(st, x_io, idx, w)


def test_decode_layers_matches_per_call_path(api):
    """Same layers through moe_route + moe_expert_q4_gateup + moe_expert_q4_down_combine."""
    d, f, E, k, L = 2816, 704, 128, 8, 2
    st = Stack(api, d, f, E, k, L, seed=13)
    x0 = synth.tokens(1, d, 13)[0]
    x_io, idx, w = st.run(api, x0)
    dm = st.dm
    ws = lambda c: torch.zeros(max(api.moe_workspace_size(c, 1, dm), 256), dtype=torch.uint8, device="cuda")
    x = torch.from_numpy(x0[None, :]).cuda()
    for l in range(L):
        h = torch.empty(1, d, device="cuda")
        i2 = torch.empty(1, k, dtype=torch.int32, device="cuda")
        w2 = torch.empty(1, k, device="cuda")
        api.moe_route(x, st.nw_d[l], 1e-6, st.rw_d[l], st.bias_d[l], 1, dm, h, i2, w2, ws(0))
        arena_l = st.arena[l * E * st.stride:(l + 1) * E * st.stride]
        act = torch.empty(k, f, device="cuda")
        api.moe_expert_q4_gateup(h, i2, st.tables[l], E, arena_l, st.stride, None, None, None, 0, 1, dm,
                                 api.MOE_PREC_FP32, act, ws(2))
        y = torch.empty(1, d, device="cuda")
        api.moe_expert_q4_down_combine(act, i2, w2, st.tables[l], E, arena_l, st.stride, None, None, None, x, 1, dm,
                                       api.MOE_PREC_FP32, y, ws(3))
        torch.cuda.synchronize()
        assert np.array_equal(np.sort(i2.cpu().numpy()[0]), np.sort(idx[l]))
        assert row_rel_err(y.cpu().numpy()[0] - x_io[l], x_io[l + 1] - x_io[l]) < TOL_FP32
        x = torch.from_numpy(x_io[l + 1][None, :].copy()).cuda()  # continue from the fused path's output


def test_decode_layers_repeat_and_feedback(api):
    """Several launches on one workspace (its two region sets alternate, each
    launch clearing the set the previous one used): a fixed input gives
    identical outputs every time, and x_next is the unit-RMS rescale of the
    last layer's output."""
    d, f, E, k, L = 640, 192, 32, 8, 3
    st = Stack(api, d, f, E, k, L, seed=14)
    x0 = synth.tokens(1, d, 14)[0]
    nxt = torch.zeros(d, device="cuda")
    first = None
    for _ in range(4):
        x_io, idx, w = st.run(api, x0, x_next=nxt)
        if first is None:
            # the first launch on a fresh workspace against the oracle too
            _check_layers(st, x_io, idx, w)
            first = (x_io, idx, w)
        else:
            assert np.array_equal(first[0], x_io) and np.array_equal(first[1], idx) and np.array_equal(first[2], w)
    want = orc.rms_rescale(x_io[L].astype(np.float64), 1e-6)
    assert row_rel_err(nxt.cpu().numpy(), want) < 1e-5


def test_decode_layers_steps_feed_back_in_place(api):
    """Decode steps with x_next = x_io[0] (in place), against the oracle
    teacher-forced per layer."""
    d, f, E, k, L = 256, 128, 16, 4, 3
    st = Stack(api, d, f, E, k, L, seed=15)
    x_io = torch.zeros(L + 1, d, device="cuda")
    x_io[0].copy_(torch.from_numpy(synth.tokens(1, d, 15)[0]))
    idx = torch.zeros(L, k, dtype=torch.int32, device="cuda")
    w = torch.zeros(L, k, device="cuda")
    for step in range(5):
        before = x_io.cpu().numpy()
        api.moe_decode_layers(x_io, L, st.nw_d, 1e-6, st.rw_d, st.bias_d, st.tables, E, st.arena, E * st.stride,
                              st.stride, st.dm, idx, w, x_io[0], st.ws)
        api.moe_decode_check(st.ws)
        after = x_io.cpu().numpy()
        io = np.concatenate([before[:1], after[1:]])
        _check_layers(st, io, idx.cpu().numpy(), w.cpu().numpy())
        want = orc.rms_rescale(after[L].astype(np.float64), 1e-6)
        assert row_rel_err(after[0], want) < 1e-5, step


def test_decode_layers_rejects_bad_arguments(api):
    st = Stack(api, 256, 128, 16, 4, 1, seed=16)
    x_io = torch.zeros(2, 256, device="cuda")
    idx = torch.zeros(1, 4, dtype=torch.int32, device="cuda")
    w = torch.zeros(1, 4, device="cuda")
    with pytest.raises(api.MoeError):  # workspace too small
        api.moe_decode_layers(x_io, 1, st.nw_d, 1e-6, st.rw_d, st.bias_d, st.tables, 16, st.arena, 16 * st.stride,
                              st.stride, st.dm, idx, w, None, st.ws[:64])
    with pytest.raises(api.MoeError):  # layer stride below n_slots * slot_stride
        api.moe_decode_layers(x_io, 1, st.nw_d, 1e-6, st.rw_d, st.bias_d, st.tables, 16, st.arena, st.stride,
                              st.stride, st.dm, idx, w, None, st.ws)


def test_decode_layers_workspace_bound_to_its_shapes(api):
    """A workspace that served one shape is refused for another (its regions
    are laid out for the first): the launch writes nothing and
    moe_decode_check reports it; zero-filled again it serves the new shape."""
    a = Stack(api, 256, 128, 16, 4, 2, seed=19)
    b = Stack(api, 256, 128, 16, 4, 3, seed=20)
    x0 = synth.tokens(1, 256, 19)[0]
    a.run(api, x0)
    b.ws[:512].copy_(a.ws[:512])  # the header: launch count and the 2-layer shape's signature
    with pytest.raises(api.MoeError):
        b.run(api, x0)
    b.ws.zero_()
    x_io, idx, w = b.run(api, x0)
    _check_layers(b, x_io, idx, w)


def test_decode_layers_two_workspaces_interleaved(api):
    """Two stacks, each with its own workspace, launched alternately on one
    stream: each keeps giving the result of its first launch."""
    a = Stack(api, 256, 128, 16, 4, 2, seed=21)
    b = Stack(api, 256, 128, 24, 4, 3, seed=22)
    xa, xb = synth.tokens(1, 256, 21)[0], synth.tokens(1, 256, 22)[0]
    ra, rb = a.run(api, xa), b.run(api, xb)
    _check_layers(a, *ra)
    _check_layers(b, *rb)
    for _ in range(3):
        for st, x, ref in ((a, xa, ra), (b, xb, rb)):
            got = st.run(api, x)
            assert all(np.array_equal(u, v) for u, v in zip(got, ref))
