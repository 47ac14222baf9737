"""Paths captured as HIP graphs and replayed, as the benchmark runs them.

Every replay is checked bit for bit against the eager result of the same
calls, with eager launches on the same workspace between the replays: the
fused decode alternates its region sets by a launch count kept in the
workspace, and split-K GEMM items leave their arrival counters at zero, so a
replay must not depend on how many launches came before it.  Nothing here
clears memory inside a graph."""
import numpy as np
import pytest
import torch

import oracle as orc
import synth
from helpers import TOL_BF16, row_rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int4_routed_expert_route_amd.api as api
    api.lib()
    return api


def _capture(fn):
    """fn() once eagerly on a side stream, then captured; returns the graph."""
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        fn()
    torch.cuda.synchronize()
    return graph


def _host(ts):
    torch.cuda.synchronize()
    return [t.cpu().numpy().copy() for t in ts]


def test_fused_decode_graph_replays(api):
    d, f, E, k, L = 2816, 704, 128, 8, 3
    dm = api.dims(d, f, E, k)
    stride = api.moe_expert_blob_bytes(dm)
    blobs = np.concatenate([synth.expert_blob(d, f, 21, l, e) for l in range(L) for e in range(E)])
    arena = torch.from_numpy(blobs).cuda()
    tables = torch.arange(E, dtype=torch.int32, device="cuda").repeat(L, 1).contiguous()
    rw = torch.from_numpy(np.stack([synth.router_weight(d, E, 21, l) for l in range(L)])).cuda()
    nw = torch.from_numpy(np.stack([synth.norm_weight(d, 21, l) for l in range(L)])).cuda()
    bias = torch.from_numpy(np.stack([synth.zipf_bias(E, 21, l) for l in range(L)])).cuda()
    ws = torch.zeros(api.moe_workspace_size(api.MOE_CALL_DECODE_LAYERS, L, dm), dtype=torch.uint8, device="cuda")
    x_io = torch.zeros(L + 1, d, device="cuda")
    x_io[0].copy_(torch.from_numpy(synth.tokens(1, d, 21).reshape(-1)))
    idx = torch.zeros(L, k, dtype=torch.int32, device="cuda")
    w = torch.zeros(L, k, device="cuda")

    def launch():
        api.moe_decode_layers(x_io, L, nw, 1e-6, rw, bias, tables, E, arena, E * stride, stride, dm, idx, w, None,
                              ws)

    def clear_outputs():
        x_io[1:].zero_()
        idx.zero_()
        w.zero_()

    launch()
    want = _host([x_io, idx, w])
    api.moe_decode_check(ws)
    graph = _capture(launch)
    for r in range(3):
        clear_outputs()
        graph.replay()
        got = _host([x_io, idx, w])
        for a, b in zip(got, want):
            assert np.array_equal(a, b), f"replay {r}"
        clear_outputs()
        launch()  # eager, between replays: moves the workspace's launch count on
        got = _host([x_io, idx, w])
        for a, b in zip(got, want):
            assert np.array_equal(a, b), f"eager after replay {r}"
    api.moe_decode_check(ws)


@pytest.mark.parametrize("T", [1, 32, 200])
def test_split_k_grouped_gemm_graph_replays(api, T):
    """The grouped GEMMs captured as gate/up + down-combine: a single token
    and the 32-token batched-decode shape (the few-pairs kernel, K parts
    summed through LDS), and 200 tokens (the work-list GEMM, whose items of
    few pairs are split along K and summed through memory)."""
    d, f, E, k = 2816, 704, 128, 8
    dm = api.dims(d, f, E, k)
    stride = api.moe_expert_blob_bytes(dm)
    blobs = [synth.expert_blob(d, f, 22, 0, e) for e in range(E)]
    arena = torch.from_numpy(np.concatenate(blobs)).cuda()
    slots = torch.arange(E, dtype=torch.int32, device="cuda")
    rw = synth.router_weight(d, E, 22, 0)
    nw = synth.norm_weight(d, 22, 0)
    bias = synth.zipf_bias(E, 22, 0)
    x_np = synth.tokens(T, d, 22, stream=T)
    x = torch.from_numpy(x_np).cuda()
    h = torch.empty(T, d, device="cuda")
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, device="cuda")
    pc = api.MOE_PREC_F16_MFMA
    ws = lambda c, p=0: torch.zeros(max(api.moe_workspace_size(c, T, dm, p), 256), dtype=torch.uint8, device="cuda")
    api.moe_route(x, torch.from_numpy(nw).cuda(), 1e-6, torch.from_numpy(rw).cuda(), torch.from_numpy(bias).cuda(),
                  T, dm, h, idx, w, ws(0))
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    sp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    pp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    api.moe_permute(idx, T, dm, counts, offsets, sp, pp)
    act = torch.zeros(api.moe_act_bytes(T, dm, pc), dtype=torch.uint8, device="cuda")
    y = torch.empty(T, d, device="cuda")
    wsg, wsd = ws(2, pc), ws(3, pc)

    def launch():
        api.moe_expert_q4_gateup(h, idx, slots, E, arena, stride, offsets, sp, None, 0, T, dm, pc, act, wsg)
        api.moe_expert_q4_down_combine(act, idx, w, slots, E, arena, stride, offsets, sp, pp, x, T, dm, pc, y, wsd)

    launch()
    want = _host([act, y])
    ry, *_ = orc.moe_layer(x_np, nw, rw, bias, lambda e: blobs[e], d, f, k, idx_override=_host([idx])[0])
    assert row_rel_err(want[1] - x_np, ry - x_np) < TOL_BF16
    graph = _capture(launch)
    for r in range(3):
        act.zero_()
        y.zero_()
        graph.replay()
        got = _host([act, y])
        assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1]), f"replay {r}"
        y.zero_()
        launch()
        got = _host([act, y])
        assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1]), f"eager after replay {r}"
    counters = _host([wsg[:2048], wsd[:2048]])
    assert not counters[0].any() and not counters[1].any()
