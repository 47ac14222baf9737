"""GPU parity at the configured sizes, in the launch configurations the
benchmark times, against the C++ oracle:

* batch-1 decode through all 30 layers of the full shape in one
  moe_decode_layers launch per step, Zipf routing, slots permuted, three
  steps (the last two fed back), every layer checked teacher-forced (the
  oracle takes the GPU's input of that layer);
* the bounded cache at its full shape (30 layers, 64 of 128 slots, 512 Markov
  steps), host and device rule, LRU and LFU: hit masks and slot tables equal
  to the oracle's after every step of every layer, staged blobs byte-exact;
* steps of the device cache recorded as HIP graphs and replayed, against the
  same steps run eagerly on a twin cache;
* all 2048 rows of one prefill layer (fp16 MFMA path), element by element.
"""
import numpy as np
import pytest
import torch

import oracle as orc
import synth
from helpers import D, E, F, K, TOL_BF16, TOL_FP32, LayerData, check_topk, row_rel_err

pytestmark = pytest.mark.gpu

NL = synth.N_LAYERS


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int4_routed_expert_route_amd.api as api
    api.lib()
    return api


# ----------------------------------------------------------------------------- C1: 30-layer decode

class FullStack:
    """All 30 x 128 experts of the full shape resident (12.85 GB), slot order
    permuted per layer; blobs regenerated on the host only for the experts the
    oracle needs."""

    def __init__(self, api, seed):
        self.seed = seed
        self.dm = api.dims(D, F, E, K)
        self.stride = api.moe_expert_blob_bytes(self.dm)
        self.rw = np.stack([synth.router_weight(D, E, seed, l) for l in range(NL)])
        self.nw = np.stack([synth.norm_weight(D, seed, l) for l in range(NL)])
        self.bias = np.stack([synth.zipf_bias(E, seed, l) for l in range(NL)])
        self.arena = torch.empty(NL * E * self.stride, dtype=torch.uint8, device="cuda")
        tables = np.zeros((NL, E), dtype=np.int32)
        for l in range(NL):
            perm = synth.slot_permutation(E, seed, l)  # slot s holds expert perm[s]
            blobs = synth.expert_blobs(D, F, seed, l, perm.tolist(), threads=16)
            self.arena[l * E * self.stride:(l + 1) * E * self.stride].copy_(torch.from_numpy(np.concatenate(blobs)))
            tables[l, perm] = np.arange(E, dtype=np.int32)
        self.tables = torch.from_numpy(tables).cuda()
        self.rw_d = torch.from_numpy(self.rw).cuda()
        self.nw_d = torch.from_numpy(self.nw).cuda()
        self.bias_d = torch.from_numpy(self.bias).cuda()
        self.ws = torch.zeros(api.moe_workspace_size(api.MOE_CALL_DECODE_LAYERS, NL, self.dm), dtype=torch.uint8,
                              device="cuda")
        torch.cuda.synchronize()

    def blob(self, l, e):
        return synth.expert_blob(D, F, self.seed, l, e)


def test_decode_30_layers_full_shape_teacher_forced(api):
    st = FullStack(api, seed=21)
    x = synth.tokens(1, D, 21)[0]
    swaps = 0
    for step in range(3):
        print(f"30-layer decode: step {step}", flush=True)
        x_io = torch.zeros(NL + 1, D, device="cuda")
        x_io[0].copy_(torch.from_numpy(x))
        idx = torch.zeros(NL, K, dtype=torch.int32, device="cuda")
        w = torch.zeros(NL, K, device="cuda")
        x_next = torch.zeros(D, device="cuda")
        api.moe_decode_layers(x_io, NL, st.nw_d, 1e-6, st.rw_d, st.bias_d, st.tables, E, st.arena, E * st.stride,
                              st.stride, st.dm, idx, w, x_next, st.ws)
        api.moe_decode_check(st.ws)
        xs, gi, gw = x_io.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()
        assert np.all(np.isfinite(xs))
        for l in range(NL):
            _, lg, ridx, _ = orc.route(xs[l][None, :], st.nw[l], st.rw[l], st.bias[l], K)
            swaps += check_topk(gi[l][None, :], ridx, lg)
            ry, _, rw_, _, _ = orc.moe_layer(xs[l][None, :], st.nw[l], st.rw[l], st.bias[l],
                                             lambda e, l=l: st.blob(l, e), D, F, K, idx_override=gi[l][None, :])
            assert np.allclose(gw[l], rw_[0], rtol=1e-5, atol=1e-6), (step, l)
            err = row_rel_err(xs[l + 1] - xs[l], ry[0] - xs[l])
            assert err < TOL_FP32, (step, l, err)
        want_next = orc.rms_rescale(xs[NL][None, :], 1e-6)[0]
        assert row_rel_err(x_next.cpu().numpy(), want_next) < 1e-5
        x = x_next.cpu().numpy()
    print(f"30-layer decode: {3 * NL * K} routing decisions, {swaps} accepted near-tie swaps", flush=True)


# ----------------------------------------------------------------------------- C4: the cache at full shape

class CachePool:
    """Pinned pool of NL x E blobs, device arena of S slots per layer."""

    def __init__(self, api, d, f, S, seed, fill=True):
        self.d, self.f, self.S = d, f, S
        self.dm = api.dims(d, f, E, K)
        self.blob = orc.blob_bytes(d, f)
        self.stride = api.moe_expert_blob_bytes(self.dm)
        self.seed = seed
        self.pool = torch.empty(NL * E * self.blob, dtype=torch.uint8, pin_memory=True)
        for l in range(NL):
            blobs = synth.expert_blobs(d, f, seed, l, range(E), threads=16)
            self.pool[l * E * self.blob:(l + 1) * E * self.blob].copy_(torch.from_numpy(np.concatenate(blobs)))
        self.arena = torch.full((NL * S * self.stride,), 0xA5, dtype=torch.uint8, device="cuda")
        self.tables = torch.zeros(NL, E, dtype=torch.int32, device="cuda")
        self.cache = api.MoeCache(NL, E, S, K, self.pool, self.blob, self.arena, self.stride, self.tables)

    def slot_dev(self, l, s):
        off = (l * self.S + s) * self.stride
        return self.arena[off:off + self.blob]

    def pool_blob(self, l, e):
        off = (l * E + e) * self.blob
        return self.pool[off:off + self.blob]

    def check_resident(self, ref):
        """Every resident slot holds its expert's blob (compared on the device)."""
        for l in range(NL):
            for s, e in enumerate(ref[l].slot_expert):
                if e >= 0:
                    assert torch.equal(self.slot_dev(l, s), self.pool_blob(l, e).cuda(non_blocking=True)), (l, s, e)


def _ref(policy):
    return [orc.LruSlotCache(64, E) if policy == "lru" else orc.LfuSlotCache(64, E) for _ in range(NL)]


@pytest.mark.parametrize("mode", ["host", "device"])
@pytest.mark.parametrize("policy", ["lru", "lfu"])
def test_cache_full_shape_follows_oracle(api, mode, policy):
    """64 of 128 slots, 30 layers, 512 Markov(0.8) steps.  Blobs of the small
    shape (d=128, f=64) keep the pool small; the rule does not depend on the
    blob size (the next test stages full-size blobs)."""
    steps, S = 512, 64
    pc = CachePool(api, 128, 64, S, seed=5)
    api.moe_cache_set_policy(pc.cache, 0 if policy == "lru" else 1, 0)
    if mode == "device":
        api.moe_cache_enable_device(pc.cache)
    side, compute = torch.cuda.Stream(), torch.cuda.current_stream()
    ref = _ref(policy)
    sels = [synth.markov_selections(E, K, steps, 5, l) for l in range(NL)]
    hit_dev = torch.zeros(NL, 16, dtype=torch.uint8, device="cuda")
    hits = misses = 0
    for t in range(steps):
        if t % 128 == 0:
            print(f"cache {mode}/{policy}: step {t}", flush=True)
        want = []
        for l in range(NL):
            sel = np.random.default_rng(t * 31 + l).permutation(sels[l][t]).astype(np.int32)
            if mode == "device":
                api.moe_slot_stage_device(pc.cache, l, t, torch.from_numpy(sel).cuda(), side, compute,
                                          hit_dev[l, :K])
            else:
                api.moe_slot_stage(pc.cache, l, t, torch.from_numpy(sel), side, compute, hit_dev[l, :K])
            api.moe_cache_wait(pc.cache, l, compute)
            h, installs = ref[l].step(t, sel.tolist())
            hits += sum(h)
            misses += len(installs)
            want.append((h, installs))
        torch.cuda.synchronize()
        got_hits = hit_dev[:, :K].cpu().numpy().astype(bool)
        got_tables = pc.tables.cpu().numpy()
        for l in range(NL):
            assert got_hits[l].tolist() == want[l][0], (t, l)
            assert np.array_equal(got_tables[l], np.array(ref[l].slot_of_expert(), np.int32)), (t, l)
            for e, s, _ in want[l][1]:
                assert torch.equal(pc.slot_dev(l, s), pc.pool_blob(l, e).cuda()), (t, l, e, s)
    st = api.moe_cache_stats(pc.cache)
    assert (st.hits, st.misses, st.bytes_staged) == (hits, misses, misses * pc.blob)
    se = torch.zeros(NL, S, dtype=torch.int32)
    stp = torch.zeros(NL, S, dtype=torch.int64)
    api.moe_cache_export(pc.cache, se, stp)
    for l in range(NL):
        assert se[l].tolist() == ref[l].slot_expert and stp[l].tolist() == ref[l].stamp, l
    if policy == "lfu":
        counts = torch.zeros(NL, E, dtype=torch.int64)
        api.moe_cache_export_usage(pc.cache, counts, None)
        for l in range(NL):
            assert counts[l].tolist() == ref[l].counts(), l
    print(f"cache {mode}/{policy}: hit rate {hits / (hits + misses):.4f}, {misses} misses", flush=True)
    pc.cache.close()


def test_cache_full_shape_full_blobs_device(api):
    """The same at the real blob size (3,345,408 B, a 12.85 GB pinned pool and
    a 6.42 GB arena), device rule, LRU: tables every step, every resident
    slot's bytes at the end."""
    steps, S = 512, 64
    pc = CachePool(api, D, F, S, seed=6)
    api.moe_cache_enable_device(pc.cache)
    side, compute = torch.cuda.Stream(), torch.cuda.current_stream()
    ref = _ref("lru")
    sels = [synth.markov_selections(E, K, steps, 6, l) for l in range(NL)]
    hit_dev = torch.zeros(NL, 16, dtype=torch.uint8, device="cuda")
    for t in range(steps):
        if t % 128 == 0:
            print(f"cache full blobs: step {t}", flush=True)
        want = []
        for l in range(NL):
            sel = sels[l][t][::-1].copy()
            api.moe_slot_stage_device(pc.cache, l, t, torch.from_numpy(sel).cuda(), side, compute, hit_dev[l, :K])
            api.moe_cache_wait(pc.cache, l, compute)
            want.append(ref[l].step(t, sel.tolist())[0])
        torch.cuda.synchronize()
        got_hits = hit_dev[:, :K].cpu().numpy().astype(bool)
        got_tables = pc.tables.cpu().numpy()
        for l in range(NL):
            assert got_hits[l].tolist() == want[l], (t, l)
            assert np.array_equal(got_tables[l], np.array(ref[l].slot_of_expert(), np.int32)), (t, l)
    pc.check_resident(ref)
    st = api.moe_cache_stats(pc.cache)
    assert st.bytes_staged == st.misses * 3_345_408
    pc.cache.close()


def test_device_cache_steps_as_graphs(api):
    """Steps of the device cache recorded as HIP graphs (one per step, as the
    benchmark records them) and replayed, one of them twice, with eager work
    and synchronisations between replays; a twin cache runs the same steps
    eagerly.  Hit masks, device tables and statistics agree after every
    replay."""
    steps, warm, S, nl = 24, 8, 64, 2
    twins = []
    for _ in range(2):
        pc = CachePool(api, 128, 64, S, seed=7)
        api.moe_cache_enable_device(pc.cache)
        twins.append(pc)
    a, b = twins
    side_a, side_b = torch.cuda.Stream(), torch.cuda.Stream()
    sels = [synth.markov_selections(E, K, steps, 7, l) for l in range(nl)]
    sel_dev = torch.from_numpy(np.stack([np.stack([sels[l][t] for l in range(nl)]) for t in range(steps)])).cuda()
    hit_a = torch.zeros(nl, 16, dtype=torch.uint8, device="cuda")
    hit_b = torch.zeros(nl, 16, dtype=torch.uint8, device="cuda")

    def step(pc, side, hit, t):
        compute = torch.cuda.current_stream()
        for l in range(nl):
            api.moe_slot_stage_device(pc.cache, l, t, sel_dev[t, l], side, compute, hit[l, :K])
            api.moe_cache_wait(pc.cache, l, compute)

    for t in range(warm):
        step(a, side_a, hit_a, t)
        step(b, side_b, hit_b, t)
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    graphs = {}
    for t in range(warm, steps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            step(b, side_b, hit_b, t)
        graphs[t] = g
    torch.cuda.synchronize()
    order = list(range(warm, steps))
    order.insert(3, order[2])  # one step replayed a second time: all hits
    for t in order:
        step(a, side_a, hit_a, t)
        graphs[t].replay()
        junk = torch.randn(1 << 16, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(hit_a[:, :K], hit_b[:, :K]), t
        assert torch.equal(a.tables, b.tables), t
    sa, sb = api.moe_cache_stats(a.cache), api.moe_cache_stats(b.cache)
    assert (sa.hits, sa.misses, sa.bytes_staged) == (sb.hits, sb.misses, sb.bytes_staged)
    ref = [orc.LruSlotCache(S, E) for _ in range(nl)]
    for t in list(range(warm)) + order:
        for l in range(nl):
            ref[l].step(t, sels[l][t].tolist())
    for l in range(nl):
        assert np.array_equal(b.tables[l].cpu().numpy(), np.array(ref[l].slot_of_expert(), np.int32)), l
    for pc in twins:
        pc.cache.close()


# ----------------------------------------------------------------------------- C3: a whole prefill layer

def test_prefill_layer_all_rows(api):
    """Every one of the 2048 tokens of one prefill layer (Zipf routing, fp16
    MFMA path, the benchmark's launch configuration), element by element
    against the oracle at 1e-2 per row, and the act of every pair."""
    from test_gpu_prefill import run_prefill
    T = 2048
    layer = LayerData(seed=0, layer=1)
    arena = torch.from_numpy(np.concatenate([layer.blobs[e] for e in range(E)])).cuda()
    x_np = synth.tokens(T, D, seed=0, stream=98)
    out = run_prefill(api, x_np, layer, arena, D, F, E, K, prec="f16")
    gi = out["idx"].cpu().numpy()
    counts = out["counts"].cpu().numpy()
    assert counts.sum() == T * K and counts.max() > 500
    _, lg, ridx, _ = orc.route(x_np, layer.norm_w, layer.router_w, layer.bias, K)
    swaps = check_topk(gi, ridx, lg)
    print(f"prefill layer: {T * K} routing decisions, {swaps} accepted near-tie swaps", flush=True)
    ry, _, _, rh, _ = orc.moe_layer(x_np, layer.norm_w, layer.router_w, layer.bias, layer.blob_of, D, F, K,
                                    idx_override=gi)
    y = out["y"].cpu().numpy()
    assert np.all(np.isfinite(y))
    e_y = row_rel_err(y - x_np, ry - x_np)
    print(f"prefill layer: max row rel err of the MoE output over all {T} rows {e_y:.3e}", flush=True)
    assert e_y < TOL_BF16
    assert row_rel_err(y, ry) < TOL_BF16
    # act of every pair, grouped by expert.  act is an intermediate held as
    # fp16 with one power-of-two exponent per (expert tile, 64-column group),
    # so its rounding is relative to the expert's largest value there, not to
    # each row's own: the error is measured against the expert's maximum.
    worst = 0.0
    for e in np.unique(gi):
        rows = np.argwhere(gi == e)
        ract = orc.expert_gateup(layer.blobs[int(e)], rh[rows[:, 0]], D, F).astype(np.float64)
        got = out["act"][rows[:, 0] * K + rows[:, 1]]
        err = float(np.abs(got - ract).max() / np.abs(ract).max())
        worst = max(worst, err)
        assert err < TOL_BF16, (e, err)
    print(f"prefill layer: act error relative to each expert's maximum, worst {worst:.3e}", flush=True)
