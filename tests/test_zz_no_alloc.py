"""moe_route_noalloc (static per-device scratch, nothing allocated) against
moe_route with a caller workspace, through the C ABI: the same bits on every
output, over calls in a row that switch between the fused small path and the
split router path, the later ones smaller than the earlier."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

D, F, E, K = synth.D_MODEL, synth.D_FF, synth.N_EXPERTS, synth.TOP_K


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int4_routed_expert_route_amd.api as api
    api.lib()
    return api


@pytest.fixture(scope="module")
def layer():
    return dict(router_w=torch.from_numpy(synth.router_weight(D, E, 0, 4)).cuda(),
                bias=torch.from_numpy(synth.zipf_bias(E, 0, 4)).cuda(),
                norm_w=torch.from_numpy(synth.norm_weight(D, 0, 4)).cuda())


def _outs(T):
    return (torch.empty(T, D, device="cuda"), torch.full((T, K), -1, dtype=torch.int32, device="cuda"),
            torch.full((T, K), -1.0, device="cuda"))


@pytest.mark.parametrize("sizes", [(300, 5), (2048, 40, 1), (8, 3)])
def test_route_noalloc_matches_route(api, layer, sizes):
    dm = api.dims(D, F, E, K)
    for n, T in enumerate(sizes):
        print(f"no-alloc route: call {n} T={T}", flush=True)
        x = torch.from_numpy(synth.tokens(T, D, seed=7, stream=T)).cuda()
        for norm, bias in ((True, True), (False, False)):
            ref = _outs(T)
            ws = torch.zeros(api.moe_workspace_size(api.MOE_CALL_ROUTE, T, dm), dtype=torch.uint8, device="cuda")
            api.moe_route(x, layer["norm_w"] if norm else None, 1e-6, layer["router_w"],
                          layer["bias"] if bias else None, T, dm, *ref, ws)
            got = _outs(T)
            api.moe_route_noalloc(x, layer["norm_w"] if norm else None, 1e-6, layer["router_w"],
                                  layer["bias"] if bias else None, T, dm, *got)
            torch.cuda.synchronize()
            for r, g, name in zip(ref, got, ("h", "topk_idx", "topk_w")):
                a, b = r.cpu().numpy(), g.cpu().numpy()
                assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                      b.view(np.uint32) if b.dtype == np.float32 else b), (T, norm, name)
            assert (got[1].cpu().numpy() >= 0).all()
