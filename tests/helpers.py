"""Shared test utilities: device buffers for seeded layers, and the comparison
rules (certified top-k, per-row relative error)."""
from __future__ import annotations

import numpy as np

import synth

D, F, E, K = synth.D_MODEL, synth.D_FF, synth.N_EXPERTS, synth.TOP_K

TOL_FP32 = 2e-3   # max |gpu - ref| / max |ref| per output row, fp32-accumulate path
TOL_BF16 = 1e-2   # same, 16-bit-operand MFMA path (fp16 operands)


def row_rel_err(gpu, ref) -> float:
    """max over rows of max_i |gpu_i - ref_i| / max_i |ref_i|."""
    gpu = np.atleast_2d(np.asarray(gpu, dtype=np.float64))
    ref = np.atleast_2d(np.asarray(ref, dtype=np.float64))
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    if not np.all(np.isfinite(gpu)):
        return float("inf")
    num = np.abs(gpu - ref).max(axis=1)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return float((num / den).max())


def check_topk(gpu_idx, oracle_idx, logits64, tau_rel=1e-4):
    """Routing parity.  A rank where GPU and oracle agree must agree exactly;
    a rank where they differ is accepted only as a near-tie: the two experts'
    float64 logits differ by at most tau = tau_rel * max(1, |logit|).  Returns
    the number of accepted near-tie differences."""
    gpu_idx = np.asarray(gpu_idx)
    oracle_idx = np.asarray(oracle_idx)
    n_swaps = 0
    for t in range(gpu_idx.shape[0]):
        g, o, lg = gpu_idx[t], oracle_idx[t], logits64[t]
        assert len(set(g.tolist())) == len(g), f"token {t}: repeated expert {g}"
        assert np.all((g >= 0) & (g < lg.shape[0])), f"token {t}: id out of range {g}"
        for j in range(len(g)):
            if g[j] != o[j]:
                tau = tau_rel * max(1.0, abs(lg[o[j]]))
                assert abs(lg[g[j]] - lg[o[j]]) <= tau, (
                    f"token {t} rank {j}: gpu {g[j]} ({lg[g[j]]}) vs oracle {o[j]} ({lg[o[j]]})")
                n_swaps += 1
        # the chosen set must dominate everything left out, up to tau
        left = np.setdiff1d(np.arange(lg.shape[0]), g)
        if left.size:
            tau = tau_rel * max(1.0, abs(lg[g].min()))
            assert lg[left].max() <= lg[g].min() + tau, f"token {t}: unselected expert beats a selected one"
    return n_swaps


class LayerData:
    """One seeded MoE layer on the host (blobs, router, norm, bias).

    offset_weights=True redraws every group's bias as U(-0.1, 0.1),
    independent of its scale: the weights then carry a mean of about +0.09,
    so sums over near-constant inputs add up coherently (large activations)."""

    def __init__(self, seed: int, layer: int, zipf: bool = True, norm: bool = True, experts=None,
                 offset_weights: bool = False):
        self.seed, self.layer = seed, layer
        self.router_w = synth.router_weight(D, E, seed, layer)
        self.bias = synth.zipf_bias(E, seed, layer) if zipf else None
        self.norm_w = synth.norm_weight(D, seed, layer) if norm else None
        ids = range(E) if experts is None else experts
        self.blobs = dict(zip(ids, synth.expert_blobs(D, F, seed, layer, ids)))
        if offset_weights:
            nib, n_pairs = synth.blob_payload_sizes(D, F)
            for e, b in self.blobs.items():
                pairs = b[nib:].view(np.float16).reshape(n_pairs, 2)
                pairs[:, 1] = synth.rng(seed, 99, layer, e).uniform(-0.1, 0.1, n_pairs).astype(np.float16)

    def blob_of(self, e):
        return self.blobs[e]


# Stored position of column j inside a block of 8 in the MFMA act layout.
ACT_POS = np.array([2 * (j % 4) + j // 4 for j in range(8)])


def decode_scaled_act(buf, rows, cols, dtype):
    """Block-scaled act buffer of the MFMA path (16-bit values [rows][cols] in
    the 0,4,1,5,2,6,3,7 order inside each block of 8, then int8 exponents
    [rows][cols/64]) -> float64 numpy [rows][cols] in natural column order."""
    import torch
    b = buf.detach().cpu()
    nval = rows * cols * 2
    vals = b[:nval].view(dtype).reshape(rows, cols).float().numpy().astype(np.float64)
    vals = vals.reshape(rows, cols // 8, 8)[:, :, ACT_POS].reshape(rows, cols)
    ex = b[nval:nval + rows * (cols // 64)].view(torch.int8).reshape(rows, cols // 64).numpy().astype(np.int64)
    return vals * np.repeat(np.exp2(ex.astype(np.float64)), 64, axis=1)
