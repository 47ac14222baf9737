"""Seeded synthetic inputs for the routed int4 mixture-of-experts layer.

This module is shared by the tests, the benchmark and the oracle checks.  It
draws random numbers and nothing else: it holds none of the layer's arithmetic
(no dequantisation, no matvec, no routing).  Every tensor comes from its own
counter-keyed stream ``(seed, tag, layer, index)`` so that any single expert
blob, router or token batch can be regenerated on its own, on any machine,
without materialising the whole 12.9 GB pool.

Shapes follow the model the pages describe: 30 MoE layers of 128 experts, 8
selected per token, int4 weights in affine groups of 64 along the input
dimension with a 16-bit scale and bias per group (TurboFieldfare video
transcript, paragraphs on the 128 experts and on the two weight piles;
"Optimizing a 14.3 GB model for an 8 GB machine", section "Vectorization
helped when it respected the storage layout").  The value distributions are
the synthetic recipe of this library (nibbles uniform 0..15, scale
s ~ U(0.005, 0.02), bias -s * (7.5 + U(-1, 1)), router N(0, 0.02^2), norm
weight N(1, 0.1^2), tokens N(0, 1), Zipf(1.1) expert popularity).

The bias is the group's minimum, as an affine quantiser stores it, so that
the dequantised weights s * q + b are centred near zero with a small offset
per group, like those of a trained model.  (A bias drawn independently of
the scale leaves every weight with a mean of about +0.09; every expert's
output then points along one common direction, and after a single MoE layer
all tokens are nearly parallel and select the same experts.)
"""
from __future__ import annotations

import numpy as np
from concurrent.futures import ThreadPoolExecutor

# stream tags
_BLOB, _ROUTER, _ZIPF, _NORM, _TOKENS, _MARKOV, _SHARED, _PERM = 1, 2, 3, 4, 5, 6, 7, 8

D_MODEL = 2816
D_FF = 704
N_EXPERTS = 128
TOP_K = 8
N_LAYERS = 30
GROUP = 64


def rng(*key: int) -> np.random.Generator:
    """Independent PCG64 stream for an integer key tuple."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def blob_payload_sizes(d: int, f: int) -> tuple[int, int]:
    """(nibble bytes, number of (scale, bias) pairs) of one expert.

    The expert blob stores all packed nibbles of its three matrices first and
    all (scale, bias) fp16 pairs after them; since every nibble and every
    pair is drawn independently, the generator needs only these two counts.
    """
    n_weights = 3 * d * f
    return n_weights // 2, n_weights // GROUP


def expert_blob(d: int, f: int, seed: int, layer: int, expert: int) -> np.ndarray:
    """One expert blob (uint8): uniform nibbles, then fp16 (scale, bias) pairs
    with the bias at the group's minimum (weights centred near zero)."""
    nib_bytes, n_pairs = blob_payload_sizes(d, f)
    g = rng(seed, _BLOB, layer, expert)
    out = np.empty(nib_bytes + 4 * n_pairs, dtype=np.uint8)
    out[:nib_bytes] = np.frombuffer(g.bytes(nib_bytes), dtype=np.uint8)
    sb = np.empty((n_pairs, 2), dtype=np.float16)
    scale = g.uniform(0.005, 0.02, n_pairs)
    sb[:, 0] = scale.astype(np.float16)
    sb[:, 1] = (-scale * (7.5 + g.uniform(-1.0, 1.0, n_pairs))).astype(np.float16)
    out[nib_bytes:] = sb.reshape(-1).view(np.uint8)
    return out


def expert_blobs(d: int, f: int, seed: int, layer: int, experts, threads: int = 8) -> list[np.ndarray]:
    """Several blobs of one layer, generated on a small thread pool."""
    experts = list(experts)
    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        return list(ex.map(lambda e: expert_blob(d, f, seed, layer, e), experts))


def router_weight(d: int, n_experts: int, seed: int, layer: int) -> np.ndarray:
    """fp32 router matrix [E, d] ~ N(0, 0.02^2)."""
    return rng(seed, _ROUTER, layer).normal(0.0, 0.02, (n_experts, d)).astype(np.float32)


def zipf_bias(n_experts: int, seed: int, layer: int, s: float = 1.1) -> np.ndarray:
    """Additive router bias ln(pi_e) for a Zipf(s) popularity over a seeded
    per-layer permutation of the experts (fp32 [E])."""
    perm = rng(seed, _ZIPF, layer).permutation(n_experts)
    ranks = np.empty(n_experts, dtype=np.float64)
    ranks[perm] = np.arange(1, n_experts + 1, dtype=np.float64)
    p = ranks ** (-s)
    p /= p.sum()
    return np.log(p).astype(np.float32)


def zipf_probs(n_experts: int, seed: int, layer: int, s: float = 1.1) -> np.ndarray:
    return np.exp(zipf_bias(n_experts, seed, layer, s).astype(np.float64))


def norm_weight(d: int, seed: int, layer: int) -> np.ndarray:
    """RMSNorm weight [d] ~ N(1, 0.1^2), fp32."""
    return rng(seed, _NORM, layer).normal(1.0, 0.1, d).astype(np.float32)


def tokens(T: int, d: int, seed: int, stream: int = 0) -> np.ndarray:
    """Token activations [T, d] ~ N(0, 1), fp32."""
    return rng(seed, _TOKENS, stream).normal(0.0, 1.0, (T, d)).astype(np.float32)


def markov_selections(n_experts: int, k: int, steps: int, seed: int, layer: int,
                      keep: float = 0.8, refill: str = "zipf") -> np.ndarray:
    """Expert sets with token-to-token locality, int32 [steps, k] (each row
    sorted ascending).  Step 0 draws k experts without replacement from the
    prior; every later step keeps each previous expert with probability
    ``keep`` and refills from the prior restricted to the experts not kept.
    ``refill`` is "zipf" (the layer's Zipf(1.1) prior) or "uniform"."""
    g = rng(seed, _MARKOV, layer, 0 if refill == "zipf" else 1)
    prior = zipf_probs(n_experts, seed, layer) if refill == "zipf" else np.full(n_experts, 1.0 / n_experts)
    prior = prior / prior.sum()  # the Zipf bias is fp32: renormalise in fp64 for Generator.choice
    out = np.empty((steps, k), dtype=np.int32)
    cur = g.choice(n_experts, size=k, replace=False, p=prior)
    out[0] = np.sort(cur)
    for t in range(1, steps):
        kept = [e for e in cur if g.random() < keep]
        need = k - len(kept)
        if need:
            p = prior.copy()
            p[kept] = 0.0
            p /= p.sum()
            new = g.choice(n_experts, size=need, replace=False, p=p)
            cur = np.array(list(kept) + list(new))
        else:
            cur = np.array(kept)
        out[t] = np.sort(cur)
    return out


def selection_bias(selection: np.ndarray, n_experts: int, boost: float = 64.0) -> np.ndarray:
    """Router bias that forces a selection: +boost on the chosen experts, 0
    elsewhere (fp32 [..., E])."""
    sel = np.asarray(selection)
    out = np.zeros(sel.shape[:-1] + (n_experts,), dtype=np.float32)
    np.put_along_axis(out, sel.astype(np.int64), np.float32(boost), axis=-1)
    return out


def shared_weight_bf16(rows: int, cols: int, seed: int, layer: int) -> np.ndarray:
    """Dense shared-path weight as bf16 bit patterns (uint16 [rows, cols]),
    values ~ N(0, 0.02^2) rounded to nearest-even bf16."""
    w = rng(seed, _SHARED, layer).normal(0.0, 0.02, (rows, cols)).astype(np.float32)
    bits = w.view(np.uint32).astype(np.uint64)
    rounded = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def slot_permutation(n: int, seed: int, layer: int) -> np.ndarray:
    """A seeded permutation used to scatter experts over slots (int32 [n])."""
    return rng(seed, _PERM, layer).permutation(n).astype(np.int32)
