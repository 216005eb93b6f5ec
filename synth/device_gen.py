"""Device-side seeded inputs for the large workloads.

One layer of the 1M-token cache is 2 x 2 GiB of bf16, and the ragged batch
of 16 sequences up to 32K tokens is 2 x 1 GiB: too large to draw on the
host per run, so they are drawn on the GPU with torch's Philox generator:
float32 N(0, 1) per KV head, scaled by 1/sqrt(128), rounded once to bf16.
Draw order per layer: K (head by head), V (head by head), then the query
and tree tensors.  Small integer structure (context lengths, padding,
parents) comes from the host generators.  Like the host generators, this
holds no attention or acceptance arithmetic.
"""
from __future__ import annotations

import math

import numpy as np

from .generators import SEEDS, layered_tree, pad_groups

L_1M = 1 << 20


def _normal_bf16(shape, gen, device, scale):
    import torch
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    x.mul_(scale)
    return x.to(torch.bfloat16)


def layer_1m(layer: int, *, L: int = L_1M, Hq: int = 32, Hkv: int = 8, D: int = 128,
             n_chain: int = 3, device="cuda", seed: int = SEEDS[4],
             value_scale: float | None = None) -> dict:
    """Cache K/V ``[1, Hkv, L, D]``, the verify queries of a 3-token chain,
    its tree K/V, the 3 chained draft queries and 3 single draft queries;
    every draw N(0,1)/sqrt(D), or N(0,1) times ``value_scale``."""
    import torch
    s = 1.0 / math.sqrt(D) if value_scale is None else value_scale
    gen = torch.Generator(device=device)
    gen.manual_seed(seed + layer)
    k = torch.empty((1, Hkv, L, D), dtype=torch.bfloat16, device=device)
    v = torch.empty_like(k)
    for h in range(Hkv):
        k[0, h] = _normal_bf16((L, D), gen, device, s)
    for h in range(Hkv):
        v[0, h] = _normal_bf16((L, D), gen, device, s)
    return dict(
        k=k, v=v,
        verify_q=_normal_bf16((1, n_chain, Hq, D), gen, device, s),
        tree_k=_normal_bf16((1, Hkv, n_chain, D), gen, device, s),
        tree_v=_normal_bf16((1, Hkv, n_chain, D), gen, device, s),
        ctx_q=_normal_bf16((1, n_chain, Hq, D), gen, device, s),
        fwd_q=[_normal_bf16((1, 1, Hq, D), gen, device, s) for _ in range(n_chain)],
    )


def ragged_batch(widths=(10, 14, 12, 8), *, B: int = 16, lo: int = 2048, hi: int = 32768,
                 Hq: int = 32, Hkv: int = 8, D: int = 128, device="cuda",
                 seed: int = SEEDS[5], value_scale: float | None = None,
                 q_scale: float = 1.0) -> dict:
    """Ragged batch: L_b ~ U{lo..hi} (host PCG64), tail padding in groups of
    5 over the last 32 verify steps, a layered tree of the given widths with
    parents uniform over the previous depth (host), and q, cache K/V
    ``[B, Hkv, hi, D]``, tree K/V drawn on the device.  ``value_scale``
    defaults to 1/sqrt(D); the queries are further multiplied by q_scale
    (value_scale 1.0 with q_scale 4 gives a peaked variant: scores with a
    spread of about 4, so a few keys carry most of each softmax)."""
    import torch
    s = 1.0 / math.sqrt(D) if value_scale is None else value_scale
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi + 1, size=B).astype(np.int32)
    pad = np.zeros((B, hi), dtype=np.uint8)
    for b in range(B):
        pad[b, :lens[b]] = pad_groups(rng, int(lens[b]))
    tree = layered_tree(rng, widths)
    N = tree.n
    gen = torch.Generator(device=device)
    gen.manual_seed(seed + 17)
    k = torch.empty((B, Hkv, hi, D), dtype=torch.bfloat16, device=device)
    v = torch.empty_like(k)
    for b in range(B):
        k[b] = _normal_bf16((Hkv, hi, D), gen, device, s)
    for b in range(B):
        v[b] = _normal_bf16((Hkv, hi, D), gen, device, s)
    return dict(
        lens=lens, pad=pad, tree=tree, k=k, v=v,
        verify_q=_normal_bf16((B, N, Hq, D), gen, device, s * q_scale),
        tree_k=_normal_bf16((B, Hkv, N, D), gen, device, s),
        tree_v=_normal_bf16((B, Hkv, N, D), gen, device, s),
    )
