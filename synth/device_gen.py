"""Device-side seeded inputs for the million-token workload.

One layer of the 1M-token cache is 2 x 2 GiB of bf16, too large to draw on
the host per run, so it is drawn on the GPU with torch's Philox generator:
float32 N(0, 1) per KV head, scaled by 1/sqrt(128), rounded once to bf16.
Draw order per layer: K (head by head), V (head by head), then the query
and tree tensors.  Like the host generators, this holds no attention or
acceptance arithmetic.
"""
from __future__ import annotations

import math

from .generators import SEEDS

L_1M = 1 << 20


def _normal_bf16(shape, gen, device, scale):
    import torch
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    x.mul_(scale)
    return x.to(torch.bfloat16)


def layer_1m(layer: int, *, L: int = L_1M, Hq: int = 32, Hkv: int = 8, D: int = 128,
             n_chain: int = 3, device="cuda", seed: int = SEEDS[4]) -> dict:
    """Cache K/V ``[1, Hkv, L, D]``, the verify queries of a 3-token chain,
    its tree K/V, the 3 chained draft queries and 3 single draft queries."""
    import torch
    s = 1.0 / math.sqrt(D)
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
