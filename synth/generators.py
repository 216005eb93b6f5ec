"""Seeded input generators for the five workloads and for ad-hoc test shapes.

Every draw uses NumPy's PCG64 (``numpy.random.default_rng``).  Floating-point
tensors are drawn as float32 N(0, 1), optionally scaled, and, for bf16
workloads, rounded to bf16 with round-to-nearest-even and returned as raw
uint16 bit patterns.  Both the oracle and the HIP path start from these same
bits, so neither side sees a value the other does not.

Shapes follow the cache layout of the library: q ``[B, T, Hq, D]``,
K and V ``[B, Hkv, L_cap, D]`` with D contiguous, ``cache_len[B]`` int32.

Workload shapes (from the pages' experiments, see the design notes):
  * tiny fp32 case: B=1, Hq=2, Hkv=1, D=64, L=512, full binary tree of depth 3;
  * 4K: Llama-3-8B-shaped layer (32 q heads, 8 KV heads, D=128), budget 256;
  * 16K: batch 8, budgets 256..2048, 64-node tree with widths 10/18/18/18;
  * 1M: 32 layers of 1,048,576 tokens (generated on the device, per layer);
  * ragged: batch 16, contexts U[2048, 32768], 44- and 64-node trees, padding.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "SEEDS", "PLANT_LOGIT",
    "round_to_bf16_bits", "draw_normal",
    "AttnCase", "make_attn_case",
    "budget_indices", "Tree", "heap_tree", "chain_tree", "layered_tree",
    "draft_tokens", "plant_acceptance", "AcceptCase",
    "make_accept_case", "pad_groups", "config_tiny", "config_4k", "config_8k", "config_16k",
    "config_ragged",
]

# Seed 1000 c for workload c = 1..5; the 8K point between the 4K and 16K
# workloads (BudgetDraft sweeps its budgets at 4K, 8K and 16K) takes 3500.
SEEDS = {1: 1000, 2: 2000, 3: 3000, 4: 4000, 5: 5000, "8k": 3500}
PLANT_LOGIT = 10.0


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    r = ((u + bias) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def draw_normal(rng: np.random.Generator, shape, scale: float, dtype: str) -> np.ndarray:
    """N(0,1) * scale drawn in float32; bf16 workloads get RNE bit patterns."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    if dtype == "bf16":
        return round_to_bf16_bits(x)
    if dtype == "f32":
        return x
    raise ValueError(dtype)


@dataclass
class AttnCase:
    """One attention problem.  Arrays are bf16 bits (uint16) or float32."""
    dtype: str
    B: int
    Hq: int
    Hkv: int
    D: int
    L_cap: int
    scale: float
    q: np.ndarray              # [B, T, Hq, D]
    k: np.ndarray              # [B, Hkv, L_cap, D]
    v: np.ndarray              # [B, Hkv, L_cap, D]
    cache_len: np.ndarray      # [B] int32
    extra: dict = field(default_factory=dict)


def make_attn_case(seed: int, *, B: int, Hq: int, Hkv: int, D: int, L_cap: int,
                   T: int, cache_len=None, dtype: str = "bf16",
                   value_scale: float | None = None) -> AttnCase:
    """Draw q, K, V in the fixed order q, K, V.

    ``value_scale`` multiplies the N(0,1) draws (``1/sqrt(128)`` for the bf16
    workloads, 1.0 for the tiny fp32 case and for the peaked variants).
    """
    rng = np.random.default_rng(seed)
    vs = 1.0 if value_scale is None else value_scale
    q = draw_normal(rng, (B, T, Hq, D), vs, dtype)
    k = draw_normal(rng, (B, Hkv, L_cap, D), vs, dtype)
    v = draw_normal(rng, (B, Hkv, L_cap, D), vs, dtype)
    if cache_len is None:
        cache_len = np.full(B, L_cap, dtype=np.int32)
    cache_len = np.asarray(cache_len, dtype=np.int32)
    return AttnCase(dtype, B, Hq, Hkv, D, L_cap, 1.0 / math.sqrt(D), q, k, v,
                    cache_len, {"rng": rng})


# ---------------------------------------------------------------- KV budgets

def budget_indices(rng: np.random.Generator, L: int, budget: int,
                   n_sink: int = 4) -> np.ndarray:
    """Budget list: sink [0, n_sink), the last budget/2 positions, and the rest
    drawn uniformly without replacement from the middle; sorted, int32.

    This is the budget recipe of the 4K and 16K workloads (sink 4 + recent B/2
    + uniform middle).  When L <= budget every position is taken.
    """
    if L <= budget:
        return np.arange(L, dtype=np.int32)
    recent = budget // 2
    n_mid = budget - n_sink - recent
    lo, hi = n_sink, L - recent
    mid = rng.choice(hi - lo, size=n_mid, replace=False) + lo
    sel = np.concatenate([np.arange(n_sink), mid, np.arange(L - recent, L)])
    return np.sort(sel).astype(np.int32)


# ---------------------------------------------------------------- tree shapes

@dataclass
class Tree:
    """A speculation tree as built: parent per node (-1 = child of the anchor)
    and each node's depth as placed by the builder (not derived afterwards)."""
    parents: np.ndarray   # [N] int32
    depth: np.ndarray     # [N] int32, depth-0 nodes hang off the anchor

    @property
    def n(self) -> int:
        return len(self.parents)


def heap_tree(k: int, levels: int) -> Tree:
    """Full k-ary tree with depths 0..levels in breadth-first (heap) order.

    Node 0 hangs off the anchor (parent -1); node i > 0 has parent (i-1)//k.
    """
    par, dep = [-1], [0]
    for lev in range(1, levels + 1):
        first = len(par)
        for i in range(first, first + k ** lev):
            par.append((i - 1) // k)
            dep.append(lev)
    return Tree(np.asarray(par, np.int32), np.asarray(dep, np.int32))


def chain_tree(n: int) -> Tree:
    """A chain of n speculated tokens: parents -1, 0, 1, ..., n-2."""
    return Tree(np.arange(-1, n - 1, dtype=np.int32), np.arange(n, dtype=np.int32))


def layered_tree(rng: np.random.Generator, widths) -> Tree:
    """Depth-major tree: depth-0 nodes hang off the anchor; each deeper node
    picks its parent uniformly among the nodes of the previous depth."""
    par, dep = [], []
    prev_first, prev_w = 0, 0
    for d, w in enumerate(widths):
        first = len(par)
        if d == 0:
            par.extend([-1] * w)
        else:
            par.extend((rng.integers(0, prev_w, size=w) + prev_first).tolist())
        dep.extend([d] * w)
        prev_first, prev_w = first, w
    return Tree(np.asarray(par, np.int32), np.asarray(dep, np.int32))


# ---------------------------------------------------------------- acceptance

def draft_tokens(rng: np.random.Generator, parents: np.ndarray, vocab: int) -> np.ndarray:
    """Draft token per node; siblings (same parent, the anchor included) get
    distinct tokens."""
    tok = np.empty(len(parents), dtype=np.int32)
    for p in np.unique(parents):
        kids = np.nonzero(parents == p)[0]
        tok[kids] = rng.choice(vocab, size=len(kids), replace=False)
    return tok


def plant_acceptance(rng: np.random.Generator, logits_b: np.ndarray, tokens: np.ndarray,
                     tree: Tree, depth_target: int):
    """Plant a known accepted path of ``depth_target`` draft tokens into one
    sequence's logits ``[N+1, V]`` (row 0 = anchor, row i+1 = node i).

    Returns the expected (accept_len, path, bonus) by construction: the
    planted value makes a row's maximum the chosen token, and the row after
    the last accepted node gets a token that none of its children carry.
    """
    parents = tree.parents
    d = min(depth_target, int(tree.depth.max()) + 1)
    path = []
    if d > 0:
        node = int(rng.choice(np.nonzero(tree.depth == d - 1)[0]))
        while node >= 0:
            path.append(node)
            node = int(parents[node])
        path.reverse()
        for n in path:
            logits_b[parents[n] + 1, tokens[n]] = PLANT_LOGIT
    stop_node = path[-1] if path else -1
    kid_toks = set(tokens[parents == stop_node].tolist())
    V = logits_b.shape[-1]
    while True:
        x = int(rng.integers(0, V))
        if x not in kid_toks:
            break
    logits_b[stop_node + 1, x] = PLANT_LOGIT
    return d, path, x


@dataclass
class AcceptCase:
    logits: np.ndarray        # [B, N+1, V] float32
    tokens: np.ndarray        # [B, N] int32
    parents: np.ndarray       # [N] int32 (shared across the batch)
    max_depth: int
    expected_len: np.ndarray  # [B]
    expected_path: list
    expected_bonus: np.ndarray


def make_accept_case(seed: int, tree: Tree, B: int, vocab: int,
                     depths=None) -> AcceptCase:
    """Logits N(0,1) [B, N+1, V], sibling-distinct draft tokens and a planted
    accepted depth per sequence (uniform over 0..max depth unless given)."""
    rng = np.random.default_rng(seed)
    N = tree.n
    logits = rng.standard_normal(size=(B, N + 1, vocab), dtype=np.float32)
    maxd = int(tree.depth.max()) + 1
    tokens = np.stack([draft_tokens(rng, tree.parents, vocab) for _ in range(B)])
    if depths is None:
        depths = rng.integers(0, maxd + 1, size=B)
    exp_len, exp_path, exp_bonus = [], [], []
    for b in range(B):
        d, path, x = plant_acceptance(rng, logits[b], tokens[b], tree, int(depths[b]))
        exp_len.append(d)
        exp_path.append(path)
        exp_bonus.append(x)
    return AcceptCase(logits, tokens.astype(np.int32), tree.parents.copy(), maxd,
                      np.asarray(exp_len, np.int32), exp_path,
                      np.asarray(exp_bonus, np.int32))


# ---------------------------------------------------------------- padding

def pad_groups(rng: np.random.Generator, L_b: int, n_groups: int = 32,
               group: int = 5) -> np.ndarray:
    """Per-slot pad flags (uint8, length L_b) for a sequence whose last
    ``n_groups`` verify steps each appended ``group`` slots: a ~ U{1..group}
    accepted tokens followed by ``group - a`` pads."""
    pad = np.zeros(L_b, dtype=np.uint8)
    n_groups = min(n_groups, L_b // group)
    for g in range(n_groups):
        start = L_b - (n_groups - g) * group
        a = int(rng.integers(1, group + 1))
        pad[start + a:start + group] = 1
    return pad


# ---------------------------------------------------------------- workloads

def config_tiny(seed: int = SEEDS[1]) -> dict:
    """Tiny fp32 case: B=1, Hq=2, Hkv=1, D=64, L=512; draft sink 4 + W 64 over
    one query; full binary tree (k=2, depths 0..3, N=15); vocab 1000."""
    tree = heap_tree(2, 3)
    case = make_attn_case(seed, B=1, Hq=2, Hkv=1, D=64, L_cap=512, T=1, dtype="f32")
    rng = case.extra["rng"]
    N = tree.n
    vq = draw_normal(rng, (1, N, 2, 64), 1.0, "f32")
    tk = draw_normal(rng, (1, 1, N, 64), 1.0, "f32")
    tv = draw_normal(rng, (1, 1, N, 64), 1.0, "f32")
    return dict(case=case, n_sink=4, window=64, tree=tree, verify_q=vq,
                tree_k=tk, tree_v=tv, vocab=1000)


def config_4k(seed: int = SEEDS[2], value_scale: float | None = None) -> dict:
    """4K: B=1, Hq=32, Hkv=8, D=128, bf16 N(0,1)/sqrt(128) (or N(0,1) times
    ``value_scale``, the peaked variant); draft over a budget of 256 (sink 4,
    last 128, 124 uniform middle); verify chain of 5."""
    s = 1.0 / math.sqrt(128) if value_scale is None else value_scale
    case = make_attn_case(seed, B=1, Hq=32, Hkv=8, D=128, L_cap=4096, T=1, value_scale=s)
    rng = case.extra["rng"]
    tree = chain_tree(5)
    vq = draw_normal(rng, (1, 5, 32, 128), s, "bf16")
    tk = draw_normal(rng, (1, 8, 5, 128), s, "bf16")
    tv = draw_normal(rng, (1, 8, 5, 128), s, "bf16")
    idx = budget_indices(rng, 4096, 256)[None, None, :]
    return dict(case=case, idx=idx, tree=tree, verify_q=vq, tree_k=tk, tree_v=tv,
                vocab=128256)


def config_16k(seed: int = SEEDS[3], budgets=(256, 512, 1024, 2048), L: int = 16384,
               B: int = 8, value_scale: float | None = None) -> dict:
    """16K: B=8, L=16384, budgets 256..2048 drawn per sequence (shared across
    KV heads), 64-node tree of widths 10/18/18/18 shared across the batch;
    values N(0,1)/sqrt(128), or N(0,1) times ``value_scale``."""
    s = 1.0 / math.sqrt(128) if value_scale is None else value_scale
    case = make_attn_case(seed, B=B, Hq=32, Hkv=8, D=128, L_cap=L, T=1, value_scale=s)
    rng = case.extra["rng"]
    tree = layered_tree(rng, (10, 18, 18, 18))
    N = tree.n
    vq = draw_normal(rng, (B, N, 32, 128), s, "bf16")
    tk = draw_normal(rng, (B, 8, N, 128), s, "bf16")
    tv = draw_normal(rng, (B, 8, N, 128), s, "bf16")
    idx = {bud: np.stack([budget_indices(rng, L, bud) for _ in range(B)])[:, None, :]
           for bud in budgets}
    return dict(case=case, idx=idx, tree=tree, verify_q=vq, tree_k=tk, tree_v=tv,
                vocab=128256)


def config_8k(seed: int = SEEDS["8k"], budgets=(256, 512, 1024, 2048)) -> dict:
    """8K: the 16K recipe at L = 8192 (batch 8, budgets 256..2048 per
    sequence, the 64-node tree of widths 10/18/18/18, vocab 128,256)."""
    return config_16k(seed, budgets, L=8192, B=8)


def config_ragged(seed: int = SEEDS[5], widths=(10, 14, 12, 8), B: int = 16,
                  lo: int = 2048, hi: int = 32768) -> dict:
    """Ragged batch: B=16, L_b ~ U{lo..hi}, tail padding in groups of 5,
    layered tree of the given widths (44-node 10/14/12/8 or 64-node
    10/18/18/18)."""
    s = 1.0 / math.sqrt(128)
    rng0 = np.random.default_rng(seed)
    lens = rng0.integers(lo, hi + 1, size=B).astype(np.int32)
    case = make_attn_case(seed + 1, B=B, Hq=32, Hkv=8, D=128, L_cap=hi, T=1,
                          cache_len=lens, value_scale=s)
    rng = case.extra["rng"]
    pad = np.zeros((B, hi), dtype=np.uint8)
    for b in range(B):
        pad[b, :lens[b]] = pad_groups(rng, int(lens[b]))
    tree = layered_tree(rng, widths)
    N = tree.n
    vq = draw_normal(rng, (B, N, 32, 128), s, "bf16")
    tk = draw_normal(rng, (B, 8, N, 128), s, "bf16")
    tv = draw_normal(rng, (B, 8, N, 128), s, "bf16")
    return dict(case=case, pad=pad, tree=tree, verify_q=vq, tree_k=tk, tree_v=tv,
                vocab=128256)
