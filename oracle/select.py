"""Budget selection by block-mean scoring, plain definitions (test
infrastructure only).

SpecPV (section 3.2 "Partial Verification") selects its partial KV cache at
the block level, as KV cache managers keep the cache in blocks, and keeps a
sink, the retrieved blocks and a local window as one key set; its
experiments (section 4.1) use "mean reduction" for the retrieval.
BudgetDraft (abstract) drafts over a sparse KV view under a fixed budget.

Reading of what the pages leave open:

* Blocks are the cache manager's: block c holds positions
  [c * block, (c + 1) * block).  Its summary is the mean of its keys over
  the positions below cache_len that are not padding (the "mean
  reduction"); a block with no such position has no summary (NaN).
* A KV head's queries (its G query heads times the Tq query tokens) score
  block c with the mean of their dot products with the block's mean key,
  i.e. (mean query) . (mean key); the softmax scale does not change the
  order and is left out.  With one list per sequence (``shared``: a cache
  manager's block holds every head, so a partial cache keeps whole blocks)
  the mean runs over every KV head's score as well.
* The list keeps the sink [0, n_sink) and the window
  [max(n_sink, L - window), L) of the draft view (L = cache_len), and
  chooses among the blocks that meet the middle [n_sink, L - window): the
  n_select highest scores, ties to the smaller block index, blocks without
  a summary never chosen.  A chosen block contributes its middle positions.
* The list holds the chosen positions that are not padding, in increasing
  order, then -1 entries up to the budget (a -1 entry selects nothing).
"""
from __future__ import annotations

import numpy as np

from .bf16 import as_f64


def block_means_ref(k, cache_len, block: int, n_blocks: int, pad=None) -> np.ndarray:
    """Mean key of every block: ``[B, Hkv, n_blocks, D]`` float64, NaN for a
    block with no valid position.  ``k`` is the cache ``[B, Hkv, L_cap, D]``
    (bf16 bits or float32), ``pad`` ``[B, >= L_cap]`` (nonzero = padding) or
    None."""
    B, Hkv, _, D = k.shape
    out = np.full((B, Hkv, n_blocks, D), np.nan)
    for b in range(B):
        L = int(cache_len[b])
        for c in range(n_blocks):
            pos = np.arange(c * block, min((c + 1) * block, L))
            if pad is not None:
                pos = pos[np.asarray(pad[b])[pos] == 0]
            if len(pos) == 0:
                continue
            for g in range(Hkv):
                out[b, g, c] = as_f64(k[b, g][pos]).mean(axis=0)
    return out


def candidate_blocks(L: int, block: int, n_sink: int, window: int) -> np.ndarray:
    """Blocks that meet the middle [n_sink, L - window)."""
    lo, hi = n_sink, L - window
    if hi <= lo:
        return np.zeros(0, dtype=np.int64)
    return np.arange(lo // block, (hi - 1) // block + 1)


def block_scores_ref(q, means, cache_len, block: int, n_sink: int, window: int,
                     shared: bool = False) -> np.ndarray:
    """Score of every candidate block per (sequence, KV head): ``[B, Hkv,
    n_blocks]`` float64, NaN where a block is not a candidate or has no
    summary; with ``shared``, ``[B, 1, n_blocks]``, the mean over the KV
    heads (NaN if any head has no summary).  ``q`` is ``[B, Tq, Hq, D]``."""
    B, T, Hq, D = q.shape
    Hkv, nb = means.shape[1], means.shape[2]
    G = Hq // Hkv
    sc = np.full((B, Hkv, nb), np.nan)
    for b in range(B):
        cand = candidate_blocks(int(cache_len[b]), block, n_sink, window)
        cand = cand[cand < nb]
        for g in range(Hkv):
            qbar = as_f64(q[b, :, g * G:(g + 1) * G]).reshape(-1, D).mean(axis=0)
            sc[b, g, cand] = means[b, g, cand] @ qbar
    if shared:
        return sc.mean(axis=1, keepdims=True)
    return sc


def top_blocks(scores_row: np.ndarray, n_select: int) -> np.ndarray:
    """The n_select highest finite scores, ties to the smaller block index;
    returned in increasing block order."""
    finite = np.nonzero(np.isfinite(scores_row))[0]
    order = sorted(finite.tolist(), key=lambda c: (-scores_row[c], c))
    return np.sort(np.asarray(order[:n_select], dtype=np.int64))


def select_list(L: int, pad_row, chosen, block: int, n_sink: int, window: int,
                budget: int) -> np.ndarray:
    """The budget list of one (sequence, KV head) from its chosen blocks."""
    mid_lo, mid_hi = n_sink, L - window
    pos = set(range(0, min(n_sink, L)))
    pos |= set(range(max(n_sink, L - window), L))
    for c in chosen:
        pos |= set(range(max(c * block, mid_lo), min((c + 1) * block, mid_hi)))
    lst = sorted(p for p in pos if pad_row is None or pad_row[p] == 0)
    if len(lst) > budget:
        raise ValueError("budget too small for the chosen positions")
    return np.array(lst + [-1] * (budget - len(lst)), dtype=np.int32)


def select_blocks_ref(q, k, cache_len, *, block: int, n_sink: int, window: int, n_select: int,
                      budget: int, pad=None, n_blocks: int | None = None, shared: bool = False):
    """Budget lists ``[B, Hkv, budget]`` (``[B, 1, budget]`` when shared)
    int32 chosen by block-mean scoring, with the scores and the chosen blocks
    per list."""
    B = k.shape[0]
    Hkv = 1 if shared else k.shape[1]
    if n_blocks is None:
        n_blocks = -(-k.shape[2] // block)
    means = block_means_ref(k, cache_len, block, n_blocks, pad)
    sc = block_scores_ref(q, means, cache_len, block, n_sink, window, shared)
    idx = np.zeros((B, Hkv, budget), dtype=np.int32)
    chosen = {}
    for b in range(B):
        for g in range(Hkv):
            ch = top_blocks(sc[b, g], n_select)
            chosen[(b, g)] = ch
            idx[b, g] = select_list(int(cache_len[b]), None if pad is None else pad[b], ch,
                                    block, n_sink, window, budget)
    return idx, sc, chosen
