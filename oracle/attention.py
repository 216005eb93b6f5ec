"""Draft and verify attention, plain definitions in float64 (test infrastructure).

Conventions shared with the library's interface:
  q ``[B, T, Hq, D]``; cache K, V ``[B, Hkv, L_cap, D]``; ``cache_len[b] = L_b``
  valid slots ``[0, L_b)``; query head h reads KV head ``h // (Hq // Hkv)``.
  Scores are ``scale * <q, k>``; no positional transform is applied because the
  cached keys already carry their rotary positions (Windowed-MTP review, "What
  carries the argument").  Each output row is ``sum_j softmax(s)_j V_j`` and
  ``lse = log sum_j exp(s_j)``; a row with no visible key gets 0 and -inf.
"""
from __future__ import annotations

import numpy as np

from .bf16 import as_f64


def _attend(Q: np.ndarray, K: np.ndarray, V: np.ndarray, visible: np.ndarray,
            scale: float):
    """Softmax attention of rows Q [r, D] over keys K/V [n, D], where row i
    sees key j iff visible[i, j].  Returns out [r, D], lse [r]."""
    r = Q.shape[0]
    out = np.zeros((r, V.shape[1]), dtype=np.float64)
    lse = np.full(r, -np.inf, dtype=np.float64)
    if K.shape[0] == 0:
        return out, lse
    S = scale * (Q @ K.T)                       # [r, n]
    for i in range(r):
        s = S[i][visible[i]]
        if s.size == 0:
            continue
        m = s.max()
        w = np.exp(s - m)
        z = w.sum()
        out[i] = (w / z) @ V[visible[i]]
        lse[i] = m + np.log(z)
    return out, lse


# ------------------------------------------------------------------ draft view

def draft_view(L_b: int, n_q: int, t: int, *, n_sink: int | None = None,
               window: int | None = None, idx_list=None) -> np.ndarray:
    """Key positions seen by draft query t (0-based) of n_q chained queries.

    The n_q queries are the last n_q positions of the sequence, so query t sits
    at position ``e - 1`` with ``e = L_b - n_q + t + 1`` and sees nothing at or
    after ``e`` (causal).

    Window mode (Windowed-MTP review, "What carries the argument"): the union
    of the first ``n_sink`` positions and the last ``window`` positions up to
    and including the query itself, each position counted once.

    Budget mode (BudgetDraft review, abstract): the caller's list of selected
    positions, restricted to the causal prefix.  An entry of -1 is padding
    and selects nothing, so lists of one fixed length can describe views of
    different sizes (a sequence shorter than the budget lists all of its
    positions, as SpecPV section 3.3 falls back to the whole cache when the
    sequence is shorter than the partial budget); any other position outside
    ``[0, L_b)`` is an input error.
    """
    e = L_b - n_q + t + 1
    if idx_list is None:
        sink = set(range(0, min(n_sink, e)))
        recent = set(range(max(0, e - window), e))
        return np.array(sorted(sink | recent), dtype=np.int64)
    lst = np.asarray(idx_list, dtype=np.int64)
    lst = lst[lst != -1]
    if ((lst < 0) | (lst >= L_b)).any():
        raise IndexError("budget index outside [0, cache_len)")
    return lst[lst < e]


def draft_attn_ref(q, k, v, cache_len, *, scale: float, n_sink=None, window=None,
                   idx=None, pairs=None):
    """Draft attention over the sparse view.

    ``idx`` is ``[B, Hidx, Bud]`` with Hidx = 1 (one list shared by all KV
    heads) or Hkv (one list per KV head); ``None`` selects window mode.
    ``pairs`` optionally restricts the work to a list of (b, kv_head).
    Returns out ``[B, T, Hq, D]`` and lse ``[B, T, Hq]`` (float64; rows that
    were not computed are NaN).
    """
    B, T, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.full((B, T, Hq, D), np.nan)
    lse = np.full((B, T, Hq), np.nan)
    if pairs is None:
        pairs = [(b, g) for b in range(B) for g in range(Hkv)]
    for b, g in pairs:
        L_b = int(cache_len[b])
        Kbg = as_f64(k[b, g, :L_b])
        Vbg = as_f64(v[b, g, :L_b])
        for t in range(T):
            if idx is None:
                pos = draft_view(L_b, T, t, n_sink=n_sink, window=window)
            else:
                lst = idx[b, 0 if idx.shape[1] == 1 else g]
                pos = draft_view(L_b, T, t, idx_list=lst)
            Q = as_f64(q[b, t, g * G:(g + 1) * G])
            vis = np.ones((G, len(pos)), dtype=bool)
            o, l = _attend(Q, Kbg[pos], Vbg[pos], vis, scale)
            out[b, t, g * G:(g + 1) * G] = o
            lse[b, t, g * G:(g + 1) * G] = l
    return out, lse


# ------------------------------------------------------------------ tree

def tree_depths(parents) -> np.ndarray:
    """Depth of each node: a node whose parent is -1 hangs off the anchor (the
    last committed token) and has depth 0; otherwise depth(parent) + 1.
    Parents must precede their children (SpecMemo review: a tree of
    N = sum_i k^i speculated nodes, built level by level)."""
    parents = np.asarray(parents)
    d = np.zeros(len(parents), dtype=np.int64)
    for i, p in enumerate(parents):
        if p < -1 or p >= i:
            raise ValueError("parent must be -1 or an earlier node")
        d[i] = 0 if p < 0 else d[p] + 1
    return d


def tree_ancestors(parents) -> np.ndarray:
    """anc[i, j] is True iff node j is node i or one of its ancestors."""
    parents = np.asarray(parents)
    n = len(parents)
    anc = np.zeros((n, n), dtype=bool)
    for i in range(n):
        j = i
        while j >= 0:
            anc[i, j] = True
            j = int(parents[j])
    return anc


def position_ids(cache_len, pad, parents) -> np.ndarray:
    """Remapped position of every tree node: the number of non-padding cache
    slots of its sequence plus its depth (SpecMemo review: position IDs are
    remapped so that padding is ignored).  ``pad`` is ``[B, L_cap]`` (nonzero =
    padding) or None; ``parents`` is ``[N]`` or ``[B, N]``."""
    cache_len = np.asarray(cache_len)
    B = len(cache_len)
    par = np.asarray(parents)
    out = []
    for b in range(B):
        pb = par if par.ndim == 1 else par[b]
        L_b = int(cache_len[b])
        n_pad = 0 if pad is None else int(np.count_nonzero(pad[b, :L_b]))
        out.append((L_b - n_pad) + tree_depths(pb))
    return np.stack(out).astype(np.int64)


def verify_attn_ref(q, k, v, cache_len, tree_k, tree_v, parents, *, scale: float,
                    pad=None, pairs=None, rows=None):
    """Tree-masked verify attention (SpecMemo review, "What carries the
    argument" and Figure 9).

    q ``[B, N, Hq, D]``; cache K/V ``[B, Hkv, L_cap, D]``; tree K/V
    ``[B, Hkv, N, D]`` hold the speculated nodes' keys and values; ``pad``
    ``[B, L_cap]`` (nonzero = padding, scored -inf) or None; ``parents`` is
    ``[N]`` (shared) or ``[B, N]``.  Node i attends to every non-padding slot
    of ``[0, L_b)`` and to the tree nodes on its root path, itself included.
    ``pairs`` restricts to (b, kv_head) pairs and ``rows`` to node indices.
    """
    B, N, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    par = np.asarray(parents)
    out = np.full((B, N, Hq, D), np.nan)
    lse = np.full((B, N, Hq), np.nan)
    if pairs is None:
        pairs = [(b, g) for b in range(B) for g in range(Hkv)]
    node_rows = list(range(N)) if rows is None else list(rows)
    for b, g in pairs:
        pb = par if par.ndim == 1 else par[b]
        anc = tree_ancestors(pb)
        L_b = int(cache_len[b])
        slots = np.arange(L_b)
        if pad is not None:
            slots = slots[np.asarray(pad[b, :L_b]) == 0]
        Kc = as_f64(k[b, g])[slots]
        Vc = as_f64(v[b, g])[slots]
        Kall = np.concatenate([Kc, as_f64(tree_k[b, g, :N])])
        Vall = np.concatenate([Vc, as_f64(tree_v[b, g, :N])])
        for i in node_rows:
            vis = np.concatenate([np.ones(len(slots), dtype=bool), anc[i]])
            Q = as_f64(q[b, i, g * G:(g + 1) * G])
            o, l = _attend(Q, Kall, Vall, np.broadcast_to(vis, (G, len(vis))), scale)
            out[b, i, g * G:(g + 1) * G] = o
            lse[b, i, g * G:(g + 1) * G] = l
    return out, lse
