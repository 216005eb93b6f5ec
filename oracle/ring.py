"""Draft-KV ring buffer, plain definitions (test infrastructure only).

Windowed-MTP review ("What carries the argument"): the draft attends only to
the first n_sink positions and the last W, so its KV working set is a
constant window and the draft KV pool can be compacted into a ring buffer;
the referee's remarks on the appendix pseudocode name the slot mapping
"slot = ring_base(r) + logical_pos" with the ring wrapping and a "+d slack".

Reading of what the pages leave open:

* One sequence's draft cache keeps the sink in slots [0, n_sink) and a ring
  of R slots after it: logical position p >= n_sink lives in slot
  n_sink + (p - n_sink) mod R.  The sequence's ring base is slot n_sink of
  its own rows.
* The ring must hold every position a draft query can see: the last query
  sees [L - window, L) and the first of Tq chained queries reaches back to
  L - Tq + 1 - window, so R >= window + Tq - 1 (the slack d = Tq - 1 covers
  the chained draft queries).
* cache_len stays the logical length of the sequence; it may exceed the
  ring's capacity.
"""
from __future__ import annotations

import numpy as np

from .attention import draft_attn_ref, draft_view


def ring_slot(p: int, n_sink: int, ring: int) -> int:
    """Slot of logical position p."""
    return p if p < n_sink else n_sink + (p - n_sink) % ring


def ring_from_logical(k_logical, cache_len, n_sink: int, ring: int):
    """Lay a logical cache ``[B, Hkv, L_cap, D]`` out as a ring cache
    ``[B, Hkv, n_sink + ring, D]``: each slot holds the latest position
    (below cache_len) that maps to it; slots never written are zero."""
    k_logical = np.asarray(k_logical)
    B, Hkv, _, D = k_logical.shape
    out = np.zeros((B, Hkv, n_sink + ring, D), dtype=k_logical.dtype)
    for b in range(B):
        for p in range(int(cache_len[b])):      # later positions overwrite earlier ones
            out[b, :, ring_slot(p, n_sink, ring)] = k_logical[b, :, p]
    return out


def ring_draft_ref(q, k_ring, v_ring, cache_len, *, scale: float, n_sink: int, window: int,
                   ring: int):
    """Window draft over a ring cache: the draft view of each query (logical
    positions, as in window mode), each position read from its ring slot."""
    B, T = q.shape[0], q.shape[1]
    if window + T - 1 > ring:
        raise ValueError("the ring must hold window + Tq - 1 positions")
    # rebuild, per sequence, the logical rows the views need, then reuse the
    # window-mode definition over that logical cache
    L_max = int(np.max(cache_len))
    Hkv, D = k_ring.shape[1], k_ring.shape[3]
    kl = np.zeros((B, Hkv, L_max, D), dtype=k_ring.dtype)
    vl = np.zeros((B, Hkv, L_max, D), dtype=v_ring.dtype)
    for b in range(B):
        L = int(cache_len[b])
        need = set()
        for t in range(T):
            need |= set(draft_view(L, T, t, n_sink=n_sink, window=window).tolist())
        for p in need:
            kl[b, :, p] = k_ring[b, :, ring_slot(p, n_sink, ring)]
            vl[b, :, p] = v_ring[b, :, ring_slot(p, n_sink, ring)]
    return draft_attn_ref(q, kl, vl, np.asarray(cache_len), scale=scale, n_sink=n_sink,
                          window=window)
