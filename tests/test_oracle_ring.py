"""Pins for the oracle's draft-KV ring buffer (CPU only).

Pinned against: a hand-enumerated slot table (golden/ring_slots.json); the
invariant that the positions any draft view needs occupy distinct slots when
the ring holds window + Tq - 1 positions; and torch SDPA over the explicit
view positions of the logical cache, which the window draft over the ring
must reproduce wherever the ring has wrapped.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import ring as ro
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_slots_match_the_hand_table():
    with open(os.path.join(GOLDEN, "ring_slots.json")) as f:
        fx = json.load(f)
    got = [ro.ring_slot(p, fx["n_sink"], fx["ring"]) for p in fx["positions"]]
    assert got == fx["slots"]


@pytest.mark.parametrize("T", [1, 3, 5])
def test_views_occupy_distinct_slots(T):
    for n_sink, window in ((0, 7), (4, 16), (4, 64)):
        ring = window + T - 1
        for L in list(range(T, 300, 7)) + [10 ** 6 + 3]:
            need = set()
            for t in range(T):
                need |= set(oracle.draft_view(L, T, t, n_sink=n_sink, window=window).tolist())
            slots = {ro.ring_slot(p, n_sink, ring) for p in need}
            assert len(slots) == len(need), (n_sink, window, L)
            assert max(slots) < n_sink + ring


@pytest.mark.parametrize("T", [1, 3])
@pytest.mark.parametrize("lens", [[40, 23], [300, 161], [999, 512]])
def test_ring_draft_is_sdpa_over_the_logical_view(T, lens):
    n_sink, window = 4, 24
    ring = window + T - 1 + 5                 # some slack beyond the minimum
    c = synth.make_attn_case(8500 + T + lens[0], B=2, Hq=4, Hkv=2, D=16, L_cap=max(lens), T=T,
                             cache_len=lens, dtype="f32")
    kr = ro.ring_from_logical(c.k, c.cache_len, n_sink, ring)
    vr = ro.ring_from_logical(c.v, c.cache_len, n_sink, ring)
    out, lse = oracle.ring_draft_ref(c.q, kr, vr, c.cache_len, scale=c.scale, n_sink=n_sink,
                                     window=window, ring=ring)
    for b in range(2):
        L = int(c.cache_len[b])
        for t in range(T):
            view = oracle.draft_view(L, T, t, n_sink=n_sink, window=window)
            for g in range(2):
                q = torch.from_numpy(c.q[b, t, 2 * g:2 * g + 2].astype(np.float64))[None, :, None]
                k = torch.from_numpy(c.k[b, g, view].astype(np.float64))[None, None]
                v = torch.from_numpy(c.v[b, g, view].astype(np.float64))[None, None]
                o = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=c.scale)
                np.testing.assert_allclose(out[b, t, 2 * g:2 * g + 2], o[0, :, 0].numpy(),
                                           rtol=0, atol=1e-12)


def test_a_ring_too_small_for_the_chained_queries_is_rejected():
    c = synth.make_attn_case(8600, B=1, Hq=2, Hkv=1, D=8, L_cap=50, T=3, dtype="f32")
    kr = ro.ring_from_logical(c.k, c.cache_len, 4, 10)
    with pytest.raises(ValueError):
        oracle.ring_draft_ref(c.q, kr, kr, c.cache_len, scale=c.scale, n_sink=4, window=9, ring=10)


def test_later_positions_overwrite_their_slot():
    k = np.arange(30, dtype=np.float32).reshape(1, 1, 30, 1)
    kr = ro.ring_from_logical(k, [30], 2, 8)
    # slot s >= 2 holds the latest p < 30 with 2 + (p - 2) % 8 = s
    assert kr[0, 0, :, 0].tolist() == [0, 1, 26, 27, 28, 29, 22, 23, 24, 25]
