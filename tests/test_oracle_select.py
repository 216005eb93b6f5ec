"""Pins for the oracle's budget selection by block-mean scoring (CPU only).

Pinned against: closed forms of block means over a ramp of keys; the mean
of every pairwise query-key score of a block, computed with torch matmul;
exhaustive enumeration of k-subsets for the top-k rule; attention over the
emitted lists (SDPA for a list covering everything, the window draft for a
list of sink and window only); a planted block that must be chosen.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import select as sel
import synth


def ramp_cache(B, Hkv, L_cap, D):
    """K[b, g, j, :] = (j + 1) * u_g with u_g = (g + 1) * [1, 2, ..., D]
    (small integers, exact in float32)."""
    j = np.arange(L_cap, dtype=np.float64) + 1
    u = np.arange(1, D + 1)[None, :] * np.arange(1, Hkv + 1)[:, None]
    k = j[None, None, :, None] * u[None, :, None, :]
    return np.broadcast_to(k, (B, Hkv, L_cap, D)).astype(np.float32)


def test_block_means_of_a_ramp_closed_form():
    B, Hkv, D, bs, L_cap = 2, 2, 8, 16, 80
    k = ramp_cache(B, Hkv, L_cap, D)
    lens = np.array([80, 45])
    pad = np.zeros((B, L_cap), dtype=np.uint8)
    pad[1, [17, 18, 30]] = 1              # sequence 1: pads inside block 1
    m = oracle.block_means_ref(k, lens, bs, 5, pad)
    u = k[0, :, 0, :].astype(np.float64)  # (0 + 1) * u
    for b in range(B):
        L = int(lens[b])
        for c in range(5):
            pos = [p for p in range(c * bs, min((c + 1) * bs, L)) if not pad[b, p]]
            if not pos:
                assert np.all(np.isnan(m[b, :, c]))
                continue
            # mean of (p + 1) over the listed positions, times u
            s = sum(p + 1 for p in pos) / len(pos)
            np.testing.assert_allclose(m[b, :, c], s * u, rtol=1e-12)
    # sequence 1 has 45 tokens: block 2 covers 32..44, block 3 is empty
    np.testing.assert_allclose(m[1, 0, 2], (33 + 45) / 2 * u[0], rtol=1e-12)
    assert np.all(np.isnan(m[1, :, 3]))


@pytest.mark.parametrize("seed", range(3))
def test_block_score_is_the_mean_of_all_its_pairwise_scores(seed):
    """(mean query) . (mean key) equals the mean of q_r . k_j over the
    group's query rows r and the block's valid positions j (bilinearity),
    computed here as one matmul."""
    c = synth.make_attn_case(6100 + seed, B=2, Hq=8, Hkv=2, D=32, L_cap=96, T=3,
                             cache_len=[96, 70], dtype="bf16", value_scale=1.0)
    pad = (np.random.default_rng(seed).random((2, 96)) < 0.15).astype(np.uint8)
    bs, sink, win = 8, 4, 20
    means = oracle.block_means_ref(c.k, c.cache_len, bs, 12, pad)
    sc = oracle.block_scores_ref(c.q, means, c.cache_len, bs, sink, win)
    G = 4
    for b in range(2):
        L = int(c.cache_len[b])
        for g in range(2):
            Q = torch.from_numpy(oracle.as_f64(c.q[b, :, g * G:(g + 1) * G]).reshape(-1, 32))
            for blk in range(12):
                pos = [p for p in range(blk * bs, min((blk + 1) * bs, L)) if not pad[b, p]]
                is_cand = blk in sel.candidate_blocks(L, bs, sink, win).tolist()
                if not pos or not is_cand:
                    assert np.isnan(sc[b, g, blk])
                    continue
                K = torch.from_numpy(oracle.as_f64(c.k[b, g])[pos])
                want = (Q @ K.T).mean().item()
                assert abs(sc[b, g, blk] - want) <= 1e-12 * max(1.0, abs(want))


@pytest.mark.parametrize("seed", range(40))
def test_top_blocks_equals_best_subset_enumeration(seed):
    """Top-k with ties to the smaller index = among the k-subsets of blocks
    with a score, the one of largest score sum, then the lexicographically
    smallest; every block with a score when fewer than k have one."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 9))
    s = rng.integers(0, 4, size=n).astype(np.float64)          # frequent ties
    s[rng.random(n) < 0.2] = np.nan
    k = int(rng.integers(0, n + 2))
    got = sel.top_blocks(s, k).tolist()
    finite = [i for i in range(n) if np.isfinite(s[i])]
    if k >= len(finite):
        assert got == finite
        return
    best = max(itertools.combinations(finite, k), key=lambda t: (sum(s[i] for i in t),
                                                                   [-i for i in t]))
    assert got == list(best)


def test_selecting_every_block_lists_every_position_and_gives_full_attention():
    c = synth.make_attn_case(6200, B=2, Hq=4, Hkv=2, D=16, L_cap=90, T=1,
                             cache_len=[90, 61], dtype="f32")
    idx, _, _ = oracle.select_blocks_ref(c.q, c.k, c.cache_len, block=8, n_sink=4, window=10,
                                         n_select=100, budget=100)
    for b in range(2):
        L = int(c.cache_len[b])
        for g in range(2):
            np.testing.assert_array_equal(idx[b, g, :L], np.arange(L))
            assert np.all(idx[b, g, L:] == -1)
    out, _ = oracle.draft_attn_ref(c.q, c.k, c.v, c.cache_len, scale=c.scale, idx=idx)
    for b in range(2):
        L = int(c.cache_len[b])
        q = torch.from_numpy(oracle.as_f64(c.q[b]).transpose(1, 0, 2))[None]
        kk = torch.from_numpy(oracle.as_f64(c.k[b, :, :L]))[None]
        vv = torch.from_numpy(oracle.as_f64(c.v[b, :, :L]))[None]
        ref = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, scale=c.scale,
                                                               enable_gqa=True)
        np.testing.assert_allclose(out[b], ref[0].numpy().transpose(1, 0, 2), rtol=0,
                                   atol=1e-12)


@pytest.mark.parametrize("T", [1, 3])
def test_selecting_no_block_is_the_window_draft(T):
    """With no block chosen the list is the sink and the window ending at
    cache_len: for the last query (the one at position cache_len - 1) that is
    the window draft's view."""
    c = synth.make_attn_case(6300 + T, B=2, Hq=4, Hkv=1, D=16, L_cap=120, T=T,
                             cache_len=[120, 77], dtype="f32")
    idx, _, _ = oracle.select_blocks_ref(c.q, c.k, c.cache_len, block=16, n_sink=4, window=24,
                                         n_select=0, budget=40)
    got, lse_g = oracle.draft_attn_ref(c.q, c.k, c.v, c.cache_len, scale=c.scale, idx=idx)
    want, lse_w = oracle.draft_attn_ref(c.q, c.k, c.v, c.cache_len, scale=c.scale, n_sink=4,
                                        window=24)
    np.testing.assert_allclose(got[:, T - 1], want[:, T - 1], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse_g[:, T - 1], lse_w[:, T - 1], rtol=0, atol=1e-13)


def test_planted_block_is_chosen():
    """A block whose keys point along the group's mean query has by far the
    largest score, so it is the one block chosen."""
    c = synth.make_attn_case(6400, B=1, Hq=4, Hkv=2, D=32, L_cap=256, T=2,
                             cache_len=[256], dtype="f32", value_scale=0.1)
    k = c.k.copy()
    G = 2
    for g, blk in ((0, 5), (1, 11)):
        qbar = c.q[0, :, g * G:(g + 1) * G].reshape(-1, 32).mean(axis=0)
        k[0, g, blk * 16:(blk + 1) * 16] = 3 * qbar / np.linalg.norm(qbar)
    idx, sc, chosen = oracle.select_blocks_ref(c.q, k, c.cache_len, block=16, n_sink=4,
                                               window=32, n_select=1, budget=4 + 32 + 16)
    assert chosen[(0, 0)].tolist() == [5] and chosen[(0, 1)].tolist() == [11]
    assert set(range(80, 96)) <= set(idx[0, 0].tolist())
    assert set(range(176, 192)) <= set(idx[0, 1].tolist())


def test_lists_skip_pads_stay_sorted_and_within_the_view():
    rng = np.random.default_rng(6500)
    c = synth.make_attn_case(6500, B=3, Hq=8, Hkv=2, D=16, L_cap=300, T=1,
                             cache_len=[300, 211, 40], dtype="bf16", value_scale=1.0)
    pad = (rng.random((3, 300)) < 0.1).astype(np.uint8)
    bs, sink, win, nsel = 16, 4, 32, 5
    budget = sink + win + nsel * bs
    idx, sc, chosen = oracle.select_blocks_ref(c.q, c.k, c.cache_len, block=bs, n_sink=sink,
                                               window=win, n_select=nsel, budget=budget, pad=pad)
    for b in range(3):
        L = int(c.cache_len[b])
        for g in range(2):
            lst = idx[b, g][idx[b, g] >= 0]
            assert np.all(np.diff(lst) > 0)
            assert np.all(idx[b, g, len(lst):] == -1)
            assert not pad[b, lst].any()
            allowed = set(range(min(sink, L))) | set(range(max(sink, L - win), L))
            for blk in chosen[(b, g)]:
                allowed |= set(range(max(blk * bs, sink), min((blk + 1) * bs, L - win)))
            assert set(lst.tolist()) == {p for p in allowed if not pad[b, p]}
            assert len(chosen[(b, g)]) == min(nsel, int(np.isfinite(sc[b, g]).sum()))
    # sequence 2 (40 tokens) is shorter than sink + window: every non-pad position
    lst = idx[2, 0][idx[2, 0] >= 0]
    np.testing.assert_array_equal(lst, [p for p in range(40) if not pad[2, p]])


@pytest.mark.parametrize("seed", range(2))
def test_shared_score_is_the_mean_over_every_head_of_its_pairwise_scores(seed):
    """One list per sequence: a block's score is the mean over the KV heads
    of each head's mean pairwise query-key score (every query head paired
    with its own KV head)."""
    c = synth.make_attn_case(6600 + seed, B=1, Hq=8, Hkv=4, D=16, L_cap=64, T=2,
                             cache_len=[64], dtype="f32", value_scale=1.0)
    means = oracle.block_means_ref(c.k, c.cache_len, 8, 8)
    sc = oracle.block_scores_ref(c.q, means, c.cache_len, 8, 4, 8, shared=True)
    assert sc.shape == (1, 1, 8)
    for blk in sel.candidate_blocks(64, 8, 4, 8):
        per_head = []
        for g in range(4):
            Q = torch.from_numpy(c.q[0, :, 2 * g:2 * g + 2].reshape(-1, 16).astype(np.float64))
            K = torch.from_numpy(c.k[0, g, blk * 8:(blk + 1) * 8].astype(np.float64))
            per_head.append((Q @ K.T).mean().item())
        assert abs(sc[0, 0, blk] - np.mean(per_head)) <= 1e-12


def test_shared_lists_have_one_row_per_sequence():
    c = synth.make_attn_case(6700, B=2, Hq=8, Hkv=2, D=16, L_cap=200, T=1,
                             cache_len=[200, 150], dtype="f32")
    idx, sc, chosen = oracle.select_blocks_ref(c.q, c.k, c.cache_len, block=16, n_sink=4,
                                               window=32, n_select=3, budget=4 + 32 + 48,
                                               shared=True)
    assert idx.shape == (2, 1, 84) and sc.shape[1] == 1
    assert set(chosen) == {(0, 0), (1, 0)}
