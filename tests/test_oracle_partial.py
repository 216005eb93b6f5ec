"""Pins for the oracle's partial verification (CPU only).

Pinned against: a marked cache (each key names its own position) for the
gather; the full-cache verify oracle when the list names every position;
torch SDPA over the listed positions plus the node's root path on the
original cache; invariance to the order of the list; a KV commit into the
partial cache followed by the next verify; and the hand-enumerated
full/partial schedule of SpecPV section 3.3 (golden/verify_mode_specpv.json).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import partial as po
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_gather_of_a_marked_cache():
    B, Hkv, L, D = 2, 3, 40, 4
    k = np.zeros((B, Hkv, L, D), dtype=np.float32) + np.arange(L, dtype=np.float32)[None, None, :, None]
    idx = np.array([[[0, 5, 6, -1, 39, -1]], [[3, -1, 30, 2, -1, -1]]], dtype=np.int32)
    pk, pv, pad, length, err = oracle.gather_ref(k, -k, [40, 30], idx, capacity=8)
    assert err == po.ERR_INDEX                        # 30 = cache_len: one past the end
    np.testing.assert_array_equal(length, [6, 6])
    np.testing.assert_array_equal(pad, [[0, 0, 0, 1, 0, 1, 0, 0], [0, 1, 1, 0, 1, 1, 0, 0]])
    np.testing.assert_array_equal(pk[0, :, :, 0], [[0, 5, 6, 0, 39, 0, 0, 0]] * 3)
    np.testing.assert_array_equal(pk[1, :, :, 0], [[3, 0, 0, 2, 0, 0, 0, 0]] * 3)
    np.testing.assert_array_equal(pv, -pk)
    with pytest.raises(ValueError):
        oracle.gather_ref(k, k, [40, 30], np.zeros((2, 3, 4), np.int32), capacity=8)


def tree_case(seed, *, B=2, L=60, widths=(2, 3, 2)):
    rng = np.random.default_rng(seed)
    tree = synth.layered_tree(rng, widths)
    c = synth.make_attn_case(seed, B=B, Hq=4, Hkv=2, D=16, L_cap=L, T=1,
                             cache_len=[L, L - 17], dtype="f32")
    q = synth.draw_normal(rng, (B, tree.n, 4, 16), 1.0, "f32")
    tk = synth.draw_normal(rng, (B, 2, tree.n, 16), 1.0, "f32")
    tv = synth.draw_normal(rng, (B, 2, tree.n, 16), 1.0, "f32")
    return c, tree, q, tk, tv, rng


def partial_verify(c, tree, q, tk, tv, idx, cap):
    pk, pv, pad, length, err = oracle.gather_ref(c.k, c.v, c.cache_len, idx, cap)
    assert err == 0
    return oracle.verify_attn_ref(q, pk, pv, length, tk, tv, tree.parents, scale=c.scale, pad=pad)


def test_list_of_every_position_gives_the_full_verify():
    c, tree, q, tk, tv, _ = tree_case(7700)
    idx = np.full((2, 1, 64), -1, dtype=np.int32)
    for b in range(2):
        L = int(c.cache_len[b])
        idx[b, 0, :L] = np.arange(L)
    got, lse = partial_verify(c, tree, q, tk, tv, idx, 64)
    want, lse_w = oracle.verify_attn_ref(q, c.k, c.v, c.cache_len, tk, tv, tree.parents,
                                         scale=c.scale)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse_w, rtol=0, atol=1e-13)


@pytest.mark.parametrize("seed", range(3))
def test_partial_verify_is_sdpa_over_the_listed_positions_and_the_path(seed):
    c, tree, q, tk, tv, rng = tree_case(7800 + seed)
    idx = np.full((2, 1, 40), -1, dtype=np.int32)
    for b in range(2):
        L = int(c.cache_len[b])
        lst = np.sort(rng.choice(L, 25, replace=False))
        slots = np.sort(rng.choice(40, 25, replace=False))
        idx[b, 0, slots] = lst
    got, _ = partial_verify(c, tree, q, tk, tv, idx, 48)
    anc = oracle.tree_ancestors(tree.parents)
    for b in range(2):
        L = int(c.cache_len[b])
        listed = np.zeros(L, dtype=bool)
        listed[idx[b, 0][idx[b, 0] >= 0]] = True
        for i in range(tree.n):
            for g in range(2):
                K = np.concatenate([c.k[b, g, :L], tk[b, g]]).astype(np.float64)
                V = np.concatenate([c.v[b, g, :L], tv[b, g]]).astype(np.float64)
                mask = np.concatenate([listed, anc[i]])
                qq = torch.from_numpy(q[b, i, 2 * g:2 * g + 2].astype(np.float64))[None, :, None]
                o = torch.nn.functional.scaled_dot_product_attention(
                    qq, torch.from_numpy(K)[None, None], torch.from_numpy(V)[None, None],
                    attn_mask=torch.from_numpy(mask)[None, None, None], scale=c.scale)
                np.testing.assert_allclose(got[b, i, 2 * g:2 * g + 2], o[0, :, 0].numpy(),
                                           rtol=0, atol=1e-12)


def test_order_of_the_list_does_not_change_the_verify():
    c, tree, q, tk, tv, rng = tree_case(7900)
    idx = np.full((2, 1, 30), -1, dtype=np.int32)
    for b in range(2):
        idx[b, 0, :20] = np.sort(rng.choice(int(c.cache_len[b]), 20, replace=False))
    perm = idx[:, :, rng.permutation(30)]
    a, _ = partial_verify(c, tree, q, tk, tv, idx, 32)
    b2, _ = partial_verify(c, tree, q, tk, tv, perm, 32)
    np.testing.assert_allclose(a, b2, rtol=0, atol=1e-13)


def test_buffer_commit_then_verify():
    """Accepted tokens go into the partial cache's buffer through the KV
    commit; the next partial verify sees the listed positions, the committed
    path and its own ancestors."""
    c, tree, q, tk, tv, rng = tree_case(8000)
    idx = np.full((2, 1, 30), -1, dtype=np.int32)
    for b in range(2):
        idx[b, 0, :22] = np.sort(rng.choice(int(c.cache_len[b]), 22, replace=False))
    pk, pv, pad, length, _ = oracle.gather_ref(c.k, c.v, c.cache_len, idx, 48)
    alen = np.array([2, 1])
    node2 = [j for j in range(tree.n) if tree.parents[j] >= 0][0]
    apath = np.array([[tree.parents[node2], node2], [0, -1]], dtype=np.int32)
    pk2, pv2, len2, pad2, P, err = oracle.commit_ref(pk, pv, length, pad, tk, tv, alen, apath, 2)
    assert err == 0 and P == 3
    q2 = synth.draw_normal(rng, (2, tree.n, 4, 16), 1.0, "f32")
    got, _ = oracle.verify_attn_ref(q2, pk2, pv2, len2, tk, tv, tree.parents, scale=c.scale,
                                    pad=pad2)
    anc = oracle.tree_ancestors(tree.parents)
    for b in range(2):
        # listed positions, the committed path, then the bonus token's slot,
        # which the commit keeps valid and the caller's next forward pass
        # fills (here it still holds the gather's zeros)
        zero = np.zeros((2, 16), dtype=np.float32)
        keys = [c.k[b, :, p] for p in idx[b, 0] if p >= 0] + \
            [tk[b, :, n] for n in apath[b, :alen[b]]] + [zero]
        vals = [c.v[b, :, p] for p in idx[b, 0] if p >= 0] + \
            [tv[b, :, n] for n in apath[b, :alen[b]]] + [zero]
        for i in (0, tree.n - 1):
            kk = np.stack(keys + [tk[b, :, j] for j in np.nonzero(anc[i])[0]], axis=1)
            vv = np.stack(vals + [tv[b, :, j] for j in np.nonzero(anc[i])[0]], axis=1)
            for g in range(2):
                qq = torch.from_numpy(q2[b, i, 2 * g:2 * g + 2].astype(np.float64))[None, :, None]
                o = torch.nn.functional.scaled_dot_product_attention(
                    qq, torch.from_numpy(kk[g].astype(np.float64))[None, None],
                    torch.from_numpy(vv[g].astype(np.float64))[None, None], scale=c.scale)
                np.testing.assert_allclose(got[b, i, 2 * g:2 * g + 2], o[0, :, 0].numpy(),
                                           rtol=0, atol=1e-12)


def test_full_or_partial_schedule_matches_the_hand_table():
    with open(os.path.join(GOLDEN, "verify_mode_specpv.json")) as f:
        fx = json.load(f)
    for case in fx["cases"]:
        *args, mode = case
        assert oracle.verify_mode_ref(*args) == mode, case
