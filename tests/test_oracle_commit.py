"""Pins for the oracle's KV commit of the accepted path (CPU only).

Pinned against: the hand-enumerated toy batch of SpecMemo's Figure 9
(``golden/kv_commit_figure9.json``); library attention (torch SDPA in fp64)
over the committed cache, which must reproduce the oracle's tree-verify
output of the deepest accepted node; the position remap of the next step;
and invariants of the compacted (pad-free) sequence.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fixture():
    with open(os.path.join(GOLDEN, "kv_commit_figure9.json")) as f:
        return json.load(f)


def _marked_cache(B, Hkv, cap, D):
    """K/V whose every element names its own (b, h, slot): value = slot."""
    k = np.zeros((B, Hkv, cap, D), dtype=np.float32)
    k += np.arange(cap, dtype=np.float32)[None, None, :, None]
    return k, -k


def test_figure9_batch():
    d = _fixture()
    B, cap, N = len(d["cache_len"]), d["capacity"], d["n_nodes"]
    k, v = _marked_cache(B, 2, cap, 4)
    # tree node n carries the value 1000 + n, so a committed slot names its node
    tk = np.zeros((B, 2, N, 4), dtype=np.float32) + (1000 + np.arange(N))[None, None, :, None]
    pad = np.zeros((B, cap), dtype=np.uint8)
    k2, v2, cl2, pad2, P, err = oracle.commit_ref(
        k, v, d["cache_len"], pad, tk, -tk, np.array(d["accept_len"]),
        np.array(d["accept_path"]), d["max_depth"])
    assert err == 0
    assert P == d["expected_P"]
    np.testing.assert_array_equal(cl2, d["expected_cache_len"])
    np.testing.assert_array_equal(pad2, np.array(d["expected_pad"], dtype=np.uint8))
    # pads appended per sequence = P - (accept_len + 1)
    for b in range(B):
        L = d["cache_len"][b]
        assert int(pad2[b, L:L + P].sum()) == d["expected_pad_counts"][b]
    node = np.where(k2[:, 0, :, 0] >= 1000, k2[:, 0, :, 0] - 1000, -1).astype(int)
    np.testing.assert_array_equal(node, np.array(d["expected_slot_node"]))
    np.testing.assert_array_equal(v2, -k2)


def _sdpa_over_cache(q, K, V, pad_row, length, scale):
    """torch SDPA in fp64 of queries q [G, D] over cache slots [0, length)
    whose pad byte is 0."""
    keep = np.nonzero(pad_row[:length] == 0)[0]
    qt = torch.from_numpy(q)[None, :, None, :].transpose(1, 2)           # [1, 1, G, D]
    kt = torch.from_numpy(K[keep])[None, None]                          # [1, 1, n, D]
    vt = torch.from_numpy(V[keep])[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return o[0, 0].numpy()


@pytest.mark.parametrize("seed", range(6))
def test_attention_over_committed_cache_equals_verify_of_deepest_node(seed):
    """Committing the accepted path and then attending over the cache (up to
    the bonus slot, which holds no key yet) gives the same result as the
    tree-verify attention of the deepest accepted node, whose keys are the
    cache plus its ancestors and itself."""
    rng = np.random.default_rng(7100 + seed)
    B, Hq, Hkv, D, cap = 3, 4, 2, 16, 96
    tree = synth.layered_tree(rng, (3, 3, 2))
    N = tree.n
    lens = rng.integers(20, 60, size=B).astype(np.int32)
    pad = np.zeros((B, cap), dtype=np.uint8)
    for b in range(B):
        pad[b, :lens[b]] = synth.pad_groups(rng, int(lens[b]), n_groups=4)
    k = rng.standard_normal((B, Hkv, cap, D))
    v = rng.standard_normal((B, Hkv, cap, D))
    tk = rng.standard_normal((B, Hkv, N, D))
    tv = rng.standard_normal((B, Hkv, N, D))
    q = rng.standard_normal((B, N, Hq, D))
    acc = synth.make_accept_case(7200 + seed, tree, B, 32, depths=[1, 2, 3])
    alen, apath, _ = oracle.accept_ref(acc.logits, acc.tokens, tree.parents, acc.max_depth)
    scale = 1 / math.sqrt(D)
    ref, _ = oracle.verify_attn_ref(q, k, v, lens, tk, tv, tree.parents, scale=scale, pad=pad)
    k2, v2, cl2, pad2, P, err = oracle.commit_ref(k, v, lens, pad, tk, tv, alen, apath,
                                                  acc.max_depth)
    assert err == 0 and P == 1 + int(alen.max())
    G = Hq // Hkv
    for b in range(B):
        tau = int(alen[b])
        assert tau >= 1
        deepest = int(apath[b, tau - 1])
        for g in range(Hkv):
            got = _sdpa_over_cache(q[b, deepest, g * G:(g + 1) * G], k2[b, g], v2[b, g],
                                   pad2[b], int(lens[b]) + tau, scale)
            np.testing.assert_allclose(got, ref[b, deepest, g * G:(g + 1) * G],
                                       rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_compacted_sequence_grows_by_path_and_bonus(seed):
    """Dropping pad slots, the committed sequence is the old one followed by
    the accepted nodes in path order and the bonus slot; slots outside the
    appended range keep their contents; every sequence grows by P."""
    rng = np.random.default_rng(7300 + seed)
    B, Hkv, D, cap = 5, 2, 8, 80
    tree = synth.layered_tree(rng, (2, 3, 3, 2))
    N = tree.n
    lens = rng.integers(10, 50, size=B).astype(np.int32)
    pad = np.zeros((B, cap), dtype=np.uint8)
    for b in range(B):
        pad[b, :lens[b]] = synth.pad_groups(rng, int(lens[b]), n_groups=3)
    k = rng.standard_normal((B, Hkv, cap, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, cap, D)).astype(np.float32)
    tk = rng.standard_normal((B, Hkv, N, D)).astype(np.float32)
    tv = rng.standard_normal((B, Hkv, N, D)).astype(np.float32)
    acc = synth.make_accept_case(7400 + seed, tree, B, 16)
    alen, apath, _ = oracle.accept_ref(acc.logits, acc.tokens, tree.parents, acc.max_depth)
    k2, v2, cl2, pad2, P, err = oracle.commit_ref(k, v, lens, pad, tk, tv, alen, apath,
                                                  acc.max_depth)
    assert err == 0
    assert P == 1 + int(alen.max())
    np.testing.assert_array_equal(cl2, lens + P)
    for b in range(B):
        L, tau = int(lens[b]), int(alen[b])
        old = np.nonzero(pad[b, :L] == 0)[0]
        new = np.nonzero(pad2[b, :L + P] == 0)[0]
        # old valid slots, then L .. L + tau (path + bonus)
        np.testing.assert_array_equal(new, np.concatenate([old, np.arange(L, L + tau + 1)]))
        for j in range(tau):
            np.testing.assert_array_equal(k2[b, :, L + j], tk[b, :, apath[b, j]])
            np.testing.assert_array_equal(v2[b, :, L + j], tv[b, :, apath[b, j]])
        # parents chain: the committed nodes form a root path
        for j in range(tau):
            assert tree.parents[apath[b, j]] == (apath[b, j - 1] if j else -1)
        untouched = np.ones(cap, dtype=bool)
        untouched[L:L + tau] = False
        np.testing.assert_array_equal(k2[b][:, untouched], k[b][:, untouched])
        np.testing.assert_array_equal(v2[b][:, untouched], v[b][:, untouched])
        np.testing.assert_array_equal(pad2[b, :L], pad[b, :L])
        np.testing.assert_array_equal(pad2[b, L + P:], pad[b, L + P:])


def test_next_positions_follow_the_bonus_token():
    """Position remap of the next step: the next tree's depth-0 nodes sit
    right after the bonus token, i.e. at (valid tokens before) + tau + 1,
    whatever padding the commit appended."""
    rng = np.random.default_rng(7500)
    B, cap = 4, 64
    lens = np.array([10, 17, 30, 22], dtype=np.int32)
    pad = np.zeros((B, cap), dtype=np.uint8)
    for b in range(B):
        pad[b, :lens[b]] = synth.pad_groups(rng, int(lens[b]), n_groups=2)
    alen = np.array([0, 3, 1, 2])
    apath = np.array([[-1, -1, -1], [0, 1, 2], [1, -1, -1], [0, 1, -1]])
    z = np.zeros((B, 1, cap, 2), dtype=np.float32)
    zt = np.zeros((B, 1, 3, 2), dtype=np.float32)
    _, _, cl2, pad2, P, err = oracle.commit_ref(z, z, lens, pad, zt, zt, alen, apath, 3)
    assert err == 0 and P == 4
    nxt = oracle.position_ids(cl2, pad2, np.array([-1, -1, 0]))
    before = oracle.position_ids(lens, pad, np.array([-1]))[:, 0]
    np.testing.assert_array_equal(nxt[:, 0], before + alen + 1)
    np.testing.assert_array_equal(nxt[:, 2], before + alen + 2)


def test_bad_accept_results_append_padding_only():
    z = np.zeros((3, 1, 16, 2), dtype=np.float32)
    tk = np.ones((3, 1, 4, 2), dtype=np.float32)
    lens = np.array([2, 3, 4])
    pad = np.zeros((3, 16), dtype=np.uint8)
    alen = np.array([5, 1, 2])                       # 5 > max_depth 3
    apath = np.array([[0, 1, 2], [7, -1, -1], [0, 1, -1]])   # node 7 >= N = 4
    k2, _, cl2, pad2, P, err = oracle.commit_ref(z, z, lens, pad, tk, tk, alen, apath, 3)
    assert err == oracle.commit.ERR_COMMIT
    assert P == 3                                    # only sequence 2 counts
    np.testing.assert_array_equal(cl2, lens + 3)
    np.testing.assert_array_equal(pad2[0, 2:5], [1, 1, 1])
    np.testing.assert_array_equal(pad2[1, 3:6], [1, 1, 1])
    np.testing.assert_array_equal(pad2[2, 4:7], [0, 0, 0])
    assert not k2[0].any() and not k2[1].any()
    assert k2[2, 0, 4:6].all() and not k2[2, 0, 6].any()


def test_accept_length_beyond_the_node_count_is_invalid():
    z = np.zeros((1, 1, 16, 2), dtype=np.float32)
    tk = np.ones((1, 1, 2, 2), dtype=np.float32)
    _, _, cl2, pad2, P, err = oracle.commit_ref(z, z, [4], np.zeros((1, 16), np.uint8), tk, tk,
                                                [3], [[0, 1, 1]], 5)
    assert err == oracle.commit.ERR_COMMIT and P == 1
    np.testing.assert_array_equal(cl2, [5])
    assert pad2[0, 4] == 1


def test_cache_overflow_leaves_the_sequence_alone():
    z = np.zeros((2, 1, 8, 2), dtype=np.float32)
    tk = np.ones((2, 1, 3, 2), dtype=np.float32)
    lens = np.array([3, 6])
    pad = np.zeros((2, 8), dtype=np.uint8)
    k2, _, cl2, pad2, P, err = oracle.commit_ref(z, z, lens, pad, tk, tk, np.array([1, 2]),
                                                 np.array([[0, -1], [0, 1]]), 2)
    assert P == 3 and err == oracle.commit.ERR_CACHE_LEN
    np.testing.assert_array_equal(cl2, [6, 6])       # 6 + 3 > 8: unchanged
    assert not k2[1].any() and not pad2[1].any()
    assert k2[0, 0, 3].all()


def test_in_place_commit_order_is_safe():
    """The GPU commit reads a group of up to 8 path rows, then writes them,
    group after group, with the tree rows aliasing the cache slots just past
    cache_len.  Since path[j] >= j, no write lands on a row a later group
    still reads: simulated here on an aliased buffer, the result equals the
    oracle's copy from separate tree rows."""
    rng = np.random.default_rng(7600)
    for trial in range(50):
        n = int(rng.integers(1, 40))
        par = np.array([-1] + [int(rng.integers(-1, i)) for i in range(1, n)], dtype=np.int32)
        depth = oracle.tree_depths(par)
        end = int(rng.integers(0, n))
        path = []
        j = end
        while j >= 0:
            path.append(j)
            j = int(par[j])
        path.reverse()
        tau, L, cap = len(path), 5, 5 + n + 3
        buf = rng.standard_normal((1, 1, cap, 3))
        tree = buf[:, :, L:L + n].copy()
        want, _, _, _, _, _ = oracle.commit_ref(buf, buf, [L], np.zeros((1, cap), np.uint8),
                                                tree, tree, [tau], [path], n)
        got = buf.copy()
        for g0 in range(0, tau, 8):
            rows = [got[0, 0, L + path[j]].copy() for j in range(g0, min(tau, g0 + 8))]
            for i, r in enumerate(rows):
                got[0, 0, L + g0 + i] = r
        np.testing.assert_array_equal(got, want)
        assert all(path[j] >= j for j in range(tau)) and depth[end] + 1 == tau


# ------------------------------------------------------------ compaction of pad slots

def _golden_compact():
    with open(os.path.join(os.path.dirname(__file__), "golden", "kv_compact.json")) as f:
        return json.load(f)


def _check_compact_golden(fn):
    """True iff `fn` (a compaction with the oracle's signature) reproduces the
    hand-enumerated fixture."""
    g = _golden_compact()
    B, cap = len(g["cache_len"]), g["capacity"]
    slot = np.broadcast_to(np.arange(cap, dtype=np.float64)[None, None, :, None], (B, 2, cap, 4))
    k2, v2, cl2, pad2, err = fn(slot, -slot, np.array(g["cache_len"]), np.array(g["pad"], np.uint8))
    if err != 0 or list(cl2) != g["expected_cache_len"]:
        return False
    for b in range(B):
        n, L = g["expected_cache_len"][b], g["cache_len"][b]
        src = np.array(g["expected_slot_source"][b], dtype=np.float64)
        if not (np.array_equal(k2[b, :, :n, :], np.broadcast_to(src[None, :, None], (2, n, 4))) and
                np.array_equal(v2[b, :, :n, :], -k2[b, :, :n, :]) and not pad2[b, :L].any()):
            return False
    return True


def test_compact_golden():
    assert _check_compact_golden(oracle.compact_ref)


def test_compact_planted_mistakes_fail_the_golden_case():
    """Two plausible mistakes: a range that stops one slot short (the last
    cached slot is never kept), and ignoring the pad bytes."""
    def range_one_short(k, v, cache_len, pad):
        return oracle.compact_ref(k, v, np.maximum(np.asarray(cache_len) - 1, 0), pad)

    def keeps_pads(k, v, cache_len, pad):
        return oracle.compact_ref(k, v, cache_len, np.zeros_like(pad))

    assert not _check_compact_golden(range_one_short)
    assert not _check_compact_golden(keeps_pads)


@pytest.mark.parametrize("seed", range(5))
def test_attention_over_compacted_cache_needs_no_mask(seed):
    """After compaction, plain attention (no mask) over the first cache_len
    slots equals attention over the padded cache with its pad slots masked;
    the oracle's tree verify over the compacted cache without pads equals its
    verify over the padded cache; the position remap is unchanged."""
    rng = np.random.default_rng(7600 + seed)
    B, Hq, Hkv, D, cap = 3, 4, 2, 16, 120
    lens = rng.integers(0, cap + 1, size=B).astype(np.int32)
    lens[0] = cap
    pad = (rng.random((B, cap)) < 0.3).astype(np.uint8)
    for b in range(B):
        pad[b, lens[b]:] = rng.integers(0, 2, size=cap - lens[b])   # bytes past cache_len ignored
    k = rng.standard_normal((B, Hkv, cap, D))
    v = rng.standard_normal((B, Hkv, cap, D))
    k2, v2, cl2, pad2, err = oracle.compact_ref(k, v, lens, pad)
    assert err == 0
    scale = 1 / math.sqrt(D)
    G = Hq // Hkv
    q = rng.standard_normal((B, Hq, D))
    for b in range(B):
        n = int(cl2[b])
        assert n == int((pad[b, :lens[b]] == 0).sum())
        assert not pad2[b, :lens[b]].any()
        for g in range(Hkv):
            if n == 0:
                continue
            masked = _sdpa_over_cache(q[b, g * G:(g + 1) * G], k[b, g], v[b, g], pad[b],
                                      int(lens[b]), scale)
            qt = torch.from_numpy(q[b, g * G:(g + 1) * G])[None, None]
            plain = torch.nn.functional.scaled_dot_product_attention(
                qt, torch.from_numpy(k2[b, g, :n])[None, None],
                torch.from_numpy(v2[b, g, :n])[None, None], scale=scale)[0, 0].numpy()
            np.testing.assert_allclose(plain, masked, rtol=0, atol=1e-12)
    tree = synth.layered_tree(rng, (2, 3))
    N = tree.n
    tk = rng.standard_normal((B, Hkv, N, D))
    tv = rng.standard_normal((B, Hkv, N, D))
    qv = rng.standard_normal((B, N, Hq, D))
    ref, lse = oracle.verify_attn_ref(qv, k, v, lens, tk, tv, tree.parents, scale=scale, pad=pad)
    got, lse2 = oracle.verify_attn_ref(qv, k2, v2, cl2, tk, tv, tree.parents, scale=scale,
                                       pad=np.zeros_like(pad))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(oracle.position_ids(cl2, np.zeros_like(pad), tree.parents),
                                  oracle.position_ids(lens, pad, tree.parents))


def test_compact_is_idempotent_and_leaves_unpadded_caches_alone():
    rng = np.random.default_rng(7700)
    B, Hkv, D, cap = 4, 2, 8, 50
    lens = np.array([50, 17, 0, 33], dtype=np.int32)
    pad = (rng.random((B, cap)) < 0.2).astype(np.uint8)
    pad[1] = 0
    k = rng.standard_normal((B, Hkv, cap, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, cap, D)).astype(np.float32)
    k1, v1, cl1, p1, e1 = oracle.compact_ref(k, v, lens, pad)
    k2, v2, cl2, p2, e2 = oracle.compact_ref(k1, v1, cl1, p1)
    assert e1 == e2 == 0
    np.testing.assert_array_equal(cl1, cl2)
    np.testing.assert_array_equal(k1, k2)
    np.testing.assert_array_equal(v1, v2)
    np.testing.assert_array_equal(k1[1], k[1])      # no pads: nothing moves
    assert cl1[1] == 17 and cl1[2] == 0


def test_compact_bad_cache_length_leaves_the_sequence_alone():
    rng = np.random.default_rng(7800)
    B, Hkv, D, cap = 3, 1, 4, 10
    lens = np.array([11, -1, 6], dtype=np.int32)
    pad = np.ones((B, cap), dtype=np.uint8)
    k = rng.standard_normal((B, Hkv, cap, D))
    k2, v2, cl2, pad2, err = oracle.compact_ref(k, k, lens, pad)
    assert err == 1
    np.testing.assert_array_equal(cl2, [11, -1, 0])
    np.testing.assert_array_equal(k2[:2], k[:2])
    np.testing.assert_array_equal(pad2[:2], pad[:2])
    assert not pad2[2, :6].any() and pad2[2, 6:].all()
