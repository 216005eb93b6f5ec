"""Pins for the oracle's draft and verify attention (CPU only).

Every check compares the oracle with something other than itself: PyTorch's
scaled_dot_product_attention in float64 on the CPU (an independent library
routine), hand-enumerated fixtures, closed forms, or a second formulation of
the same input (compacted cache, permuted index list, repeated KV heads).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def sdpa(q_rows, K, V, mask=None, scale=None):
    """torch SDPA on float64 CPU tensors.  q_rows [Hq, T, D], K/V [Hkv, n, D]."""
    q = torch.from_numpy(np.ascontiguousarray(q_rows))[None]
    k = torch.from_numpy(np.ascontiguousarray(K))[None]
    v = torch.from_numpy(np.ascontiguousarray(V))[None]
    m = None if mask is None else torch.from_numpy(mask)
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=scale,
                                       enable_gqa=True)
    return o[0].numpy()


def small_case(seed, B=2, Hq=4, Hkv=2, D=16, L=37, T=1, lens=None, dtype="f32", scale=1.0):
    return synth.make_attn_case(seed, B=B, Hq=Hq, Hkv=Hkv, D=D, L_cap=L, T=T,
                                cache_len=lens, dtype=dtype, value_scale=scale)


# --------------------------------------------------------------- draft

@pytest.mark.parametrize("T", [1, 3])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_window_covering_context_equals_full_attention(T, dtype):
    """A window that covers the whole context is full (causal) attention."""
    c = small_case(11, T=T, lens=[37, 21], dtype=dtype)
    out, lse = oracle.draft_attn_ref(c.q, c.k, c.v, c.cache_len, scale=c.scale,
                                     n_sink=2, window=40)
    for b in range(c.B):
        L = int(c.cache_len[b])
        mask = np.zeros((T, L), dtype=bool)
        for t in range(T):
            mask[t, :L - T + t + 1] = True
        q = oracle.as_f64(c.q[b]).transpose(1, 0, 2)          # [Hq, T, D]
        ref = sdpa(q, oracle.as_f64(c.k[b, :, :L]), oracle.as_f64(c.v[b, :, :L]),
                   mask, c.scale)
        np.testing.assert_allclose(out[b], ref.transpose(1, 0, 2), rtol=0, atol=1e-12)


def test_gather_of_every_position_equals_full_attention():
    c = small_case(12, B=1, lens=[37])
    idx = np.arange(37, dtype=np.int32)[None, None, :]
    out, _ = oracle.draft_attn_ref(c.q, c.k, c.v, c.cache_len, scale=c.scale, idx=idx)
    q = oracle.as_f64(c.q[0]).transpose(1, 0, 2)
    ref = sdpa(q, oracle.as_f64(c.k[0]), oracle.as_f64(c.v[0]), None, c.scale)
    np.testing.assert_allclose(out[0], ref.transpose(1, 0, 2), rtol=0, atol=1e-12)


@pytest.mark.parametrize("T", [1, 3])
def test_padded_gather_of_a_short_sequence_equals_full_attention(T):
    """A fixed-length list for a sequence shorter than the budget: every
    position once, -1 entries scattered in between.  The -1 entries select
    nothing, so the result is full causal attention (SDPA)."""
    c = small_case(15, B=1, lens=[23], T=T, L=37)
    rng = np.random.default_rng(15)
    lst = np.concatenate([np.arange(23), np.full(17, -1)]).astype(np.int32)
    idx = lst[rng.permutation(len(lst))][None, None, :]
    out, _ = oracle.draft_attn_ref(c.q, c.k, c.v, c.cache_len, scale=c.scale, idx=idx)
    mask = np.zeros((T, 23), dtype=bool)
    for t in range(T):
        mask[t, :23 - T + t + 1] = True
    q = oracle.as_f64(c.q[0]).transpose(1, 0, 2)
    ref = sdpa(q, oracle.as_f64(c.k[0, :, :23]), oracle.as_f64(c.v[0, :, :23]), mask, c.scale)
    np.testing.assert_allclose(out[0], ref.transpose(1, 0, 2), rtol=0, atol=1e-12)


def test_window_views_match_hand_enumeration():
    with open(os.path.join(GOLDEN, "draft_window_views.json")) as f:
        fx = json.load(f)
    for case in fx["cases"]:
        for t, want in enumerate(case["views"]):
            got = oracle.draft_view(case["L"], case["n_q"], t, n_sink=case["n_sink"],
                                    window=case["window"])
            assert got.tolist() == want, case


def test_window_view_size_closed_form():
    """One query over a long context sees min(L, n_sink + W) positions; with
    the Windowed-MTP operating point (n_sink 64 + W 4032) at 1M context that
    drops ~99.6% of the cache."""
    for L, s, W in [(1 << 20, 64, 4032), (1 << 20, 4, 4096), (100, 4, 96), (50, 4, 96)]:
        v = oracle.draft_view(L, 1, 0, n_sink=s, window=W)
        assert len(v) == min(L, s + W)
    assert 1 - (64 + 4032) / (1 << 20) > 0.99


def test_gather_equals_window_when_listing_the_window():
    c = small_case(13, lens=[37, 29])
    out_w, lse_w = oracle.draft_attn_ref(c.q, c.k, c.v, c.cache_len, scale=c.scale,
                                         n_sink=3, window=9)
    idx = np.zeros((2, 1, 12), dtype=np.int32)
    idx[0, 0] = np.r_[0:3, 28:37]
    idx[1, 0] = np.r_[0:3, 20:29]
    out_g, lse_g = oracle.draft_attn_ref(c.q, c.k, c.v, c.cache_len, scale=c.scale, idx=idx)
    np.testing.assert_allclose(out_g, out_w, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse_g, lse_w, rtol=0, atol=1e-14)


def test_permuting_budget_list_leaves_result_unchanged():
    c = small_case(14, lens=[37, 37])
    rng = np.random.default_rng(0)
    idx = np.stack([synth.budget_indices(rng, 37, 16) for _ in range(2)])[:, None, :]
    perm = idx[:, :, rng.permutation(16)]
    a = oracle.draft_attn_ref(c.q, c.k, c.v, c.cache_len, scale=c.scale, idx=idx)
    b = oracle.draft_attn_ref(c.q, c.k, c.v, c.cache_len, scale=c.scale, idx=perm)
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-14)


def test_per_head_budget_lists():
    """Hidx = Hkv: each KV head uses its own list; equals running each head
    alone with a shared list."""
    c = small_case(15, lens=[37, 37])
    rng = np.random.default_rng(1)
    idx = np.stack([np.stack([synth.budget_indices(rng, 37, 12) for _ in range(2)])
                    for _ in range(2)])                    # [B, Hkv, 12]
    out, _ = oracle.draft_attn_ref(c.q, c.k, c.v, c.cache_len, scale=c.scale, idx=idx)
    for g in range(2):
        o_g, _ = oracle.draft_attn_ref(c.q, c.k, c.v, c.cache_len, scale=c.scale,
                                       idx=idx[:, g:g + 1], pairs=[(0, g), (1, g)])
        np.testing.assert_allclose(out[:, :, 2 * g:2 * g + 2], o_g[:, :, 2 * g:2 * g + 2],
                                   rtol=0, atol=1e-14)


def test_gqa_equals_mha_with_repeated_heads():
    c = small_case(16, Hq=6, Hkv=2, lens=[37, 25], T=2)
    a = oracle.draft_attn_ref(c.q, c.k, c.v, c.cache_len, scale=c.scale, n_sink=4, window=7)
    k3 = np.repeat(c.k, 3, axis=1)
    v3 = np.repeat(c.v, 3, axis=1)
    b = oracle.draft_attn_ref(c.q, k3, v3, c.cache_len, scale=c.scale, n_sink=4, window=7)
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-14)


def test_softmax_rows_sum_to_one():
    """With every value row equal to 1 the output is the sum of the softmax
    weights, which must be 1."""
    c = small_case(17, lens=[37, 11], T=3)
    ones = np.ones_like(c.v)
    out, _ = oracle.draft_attn_ref(c.q, c.k, ones, c.cache_len, scale=c.scale,
                                   n_sink=2, window=5)
    assert np.abs(out - 1).max() <= 1e-12


def test_lse_closed_forms():
    """One visible key: lse = its score.  Two keys with equal scores:
    lse = score + log 2 and the output is the mean of the two values."""
    q = np.zeros((1, 1, 1, 4)); q[..., 0] = 1.0
    k = np.zeros((1, 1, 3, 4)); k[0, 0, :, 0] = [2.0, 5.0, 2.0]
    v = np.arange(12, dtype=np.float64).reshape(1, 1, 3, 4)
    idx = np.array([[[1]]], dtype=np.int32)
    out, lse = oracle.draft_attn_ref(q, k, v, np.array([3]), scale=0.5, idx=idx)
    assert lse[0, 0, 0] == 2.5 and np.array_equal(out[0, 0, 0], v[0, 0, 1])
    idx = np.array([[[0, 2]]], dtype=np.int32)
    out, lse = oracle.draft_attn_ref(q, k, v, np.array([3]), scale=0.5, idx=idx)
    assert abs(lse[0, 0, 0] - (1.0 + math.log(2))) < 1e-15
    np.testing.assert_allclose(out[0, 0, 0], (v[0, 0, 0] + v[0, 0, 2]) / 2, atol=1e-15)


def test_empty_view_row_is_zero_with_minus_inf_lse():
    """Budget mode with chained queries: the first query sees none of the
    listed positions when they all lie after it."""
    c = small_case(18, B=1, lens=[20], T=2)
    idx = np.array([[[19]]], dtype=np.int32)
    out, lse = oracle.draft_attn_ref(c.q, c.k, c.v, c.cache_len, scale=c.scale, idx=idx)
    assert np.all(out[0, 0] == 0) and np.all(np.isneginf(lse[0, 0]))
    assert np.all(np.isfinite(lse[0, 1]))


@pytest.mark.parametrize("bad", [20, -2])
def test_budget_index_out_of_range_is_an_error(bad):
    """Only -1 is padding; every other position outside [0, L) is an error."""
    c = small_case(19, B=1, lens=[20])
    with pytest.raises(IndexError):
        oracle.draft_attn_ref(c.q, c.k, c.v, c.cache_len, scale=c.scale,
                              idx=np.array([[[3, bad]]], dtype=np.int32))


# --------------------------------------------------------------- tree helpers

@pytest.mark.parametrize("k,levels", [(2, 3), (3, 2), (10, 3), (1, 5), (4, 0)])
def test_full_kary_tree_node_count(k, levels):
    """N = sum_{i=0}^{l} k^i for a full k-ary tree; depth d holds k^d nodes."""
    tree = synth.heap_tree(k, levels)
    depth = oracle.tree_depths(tree.parents)
    n_closed = levels + 1 if k == 1 else (k ** (levels + 1) - 1) // (k - 1)
    assert len(depth) == n_closed == sum(k ** i for i in range(levels + 1))
    for d in range(levels + 1):
        assert int((depth == d).sum()) == k ** d
    np.testing.assert_array_equal(depth, tree.depth)


def test_tiny_workload_tree_is_15_nodes():
    assert synth.heap_tree(2, 3).n == 15


@pytest.mark.parametrize("widths", [(10, 18, 18, 18), (10, 14, 12, 8)])
def test_layered_tree_widths(widths):
    """The 64- and 44-node trees: node count is the sum of the widths and the
    oracle's depths reproduce the builder's levels."""
    tree = synth.layered_tree(np.random.default_rng(3), widths)
    assert tree.n == sum(widths) and tree.n in (64, 44)
    np.testing.assert_array_equal(oracle.tree_depths(tree.parents), tree.depth)


def test_ancestors_of_chain_and_tree():
    anc = oracle.tree_ancestors(np.array([-1, 0, 1, 2]))
    np.testing.assert_array_equal(anc, np.tril(np.ones((4, 4), dtype=bool)))
    anc = oracle.tree_ancestors(np.array([-1, -1, 0, 1, 2]))
    want = {0: [0], 1: [1], 2: [0, 2], 3: [1, 3], 4: [0, 2, 4]}
    for i, js in want.items():
        assert np.nonzero(anc[i])[0].tolist() == js


def test_bad_parent_rejected():
    with pytest.raises(ValueError):
        oracle.tree_depths(np.array([-1, 1]))
    with pytest.raises(ValueError):
        oracle.tree_depths(np.array([-1, -2]))


def test_position_ids_match_hand_enumeration():
    with open(os.path.join(GOLDEN, "position_ids.json")) as f:
        fx = json.load(f)
    for case in fx["cases"]:
        got = oracle.position_ids(np.array(case["cache_len"]), np.array(case["pad"], np.uint8),
                                  np.array(case["parents"]))
        assert got.tolist() == case["pos_ids"]


# --------------------------------------------------------------- verify

def _tree_inputs(seed, B, N, Hq=4, Hkv=2, D=16, L=29, lens=None, dtype="f32", scale=1.0):
    c = small_case(seed, B=B, Hq=Hq, Hkv=Hkv, D=D, L=L, T=N, lens=lens, dtype=dtype, scale=scale)
    rng = c.extra["rng"]
    tk = synth.draw_normal(rng, (B, Hkv, N, D), scale, dtype)
    tv = synth.draw_normal(rng, (B, Hkv, N, D), scale, dtype)
    return c, tk, tv


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chain_equals_causal_attention(dtype):
    """A chain of speculated tokens over the cache is causal attention over
    [cache; chain]."""
    N = 5
    c, tk, tv = _tree_inputs(21, B=2, N=N, lens=[29, 17], dtype=dtype)
    par = synth.chain_tree(N).parents
    out, lse = oracle.verify_attn_ref(c.q, c.k, c.v, c.cache_len, tk, tv, par, scale=c.scale)
    for b in range(2):
        L = int(c.cache_len[b])
        K = np.concatenate([oracle.as_f64(c.k[b, :, :L]), oracle.as_f64(tk[b])], axis=1)
        V = np.concatenate([oracle.as_f64(c.v[b, :, :L]), oracle.as_f64(tv[b])], axis=1)
        mask = np.ones((N, L + N), dtype=bool)
        mask[:, L:] = np.tril(np.ones((N, N), dtype=bool))
        ref = sdpa(oracle.as_f64(c.q[b]).transpose(1, 0, 2), K, V, mask, c.scale)
        np.testing.assert_allclose(out[b], ref.transpose(1, 0, 2), rtol=0, atol=1e-12)


def test_tree_equals_per_path_causal_attention():
    """Every root-to-leaf path of the tree, run as causal attention over
    [cache; path], reproduces the tree outputs of the nodes on that path."""
    tree = synth.heap_tree(2, 3)
    N = tree.n
    c, tk, tv = _tree_inputs(22, B=1, N=N, lens=[29])
    out, _ = oracle.verify_attn_ref(c.q, c.k, c.v, c.cache_len, tk, tv, tree.parents,
                                    scale=c.scale)
    leaves = [i for i in range(N) if i not in set(tree.parents.tolist())]
    assert len(leaves) == 8
    for leaf in leaves:
        path = []
        j = leaf
        while j >= 0:
            path.append(j)
            j = int(tree.parents[j])
        path.reverse()
        K = np.concatenate([oracle.as_f64(c.k[0]), oracle.as_f64(tk[0][:, path])], axis=1)
        V = np.concatenate([oracle.as_f64(c.v[0]), oracle.as_f64(tv[0][:, path])], axis=1)
        P = len(path)
        mask = np.ones((P, 29 + P), dtype=bool)
        mask[:, 29:] = np.tril(np.ones((P, P), dtype=bool))
        qp = oracle.as_f64(c.q[0][path]).transpose(1, 0, 2)
        ref = sdpa(qp, K, V, mask, c.scale).transpose(1, 0, 2)
        np.testing.assert_allclose(out[0, path], ref, rtol=0, atol=1e-12)


def test_padding_equals_compacted_cache():
    """Masking pad slots with -inf equals deleting them, and the remapped
    positions equal the compacted sequence's positions."""
    rng = np.random.default_rng(5)
    tree = synth.layered_tree(rng, (3, 4, 2))
    N = tree.n
    lens = np.array([29, 23])
    c, tk, tv = _tree_inputs(23, B=2, N=N, lens=lens, dtype="bf16")
    pad = np.zeros((2, 29), dtype=np.uint8)
    pad[0, :29] = synth.pad_groups(rng, 29, n_groups=4, group=5)
    pad[1, :23] = synth.pad_groups(rng, 23, n_groups=3, group=5)
    pad[1, 2] = 1
    assert pad.sum() > 0
    out, lse = oracle.verify_attn_ref(c.q, c.k, c.v, c.cache_len, tk, tv, tree.parents,
                                      scale=c.scale, pad=pad)
    pos = oracle.position_ids(lens, pad, tree.parents)
    for b in range(2):
        keep = np.nonzero(pad[b, :lens[b]] == 0)[0]
        kc = np.zeros_like(c.k[b:b + 1])
        vc = np.zeros_like(c.v[b:b + 1])
        kc[:, :, :len(keep)] = c.k[b:b + 1][:, :, keep]
        vc[:, :, :len(keep)] = c.v[b:b + 1][:, :, keep]
        o2, l2 = oracle.verify_attn_ref(c.q[b:b + 1], kc, vc, np.array([len(keep)]),
                                        tk[b:b + 1], tv[b:b + 1], tree.parents, scale=c.scale)
        np.testing.assert_allclose(out[b], o2[0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[b], l2[0], rtol=0, atol=1e-13)
        np.testing.assert_array_equal(pos[b], len(keep) + tree.depth)


def test_verify_rows_sum_to_one_and_per_sequence_parents():
    rng = np.random.default_rng(6)
    N = 7
    c, tk, tv = _tree_inputs(24, B=2, N=N, lens=[29, 5])
    par = np.stack([synth.layered_tree(rng, (2, 3, 2)).parents,
                    synth.chain_tree(N).parents])
    ones = np.ones_like(c.v)
    out, _ = oracle.verify_attn_ref(c.q, c.k, ones, c.cache_len, tk, np.ones_like(tv), par,
                                    scale=c.scale)
    assert np.abs(out - 1).max() <= 1e-12
    o_shared, _ = oracle.verify_attn_ref(c.q[1:], c.k[1:], c.v[1:], c.cache_len[1:], tk[1:],
                                         tv[1:], par[1], scale=c.scale)
    o_batched, _ = oracle.verify_attn_ref(c.q, c.k, c.v, c.cache_len, tk, tv, par,
                                          scale=c.scale)
    np.testing.assert_allclose(o_batched[1], o_shared[0], rtol=0, atol=1e-14)


def test_verify_with_empty_cache_sees_only_its_path():
    """cache_len = 0: node i attends to its root path only (the row always
    contains itself, so no row is empty)."""
    N = 4
    c, tk, tv = _tree_inputs(25, B=1, N=N, lens=[0])
    par = synth.chain_tree(N).parents
    out, lse = oracle.verify_attn_ref(c.q, c.k, c.v, c.cache_len, tk, tv, par, scale=c.scale)
    assert np.all(np.isfinite(lse))
    mask = np.tril(np.ones((N, N), dtype=bool))
    ref = sdpa(oracle.as_f64(c.q[0]).transpose(1, 0, 2), oracle.as_f64(tk[0]),
               oracle.as_f64(tv[0]), mask, c.scale)
    np.testing.assert_allclose(out[0], ref.transpose(1, 0, 2), rtol=0, atol=1e-12)


def test_plant_bug_in_mask_is_caught():
    """A plausible oracle mistake (a node that also sees its siblings) would
    fail the per-path pin: check that the pin's reference differs from such a
    variant on this input."""
    tree = synth.heap_tree(2, 2)
    c, tk, tv = _tree_inputs(26, B=1, N=tree.n, lens=[9])
    out, _ = oracle.verify_attn_ref(c.q, c.k, c.v, c.cache_len, tk, tv, tree.parents,
                                    scale=c.scale)
    wrong_par = synth.chain_tree(tree.n).parents     # every earlier node visible
    bad, _ = oracle.verify_attn_ref(c.q, c.k, c.v, c.cache_len, tk, tv, wrong_par,
                                    scale=c.scale)
    assert np.abs(out - bad).max() > 1e-3
