"""Pins for the oracle's greedy tree acceptance (CPU only).

Pinned against: brute-force path enumeration, values fixed by construction
(planted accepted depths), textbook greedy speculative decoding on chains,
numpy.argmax's first-occurrence and NaN rules, and a hand-enumerated batch.
"""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def random_parents(draw_ints, n):
    return np.array([-1] + [draw_ints(-1, i - 1) for i in range(1, n)], dtype=np.int32)


@st.composite
def small_trees(draw):
    n = draw(st.integers(1, 15))
    par = [-1] + [draw(st.integers(-1, i - 1)) for i in range(1, n)]
    V = draw(st.integers(1, 16))
    B = draw(st.integers(1, 3))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    return np.array(par, dtype=np.int32), V, B, seed


@settings(max_examples=300, deadline=None)
@given(small_trees())
def test_accept_equals_bruteforce_on_small_trees(args):
    """Every tree with N <= 15 nodes and V <= 16 tokens: the oracle's flag
    propagation equals exhaustive path enumeration.  Logits are small integers
    so that ties are frequent; tokens are unconstrained (siblings may share a
    token), which exercises the deepest-then-lowest-index rule."""
    par, V, B, seed = args
    rng = np.random.default_rng(seed)
    N = len(par)
    logits = rng.integers(0, 3, size=(B, N + 1, V)).astype(np.float32)
    tokens = rng.integers(0, V, size=(B, N)).astype(np.int32)
    maxd = int(oracle.tree_depths(par).max()) + 1
    got = oracle.accept_ref(logits, tokens, par, maxd)
    want = oracle.accept_bruteforce(logits, tokens, par, maxd)
    for g, w in zip(got, want):
        np.testing.assert_array_equal(g, w)


@settings(max_examples=100, deadline=None)
@given(small_trees())
def test_accept_with_nan_rows_equals_bruteforce(args):
    par, V, B, seed = args
    rng = np.random.default_rng(seed)
    N = len(par)
    logits = rng.standard_normal(size=(B, N + 1, V)).astype(np.float32)
    logits[rng.random(size=logits.shape) < 0.1] = np.nan
    tokens = rng.integers(0, V, size=(B, N)).astype(np.int32)
    maxd = int(oracle.tree_depths(par).max()) + 1
    got = oracle.accept_ref(logits, tokens, par, maxd)
    want = oracle.accept_bruteforce(logits, tokens, par, maxd)
    for g, w in zip(got, want):
        np.testing.assert_array_equal(g, w)


def test_argmax_first_occurrence_and_nan_match_numpy():
    rng = np.random.default_rng(7)
    rows = [np.array([1.0, 3.0, 3.0, 2.0]), np.array([np.nan, 1.0, np.nan]),
            np.array([-np.inf, -np.inf]), np.array([0.0, -0.0, 0.0]),
            np.array([1.0, np.inf, np.nan, np.inf]), np.array([-0.0, 0.0])]
    rows += [rng.integers(0, 4, size=50).astype(np.float32) for _ in range(50)]
    for r in rows:
        assert oracle.argmax_ref(r) == int(np.argmax(r))


@pytest.mark.parametrize("trial", range(64))
def test_tiny_workload_planted_depths(trial):
    """Tiny workload: binary tree (N = 15), vocab 1000, 64 seeded trials; the
    accept length, path and bonus are known by construction."""
    tree = synth.heap_tree(2, 3)
    a = synth.make_accept_case(synth.SEEDS[1] + trial, tree, 1, 1000)
    lens, paths, bonus = oracle.accept_ref(a.logits, a.tokens, a.parents, a.max_depth)
    assert lens[0] == a.expected_len[0]
    assert paths[0, :lens[0]].tolist() == a.expected_path[0]
    assert np.all(paths[0, lens[0]:] == -1)
    assert bonus[0] == a.expected_bonus[0]


def test_every_depth_covered_by_planting():
    tree = synth.heap_tree(2, 3)
    seen = set()
    for trial in range(64):
        a = synth.make_accept_case(synth.SEEDS[1] + trial, tree, 1, 1000)
        seen.add(int(a.expected_len[0]))
    assert seen == {0, 1, 2, 3, 4}


@pytest.mark.parametrize("widths,B", [((10, 18, 18, 18), 8), ((10, 14, 12, 8), 16)])
def test_layered_trees_planted(widths, B):
    tree = synth.layered_tree(np.random.default_rng(9), widths)
    a = synth.make_accept_case(77, tree, B, 4096)
    lens, paths, bonus = oracle.accept_ref(a.logits, a.tokens, a.parents, a.max_depth)
    np.testing.assert_array_equal(lens, a.expected_len)
    np.testing.assert_array_equal(bonus, a.expected_bonus)
    for b in range(B):
        assert paths[b, :lens[b]].tolist() == a.expected_path[b]


@settings(max_examples=200, deadline=None)
@given(st.integers(1, 8), st.integers(2, 6), st.integers(0, 2 ** 31 - 1))
def test_chain_is_textbook_greedy_speculative_decoding(n, V, seed):
    """On a chain, acceptance is the longest prefix of draft tokens that each
    equal the greedy target of the position before, plus the target after
    the prefix as the bonus token."""
    rng = np.random.default_rng(seed)
    logits = rng.integers(0, 3, size=(1, n + 1, V)).astype(np.float32)
    tokens = rng.integers(0, V, size=(1, n)).astype(np.int32)
    targets = np.argmax(logits[0], axis=-1)
    k = 0
    while k < n and tokens[0, k] == targets[k]:
        k += 1
    lens, paths, bonus = oracle.accept_ref(logits, tokens, synth.chain_tree(n).parents, n)
    assert lens[0] == k
    assert paths[0, :k].tolist() == list(range(k))
    assert bonus[0] == targets[k]


def test_accept_length_zero():
    """tau may be 0: nothing accepted, bonus = the anchor row's target."""
    logits = np.zeros((1, 4, 5), dtype=np.float32)
    logits[0, 0, 2] = 1.0
    tokens = np.array([[1, 3, 4]], dtype=np.int32)
    lens, paths, bonus = oracle.accept_ref(logits, tokens, np.array([-1, -1, 0]), 2)
    assert lens[0] == 0 and bonus[0] == 2 and np.all(paths == -1)


def test_batched_acceptance_fixture():
    with open(os.path.join(GOLDEN, "batched_acceptance.json")) as f:
        fx = json.load(f)
    V = fx["vocab"]
    am = np.array(fx["row_argmax"])
    B, R = am.shape
    logits = np.zeros((B, R, V), dtype=np.float32)
    for b in range(B):
        for r in range(R):
            logits[b, r, am[b, r]] = 1.0
    lens, paths, bonus = oracle.accept_ref(logits, np.array(fx["tokens"], np.int32),
                                           np.array(fx["parents"]), 4)
    assert lens.tolist() == fx["accept_len"]
    assert paths.tolist() == fx["accept_path"]
    assert bonus.tolist() == fx["bonus"]


def test_rows_off_the_accepted_path_do_not_matter():
    """Only the anchor row and the rows of accepted nodes decide the result:
    rewriting every other row leaves it unchanged."""
    tree = synth.layered_tree(np.random.default_rng(4), (4, 6, 6))
    a = synth.make_accept_case(5, tree, 4, 300)
    ref = oracle.accept_ref(a.logits, a.tokens, a.parents, a.max_depth)
    rng = np.random.default_rng(6)
    lg = a.logits.copy()
    for b in range(4):
        used = {0} | {n + 1 for n in a.expected_path[b]}
        for r in range(lg.shape[1]):
            if r not in used:
                lg[b, r] = rng.standard_normal(lg.shape[2])
    got = oracle.accept_ref(lg, a.tokens, a.parents, a.max_depth)
    for g, w in zip(got, ref):
        np.testing.assert_array_equal(g, w)


def test_path_longer_than_max_depth_is_an_error():
    logits = np.zeros((1, 3, 4), dtype=np.float32)
    logits[0, :, 1] = 1.0
    tokens = np.array([[1, 1]], dtype=np.int32)
    with pytest.raises(ValueError):
        oracle.accept_ref(logits, tokens, np.array([-1, 0]), 1)


def test_planted_bug_is_caught_by_bruteforce():
    """A plausible oracle mistake -- comparing a node's token with its own row
    instead of its parent's -- disagrees with enumeration on this input."""
    par = np.array([-1, 0, 0, 1])
    logits = np.zeros((1, 5, 4), dtype=np.float32)
    logits[0, 0, 2] = 1; logits[0, 1, 3] = 1; logits[0, 2, 1] = 1
    tokens = np.array([[2, 3, 1, 0]], dtype=np.int32)
    lens, _, _ = oracle.accept_bruteforce(logits, tokens, par, 3)
    assert lens[0] == 2                         # node 0 (2 == row 0), node 1 (3 == row 1)
    wrong = [int(tokens[0, i] == np.argmax(logits[0, i + 1])) for i in range(4)]
    assert wrong[0] == 0                        # the mistaken rule rejects node 0
