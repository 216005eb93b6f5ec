"""GPU edge cases through the C ABI: sentinel values that must never leak
into an output, out-of-range device values (error bits and poisoned
outputs), workspace reuse, run-to-run determinism, the split count, empty
batches and acceptance corner cases (ties, NaN, -inf rows, odd vocabularies).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_close, assert_lse_close, dev, host64

pytestmark = pytest.mark.gpu

skg = pytest.importorskip("sparse_kv_attention_sink_amd")

BF16_1000 = np.uint16(0x447A)     # 1000.0 in bf16
BF16_M1000 = np.uint16(0xC47A)    # -1000.0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    skg.load()


def plant_sentinels(case, hidden):
    """Give every hidden (b, slot) a key aligned with that sequence's first
    query (times 8) and values of +-1000: any hidden slot that leaks into a
    softmax dominates it.  ``hidden`` is a boolean [B, L_cap] array."""
    k = case.k.copy()
    v = case.v.copy()
    for b in range(case.B):
        for g in range(case.Hkv):
            qv = oracle.decode_bf16(case.q[b, 0, g * (case.Hq // case.Hkv)])
            sent_k = synth.round_to_bf16_bits((8 * qv).astype(np.float32))
            slots = np.nonzero(hidden[b])[0]
            k[b, g, slots] = sent_k
            v[b, g, slots] = np.where(np.arange(case.D) % 2 == 0, BF16_1000, BF16_M1000)
    case.k, case.v = k, v
    return case


def small_case(seed, *, B=2, Hq=8, Hkv=2, D=128, L=700, T=1, lens=(700, 333)):
    return synth.make_attn_case(seed, B=B, Hq=Hq, Hkv=Hkv, D=D, L_cap=L, T=T,
                                cache_len=list(lens), dtype="bf16", value_scale=1.0)


# ------------------------------------------------------------ sentinels

@pytest.mark.parametrize("T", [1, 3])
def test_window_draft_never_reads_outside_its_view(T):
    case = small_case(11 + T, T=T)
    hidden = np.ones((case.B, case.L_cap), dtype=bool)
    sink, win = 4, 40
    for b in range(case.B):
        for t in range(T):
            hidden[b, oracle.draft_view(int(case.cache_len[b]), T, t, n_sink=sink,
                                        window=win)] = False
    plant_sentinels(case, hidden)
    out, _ = skg.spec_attn_draft_sparse(dev(case.q), dev(case.k), dev(case.v),
                                        dev(case.cache_len), n_sink=sink, window=win)
    ref, _ = oracle.draft_attn_ref(case.q, case.k, case.v, case.cache_len, scale=case.scale,
                                   n_sink=sink, window=win)
    assert_close(host64(out), ref, "bf16", "window sentinel")


def test_budget_draft_never_reads_unlisted_positions():
    case = small_case(21)
    rng = np.random.default_rng(5)
    idx = np.stack([np.sort(rng.choice(int(case.cache_len[b]), 77, replace=False))
                    for b in range(case.B)])[:, None, :].astype(np.int32)
    hidden = np.ones((case.B, case.L_cap), dtype=bool)
    for b in range(case.B):
        hidden[b, idx[b, 0]] = False
    plant_sentinels(case, hidden)
    out, _ = skg.spec_attn_draft_sparse(dev(case.q), dev(case.k), dev(case.v),
                                        dev(case.cache_len), idx=dev(idx))
    ref, _ = oracle.draft_attn_ref(case.q, case.k, case.v, case.cache_len, scale=case.scale,
                                   idx=idx)
    assert_close(host64(out), ref, "bf16", "budget sentinel")


@pytest.mark.parametrize("T", [1, 3])
def test_padding_entries_of_a_budget_list_select_nothing(T):
    """-1 entries scattered through fixed-length lists, including a run
    that fills whole 32-key tiles: the result equals the oracle, and
    sentinels on every unlisted slot (row 0 included, the row that padding
    entries stage) never leak."""
    case = small_case(51 + T, T=T)
    rng = np.random.default_rng(51)
    budget = 224
    idx = np.full((case.B, 1, budget), -1, dtype=np.int32)
    hidden = np.ones((case.B, case.L_cap), dtype=bool)
    for b, n in enumerate((120, 60)):
        pos = np.sort(rng.choice(np.arange(1, int(case.cache_len[b])), n, replace=False))
        slots = np.sort(rng.choice(np.r_[0:64, 128:budget], n, replace=False))   # [64, 128) stays -1
        idx[b, 0, slots] = pos
        hidden[b, pos] = False
    plant_sentinels(case, hidden)
    out, lse = skg.spec_attn_draft_sparse(dev(case.q), dev(case.k), dev(case.v),
                                          dev(case.cache_len), idx=dev(idx))
    ref, lse_ref = oracle.draft_attn_ref(case.q, case.k, case.v, case.cache_len,
                                         scale=case.scale, idx=idx)
    assert_close(host64(out), ref, "bf16", f"padded budget T={T}")
    assert_lse_close(lse.cpu().numpy().astype(np.float64), lse_ref, 1e-3, "padded budget lse")


def test_padded_per_head_lists_and_an_all_padding_head():
    case = small_case(55)
    rng = np.random.default_rng(55)
    budget = 96
    idx = np.full((case.B, case.Hkv, budget), -1, dtype=np.int32)
    for b in range(case.B):
        for g in range(case.Hkv):
            if (b, g) == (1, 1):
                continue                                   # nothing listed at all
            n = int(rng.integers(1, budget))
            idx[b, g, rng.choice(budget, n, replace=False)] = rng.choice(
                int(case.cache_len[b]), n, replace=False)
    out, lse = skg.spec_attn_draft_sparse(dev(case.q), dev(case.k), dev(case.v),
                                          dev(case.cache_len), idx=dev(idx))
    ref, lse_ref = oracle.draft_attn_ref(case.q, case.k, case.v, case.cache_len,
                                         scale=case.scale, idx=idx)
    got = host64(out)
    G = case.Hq // case.Hkv
    assert np.all(got[1, :, G:2 * G] == 0)
    assert np.all(np.isneginf(lse.cpu().numpy()[1, :, G:2 * G]))
    assert_close(got, ref, "bf16", "padded per-head lists")
    assert_lse_close(lse.cpu().numpy().astype(np.float64), lse_ref, 1e-3, "padded lse")


def test_padded_budget_list_fp32_path():
    case = synth.make_attn_case(57, B=2, Hq=2, Hkv=1, D=64, L_cap=300, T=2,
                                cache_len=[300, 140], dtype="f32")
    rng = np.random.default_rng(57)
    idx = np.full((2, 1, 150), -1, dtype=np.int32)
    idx[0, 0, rng.choice(150, 100, replace=False)] = rng.choice(300, 100, replace=False)
    idx[1, 0, rng.choice(150, 140, replace=False)] = np.arange(140)
    out, _ = skg.spec_attn_draft_sparse(dev(case.q), dev(case.k), dev(case.v),
                                        dev(case.cache_len), idx=dev(idx), scale=case.scale)
    ref, _ = oracle.draft_attn_ref(case.q, case.k, case.v, case.cache_len, scale=case.scale,
                                   idx=idx)
    assert_close(host64(out), ref, "f32", "padded budget fp32")


def test_negative_budget_entry_other_than_padding_is_an_error():
    case = small_case(59)
    idx = np.tile(np.arange(40, dtype=np.int32), (case.B, 1, 1))
    idx[0, 0, 5] = -1                                  # padding: fine
    idx[1, 0, 9] = -2                                  # not padding: an error
    dims = skg.make_dims(case.B, case.Hq, case.Hkv, case.D, skg.SPEC_BF16)
    ws = skg.new_workspace(skg.draft_workspace_bytes(dims, 1, 40), "cuda")
    out, _ = skg.spec_attn_draft_sparse(dev(case.q), dev(case.k), dev(case.v),
                                        dev(case.cache_len), idx=dev(idx), workspace=ws)
    assert skg.spec_device_status(ws) == skg.SPEC_DEV_INDEX
    got = host64(out)
    assert np.all(np.isnan(got[1])) and np.all(np.isfinite(got[0]))


def test_verify_never_reads_pads_or_slots_past_the_cache():
    tree = synth.layered_tree(np.random.default_rng(3), (3, 5, 4))
    case = small_case(31, T=tree.n)
    rng = np.random.default_rng(9)
    pad = np.zeros((case.B, case.L_cap), dtype=np.uint8)
    for b in range(case.B):
        L_b = int(case.cache_len[b])
        pad[b, :L_b] = synth.pad_groups(rng, L_b, n_groups=20)
        pad[b, rng.choice(L_b, 25, replace=False)] = 1          # pads anywhere in the cache
    hidden = np.ones((case.B, case.L_cap), dtype=bool)
    for b in range(case.B):
        L_b = int(case.cache_len[b])
        hidden[b, :L_b] = pad[b, :L_b] != 0
    plant_sentinels(case, hidden)
    tk = synth.draw_normal(rng, (case.B, case.Hkv, tree.n, case.D), 1.0, "bf16")
    tv = synth.draw_normal(rng, (case.B, case.Hkv, tree.n, case.D), 1.0, "bf16")
    out, _, pos = skg.spec_attn_verify_tree(dev(case.q), dev(case.k), dev(case.v),
                                            dev(case.cache_len), dev(tk), dev(tv),
                                            dev(tree.parents), pad=dev(pad))
    ref, _ = oracle.verify_attn_ref(case.q, case.k, case.v, case.cache_len, tk, tv,
                                    tree.parents, scale=case.scale, pad=pad)
    assert_close(host64(out), ref, "bf16", "verify sentinel")
    np.testing.assert_array_equal(pos.cpu().numpy(),
                                  oracle.position_ids(case.cache_len, pad, tree.parents))


@pytest.mark.parametrize("widths", [(3, 5, 4), (10, 18, 18, 18)], ids=["tree12", "tree64"])
def test_verify_tree_nodes_off_the_ancestor_path_never_leak(widths):
    """Sentinel tree nodes: every leaf and every other depth-1 node gets a key
    aligned with the first query of its KV head's group (times 8) and values
    of +-1000.  A node sees a sentinel only if it is on its own root path, so
    any sibling, cousin or descendant that leaked into another node's softmax
    would dominate it; the oracle's outputs (which include the sentinels
    exactly where the tree says) must be matched on every node."""
    tree = synth.layered_tree(np.random.default_rng(17), widths)
    case = small_case(41, T=tree.n)
    rng = np.random.default_rng(23)
    tk = synth.draw_normal(rng, (case.B, case.Hkv, tree.n, case.D), 1.0, "bf16")
    tv = synth.draw_normal(rng, (case.B, case.Hkv, tree.n, case.D), 1.0, "bf16")
    depth = oracle.tree_depths(tree.parents)
    leaves = set(range(tree.n)) - set(int(p) for p in tree.parents if p >= 0)
    sent = sorted(leaves | {i for i in range(tree.n) if depth[i] == 1 and i % 2 == 0})
    G = case.Hq // case.Hkv
    for b in range(case.B):
        for g in range(case.Hkv):
            qv = oracle.decode_bf16(case.q[b, 0, g * G])
            tk[b, g, sent] = synth.round_to_bf16_bits((8 * qv).astype(np.float32))
            tv[b, g, sent] = np.where(np.arange(case.D) % 2 == 0, BF16_1000, BF16_M1000)
    out, _, _ = skg.spec_attn_verify_tree(dev(case.q), dev(case.k), dev(case.v),
                                          dev(case.cache_len), dev(tk), dev(tv),
                                          dev(tree.parents))
    torch.cuda.synchronize()
    ref, _ = oracle.verify_attn_ref(case.q, case.k, case.v, case.cache_len, tk, tv,
                                    tree.parents, scale=case.scale)
    assert_close(host64(out), ref, "bf16", f"tree sentinel {tree.n} nodes")
    # the sentinels really dominate where they are visible: a node on whose
    # path one lies has an output of order 1000 for that head group's first head
    anc = oracle.tree_ancestors(tree.parents)          # anc[i, j]: j on the root path of i
    on_path = [i for i in range(tree.n) if anc[i, sent].any()]
    assert on_path and np.abs(ref[0, on_path, 0]).max() > 100


def test_cache_whose_address_has_bit_31_of_its_low_word_set():
    """Regression: the scalar base of a tile copy is rebuilt from two 32-bit
    halves; the low half must not be sign-extended.  K and V are placed
    where the low 32 bits of their addresses are at or above 2^31."""
    tree = synth.layered_tree(np.random.default_rng(4), (4, 6, 8))       # 18 nodes: shared ring
    case = small_case(33, T=tree.n)
    nbytes = case.k.size * 2
    # (the pool spans a whole 4 GiB period of the low word, so the first
    # offset whose low word is 2^31, rounded up to 256 bytes, lies inside it
    # wherever the allocator puts the pool)
    pool = torch.empty((1 << 32) + 4 * nbytes + 4096, dtype=torch.uint8, device="cuda")
    base = pool.data_ptr()
    off = (((1 << 31) - (base & 0xFFFFFFFF)) % (1 << 32) + 255) // 256 * 256
    assert off + 2 * nbytes <= pool.numel()

    def place(a, at):
        t = pool[at:at + nbytes].view(torch.bfloat16).view(a.shape)
        t.copy_(dev(a))
        assert (t.data_ptr() & 0xFFFFFFFF) >= (1 << 31)
        return t

    k = place(case.k, off)
    v = place(case.v, off + nbytes)
    rng = np.random.default_rng(10)
    tk = synth.draw_normal(rng, (case.B, case.Hkv, tree.n, case.D), 1.0, "bf16")
    tv = synth.draw_normal(rng, (case.B, case.Hkv, tree.n, case.D), 1.0, "bf16")
    out, _, _ = skg.spec_attn_verify_tree(dev(case.q), k, v, dev(case.cache_len), dev(tk), dev(tv),
                                          dev(tree.parents))
    ref, _ = oracle.verify_attn_ref(case.q, case.k, case.v, case.cache_len, tk, tv, tree.parents,
                                    scale=case.scale)
    assert_close(host64(out), ref, "bf16", "verify, high low-word base")
    del pool


# ------------------------------------------------------------ device range errors

def test_out_of_range_budget_index_poisons_only_its_head():
    case = small_case(41)
    rng = np.random.default_rng(1)
    idx = np.stack([np.stack([np.sort(rng.choice(int(case.cache_len[b]), 50, replace=False))
                              for _ in range(case.Hkv)]) for b in range(case.B)]).astype(np.int32)
    idx[1, 1, 7] = int(case.cache_len[1])             # one past the end: sequence 1, KV head 1
    dims = skg.make_dims(case.B, case.Hq, case.Hkv, case.D, skg.SPEC_BF16)
    ws = skg.new_workspace(skg.draft_workspace_bytes(dims, 1, 50), "cuda")
    out, lse = skg.spec_attn_draft_sparse(dev(case.q), dev(case.k), dev(case.v),
                                          dev(case.cache_len), idx=dev(idx), workspace=ws)
    assert skg.spec_device_status(ws) == skg.SPEC_DEV_INDEX
    assert skg.spec_device_status(ws) == 0                      # reading clears it
    got = host64(out)
    G = case.Hq // case.Hkv
    assert np.all(np.isnan(got[1, :, G:2 * G]))
    assert np.all(np.isnan(lse.cpu().numpy()[1, :, G:2 * G]))
    ok = np.ones(got.shape, dtype=bool)
    ok[1, :, G:2 * G] = False
    ref, _ = oracle.draft_attn_ref(case.q, case.k, case.v, case.cache_len, scale=case.scale,
                                   idx=np.where(idx < case.cache_len[:, None, None], idx, 0))
    assert_close(np.where(ok, got, np.nan), np.where(ok, ref, np.nan), "bf16", "other heads")


def test_bad_parent_poisons_only_its_sequence():
    N = 6
    case = small_case(51, T=N)
    par = np.array([[-1, 0, 0, 1, 2, 3], [-1, 0, 3, 1, 2, 3]], dtype=np.int32)  # node 2 -> 3
    rng = np.random.default_rng(2)
    tk = synth.draw_normal(rng, (case.B, case.Hkv, N, case.D), 1.0, "bf16")
    tv = synth.draw_normal(rng, (case.B, case.Hkv, N, case.D), 1.0, "bf16")
    dims = skg.make_dims(case.B, case.Hq, case.Hkv, case.D, skg.SPEC_BF16)
    ws = skg.new_workspace(skg.verify_workspace_bytes(dims, N, case.L_cap), "cuda")
    out, _, pos = skg.spec_attn_verify_tree(dev(case.q), dev(case.k), dev(case.v),
                                            dev(case.cache_len), dev(tk), dev(tv), dev(par),
                                            workspace=ws)
    assert skg.spec_device_status(ws) == skg.SPEC_DEV_PARENT
    got = host64(out)
    assert np.all(np.isnan(got[1]))
    np.testing.assert_array_equal(pos.cpu().numpy()[1], -1)
    ref, _ = oracle.verify_attn_ref(case.q[:1], case.k[:1], case.v[:1], case.cache_len[:1],
                                    tk[:1], tv[:1], par[0], scale=case.scale)
    assert_close(got[:1], ref, "bf16", "valid sequence")


@pytest.mark.parametrize("kind", ["draft", "verify"])
def test_bad_cache_len_is_reported(kind):
    case = small_case(61, T=3 if kind == "draft" else 2, lens=(701, 2))
    dims = skg.make_dims(case.B, case.Hq, case.Hkv, case.D, skg.SPEC_BF16)
    if kind == "draft":           # 701 > capacity 700, and 2 < the 3 draft queries
        ws = skg.new_workspace(skg.draft_workspace_bytes(dims, 3, 700), "cuda")
        out, _ = skg.spec_attn_draft_sparse(dev(case.q), dev(case.k), dev(case.v),
                                            dev(case.cache_len), n_sink=4, window=64,
                                            workspace=ws)
        assert skg.spec_device_status(ws) == skg.SPEC_DEV_CACHE_LEN
        assert np.all(np.isnan(host64(out)))
    else:                          # 701 > capacity; the second sequence is valid
        par = np.array([-1, 0], dtype=np.int32)
        rng = np.random.default_rng(4)
        tk = synth.draw_normal(rng, (case.B, case.Hkv, 2, case.D), 1.0, "bf16")
        tv = synth.draw_normal(rng, (case.B, case.Hkv, 2, case.D), 1.0, "bf16")
        ws = skg.new_workspace(skg.verify_workspace_bytes(dims, 2, case.L_cap), "cuda")
        out, _, pos = skg.spec_attn_verify_tree(dev(case.q), dev(case.k), dev(case.v),
                                                dev(case.cache_len), dev(tk), dev(tv), dev(par),
                                                workspace=ws)
        assert skg.spec_device_status(ws) == skg.SPEC_DEV_CACHE_LEN
        got = host64(out)
        assert np.all(np.isnan(got[0]))
        np.testing.assert_array_equal(pos.cpu().numpy()[0], -1)
        ref, _ = oracle.verify_attn_ref(case.q[1:], case.k[1:], case.v[1:], case.cache_len[1:],
                                        tk[1:], tv[1:], par, scale=case.scale)
        assert_close(got[1:], ref, "bf16", "valid sequence")


def test_accept_path_longer_than_max_depth_is_reported():
    tree = synth.chain_tree(5)
    a = synth.make_accept_case(77, tree, 2, 300, depths=[5, 1])
    ws = skg.new_workspace(skg.accept_workspace_bytes(2, 5, 300), "cuda")
    lens, paths, bonus = skg.spec_accept_greedy(dev(a.logits), dev(a.tokens), dev(a.parents), 3,
                                                workspace=ws)
    assert skg.spec_device_status(ws) == skg.SPEC_DEV_DEPTH
    ref_len, ref_path, ref_bonus = oracle.accept_ref(a.logits, a.tokens, a.parents, 5)
    np.testing.assert_array_equal(lens.cpu().numpy(), ref_len)
    np.testing.assert_array_equal(paths.cpu().numpy(), ref_path[:, :3])
    np.testing.assert_array_equal(bonus.cpu().numpy(), ref_bonus)


# ------------------------------------------------------------ reuse, determinism, splits

def test_workspace_reuse_and_bitwise_determinism():
    """Three calls on one workspace and one on a fresh workspace give the
    same bits: the merge counters return to zero after every call."""
    tree = synth.layered_tree(np.random.default_rng(8), (10, 18, 18, 18))
    case = synth.make_attn_case(71, B=2, Hq=32, Hkv=8, D=128, L_cap=6000, T=tree.n,
                                cache_len=[6000, 4321], dtype="bf16",
                                value_scale=1 / math.sqrt(128))
    rng = np.random.default_rng(6)
    tk = dev(synth.draw_normal(rng, (2, 8, tree.n, 128), 1 / math.sqrt(128), "bf16"))
    tv = dev(synth.draw_normal(rng, (2, 8, tree.n, 128), 1 / math.sqrt(128), "bf16"))
    args = (dev(case.q), dev(case.k), dev(case.v), dev(case.cache_len), tk, tv, dev(tree.parents))
    dims = skg.make_dims(2, 32, 8, 128, skg.SPEC_BF16)
    ws = skg.new_workspace(skg.verify_workspace_bytes(dims, tree.n, 6000), "cuda")
    runs = [skg.spec_attn_verify_tree(*args, workspace=ws) for _ in range(3)]
    runs.append(skg.spec_attn_verify_tree(*args))
    torch.cuda.synchronize()
    for r in runs[1:]:
        for x, y in zip(runs[0], r):
            assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                               y.view(torch.int16) if y.dtype == torch.bfloat16 else y)
    ref, _ = oracle.verify_attn_ref(case.q, case.k, case.v, case.cache_len,
                                    tk.view(torch.int16).cpu().numpy().view(np.uint16),
                                    tv.view(torch.int16).cpu().numpy().view(np.uint16),
                                    tree.parents, scale=case.scale, pairs=[(0, 0), (1, 7)])
    assert_close(host64(runs[0][0]), ref, "bf16", "reused workspace")


def test_split_count_does_not_change_the_result():
    """The same sequences in a cache of 20x the capacity get a different split
    plan (verify splits follow the capacity); both results stay within the
    bar of the oracle and of each other."""
    case = small_case(81, T=3, L=2000, lens=(2000, 1500))
    par = np.array([-1, 0, 1], dtype=np.int32)
    rng = np.random.default_rng(12)
    tk = synth.draw_normal(rng, (case.B, case.Hkv, 3, case.D), 1.0, "bf16")
    tv = synth.draw_normal(rng, (case.B, case.Hkv, 3, case.D), 1.0, "bf16")
    big_k = np.zeros((case.B, case.Hkv, 40000, case.D), dtype=np.uint16)
    big_v = np.zeros_like(big_k)
    big_k[:, :, :2000] = case.k
    big_v[:, :, :2000] = case.v
    dims = skg.make_dims(case.B, case.Hq, case.Hkv, case.D, skg.SPEC_BF16)
    assert skg.verify_workspace_bytes(dims, 3, 2000) != skg.verify_workspace_bytes(dims, 3, 40000)
    rest = (dev(case.cache_len), dev(tk), dev(tv), dev(par))
    a, _, _ = skg.spec_attn_verify_tree(dev(case.q), dev(case.k), dev(case.v), *rest)
    b, _, _ = skg.spec_attn_verify_tree(dev(case.q), dev(big_k), dev(big_v), *rest)
    ref, _ = oracle.verify_attn_ref(case.q, case.k, case.v, case.cache_len, tk, tv, par,
                                    scale=case.scale)
    assert_close(host64(a), ref, "bf16", "capacity 2000")
    assert_close(host64(b), ref, "bf16", "capacity 40000")
    assert_close(host64(a), host64(b), "bf16", "the two plans")


# ------------------------------------------------------------ empty batch

def test_empty_batch_through_the_binding():
    q = torch.empty((0, 1, 8, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((0, 2, 64, 128), dtype=torch.bfloat16, device="cuda")
    cl = torch.empty((0,), dtype=torch.int32, device="cuda")
    out, lse = skg.spec_attn_draft_sparse(q, k, k, cl, n_sink=4, window=16)
    assert out.shape == (0, 1, 8, 128)
    vq = torch.empty((0, 3, 8, 128), dtype=torch.bfloat16, device="cuda")
    tk = torch.empty((0, 2, 3, 128), dtype=torch.bfloat16, device="cuda")
    par = torch.tensor([-1, 0, 1], dtype=torch.int32, device="cuda")
    out, lse, pos = skg.spec_attn_verify_tree(vq, k, k, cl, tk, tk, par)
    assert pos.shape == (0, 3)
    logits = torch.empty((0, 4, 100), dtype=torch.float32, device="cuda")
    tok = torch.empty((0, 3), dtype=torch.int32, device="cuda")
    lens, _, _ = skg.spec_accept_greedy(logits, tok, par, 3)
    torch.cuda.synchronize()
    assert lens.shape == (0,)


# ------------------------------------------------------------ acceptance corners

def accept_corner_case(V, seed):
    """Logits with exact ties, NaN entries, all -inf rows and planted matches,
    per-sequence parents, and a vocabulary that is not a multiple of 4."""
    rng = np.random.default_rng(seed)
    B, N = 4, 9
    par = np.stack([synth.layered_tree(rng, (2, 3, 4)).parents for _ in range(B)])
    logits = rng.integers(-3, 3, size=(B, N + 1, V)).astype(np.float32)   # many ties
    logits[0, 2] = -np.inf                                                 # all -inf row
    logits[1, 0, V // 2] = np.nan                                          # NaN wins
    logits[1, 3, [min(1, V - 1), V - 1]] = np.nan                          # first NaN wins
    logits[2, 5, :] = 7.0                                                  # all tied
    tokens = rng.integers(0, V, size=(B, N)).astype(np.int32)
    for b in range(B):                                                     # plant some matches
        for i in range(N):
            if rng.random() < 0.6:
                p = int(par[b, i])
                tokens[b, i] = oracle.argmax_ref(logits[b, p + 1])
    return logits, tokens, par.astype(np.int32)


# (1, 7, 1001: one slice per row; 128,256: 31 slices merged per row, then per
# sequence; 300,001: 73 slices, more than one wavefront merges, so every
# slice arrives on the sequence's counter and the walk merges them)
@pytest.mark.parametrize("V", [1, 7, 1001, 128256, 300001])
def test_accept_corner_cases_bit_exact(V):
    logits, tokens, par = accept_corner_case(V, V)
    got = skg.spec_accept_greedy(dev(logits), dev(tokens), dev(par), 4)
    torch.cuda.synchronize()
    ref = oracle.accept_ref(logits, tokens, par, 4)
    for x, r in zip(got, ref):
        np.testing.assert_array_equal(x.cpu().numpy(), r)


def test_accept_unaligned_rows():
    """Rows of an odd vocabulary start at every alignment mod 16 bytes."""
    logits, tokens, par = accept_corner_case(4099, 3)
    got = skg.spec_accept_greedy(dev(logits), dev(tokens), dev(par), 4)
    torch.cuda.synchronize()
    for x, r in zip(got, oracle.accept_ref(logits, tokens, par, 4)):
        np.testing.assert_array_equal(x.cpu().numpy(), r)
