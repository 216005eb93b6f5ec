"""GPU parity of the KV commit of the accepted path: bit-exact against the
oracle (the commit moves bytes), on small batches compared whole, on the 16K
and ragged workloads compared over every sequence's appended window, with the
tree K/V aliasing the cache, and on the error paths."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import dev

pytestmark = pytest.mark.gpu

skg = pytest.importorskip("sparse_kv_attention_sink_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    skg.load()


def bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def gpu_commit(k, v, lens, pad, tk, tv, alen, apath, *, ws=None):
    """Run the library's commit on device copies; return host arrays, P and
    the device error bits."""
    kd, vd = dev(k), dev(v)
    cl, pd = dev(np.asarray(lens, np.int32)), dev(pad)
    ws = ws if ws is not None else skg.new_workspace(skg.commit_workspace_bytes(), "cuda")
    n = skg.spec_kv_commit(kd, vd, cl, pd, dev(tk), dev(tv), dev(np.asarray(alen, np.int32)),
                           dev(np.asarray(apath, np.int32)), workspace=ws)
    err = skg.spec_device_status(ws)
    return bits(kd), bits(vd), cl.cpu().numpy(), pd.cpu().numpy(), int(n.item()), err


def assert_same(got, want):
    k, v, cl, pad, P, err = got
    wk, wv, wcl, wpad, wP, werr = want
    assert P == wP
    assert err == werr
    np.testing.assert_array_equal(cl, wcl)
    np.testing.assert_array_equal(pad, wpad)
    np.testing.assert_array_equal(k, wk)
    np.testing.assert_array_equal(v, wv)


def small_case(seed, *, B=5, Hkv=2, D=128, cap=128, dtype="bf16", widths=(3, 4, 3, 2),
               depths=None):
    rng = np.random.default_rng(seed)
    tree = synth.layered_tree(rng, widths)
    N = tree.n
    lens = rng.integers(8, cap - 12, size=B).astype(np.int32)
    pad = np.zeros((B, cap), dtype=np.uint8)
    for b in range(B):
        pad[b, :lens[b]] = synth.pad_groups(rng, int(lens[b]), n_groups=3)
    k = synth.draw_normal(rng, (B, Hkv, cap, D), 1.0, dtype)
    v = synth.draw_normal(rng, (B, Hkv, cap, D), 1.0, dtype)
    tk = synth.draw_normal(rng, (B, Hkv, N, D), 1.0, dtype)
    tv = synth.draw_normal(rng, (B, Hkv, N, D), 1.0, dtype)
    acc = synth.make_accept_case(seed + 1, tree, B, 24, depths=depths)
    alen, apath, _ = oracle.accept_ref(acc.logits, acc.tokens, tree.parents, acc.max_depth)
    return k, v, lens, pad, tk, tv, alen, apath, acc.max_depth


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
def test_small_batches_whole(dtype, D):
    for seed in (8100, 8101, 8102):
        k, v, lens, pad, tk, tv, alen, apath, md = small_case(seed, D=D, dtype=dtype)
        want = oracle.commit_ref(k, v, lens, pad, tk, tv, alen, apath, md)
        assert_same(gpu_commit(k, v, lens, pad, tk, tv, alen, apath), want)


def test_every_depth_including_none_and_full():
    """Planted depths 0 (nothing accepted: only the bonus slot) through the
    tree's full depth in one batch."""
    k, v, lens, pad, tk, tv, alen, apath, md = small_case(8110, B=5, depths=[0, 1, 2, 3, 4])
    assert sorted(alen.tolist()) == [0, 1, 2, 3, 4]
    want = oracle.commit_ref(k, v, lens, pad, tk, tv, alen, apath, md)
    assert want[4] == 5
    assert_same(gpu_commit(k, v, lens, pad, tk, tv, alen, apath), want)


def test_all_sequences_accept_nothing():
    k, v, lens, pad, tk, tv, alen, apath, md = small_case(8111, depths=[0] * 5)
    want = oracle.commit_ref(k, v, lens, pad, tk, tv, alen, apath, md)
    assert want[4] == 1
    assert_same(gpu_commit(k, v, lens, pad, tk, tv, alen, apath), want)


def test_long_chain_paths_span_several_copy_groups():
    """A 20-node chain accepted to depth 20: the copy moves rows in groups
    of 8, so the path spans three groups."""
    rng = np.random.default_rng(8120)
    B, Hkv, D, cap = 3, 4, 128, 96
    N = 20
    lens = np.array([10, 40, 70], dtype=np.int32)
    pad = np.zeros((B, cap), dtype=np.uint8)
    k = synth.draw_normal(rng, (B, Hkv, cap, D), 1.0, "bf16")
    v = synth.draw_normal(rng, (B, Hkv, cap, D), 1.0, "bf16")
    tk = synth.draw_normal(rng, (B, Hkv, N, D), 1.0, "bf16")
    tv = synth.draw_normal(rng, (B, Hkv, N, D), 1.0, "bf16")
    alen = np.array([20, 13, 7], dtype=np.int32)
    apath = np.array([list(range(20)), list(range(13)) + [-1] * 7, list(range(7)) + [-1] * 13],
                     dtype=np.int32)
    want = oracle.commit_ref(k, v, lens, pad, tk, tv, alen, apath, 20)
    assert_same(gpu_commit(k, v, lens, pad, tk, tv, alen, apath), want)


@pytest.mark.parametrize("offset", [0, 3])
def test_tree_aliasing_the_cache_commits_in_place(offset):
    """Verify wrote the tree K/V into the cache just past cache_len (node n
    at slot L + offset + n); the commit compacts the accepted path in place."""
    rng = np.random.default_rng(8130 + offset)
    B, Hkv, D, cap, L = 4, 2, 128, 160, 50
    tree = synth.layered_tree(rng, (4, 6, 6, 6, 6, 6, 6, 6, 6, 6, 6))   # depth 11, 64 nodes
    N = tree.n
    k = synth.draw_normal(rng, (B, Hkv, cap, D), 1.0, "bf16")
    v = synth.draw_normal(rng, (B, Hkv, cap, D), 1.0, "bf16")
    lens = np.full(B, L, dtype=np.int32)
    pad = np.zeros((B, cap), dtype=np.uint8)
    acc = synth.make_accept_case(8140 + offset, tree, B, 24, depths=[11, 9, 0, 5])
    alen, apath, _ = oracle.accept_ref(acc.logits, acc.tokens, tree.parents, acc.max_depth)
    s0 = L + offset
    want = oracle.commit_ref(k, v, lens, pad, k[:, :, s0:s0 + N], v[:, :, s0:s0 + N], alen, apath,
                             acc.max_depth)
    kd, vd = dev(k), dev(v)
    cl, pd = dev(lens), dev(pad)
    ws = skg.new_workspace(skg.commit_workspace_bytes(), "cuda")
    n = skg.spec_kv_commit(kd, vd, cl, pd, kd[:, :, s0:s0 + N], vd[:, :, s0:s0 + N],
                           dev(alen.astype(np.int32)), dev(apath.astype(np.int32)), workspace=ws)
    err = skg.spec_device_status(ws)
    assert_same((bits(kd), bits(vd), cl.cpu().numpy(), pd.cpu().numpy(), int(n.item()), err), want)


def test_bad_acceptance_results_and_overflow():
    k, v, lens, pad, tk, tv, alen, apath, md = small_case(8150, B=6, cap=64)
    N = tk.shape[2]
    alen = alen.copy()
    apath = apath.copy()
    alen[0] = md + 1                        # longer than max_depth
    alen[1] = -1
    alen[2] = 1
    apath[2, 0] = N                         # a node past the tree
    lens = lens.copy()
    lens[3] = 64 - 1                        # no room for P slots
    lens[4] = -5
    want = oracle.commit_ref(k, v, lens, pad, tk, tv, alen, apath, md)
    assert want[5] == oracle.commit.ERR_COMMIT | oracle.commit.ERR_CACHE_LEN
    assert_same(gpu_commit(k, v, lens, pad, tk, tv, alen, apath), want)


def test_batch_larger_than_a_workgroup():
    """300 sequences: every workgroup scans the whole batch for P."""
    rng = np.random.default_rng(8160)
    B, Hkv, D, cap = 300, 1, 64, 24
    tree = synth.chain_tree(4)
    lens = rng.integers(0, 12, size=B).astype(np.int32)
    pad = (rng.random((B, cap)) < 0.2).astype(np.uint8)
    k = synth.draw_normal(rng, (B, Hkv, cap, D), 1.0, "bf16")
    v = synth.draw_normal(rng, (B, Hkv, cap, D), 1.0, "bf16")
    tk = synth.draw_normal(rng, (B, Hkv, 4, D), 1.0, "bf16")
    tv = synth.draw_normal(rng, (B, Hkv, 4, D), 1.0, "bf16")
    alen = rng.integers(0, 3, size=B).astype(np.int32)
    alen[217] = 4                            # the one sequence that sets P
    apath = np.tile(np.arange(4, dtype=np.int32), (B, 1))
    want = oracle.commit_ref(k, v, lens, pad, tk, tv, alen, apath, 4)
    assert want[4] == 5
    assert_same(gpu_commit(k, v, lens, pad, tk, tv, alen, apath), want)


def test_two_commits_in_a_row_reuse_the_workspace():
    k, v, lens, pad, tk, tv, alen, apath, md = small_case(8170, cap=128)
    want1 = oracle.commit_ref(k, v, lens, pad, tk, tv, alen, apath, md)
    alen2 = np.roll(alen, 1)
    apath2 = np.roll(apath, 1, axis=0)
    want2 = oracle.commit_ref(want1[0], want1[1], want1[2], want1[3], tk[::-1], tv[::-1], alen2,
                              apath2, md)
    kd, vd = dev(k), dev(v)
    cl, pd = dev(lens), dev(pad)
    ws = skg.new_workspace(skg.commit_workspace_bytes(), "cuda")
    skg.spec_kv_commit(kd, vd, cl, pd, dev(tk), dev(tv), dev(alen), dev(apath), workspace=ws)
    n = skg.spec_kv_commit(kd, vd, cl, pd, dev(np.ascontiguousarray(tk[::-1])),
                           dev(np.ascontiguousarray(tv[::-1])), dev(alen2), dev(apath2),
                           workspace=ws)
    err = skg.spec_device_status(ws)
    assert_same((bits(kd), bits(vd), cl.cpu().numpy(), pd.cpu().numpy(), int(n.item()), err),
                want2)


# ------------------------------------------------------------ workloads

def windowed_check(k_dev, v_dev, k_host_rows, v_host_rows, lens, pad, tk, tv, alen, apath, md,
                   margin=4):
    """Commit on the full-size device cache; compare every sequence's window
    [L_b - margin, L_b + P + margin) with the oracle run on that window."""
    B = len(lens)
    cl, pd = dev(lens), dev(pad)
    ws = skg.new_workspace(skg.commit_workspace_bytes(), "cuda")
    n = skg.spec_kv_commit(k_dev, v_dev, cl, pd, dev(tk), dev(tv), dev(alen), dev(apath),
                           workspace=ws)
    err = skg.spec_device_status(ws)
    _, _, wcl, wpad, wP, werr = oracle.commit_ref(np.zeros((B, 1, k_dev.shape[2], 1), np.uint8),
                                                  np.zeros((B, 1, k_dev.shape[2], 1), np.uint8),
                                                  lens, pad, np.zeros((B, 1, tk.shape[2], 1)),
                                                  np.zeros((B, 1, tk.shape[2], 1)), alen, apath, md)
    assert int(n.item()) == wP and err == werr
    np.testing.assert_array_equal(cl.cpu().numpy(), wcl)
    np.testing.assert_array_equal(pd.cpu().numpy(), wpad)
    W = 2 * margin + wP
    rel = np.full(B, margin, dtype=np.int32)
    wk, wv, _, _, _, _ = oracle.commit_ref(k_host_rows, v_host_rows, rel,
                                           np.zeros((B, W), np.uint8), tk, tv, alen, apath, md)
    for b in range(B):
        lo = int(lens[b]) - margin
        np.testing.assert_array_equal(bits(k_dev[b, :, lo:lo + W]), wk[b])
        np.testing.assert_array_equal(bits(v_dev[b, :, lo:lo + W]), wv[b])


def window_rows(t: torch.Tensor, lens, margin, W):
    return np.stack([bits(t[b, :, int(lens[b]) - margin:int(lens[b]) - margin + W])
                     for b in range(len(lens))])


def test_16k_batch_commit_windows():
    """Batch 8, 16,384-token caches (capacity 16,448), 64-node tree of widths
    10/18/18/18, planted acceptance depths 0..4."""
    rng = np.random.default_rng(8200)
    B, Hkv, D, L, cap = 8, 8, 128, 16384, 16448
    tree = synth.layered_tree(rng, (10, 18, 18, 18))
    g = torch.Generator(device="cuda")
    g.manual_seed(8201)
    k = torch.randn((B, Hkv, cap, D), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((B, Hkv, cap, D), generator=g, device="cuda").to(torch.bfloat16)
    lens = np.full(B, L, dtype=np.int32)
    pad = np.zeros((B, cap), dtype=np.uint8)
    tk = synth.draw_normal(rng, (B, Hkv, tree.n, D), 1.0, "bf16")
    tv = synth.draw_normal(rng, (B, Hkv, tree.n, D), 1.0, "bf16")
    acc = synth.make_accept_case(8202, tree, B, 128256)
    alen, apath, _ = oracle.accept_ref(acc.logits, acc.tokens, tree.parents, acc.max_depth)
    P = 1 + int(alen.max())
    kh, vh = window_rows(k, lens, 4, 8 + P), window_rows(v, lens, 4, 8 + P)
    windowed_check(k, v, kh, vh, lens, pad, tk, tv, alen.astype(np.int32),
                   apath.astype(np.int32), acc.max_depth)


@pytest.mark.parametrize("widths", [(10, 14, 12, 8), (10, 18, 18, 18)], ids=["tree44", "tree64"])
def test_ragged_batch_commit_windows(widths):
    """Batch 16, cache lengths 2,048..32,768 with tail padding in groups of 5
    (the ragged workload), capacity 32,832."""
    d = synth.config_ragged(widths=widths)
    c = d["case"]
    B, cap = c.B, 32832
    rng = np.random.default_rng(8210)
    g = torch.Generator(device="cuda")
    g.manual_seed(8211)
    k = torch.randn((B, 8, cap, 128), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((B, 8, cap, 128), generator=g, device="cuda").to(torch.bfloat16)
    pad = np.zeros((B, cap), dtype=np.uint8)
    pad[:, :d["pad"].shape[1]] = d["pad"]
    tree = d["tree"]
    acc = synth.make_accept_case(8212, tree, B, 128256)
    alen, apath, _ = oracle.accept_ref(acc.logits, acc.tokens, tree.parents, acc.max_depth)
    P = 1 + int(alen.max())
    lens = c.cache_len
    kh, vh = window_rows(k, lens, 4, 8 + P), window_rows(v, lens, 4, 8 + P)
    windowed_check(k, v, kh, vh, lens, pad, d["tree_k"], d["tree_v"], alen.astype(np.int32),
                   apath.astype(np.int32), acc.max_depth)
    del rng
