"""GPU parity of partial verification: the partial-cache gather bit-exact
against the oracle; shared (one list per sequence) block selection; and the
whole path (shared selection -> gather -> tree verify over the partial cache,
then a KV commit into its buffer and the next verify) against the oracle, on
small shapes, the 16K batch and the million-token layer (sampled pairs)."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import select as sel
import synth
from helpers import assert_close, dev, host64

pytestmark = pytest.mark.gpu

skg = pytest.importorskip("sparse_kv_attention_sink_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    skg.load()


def bits(t):
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 128)])
def test_gather_bit_exact(dtype, D):
    rng = np.random.default_rng(9800 + D)
    B, Hkv, L_cap = 3, 4, 300
    k = synth.draw_normal(rng, (B, Hkv, L_cap, D), 1.0, dtype)
    v = synth.draw_normal(rng, (B, Hkv, L_cap, D), 1.0, dtype)
    lens = np.array([300, 150, 40], dtype=np.int32)
    budget, cap = 100, 120
    idx = np.full((B, 1, budget), -1, dtype=np.int32)
    for b in range(B):
        n = min(int(lens[b]), 80)
        idx[b, 0, rng.choice(budget, n, replace=False)] = rng.choice(int(lens[b]), n, replace=False)
    want = oracle.gather_ref(k, v, lens, idx, cap)
    pk, pv, plen, ppad = skg.spec_kv_gather(dev(k), dev(v), dev(lens), dev(idx), capacity=cap)
    ws = skg.new_workspace(256, "cuda")
    pk2, pv2, plen2, ppad2 = skg.spec_kv_gather(dev(k), dev(v), dev(lens), dev(idx), capacity=cap,
                                                workspace=ws)
    assert skg.spec_device_status(ws) == 0
    for got in ((pk, pv, plen, ppad), (pk2, pv2, plen2, ppad2)):
        np.testing.assert_array_equal(bits(got[0]), want[0])
        np.testing.assert_array_equal(bits(got[1]), want[1])
        np.testing.assert_array_equal(got[2].cpu().numpy(), want[3])
        np.testing.assert_array_equal(got[3].cpu().numpy()[:, :cap], want[2])


def test_gather_bad_entries_and_bad_length():
    rng = np.random.default_rng(9810)
    k = synth.draw_normal(rng, (2, 2, 64, 128), 1.0, "bf16")
    lens = np.array([64, 30], dtype=np.int32)
    idx = np.tile(np.arange(40, dtype=np.int32), (2, 1, 1))   # 30..39 are past sequence 1
    ws = skg.new_workspace(256, "cuda")
    pk, pv, plen, ppad = skg.spec_kv_gather(dev(k), dev(k), dev(lens), dev(idx), workspace=ws)
    assert skg.spec_device_status(ws) == skg.SPEC_DEV_INDEX
    want = oracle.gather_ref(k, k, lens, idx, 40)
    np.testing.assert_array_equal(bits(pk), want[0])
    np.testing.assert_array_equal(ppad.cpu().numpy()[:, :40], want[2])
    lens2 = np.array([64, 65], dtype=np.int32)               # one past the capacity
    pk, pv, plen, ppad = skg.spec_kv_gather(dev(k), dev(k), dev(lens2), dev(idx), workspace=ws)
    assert skg.spec_device_status(ws) == skg.SPEC_DEV_CACHE_LEN
    assert np.all(ppad.cpu().numpy()[1, :40] == 1) and not bits(pk)[1].any()


def shared_select(q, k, lens, *, block, n_sink, window, n_select, budget, pad=None):
    kd, cl = dev(k), dev(np.asarray(lens, np.int32))
    pd = None if pad is None else dev(pad)
    means = skg.spec_block_means(kd, cl, block, pad=pd)
    idx, sc = skg.spec_select_blocks(dev(q), means, cl, block=block, capacity=k.shape[2],
                                     n_sink=n_sink, window=window, n_select=n_select,
                                     budget=budget, pad=pd, shared=True, want_scores=True)
    return kd, cl, idx, sc.cpu().numpy()


def check_shared(q, k, lens, idx, gsc, *, block, n_sink, window, n_select, budget, pad=None):
    nb = gsc.shape[2]
    means = oracle.block_means_ref(k, lens, block, nb, pad)
    sc = oracle.block_scores_ref(q, means, lens, block, n_sink, window, shared=True)
    sf = np.isfinite(sc)
    assert np.array_equal(sf, np.isfinite(gsc))
    eps = 1e-4 * max(1.0, np.abs(sc[sf]).max())
    np.testing.assert_allclose(gsc[sf], sc[sf], rtol=0, atol=eps)
    gidx = idx.cpu().numpy()
    for b in range(len(lens)):
        mine = sel.top_blocks(gsc[b, 0].astype(np.float64), n_select)
        want = sel.select_list(int(lens[b]), None if pad is None else pad[b], mine, block, n_sink,
                               window, budget)
        np.testing.assert_array_equal(gidx[b, 0], want)


def partial_path(q, k, v, lens, tree, tk, tv, *, block, n_sink, window, n_select, budget,
                 buffer, pad=None, pairs=None, scale=None):
    """Shared selection, gather, verify over the partial cache; returns the
    GPU outputs, the lists and the oracle's verify over the same lists."""
    kd, cl, idx, gsc = shared_select(q, k, lens, block=block, n_sink=n_sink, window=window,
                                     n_select=n_select, budget=budget, pad=pad)
    pk, pv, plen, ppad = skg.spec_kv_gather(kd, dev(v), cl, idx, capacity=budget + buffer)
    out, lse, _ = skg.spec_attn_verify_tree(dev(q), pk, pv, plen, dev(tk), dev(tv),
                                            dev(tree.parents), pad=ppad, scale=scale)
    torch.cuda.synchronize()
    gidx = idx.cpu().numpy()
    okk, okv, opad, olen, err = oracle.gather_ref(k, v, lens, gidx, budget + buffer)
    assert err == 0
    ref, _ = oracle.verify_attn_ref(q, okk, okv, olen, tk, tv, tree.parents, scale=scale,
                                    pad=opad, pairs=pairs)
    return host64(out), ref, gidx, gsc, (pk, pv, plen, ppad)


def test_small_partial_verify_then_commit_into_the_buffer():
    rng = np.random.default_rng(9900)
    B, Hq, Hkv, D, L_cap = 3, 8, 2, 128, 700
    tree = synth.layered_tree(rng, (3, 4, 3))
    c = synth.make_attn_case(9901, B=B, Hq=Hq, Hkv=Hkv, D=D, L_cap=L_cap, T=tree.n,
                             cache_len=[700, 512, 333], value_scale=1.0)
    tk = synth.draw_normal(rng, (B, Hkv, tree.n, D), 1.0, "bf16")
    tv = synth.draw_normal(rng, (B, Hkv, tree.n, D), 1.0, "bf16")
    kw = dict(block=16, n_sink=4, window=64, n_select=5, budget=4 + 64 + 80)
    got, ref, gidx, gsc, part = partial_path(c.q, c.k, c.v, c.cache_len, tree, tk, tv, buffer=16,
                                             scale=c.scale, **kw)
    check_shared(c.q, c.k, c.cache_len, dev(gidx), gsc, **kw)
    assert_close(got, ref, "bf16", "partial verify")
    # accept a path per sequence and commit it into the partial cache's buffer
    acc = synth.make_accept_case(9902, tree, B, 32, depths=[2, 0, 3])
    alen, apath, _ = oracle.accept_ref(acc.logits, acc.tokens, tree.parents, acc.max_depth)
    pk, pv, plen, ppad = part
    skg.spec_kv_commit(pk, pv, plen, ppad, dev(tk), dev(tv), dev(alen.astype(np.int32)),
                       dev(apath.astype(np.int32)))
    okk, okv, opad, olen, _ = oracle.gather_ref(c.k, c.v, c.cache_len, gidx, kw["budget"] + 16)
    okk, okv, olen, opad, P, err = oracle.commit_ref(okk, okv, olen, opad, tk, tv, alen, apath,
                                                     acc.max_depth)
    assert err == 0
    np.testing.assert_array_equal(bits(pk), okk)
    np.testing.assert_array_equal(plen.cpu().numpy(), olen)
    q2 = synth.draw_normal(rng, c.q.shape, 1.0, "bf16")
    out, _, _ = skg.spec_attn_verify_tree(dev(q2), pk, pv, plen, dev(tk), dev(tv),
                                          dev(tree.parents), pad=ppad, scale=c.scale)
    ref2, _ = oracle.verify_attn_ref(q2, okk, okv, olen, tk, tv, tree.parents, scale=c.scale,
                                     pad=opad)
    assert_close(host64(out), ref2, "bf16", "verify after the buffer commit")


def test_partial_verify_16k_batch():
    """Batch 8 at 16,384 tokens, the 64-node tree, a 2,048-slot partial
    budget (sink 4, window 1,024, blocks of 16) and a 128-slot buffer."""
    rng = np.random.default_rng(9950)
    B, L, D = 8, 16384, 128
    s = 1 / math.sqrt(D)
    tree = synth.layered_tree(rng, (10, 18, 18, 18))
    k = synth.draw_normal(rng, (B, 8, L, D), s, "bf16")
    v = synth.draw_normal(rng, (B, 8, L, D), s, "bf16")
    q = synth.draw_normal(rng, (B, tree.n, 32, D), s, "bf16")
    tk = synth.draw_normal(rng, (B, 8, tree.n, D), s, "bf16")
    tv = synth.draw_normal(rng, (B, 8, tree.n, D), s, "bf16")
    lens = np.full(B, L, dtype=np.int32)
    kw = dict(block=16, n_sink=4, window=1024, n_select=63, budget=2048)
    pairs = [(0, 0), (4, 3), (7, 7)]
    got, ref, gidx, gsc, _ = partial_path(q, k, v, lens, tree, tk, tv, buffer=128, pairs=pairs,
                                          scale=s, **kw)
    check_shared(q, k, lens, dev(gidx), gsc, **kw)
    assert_close(got, ref, "bf16", "partial verify at 16K")


def test_partial_verify_1m_layer_sampled():
    """The million-token layer: chain-3 verify over a 4,096-slot partial
    cache (sink 4, window 2,048, blocks of 128) plus a 64-slot buffer,
    against the oracle's verify over the same list (two KV heads)."""
    import synth.device_gen as dg
    d = dg.layer_1m(0)
    L = 1 << 20
    k, v = d["k"], d["v"]
    cl = torch.tensor([L], dtype=torch.int32, device="cuda")
    block, budget = 128, 4096
    means = skg.spec_block_means(k, cl, block)
    kw = dict(block=block, capacity=L, n_sink=4, window=2048, n_select=(budget - 4 - 2048) // block,
              budget=budget, shared=True)
    idx, sc = skg.spec_select_blocks(d["verify_q"], means, cl, want_scores=True, **kw)
    pk, pv, plen, ppad = skg.spec_kv_gather(k, v, cl, idx, capacity=budget + 64)
    par = torch.tensor([-1, 0, 1], dtype=torch.int32, device="cuda")
    out, _, _ = skg.spec_attn_verify_tree(d["verify_q"], pk, pv, plen, d["tree_k"], d["tree_v"],
                                          par, pad=ppad)
    torch.cuda.synchronize()
    gidx = idx.cpu().numpy()
    gsc = sc.cpu().numpy()
    mine = sel.top_blocks(gsc[0, 0].astype(np.float64), kw["n_select"])
    assert np.array_equal(gidx[0, 0], sel.select_list(L, None, mine, block, 4, 2048, budget))
    lst = gidx[0, 0][gidx[0, 0] >= 0]
    got = host64(out)
    G = 4
    for g in (1, 6):
        kk = bits(k[0, g].index_select(0, torch.from_numpy(lst).long().cuda()))[None, None]
        vv = bits(v[0, g].index_select(0, torch.from_numpy(lst).long().cuda()))[None, None]
        qq = bits(d["verify_q"][:, :, g * G:(g + 1) * G])
        tk = bits(d["tree_k"][:, g:g + 1])
        tv = bits(d["tree_v"][:, g:g + 1])
        ref, _ = oracle.verify_attn_ref(qq, kk, vv, np.array([len(lst)]), tk, tv,
                                        np.array([-1, 0, 1]), scale=1 / math.sqrt(128))
        assert_close(got[:, :, g * G:(g + 1) * G], ref, "bf16", f"1M partial verify head {g}")
    del d
    torch.cuda.empty_cache()
