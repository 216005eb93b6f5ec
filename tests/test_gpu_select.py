"""GPU parity of budget selection by block-mean scoring.

The block means are compared with the fp64 oracle within the rounding of an
fp32 sum.  The selection is a decision on fp32 scores: the kernel's scores
must match the oracle's within that rounding, its chosen blocks must be
exactly the top n_select of its own scores (ties to the smaller index), and
must equal the oracle's choice wherever the oracle's scores leave a margin
larger than the rounding at the boundary; the emitted list must equal, bit
for bit, the oracle's list built from the kernel's choice.  End to end, a
draft over the emitted list matches the oracle's draft over the same list.
"""
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


def run_select(q, k, lens, *, block, n_sink, window, n_select, budget, pad=None, ws=None):
    kd = dev(k)
    cl = dev(np.asarray(lens, np.int32))
    pd = None if pad is None else dev(pad)
    if ws is None:
        nb = -(-k.shape[2] // block)
        dims = skg.make_dims(k.shape[0], q.shape[2], k.shape[1], k.shape[3],
                             skg.SPEC_BF16 if k.dtype == np.uint16 else skg.SPEC_F32)
        ws = skg.new_workspace(skg.select_workspace_bytes(dims, nb), "cuda")
    means = skg.spec_block_means(kd, cl, block, pad=pd, workspace=ws)
    idx, scores = skg.spec_select_blocks(dev(q), means, cl, block=block, capacity=k.shape[2],
                                         n_sink=n_sink, window=window, n_select=n_select,
                                         budget=budget, pad=pd, want_scores=True, workspace=ws)
    err = skg.spec_device_status(ws)
    return means.cpu().numpy(), idx.cpu().numpy(), scores.cpu().numpy(), err


def check_selection(q, k, lens, gm, gidx, gsc, *, block, n_sink, window, n_select, budget,
                    pad=None):
    B, Hkv = k.shape[0], k.shape[1]
    nb = gm.shape[2]
    means = oracle.block_means_ref(k, lens, block, nb, pad)
    fin = np.isfinite(means)
    assert np.array_equal(fin, np.isfinite(gm)), "blocks with a mean differ"
    scale = max(1.0, np.abs(means[fin]).max()) if fin.any() else 1.0
    np.testing.assert_allclose(gm[fin], means[fin], rtol=0, atol=2e-6 * scale)
    sc = oracle.block_scores_ref(q, means, lens, block, n_sink, window)
    sf = np.isfinite(sc)
    assert np.array_equal(sf, np.isfinite(gsc)), "scored blocks differ"
    qmax = np.abs(oracle.as_f64(q)).max()
    eps = 1e-5 * max(1.0, qmax * (np.abs(means[fin]).max() if fin.any() else 1.0)) * q.shape[-1]
    np.testing.assert_allclose(gsc[sf], sc[sf], rtol=0, atol=eps)
    for b in range(B):
        for g in range(Hkv):
            mine = sel.top_blocks(gsc[b, g].astype(np.float64), n_select)
            want = sel.select_list(int(lens[b]), None if pad is None else pad[b], mine, block,
                                   n_sink, window, budget)
            np.testing.assert_array_equal(gidx[b, g], want, err_msg=f"list of pair ({b}, {g})")
            ref = sel.top_blocks(sc[b, g], n_select)
            if len(ref) and len(ref) < int(sf[b, g].sum()):
                s_sorted = np.sort(sc[b, g][sf[b, g]])[::-1]
                gap = s_sorted[len(ref) - 1] - s_sorted[len(ref)]
                if gap > 2 * eps:
                    np.testing.assert_array_equal(mine, ref)
                else:
                    assert np.all(sc[b, g][mine] >= s_sorted[len(ref) - 1] - 2 * eps)
            else:
                np.testing.assert_array_equal(mine, ref)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
def test_small_shapes_with_pads_and_partial_blocks(dtype, D):
    c = synth.make_attn_case(9100 + D, B=3, Hq=8, Hkv=2, D=D, L_cap=520, T=2,
                             cache_len=[520, 301, 60], dtype=dtype, value_scale=1.0)
    pad = (np.random.default_rng(9100).random((3, 520)) < 0.08).astype(np.uint8)
    pad[0, 160:176] = 1                                  # one block entirely padding
    kw = dict(block=16, n_sink=4, window=64, n_select=6, budget=4 + 64 + 6 * 16)
    gm, gidx, gsc, err = run_select(c.q, c.k, c.cache_len, pad=pad, **kw)
    assert err == 0
    assert np.all(np.isnan(gm[0, :, 10]))
    check_selection(c.q, c.k, c.cache_len, gm, gidx, gsc, pad=pad, **kw)


def test_ties_go_to_the_smaller_block():
    """Several blocks with identical keys have bitwise equal means and
    scores; the smaller indices are chosen."""
    c = synth.make_attn_case(9200, B=1, Hq=4, Hkv=1, D=128, L_cap=512, T=1,
                             cache_len=[512], dtype="bf16", value_scale=1.0)
    k = c.k.copy()
    qbar = oracle.as_f64(c.q[0, 0]).mean(axis=0)
    kb = synth.round_to_bf16_bits((4 * qbar / np.linalg.norm(qbar)).astype(np.float32))
    for blk in (5, 9, 13, 20, 27):
        k[0, 0, blk * 16:(blk + 1) * 16] = kb             # five equal best blocks
    kw = dict(block=16, n_sink=4, window=32, n_select=3, budget=4 + 32 + 3 * 16)
    gm, gidx, gsc, err = run_select(c.q, k, c.cache_len, **kw)
    assert err == 0
    assert gsc[0, 0, 5] == gsc[0, 0, 9] == gsc[0, 0, 27]
    assert sel.top_blocks(gsc[0, 0].astype(np.float64), 3).tolist() == [5, 9, 13]
    check_selection(c.q, k, c.cache_len, gm, gidx, gsc, **kw)


@pytest.mark.parametrize("n_select,L", [(0, 400), (100, 400), (8, 50), (8, 70)])
def test_no_block_every_block_and_short_sequences(n_select, L):
    c = synth.make_attn_case(9300 + n_select + L, B=2, Hq=8, Hkv=2, D=128, L_cap=400, T=1,
                             cache_len=[L, max(1, L // 3)], dtype="bf16", value_scale=1.0)
    kw = dict(block=16, n_sink=4, window=48, n_select=n_select,
              budget=4 + 48 + n_select * 16 + 7)
    gm, gidx, gsc, err = run_select(c.q, c.k, c.cache_len, **kw)
    assert err == 0
    check_selection(c.q, c.k, c.cache_len, gm, gidx, gsc, **kw)


def test_incremental_block_refresh_touches_only_its_blocks():
    c = synth.make_attn_case(9400, B=2, Hq=8, Hkv=2, D=128, L_cap=256, T=1,
                             cache_len=[256, 200], dtype="bf16", value_scale=1.0)
    kd, cl = dev(c.k), dev(c.cache_len)
    means = torch.full((2, 2, 16, 128), 7.0, dtype=torch.float32, device="cuda")
    skg.spec_block_means(kd, cl, 16, first_block=5, n_blocks=3, means=means)
    got = means.cpu().numpy()
    ref = oracle.block_means_ref(c.k, c.cache_len, 16, 16)
    np.testing.assert_allclose(got[:, :, 5:8], ref[:, :, 5:8], rtol=0, atol=2e-6)
    assert np.all(got[:, :, :5] == 7.0) and np.all(got[:, :, 8:] == 7.0)


def test_bad_cache_len_is_reported():
    c = synth.make_attn_case(9500, B=2, Hq=8, Hkv=2, D=128, L_cap=128, T=1,
                             cache_len=[128, 128], dtype="bf16", value_scale=1.0)
    lens = np.array([128, 129], dtype=np.int32)        # one past the capacity
    gm, gidx, gsc, err = run_select(c.q, c.k, lens, block=16, n_sink=4, window=16, n_select=2,
                                    budget=52)
    assert err == skg.SPEC_DEV_CACHE_LEN
    assert np.all(np.isnan(gm[1])) and np.all(gidx[1] == -1) and np.all(np.isnan(gsc[1]))
    assert np.all(gidx[0, :, :20] >= 0)


@pytest.fixture(scope="module")
def batch16k():
    rng = np.random.default_rng(9600)
    B, L, D = 8, 16384, 128
    s = 1 / math.sqrt(D)
    k = synth.draw_normal(rng, (B, 8, L, D), s, "bf16")
    v = synth.draw_normal(rng, (B, 8, L, D), s, "bf16")
    q = synth.draw_normal(rng, (B, 1, 32, D), s, "bf16")
    return q, k, v, np.full(B, L, dtype=np.int32)


@pytest.mark.parametrize("budget", [256, 512, 1024, 2048])
def test_16k_batch_selection_and_draft_over_its_lists(batch16k, budget):
    """Batch 8 at 16,384 tokens, blocks of 16, window budget/2, sink 4 and
    as many blocks as the rest of the budget holds; then the draft over the
    emitted lists (sampled pairs) against the oracle's draft."""
    q, k, v, lens = batch16k
    s = 1 / math.sqrt(128)
    win = budget // 2
    nsel = (budget - 4 - win) // 16
    kw = dict(block=16, n_sink=4, window=win, n_select=nsel, budget=budget)
    gm, gidx, gsc, err = run_select(q, k, lens, **kw)
    assert err == 0
    check_selection(q, k, lens, gm, gidx, gsc, **kw)
    out, _ = skg.spec_attn_draft_sparse(dev(q), dev(k), dev(v), dev(lens), idx=dev(gidx))
    torch.cuda.synchronize()
    got = host64(out)
    pairs = [(0, 0), (3, 5), (7, 7)]
    ref, _ = oracle.draft_attn_ref(q, k, v, lens, scale=s, idx=gidx, pairs=pairs)
    assert_close(got, ref, "bf16", f"draft over the selected lists, budget {budget}")


def test_ragged_padded_batch_with_three_queries():
    """The ragged workload's shape (2K..32K tokens, tail padding in groups of
    5), three query tokens per sequence, blocks of 32."""
    d = synth.config_ragged(widths=(10, 14, 12, 8), B=6, hi=32768)
    c = d["case"]
    rng = np.random.default_rng(9700)
    q = synth.draw_normal(rng, (6, 3, 32, 128), 1 / math.sqrt(128), "bf16")
    kw = dict(block=32, n_sink=4, window=512, n_select=24, budget=4 + 512 + 24 * 32)
    k = c.k[:6]
    gm, gidx, gsc, err = run_select(q, k, c.cache_len[:6], pad=d["pad"][:6], **kw)
    assert err == 0
    check_selection(q, k, c.cache_len[:6], gm, gidx, gsc, pad=d["pad"][:6], **kw)
