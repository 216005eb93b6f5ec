"""GPU parity of the compaction of a cache's pad slots: bit-exact against the
oracle (rows move as bytes) over every sequence's new length, the cleared pad
bytes, the new lengths, the untouched slots past the old length, and the
error path; pads anywhere, at the tail only, everywhere, nowhere; several
chunks and passes; strided caches; the ragged workload at full size."""
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


def run_compact(kd, vd, lens, pad, ws=None):
    cl, pd = dev(np.asarray(lens, np.int32)), dev(pad)
    ws = ws if ws is not None else skg.new_workspace(skg.compact_workspace_bytes(kd.shape[0]), "cuda")
    skg.spec_kv_compact(kd, vd, cl, pd, workspace=ws)
    err = skg.spec_device_status(ws)
    return bits(kd), bits(vd), cl.cpu().numpy(), pd.cpu().numpy(), err


def check(k, v, lens, pad, got):
    """Compare with the oracle: rows below the new length, lengths, pad bytes
    (all of them: below the old length cleared, the rest untouched), rows at
    or past the old length untouched, error bits."""
    gk, gv, gcl, gpad, gerr = got
    wk, wv, wcl, wpad, werr = oracle.compact_ref(k, v, lens, pad)
    assert gerr == werr
    np.testing.assert_array_equal(gcl, wcl)
    np.testing.assert_array_equal(gpad, wpad)
    for b in range(len(lens)):
        L = int(lens[b])
        n = int(wcl[b]) if 0 <= L <= k.shape[2] else 0
        np.testing.assert_array_equal(gk[b, :, :n], wk[b, :, :n])
        np.testing.assert_array_equal(gv[b, :, :n], wv[b, :, :n])
        hi = max(L, 0) if 0 <= L <= k.shape[2] else 0
        np.testing.assert_array_equal(gk[b, :, hi:], k[b, :, hi:])   # past the old length (or a bad one: all)
        np.testing.assert_array_equal(gv[b, :, hi:], v[b, :, hi:])


def case(seed, *, B=4, Hkv=2, D=128, cap=700, dtype="bf16", p=0.1, lens=None):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, cap + 1, size=B).astype(np.int32) if lens is None else np.asarray(lens, np.int32)
    k = synth.draw_normal(rng, (B, Hkv, cap, D), 1.0, dtype)
    v = synth.draw_normal(rng, (B, Hkv, cap, D), 1.0, dtype)
    pad = (rng.random((B, (cap + 3) // 4 * 4)) < p).astype(np.uint8)
    return rng, k, v, lens, pad


def to_dev(a, dtype):
    t = dev(a)
    return t.view(torch.bfloat16) if dtype == "bf16" else t


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
@pytest.mark.parametrize("p", [0.02, 0.3])
def test_random_pads(dtype, D, p):
    rng, k, v, lens, pad = case(8100 + D + int(100 * p), D=D, dtype=dtype, p=p, lens=[700, 1, 517, 0])
    check(k, v, lens, pad, run_compact(to_dev(k, dtype), to_dev(v, dtype), lens, pad))


def test_tail_pad_groups_as_commits_leave_them():
    rng, k, v, lens, _ = case(8200, B=6, cap=2000, lens=[2000, 1999, 1500, 161, 5, 37])
    pad = np.zeros((6, 2000), dtype=np.uint8)
    for b in range(6):
        pad[b, :lens[b]] = synth.pad_groups(rng, int(lens[b]))
    check(k, v, lens, pad, run_compact(to_dev(k, "bf16"), to_dev(v, "bf16"), lens, pad))


def test_no_pads_every_slot_a_pad_and_a_pad_at_slot_zero():
    rng, k, v, lens, _ = case(8300, B=4, cap=300, lens=[300, 300, 300, 257])
    pad = np.zeros((4, 300), dtype=np.uint8)
    pad[1] = 1
    pad[2, 0] = 1
    pad[3, 1:256] = 1          # a whole chunk of pads, then valid slots
    check(k, v, lens, pad, run_compact(to_dev(k, "bf16"), to_dev(v, "bf16"), lens, pad))


def test_moves_across_many_chunks_and_passes():
    """A pad early in a long sequence: every later row moves, through many
    256-slot chunks (f32 at D = 128: 32 pieces per row, 64 rows per pass)."""
    rng, k, v, lens, _ = case(8400, B=2, Hkv=3, D=128, cap=5000, dtype="f32", lens=[5000, 4321])
    pad = np.zeros((2, 5000), dtype=np.uint8)
    pad[0, 3] = 1
    pad[0, 4000:4010] = 1
    pad[1] = (rng.random(5000) < 0.5).astype(np.uint8)
    check(k, v, lens, pad, run_compact(to_dev(k, "f32"), to_dev(v, "f32"), lens, pad))


def test_strided_cache_and_unaligned_pad_rows():
    """K and V inside larger buffers (row stride above D, head and batch
    strides with gaps), and a pad row stride that is a multiple of 4 but not
    of 16, so the 16-byte scan starts after an unaligned head."""
    rng = np.random.default_rng(8500)
    B, Hkv, D, cap = 3, 2, 64, 301
    big = synth.draw_normal(rng, (B, Hkv + 1, cap + 7, D + 8), 1.0, "bf16")
    bigv = synth.draw_normal(rng, (B, Hkv + 1, cap + 7, D + 8), 1.0, "bf16")
    lens = np.array([301, 250, 99], dtype=np.int32)
    pad = (rng.random((B, 308)) < 0.2).astype(np.uint8)
    kd_big, vd_big = to_dev(big, "bf16"), to_dev(bigv, "bf16")
    kd, vd = kd_big[:, :Hkv, :cap, :D], vd_big[:, :Hkv, :cap, :D]
    k, v = big[:, :Hkv, :cap, :D].copy(), bigv[:, :Hkv, :cap, :D].copy()
    got = run_compact(kd, vd, lens, pad)
    check(k, v, lens, pad, got)
    # the bytes outside the views are untouched
    np.testing.assert_array_equal(bits(kd_big)[:, Hkv:], big[:, Hkv:])
    np.testing.assert_array_equal(bits(kd_big)[:, :, cap:], big[:, :, cap:])
    np.testing.assert_array_equal(bits(kd_big)[..., D:], big[..., D:])


def test_bad_cache_length_leaves_the_sequence_alone():
    rng, k, v, lens, pad = case(8600, B=3, cap=100, lens=[101, -1, 60], p=0.3)
    got = run_compact(to_dev(k, "bf16"), to_dev(v, "bf16"), lens, pad)
    assert got[4] == skg.SPEC_DEV_CACHE_LEN
    check(k, v, lens, pad, got)


def test_commit_then_compact_then_verify_matches_the_padded_verify():
    """A commit leaves pads; after compaction the verify over the compacted
    cache without a pad mask equals the verify over the padded cache, and the
    position ids are the same."""
    rng = np.random.default_rng(8700)
    B, Hq, Hkv, D, cap = 3, 8, 2, 128, 400
    tree = synth.layered_tree(rng, (3, 4, 3))
    N = tree.n
    lens = np.array([300, 123, 390 - 20], dtype=np.int32)
    k = synth.draw_normal(rng, (B, Hkv, cap, D), 1.0, "bf16")
    v = synth.draw_normal(rng, (B, Hkv, cap, D), 1.0, "bf16")
    pad = np.zeros((B, cap), dtype=np.uint8)
    for b in range(B):
        pad[b, :lens[b]] = synth.pad_groups(rng, int(lens[b]), n_groups=8)
    tk = synth.draw_normal(rng, (B, Hkv, N, D), 1.0, "bf16")
    tv = synth.draw_normal(rng, (B, Hkv, N, D), 1.0, "bf16")
    acc = synth.make_accept_case(8701, tree, B, 64, depths=[1, 3, 0])
    alen, apath, _ = oracle.accept_ref(acc.logits, acc.tokens, tree.parents, acc.max_depth)
    kd, vd = to_dev(k, "bf16"), to_dev(v, "bf16")
    cl, pd = dev(lens), dev(pad)
    ws = skg.new_workspace(skg.commit_workspace_bytes(), "cuda")
    skg.spec_kv_commit(kd, vd, cl, pd, to_dev(tk, "bf16"), to_dev(tv, "bf16"), dev(alen.astype(np.int32)),
                       dev(apath.astype(np.int32)), workspace=ws)
    assert skg.spec_device_status(ws) == 0
    q = to_dev(synth.draw_normal(rng, (B, N, Hq, D), 1.0, "bf16"), "bf16")
    tk2 = to_dev(synth.draw_normal(rng, (B, Hkv, N, D), 1.0, "bf16"), "bf16")
    tv2 = to_dev(synth.draw_normal(rng, (B, Hkv, N, D), 1.0, "bf16"), "bf16")
    parents = dev(tree.parents)
    wsv = skg.new_workspace(skg.verify_workspace_bytes(skg.make_dims(B, Hq, Hkv, D, skg.SPEC_BF16), N, cap), "cuda")
    o1, l1, p1 = skg.spec_attn_verify_tree(q, kd, vd, cl, tk2, tv2, parents, pad=pd, workspace=wsv)
    o1, p1 = o1.float().cpu(), p1.cpu()
    wsc = skg.new_workspace(skg.compact_workspace_bytes(B), "cuda")
    skg.spec_kv_compact(kd, vd, cl, pd, workspace=wsc)
    assert skg.spec_device_status(wsc) == 0
    assert not bool(pd.any())
    o2, l2, p2 = skg.spec_attn_verify_tree(q, kd, vd, cl, tk2, tv2, parents, pad=pd, workspace=wsv)
    o3, l3, p3 = skg.spec_attn_verify_tree(q, kd, vd, cl, tk2, tv2, parents, workspace=wsv)
    assert skg.spec_device_status(wsv) == 0
    np.testing.assert_array_equal(p2.cpu().numpy(), p1.numpy())
    np.testing.assert_array_equal(p3.cpu().numpy(), p1.numpy())
    for o in (o2, o3):
        np.testing.assert_allclose(o.float().cpu().numpy(), o1.numpy(), rtol=0, atol=1e-2)
        rel = float((o.float().cpu() - o1).norm() / o1.norm())
        assert rel <= 1e-2


def test_ragged_workload_at_full_size():
    """The ragged batch of 16 (contexts 2K-32K with the tail pad pattern):
    compared with the oracle over every sequence's last 400 kept slots and
    its first pad's neighbourhood, plus the lengths and pad bytes."""
    rng = np.random.default_rng(8800)
    B, Hkv, D, cap = 16, 8, 128, 32768
    lens = rng.integers(2048, cap + 1, size=B).astype(np.int32)
    pad = np.zeros((B, cap), dtype=np.uint8)
    for b in range(B):
        pad[b, :lens[b]] = synth.pad_groups(rng, int(lens[b]))
    g = torch.Generator(device="cuda")
    g.manual_seed(8801)
    kd = torch.randn((B, Hkv, cap, D), generator=g, device="cuda").to(torch.bfloat16)
    vd = torch.randn((B, Hkv, cap, D), generator=g, device="cuda").to(torch.bfloat16)
    k0 = bits(kd)
    v0 = bits(vd)
    gk, gv, gcl, gpad, gerr = run_compact(kd, vd, lens, pad)
    assert gerr == 0
    for b in range(B):
        L = int(lens[b])
        keep = np.nonzero(pad[b, :L] == 0)[0]
        n = len(keep)
        assert gcl[b] == n
        assert not gpad[b, :L].any()
        f = int(np.argmax(pad[b, :L])) if pad[b, :L].any() else L
        sl = np.arange(max(0, f - 8), n)
        np.testing.assert_array_equal(gk[b][:, sl], k0[b][:, keep[sl]])
        np.testing.assert_array_equal(gv[b][:, sl], v0[b][:, keep[sl]])
        np.testing.assert_array_equal(gk[b][:, :max(0, f - 8)], k0[b][:, :max(0, f - 8)])


def test_long_pad_rows_are_scanned_in_slices():
    """Capacities above 64 Ki slots scan the pad bytes in 64 slices per
    sequence (a launch of its own); lengths that do not divide evenly, pads
    in the first slice, in a middle one and at the tail, and a sequence with
    no pad."""
    rng = np.random.default_rng(8900)
    B, Hkv, D, cap = 3, 2, 64, 131084
    lens = np.array([131084, 100003, 70001], dtype=np.int32)
    k = synth.draw_normal(rng, (B, Hkv, cap, D), 1.0, "bf16")
    v = synth.draw_normal(rng, (B, Hkv, cap, D), 1.0, "bf16")
    pad = np.zeros((B, cap), dtype=np.uint8)
    pad[0] = (rng.random(cap) < 0.01).astype(np.uint8)
    pad[1, 70000] = 1
    pad[1, 100003 - 100:100003] = (rng.random(100) < 0.5).astype(np.uint8)
    pad[1, 100003:] = 1                      # past cache_len: ignored
    got = run_compact(to_dev(k, "bf16"), to_dev(v, "bf16"), lens, pad)
    check(k, v, lens, pad, got)
    assert got[2][2] == 70001
