"""GPU parity of the window draft over a draft-KV ring buffer: bitwise equal
to the window draft over the logical cache (the same keys in the same view
order, so the same tiles and splits), and within the bar of the oracle,
for wrapped and unwrapped rings, one and three chained queries, bf16 and
fp32, at small sizes and at the million-token layer."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import ring as ro
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


@pytest.mark.parametrize("T", [1, 3])
@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_ring_equals_window_draft_and_oracle(T, dtype, D):
    n_sink, window = 4, 200
    ring = window + T - 1 + 37
    # lengths: short (no wrap), just past one lap, many laps, window start at the wrap
    lens = [150, n_sink + ring + 5, 2000, n_sink + 3 * ring + T - 1 + window]
    c = synth.make_attn_case(10000 + T + D, B=len(lens), Hq=8, Hkv=2, D=D, L_cap=max(lens), T=T,
                             cache_len=lens, dtype=dtype, value_scale=1.0)
    kr = ro.ring_from_logical(c.k, c.cache_len, n_sink, ring)
    vr = ro.ring_from_logical(c.v, c.cache_len, n_sink, ring)
    cl = dev(c.cache_len)
    out_r, lse_r = skg.spec_attn_draft_ring(dev(c.q), dev(kr), dev(vr), cl, n_sink=n_sink,
                                            window=window, ring=ring, scale=c.scale)
    out_w, lse_w = skg.spec_attn_draft_sparse(dev(c.q), dev(c.k), dev(c.v), cl, n_sink=n_sink,
                                              window=window, scale=c.scale)
    np.testing.assert_array_equal(bits(out_r), bits(out_w))
    np.testing.assert_array_equal(lse_r.cpu().numpy(), lse_w.cpu().numpy())
    ref, _ = oracle.ring_draft_ref(c.q, kr, vr, c.cache_len, scale=c.scale, n_sink=n_sink,
                                   window=window, ring=ring)
    assert_close(host64(out_r), ref, dtype, f"ring draft T={T}")


def test_ring_with_no_sink_and_minimum_size():
    T, window = 3, 64
    ring = window + T - 1
    c = synth.make_attn_case(10100, B=2, Hq=4, Hkv=1, D=128, L_cap=900, T=T,
                             cache_len=[900, 66], value_scale=1.0)
    kr = ro.ring_from_logical(c.k, c.cache_len, 0, ring)
    vr = ro.ring_from_logical(c.v, c.cache_len, 0, ring)
    out, _ = skg.spec_attn_draft_ring(dev(c.q), dev(kr), dev(vr), dev(c.cache_len), n_sink=0,
                                      window=window, ring=ring, scale=c.scale)
    ref, _ = oracle.ring_draft_ref(c.q, kr, vr, c.cache_len, scale=c.scale, n_sink=0,
                                   window=window, ring=ring)
    assert_close(host64(out), ref, "bf16", "ring without sink")


def test_short_cache_len_is_reported():
    c = synth.make_attn_case(10200, B=2, Hq=4, Hkv=1, D=128, L_cap=80, T=3,
                             cache_len=[80, 80], value_scale=1.0)
    dims = skg.make_dims(2, 4, 1, 128, skg.SPEC_BF16)
    ws = skg.new_workspace(skg.draft_workspace_bytes(dims, 3, 4 + 32 + 2), "cuda")
    lens = np.array([5000, 2], dtype=np.int32)          # the second is shorter than Tq
    kr = dev(c.k[:, :, :4 + 40])
    out, _ = skg.spec_attn_draft_ring(dev(c.q), kr, kr, dev(lens), n_sink=4, window=32, ring=40,
                                      workspace=ws)
    assert skg.spec_device_status(ws) == skg.SPEC_DEV_CACHE_LEN
    got = host64(out)
    assert np.all(np.isnan(got[1])) and np.all(np.isfinite(got[0]))


@pytest.mark.parametrize("which", ["ctx", "fwd"])
def test_1m_ring_draft_equals_the_window_draft(which):
    """The million-token layer: the draft over a ring of window + 2 slots
    (after the 4 sink slots) holding the positions the views need, bitwise
    against the window draft over the full 1,048,576-token cache."""
    import synth.device_gen as dg
    d = dg.layer_1m(0)
    L = 1 << 20
    q = d["ctx_q"] if which == "ctx" else d["fwd_q"][0]
    T = q.shape[1]
    n_sink, window = 4, 4096
    ring = window + 2
    cl = torch.tensor([L], dtype=torch.int32, device="cuda")
    pos = torch.arange(L - ring, L, device="cuda")
    slots = n_sink + (pos - n_sink) % ring
    kr = torch.zeros((1, 8, n_sink + ring, 128), dtype=torch.bfloat16, device="cuda")
    vr = torch.zeros_like(kr)
    kr[:, :, :n_sink] = d["k"][:, :, :n_sink]
    vr[:, :, :n_sink] = d["v"][:, :, :n_sink]
    kr[:, :, slots] = d["k"][:, :, pos]
    vr[:, :, slots] = d["v"][:, :, pos]
    out_r, lse_r = skg.spec_attn_draft_ring(q, kr, vr, cl, n_sink=n_sink, window=window, ring=ring)
    out_w, lse_w = skg.spec_attn_draft_sparse(q, d["k"], d["v"], cl, n_sink=n_sink, window=window)
    np.testing.assert_array_equal(bits(out_r), bits(out_w))
    np.testing.assert_array_equal(lse_r.cpu().numpy(), lse_w.cpu().numpy())
    del d
    torch.cuda.empty_cache()
