"""spec_attn_verify_tree_noalloc through the C ABI: the verify on the
library's static scratch equals spec_attn_verify_tree on a caller workspace,
bit for bit, on two calls in a row (the second with a smaller input, so it
runs on what the first left in the array), and allocates no device memory.
(The refusal of a shape whose scratch exceeds the array is checked on the
CPU, in tests/test_abi.py, since it happens before any launch.)"""
import math

import numpy as np
import pytest
import torch

import synth
from helpers import dev

pytestmark = pytest.mark.gpu

skg = pytest.importorskip("sparse_kv_attention_sink_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    skg.load()


def _case(seed, B, L_cap, lens, widths, pad_tail):
    s = 1 / math.sqrt(128)
    rng = np.random.default_rng(seed)
    tree = synth.layered_tree(rng, widths)
    case = synth.make_attn_case(seed + 1, B=B, Hq=32, Hkv=8, D=128, L_cap=L_cap, T=tree.n,
                                cache_len=lens, value_scale=s)
    pad = np.zeros((B, L_cap), dtype=np.uint8)
    if pad_tail:
        for b in range(B):
            pad[b, :lens[b]] = synth.pad_groups(rng, int(lens[b]))
    tk = synth.draw_normal(rng, (B, 8, tree.n, 128), s, "bf16")
    tv = synth.draw_normal(rng, (B, 8, tree.n, 128), s, "bf16")
    return dict(q=dev(case.q), k=dev(case.k), v=dev(case.v), cl=dev(case.cache_len),
                tk=dev(tk), tv=dev(tv), par=dev(tree.parents), pad=dev(pad) if pad_tail else None)


def _run_both(c):
    ref = skg.spec_attn_verify_tree(c["q"], c["k"], c["v"], c["cl"], c["tk"], c["tv"], c["par"],
                                    pad=c["pad"])
    out = torch.empty_like(c["q"])
    lse = torch.empty(c["q"].shape[:3], dtype=torch.float32, device="cuda")
    pos = torch.empty(c["q"].shape[:2], dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    skg.spec_attn_verify_tree_noalloc(c["q"], c["k"], c["v"], c["cl"], c["tk"], c["tv"], c["par"],
                                      out=out, lse=lse, pos_ids=pos, pad=c["pad"])
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    return ref, (out, lse, pos), free0, free1


def _same(a, b):
    a = a.view(torch.int16) if a.dtype == torch.bfloat16 else a
    b = b.view(torch.int16) if b.dtype == torch.bfloat16 else b
    return torch.equal(a, b)


def test_noalloc_verify_equals_the_workspace_verify_on_two_calls():
    big = _case(9100, 2, 6000, [6000, 4321], (10, 18, 18, 18), pad_tail=True)
    small = _case(9200, 1, 1000, [777], (1, 1, 1, 1, 1), pad_tail=False)
    for name, c in (("64-node tree, batch 2, 6000 slots", big), ("chain of 5, batch 1, 777 keys", small)):
        ref, got, free0, free1 = _run_both(c)
        for x, y, what in zip(ref, got, ("out", "lse", "pos_ids")):
            assert _same(x, y), f"{name}: {what} differs from spec_attn_verify_tree"
        assert np.all(np.isfinite(got[0].float().cpu().numpy()))
        if name.startswith("chain"):
            # the array was mapped by the first call: the second allocates nothing
            assert free1 == free0, f"device memory changed by {free0 - free1} bytes"
