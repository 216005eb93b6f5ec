"""HIP-graph capture of the library calls: every call is a plain kernel
launch on the caller's stream (no allocation, memset or synchronisation), so
a step of draft, verify and acceptance calls captures as it is.  Each replay,
with eager work and synchronisations in between, must reproduce the eager
results: bitwise for these fixed split plans, and the acceptance outputs
exactly."""
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


def test_replays_of_a_captured_step_equal_the_eager_step():
    rng = np.random.default_rng(9100)
    B, Hq, Hkv, D, L, V = 4, 16, 4, 128, 3000, 5000
    tree = synth.layered_tree(rng, (4, 6, 6))
    N = tree.n
    k = dev(synth.draw_normal(rng, (B, Hkv, L, D), 1.0, "bf16"))
    v = dev(synth.draw_normal(rng, (B, Hkv, L, D), 1.0, "bf16"))
    lens = dev(np.array([3000, 2500, 1234, 77], np.int32))
    pad = np.zeros((B, L), dtype=np.uint8)
    for b, n in enumerate([3000, 2500, 1234, 77]):
        pad[b, :n] = synth.pad_groups(rng, n, n_groups=6)
    pad = dev(pad)
    idx = dev(np.stack([np.sort(rng.choice(n, size=64, replace=False)) for n in [3000, 2500, 1234, 77]])
              [:, None, :].astype(np.int32))
    qd = dev(synth.draw_normal(rng, (B, 1, Hq, D), 1.0, "bf16"))
    qw = dev(synth.draw_normal(rng, (B, 3, Hq, D), 1.0, "bf16"))
    qv = dev(synth.draw_normal(rng, (B, N, Hq, D), 1.0, "bf16"))
    tk = dev(synth.draw_normal(rng, (B, Hkv, N, D), 1.0, "bf16"))
    tv = dev(synth.draw_normal(rng, (B, Hkv, N, D), 1.0, "bf16"))
    parents = dev(tree.parents)
    logits = torch.randn((B, N + 1, V), device="cuda")
    am = logits.argmax(-1)                                     # every node carries its parent's target:
    tokens = am[:, torch.from_numpy(tree.parents.astype(np.int64) + 1).cuda()].to(torch.int32).contiguous()
    dims = skg.make_dims(B, Hq, Hkv, D, skg.SPEC_BF16)
    ws_g = skg.new_workspace(skg.draft_workspace_bytes(dims, 1, 64), "cuda")
    ws_w = skg.new_workspace(skg.draft_workspace_bytes(dims, 3, 4 + 200 + 2), "cuda")
    ws_v = skg.new_workspace(skg.verify_workspace_bytes(dims, N, L), "cuda")
    ws_a = skg.new_workspace(skg.accept_workspace_bytes(B, N, V), "cuda")
    outs = dict(g=torch.empty((B, 1, Hq, D), dtype=torch.bfloat16, device="cuda"),
                w=torch.empty((B, 3, Hq, D), dtype=torch.bfloat16, device="cuda"),
                v=torch.empty((B, N, Hq, D), dtype=torch.bfloat16, device="cuda"),
                vl=torch.empty((B, N, Hq), dtype=torch.float32, device="cuda"),
                vp=torch.empty((B, N), dtype=torch.int32, device="cuda"),
                al=torch.empty(B, dtype=torch.int32, device="cuda"),
                ap=torch.empty((B, 3), dtype=torch.int32, device="cuda"),
                bo=torch.empty(B, dtype=torch.int32, device="cuda"))

    def step():
        skg.spec_attn_draft_sparse(qd, k, v, lens, idx=idx, out=outs["g"], workspace=ws_g)
        skg.spec_attn_draft_sparse(qw, k, v, lens, n_sink=4, window=200, out=outs["w"], workspace=ws_w)
        skg.spec_attn_verify_tree(qv, k, v, lens, tk, tv, parents, pad=pad, out=outs["v"], lse=outs["vl"],
                                  pos_ids=outs["vp"], workspace=ws_v)
        skg.spec_accept_greedy(logits, tokens, parents, 3, accept_len=outs["al"], accept_path=outs["ap"],
                               bonus=outs["bo"], workspace=ws_a)

    step()
    torch.cuda.synchronize()
    eager = {n: t.clone() for n, t in outs.items()}
    assert int(eager["al"].min()) == 3

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        for t in outs.values():
            t.zero_()                       # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n, t in outs.items():
            assert torch.equal(t, eager[n]), (rep, n)
        step()                              # and an eager step, after a replay
        torch.cuda.synchronize()
        for n, t in outs.items():
            assert torch.equal(t, eager[n]), (rep, "eager", n)
    for w in (ws_g, ws_w, ws_v, ws_a):
        assert skg.spec_device_status(w) == 0
