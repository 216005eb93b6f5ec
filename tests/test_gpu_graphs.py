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


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _chain_to(parents, node):
    path = []
    while node >= 0:
        path.append(int(node))
        node = int(parents[node])
    return path[::-1]


@pytest.mark.parametrize("cap", [4096, 70000])
def test_replays_of_a_captured_commit_and_compaction_equal_the_eager_calls(cap):
    """A KV commit followed by pad compaction (above 65,536 slots with the
    sliced pad scan), captured once.  Every replay starts from the same cache
    and must leave exactly what the eager calls leave, which in turn is what
    the oracle's commit and compaction give."""
    import oracle
    rng = np.random.default_rng(9200 + cap)
    B, Hkv, D, depth = 2, 2, 128, 3
    tree = synth.layered_tree(rng, (3, 4, 3))
    N = tree.n
    lens_np = np.array([cap - 40, cap // 3], np.int32)
    k_np = synth.draw_normal(rng, (B, Hkv, cap, D), 1.0, "bf16")
    v_np = synth.draw_normal(rng, (B, Hkv, cap, D), 1.0, "bf16")
    pad_np = np.zeros((B, cap), dtype=np.uint8)
    for b in range(B):
        pad_np[b, :lens_np[b]] = synth.pad_groups(rng, int(lens_np[b]), n_groups=6)
    tk_np = synth.draw_normal(rng, (B, Hkv, N, D), 1.0, "bf16")
    tv_np = synth.draw_normal(rng, (B, Hkv, N, D), 1.0, "bf16")
    deep = _chain_to(tree.parents, N - 1)
    assert len(deep) == depth
    al_np = np.array([depth, 1], np.int32)
    ap_np = np.full((B, depth), -1, np.int32)
    ap_np[0] = deep
    ap_np[1, 0] = deep[0]

    start = dict(k=dev(k_np), v=dev(v_np), cl=dev(lens_np), pad=dev(pad_np))
    state = {n: t.clone() for n, t in start.items()}
    tk, tv, al, ap = dev(tk_np), dev(tv_np), dev(al_np), dev(ap_np)
    n_app = torch.empty(1, dtype=torch.int32, device="cuda")
    ws_c = skg.new_workspace(skg.commit_workspace_bytes(), "cuda")
    ws_x = skg.new_workspace(skg.compact_workspace_bytes(B), "cuda")

    def reset():
        for n, t in state.items():
            t.copy_(start[n])

    def step():
        skg.spec_kv_commit(state["k"], state["v"], state["cl"], state["pad"], tk, tv, al, ap,
                           n_appended=n_app, workspace=ws_c)
        skg.spec_kv_compact(state["k"], state["v"], state["cl"], state["pad"], workspace=ws_x)

    step()
    torch.cuda.synchronize()
    eager = {n: t.clone() for n, t in state.items()}
    eager_n = n_app.clone()

    ck, cv, ccl, cpad, P, cerr = oracle.commit_ref(k_np, v_np, lens_np, pad_np, tk_np, tv_np,
                                                   al_np, ap_np, depth)
    wk, wv, wcl, wpad, werr = oracle.compact_ref(ck, cv, ccl, cpad)
    assert cerr == 0 and werr == 0
    assert int(eager_n[0]) == P
    np.testing.assert_array_equal(eager["cl"].cpu().numpy(), wcl)
    np.testing.assert_array_equal(eager["pad"].cpu().numpy(), wpad)
    gk, gv = _bits(eager["k"]), _bits(eager["v"])
    for b in range(B):
        n = int(wcl[b])
        np.testing.assert_array_equal(gk[b, :, :n], wk[b, :, :n])
        np.testing.assert_array_equal(gv[b, :, :n], wv[b, :, :n])

    reset()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    reset()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        reset()                             # eager work between the replays
        n_app.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n, t in state.items():
            assert torch.equal(t, eager[n]), (rep, n)
        assert torch.equal(n_app, eager_n), rep
    for w in (ws_c, ws_x):
        assert skg.spec_device_status(w) == 0
