"""One workspace, zero-filled once, shared by every kind of call in a decode
loop: window and budget drafts, tree verify, acceptance, budget selection,
pad compaction, the fp32 path and a long pooled verify, at different shapes,
twice over.  Every output must equal, bit for bit, the same call made on a
fresh workspace: no call may leave anything behind that another call reads
as a counter.
"""
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


def _bits(x):
    if isinstance(x, (tuple, list)):
        return [_bits(y) for y in x]
    if x is None:
        return None
    x = x.detach()
    if x.dtype == torch.bfloat16:
        x = x.view(torch.int16)
    elif x.dtype == torch.float32:
        x = x.view(torch.int32)
    return x.cpu().numpy().copy()


def _equal(a, b):
    if isinstance(a, list):
        return len(a) == len(b) and all(_equal(x, y) for x, y in zip(a, b))
    if a is None:
        return b is None
    return np.array_equal(a, b)


def _calls():
    """(name, fn(workspace) -> outputs, workspace bytes) for a decode loop's
    calls at several shapes."""
    s = 1 / math.sqrt(128)
    rng = np.random.default_rng(4242)
    tree = synth.layered_tree(rng, (10, 18, 18, 18))
    case = synth.make_attn_case(4243, B=2, Hq=32, Hkv=8, D=128, L_cap=6000, T=tree.n,
                                cache_len=[6000, 4321], value_scale=s)
    q, k, v, cl = dev(case.q), dev(case.k), dev(case.v), dev(case.cache_len)
    tk = dev(synth.draw_normal(rng, (2, 8, tree.n, 128), s, "bf16"))
    tv = dev(synth.draw_normal(rng, (2, 8, tree.n, 128), s, "bf16"))
    par = dev(tree.parents)
    pad = np.zeros((2, 6000), dtype=np.uint8)
    for b in range(2):
        pad[b, :case.cache_len[b]] = synth.pad_groups(rng, int(case.cache_len[b]))
    padd = dev(pad)
    q3 = q[:, :3].contiguous()
    q1 = q[:, :1].contiguous()
    idx = np.stack([np.stack([synth.budget_indices(rng, int(case.cache_len[b]), 700)
                              for _ in range(8)]) for b in range(2)])
    idxd = dev(idx)
    acc = synth.make_accept_case(4244, tree, 2, 5000)
    logits, toks, apar = dev(acc.logits), dev(acc.tokens), dev(acc.parents)
    # a long single sequence whose chain verify takes chunks from the pool
    # (63 splits of 33 tiles over 65,536 keys)
    lcase = synth.make_attn_case(4245, B=1, Hq=32, Hkv=8, D=128, L_cap=65536, T=3,
                                 value_scale=s)
    lq, lk, lv, lcl = dev(lcase.q), dev(lcase.k), dev(lcase.v), dev(lcase.cache_len)
    ltk = dev(synth.draw_normal(rng, (1, 8, 3, 128), s, "bf16"))
    ltv = dev(synth.draw_normal(rng, (1, 8, 3, 128), s, "bf16"))
    lpar = dev(np.array([-1, 0, 1], dtype=np.int32))
    # fp32 tiny case
    fcase = synth.make_attn_case(4246, B=1, Hq=2, Hkv=1, D=64, L_cap=512, T=15, dtype="f32")
    ftree = synth.heap_tree(2, 3)
    frng = np.random.default_rng(4247)
    ftk = dev(synth.draw_normal(frng, (1, 1, 15, 64), 1.0, "f32"))
    ftv = dev(synth.draw_normal(frng, (1, 1, 15, 64), 1.0, "f32"))
    means = skg.spec_block_means(k, cl, 16, pad=padd)
    torch.cuda.synchronize()

    dims = skg.make_dims(2, 32, 8, 128, skg.SPEC_BF16)
    ldims = skg.make_dims(1, 32, 8, 128, skg.SPEC_BF16)
    fdims = skg.make_dims(1, 2, 1, 64, skg.SPEC_F32)

    def compact(ws):
        kk, vv, cc, pp = k.clone(), v.clone(), cl.clone(), padd.clone()
        skg.spec_kv_compact(kk, vv, cc, pp, workspace=ws)
        return kk, vv, cc, pp

    return [
        ("window draft, 3 queries",
         lambda ws: skg.spec_attn_draft_sparse(q3, k, v, cl, n_sink=4, window=256, workspace=ws),
         skg.draft_workspace_bytes(dims, 3, 4 + 256 + 2)),
        ("budget draft, per-head lists of 700",
         lambda ws: skg.spec_attn_draft_sparse(q1, k, v, cl, idx=idxd, workspace=ws),
         skg.draft_workspace_bytes(dims, 1, 700)),
        ("padded 64-node tree verify",
         lambda ws: skg.spec_attn_verify_tree(q, k, v, cl, tk, tv, par, pad=padd, workspace=ws),
         skg.verify_workspace_bytes(dims, tree.n, 6000)),
        ("acceptance",
         lambda ws: skg.spec_accept_greedy(logits, toks, apar, acc.max_depth, workspace=ws),
         skg.accept_workspace_bytes(2, tree.n, 5000)),
        ("block selection",
         lambda ws: skg.spec_select_blocks(q1, means, cl, block=16, capacity=6000, n_sink=4,
                                           window=256, n_select=20, budget=600, pad=padd,
                                           workspace=ws),
         skg.select_workspace_bytes(dims, means.shape[2])),
        ("pooled chain verify over 65,536 keys (deterministic)",
         lambda ws: skg.spec_attn_verify_tree(lq, lk, lv, lcl, ltk, ltv, lpar, workspace=ws,
                                              deterministic=True),
         skg.verify_workspace_bytes(ldims, 3, 65536)),
        ("pad compaction",
         compact, skg.compact_workspace_bytes(2)),
        ("window draft, 1 query",
         lambda ws: skg.spec_attn_draft_sparse(q1, k, v, cl, n_sink=4, window=1000, workspace=ws),
         skg.draft_workspace_bytes(dims, 1, 4 + 1000)),
        ("fp32 tree verify",
         lambda ws: skg.spec_attn_verify_tree(dev(fcase.q), dev(fcase.k), dev(fcase.v),
                                              dev(fcase.cache_len), ftk, ftv,
                                              dev(ftree.parents), workspace=ws),
         skg.verify_workspace_bytes(fdims, 15, 512)),
    ]


def test_one_workspace_serves_every_call_kind_and_shape():
    calls = _calls()
    fresh = []
    for name, fn, nbytes in calls:
        fresh.append(_bits(fn(skg.new_workspace(nbytes, "cuda"))))
        torch.cuda.synchronize()
    shared = skg.new_workspace(max(n for _, _, n in calls), "cuda")
    for rnd in range(2):
        for (name, fn, _), want in zip(calls, fresh):
            got = _bits(fn(shared))
            torch.cuda.synchronize()
            assert _equal(got, want), f"round {rnd}: {name} differs on the shared workspace"
    assert skg.spec_device_status(shared) == 0
    # every counter is back at zero
    counters = shared[256:256 + (1 << 20)]
    assert int(counters.count_nonzero()) == 0


def test_calls_on_separate_streams_with_separate_workspaces():
    """Every kind of call at once, each on a stream and a workspace of its
    own, three rounds: the calls share no hidden state (counters, scratch)
    beyond their workspaces, so every output equals, bit for bit, the same
    call run alone."""
    calls = _calls()
    alone = []
    for name, fn, nbytes in calls:
        alone.append(_bits(fn(skg.new_workspace(nbytes, "cuda"))))
        torch.cuda.synchronize()
    main = torch.cuda.current_stream()
    streams = [torch.cuda.Stream() for _ in calls]   # (default priority)
    spaces = [skg.new_workspace(nbytes, "cuda") for _, _, nbytes in calls]
    torch.cuda.synchronize()
    for rnd in range(3):
        outs = []
        for (name, fn, _), st, ws in zip(calls, streams, spaces):
            st.wait_stream(main)
            with torch.cuda.stream(st):
                outs.append(fn(ws))
        for st in streams:
            main.wait_stream(st)
        torch.cuda.synchronize()
        for (name, _, _), got, want in zip(calls, outs, alone):
            assert _equal(_bits(got), want), f"round {rnd}: {name} differs when run beside the others"
    for ws in spaces:
        assert skg.spec_device_status(ws) == 0
