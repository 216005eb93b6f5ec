#!/usr/bin/env python3
"""Benchmark of the speculative-decoding attention hot path on one MI355X.

Headline workload: the million-token windowed-draft decode step.  One
sequence with 1,048,576 cached tokens and 32 layers of bf16 KV (8 KV heads x
head_dim 128, 128 GiB resident in HBM).  Per layer: verify attention of a
3-token chain over the full cache, one draft "context" call (3 chained
queries) and 3 single-query draft calls over sink 4 + window 4096; then one
greedy acceptance over a 128256-token vocabulary.  The step time decomposes
as t_verify + t_ctx_draft + 3 t_fwd_draft (per layer) + t_accept.

Reported: algorithmic KV bytes per step / step time (GB/s, against the 8 TB/s
HBM peak), steps per second, the per-component times, the roofline position
of the dominant kernel (verify) measured with HIP events on the launch
stream, the 16K-context batch-8 step per draft budget, the 4K-context
step and the ragged batch of 16 with its 44- and 64-node trees, and the fp64
CPU oracle timed on a bounded sample of the same workload.

Inputs are seeded synthetic draws (no datasets, no weights); everything is
resident on the GPU before the timed region starts.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KV-attn HBM GB/s (% of peak) + draft+verify steps/sec, 16K and 1M ctx, 1 GPU"
HBM_PEAK_GBS = 8000.0
L1M, LAYERS, HQ, HKV, D, CHAIN, VOCAB = 1 << 20, 32, 32, 8, 128, 3, 128256
SINK, WINDOW = 4, 4096
ESZ = 2
ACCEPT_16K_BYTES = 8 * 65 * VOCAB * 4   # the acceptance's fp32 logits, 16K batch of 8, 64 nodes


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------ algorithmic bytes

def window_view_len(L, T, sink, window):
    """Keys one KV head reads for T chained queries over sink + window: the
    sink part plus the union of the T windows (each key read once)."""
    s_len = min(sink, L)
    w_start = min(max(sink, L - T + 1 - window, 0), L)
    return s_len + (L - w_start)


def draft_bytes(B, L, T, view):
    kv = B * HKV * view * 2 * D * ESZ
    q_out = 2 * B * T * HQ * D * ESZ + B * T * HQ * 4
    return kv + q_out


def verify_bytes(B, L_sum, N, pad=False):
    kv = HKV * (L_sum + B * N) * 2 * D * ESZ
    q_out = 2 * B * N * HQ * D * ESZ + B * N * HQ * 4 + B * N * 4
    return kv + q_out + (L_sum if pad else 0)


def accept_bytes(B, N, V):
    return B * (N + 1) * V * 4 + B * N * 4 * 2


def _percentiles(vals):
    """p10, p50 (median) and p90 of a list of per-call times (ms)."""
    v = sorted(vals)
    pick = lambda q: v[min(len(v) - 1, int(round(q * (len(v) - 1))))]  # noqa: E731
    return [round(pick(0.1), 5), round(pick(0.5), 5), round(pick(0.9), 5)]


# ------------------------------------------------------------ HIP graphs

def graph_replay_ms(torch, fn, reps):
    """Capture fn() (a sequence of library calls on the current stream) into
    one HIP graph and return the device time per replay over `reps` replays
    bracketed by two events: the step without host launch costs."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    graph.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        graph.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps, graph


# ------------------------------------------------------------ 1M workload

def prerecord(events, torch):
    """Record every event once outside the measured pass: a timing event
    creates its device event at its first record, which costs far more than
    a later record."""
    for e in events:
        e.record()
    torch.cuda.synchronize()


def run_1m(args, torch, skg):
    import synth.device_gen as dg
    dev = torch.device("cuda:0")
    t0 = time.time()
    layers = []
    for li in range(args.layers):
        layers.append(dg.layer_1m(li, device=dev))
        if li % 8 == 7:
            torch.cuda.synchronize()
            log(f"[bench] generated layer {li + 1}/{args.layers} ({time.time() - t0:.1f}s)")
    torch.cuda.synchronize()
    log(f"[bench] generated {args.layers} layers of 1M-token KV in {time.time() - t0:.1f}s")

    cache_len = torch.tensor([L1M], dtype=torch.int32, device=dev)
    parents = torch.tensor([-1, 0, 1], dtype=torch.int32, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(synth_seed(4) + 999)
    logits = torch.randn((1, CHAIN + 1, VOCAB), generator=g, device=dev, dtype=torch.float32)
    tokens = torch.randint(0, VOCAB, (1, CHAIN), generator=g, device=dev, dtype=torch.int32)

    dims = skg.make_dims(1, HQ, HKV, D, skg.SPEC_BF16)
    ws_v = skg.new_workspace(skg.verify_workspace_bytes(dims, CHAIN, L1M), dev)
    ws_c = skg.new_workspace(skg.draft_workspace_bytes(dims, CHAIN, SINK + WINDOW + CHAIN - 1), dev)
    ws_f = skg.new_workspace(skg.draft_workspace_bytes(dims, 1, SINK + WINDOW), dev)
    ws_a = skg.new_workspace(skg.accept_workspace_bytes(1, CHAIN, VOCAB), dev)
    v_out = torch.empty((1, CHAIN, HQ, D), dtype=torch.bfloat16, device=dev)
    v_lse = torch.empty((1, CHAIN, HQ), dtype=torch.float32, device=dev)
    v_pos = torch.empty((1, CHAIN), dtype=torch.int32, device=dev)
    c_out = torch.empty_like(v_out)
    c_lse = torch.empty_like(v_lse)
    f_out = torch.empty((1, 1, HQ, D), dtype=torch.bfloat16, device=dev)
    f_lse = torch.empty((1, 1, HQ), dtype=torch.float32, device=dev)
    acc = [torch.empty(1, dtype=torch.int32, device=dev),
           torch.empty((1, CHAIN), dtype=torch.int32, device=dev),
           torch.empty(1, dtype=torch.int32, device=dev)]

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def step(marks=None):
        for li, lay in enumerate(layers):
            e = marks[li] if marks else None
            if e: e[0].record()
            skg.spec_attn_verify_tree(lay["verify_q"], lay["k"], lay["v"], cache_len,
                                      lay["tree_k"], lay["tree_v"], parents, out=v_out, lse=v_lse,
                                      pos_ids=v_pos, workspace=ws_v)
            if e: e[1].record()
            skg.spec_attn_draft_sparse(lay["ctx_q"], lay["k"], lay["v"], cache_len, n_sink=SINK,
                                       window=WINDOW, out=c_out, lse=c_lse, workspace=ws_c)
            if e: e[2].record()
            for fq in lay["fwd_q"]:
                skg.spec_attn_draft_sparse(fq, lay["k"], lay["v"], cache_len, n_sink=SINK,
                                           window=WINDOW, out=f_out, lse=f_lse, workspace=ws_f)
            if e: e[3].record()
        skg.spec_accept_greedy(logits, tokens, parents, CHAIN, accept_len=acc[0],
                               accept_path=acc[1], bonus=acc[2], workspace=ws_a)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    for w in (ws_v, ws_c, ws_f, ws_a):
        assert skg.spec_device_status(w) == 0, "device range error during warmup"

    # The timed loop records only its two bracketing events: an event recorded
    # between two kernels idles the GPU for about 5 us, so the per-call
    # breakdown comes from a second, instrumented pass over the same steps.
    start, stop = ev(), ev()
    torch.cuda.synchronize()
    start.record()
    t_wall = time.perf_counter()
    for _ in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_step = start.elapsed_time(stop) / args.steps

    marks = [[[ev() for _ in range(4)] for _ in layers] for _ in range(args.steps)]
    prerecord([e for st in marks for m in st for e in m], torch)
    a, b = ev(), ev()
    a.record()
    for k in range(args.steps):
        step(marks[k])
    b.record()
    torch.cuda.synchronize()
    ms_step_marked = a.elapsed_time(b) / args.steps

    # The same step captured in a HIP graph and replayed.  A replay must
    # reproduce the eager step's integer outputs (position ids, acceptance)
    # exactly and its attention outputs within rounding: the long verify
    # splits take their tile chunks from a shared pool at run time, so the
    # order of the fp32 sums, and with it the last bit, can differ.
    step()
    torch.cuda.synchronize()
    att = (v_out, v_lse, c_out, c_lse, f_out, f_lse)
    ints = (v_pos, *acc)
    eager_att = [t.float().clone() for t in att]
    eager_int = [t.clone() for t in ints]
    for t in att:
        t.fill_(0)
    graph_ms, graph = graph_replay_ms(torch, step, args.steps)
    graph_ints_equal = all(bool(torch.equal(x, y)) for x, y in zip(eager_int, ints))
    graph_att_diff = max(float((x - y.float()).abs().max()) for x, y in zip(eager_att, att))
    del graph
    for w in (ws_v, ws_c, ws_f, ws_a):
        assert skg.spec_device_status(w) == 0, "device range error in the graph replays"
    assert graph_ints_equal, "graph replay changed an integer output"
    assert graph_att_diff <= 1e-2, f"graph replay moved an attention output by {graph_att_diff}"

    # The verify in both modes, back to back over every layer: the pooled
    # default and SPEC_FLAG_DETERMINISTIC (fixed split ranges), whose outputs
    # must repeat bit for bit.
    def verify_pass(det):
        for lay in layers:
            skg.spec_attn_verify_tree(lay["verify_q"], lay["k"], lay["v"], cache_len,
                                      lay["tree_k"], lay["tree_v"], parents, out=v_out, lse=v_lse,
                                      pos_ids=v_pos, workspace=ws_v, deterministic=det)
    mode_ms = {}
    n_layers = len(layers)
    for det in (False, True, False, True):
        verify_pass(det)
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        for _ in range(max(args.steps // 2, 2)):
            verify_pass(det)
        b.record()
        torch.cuda.synchronize()
        mode_ms.setdefault(det, []).append(a.elapsed_time(b) / (max(args.steps // 2, 2) * n_layers))
    det_bits = []
    for _ in range(3):
        skg.spec_attn_verify_tree(layers[0]["verify_q"], layers[0]["k"], layers[0]["v"], cache_len,
                                  layers[0]["tree_k"], layers[0]["tree_v"], parents, out=v_out,
                                  lse=v_lse, pos_ids=v_pos, workspace=ws_v, deterministic=True)
        det_bits.append((v_out.view(torch.int16).clone(), v_lse.clone()))
    torch.cuda.synchronize()
    det_equal = all(torch.equal(x[0], det_bits[0][0]) and torch.equal(x[1], det_bits[0][1])
                    for x in det_bits[1:])
    assert det_equal, "deterministic verify differs between runs"
    verify_modes = {"pooled_ms": round(min(mode_ms[False]), 4),
                    "deterministic_ms": round(min(mode_ms[True]), 4),
                    "deterministic_cost": round(min(mode_ms[True]) / min(mode_ms[False]) - 1, 4),
                    "deterministic_runs_bitwise_equal": det_equal}

    t_verify = [m[0].elapsed_time(m[1]) for st in marks for m in st]
    t_ctx = [m[1].elapsed_time(m[2]) for st in marks for m in st]
    t_fwd = [m[2].elapsed_time(m[3]) / CHAIN for st in marks for m in st]
    n = args.layers
    per_step_verify = sum(t_verify) / args.steps
    per_step_ctx = sum(t_ctx) / args.steps
    per_step_fwd = sum(t_fwd) * CHAIN / args.steps
    t_acc = max(ms_step_marked - per_step_verify - per_step_ctx - per_step_fwd, 0.0)

    vb = verify_bytes(1, L1M, CHAIN)
    cb = draft_bytes(1, L1M, CHAIN, window_view_len(L1M, CHAIN, SINK, WINDOW))
    fb = draft_bytes(1, L1M, 1, window_view_len(L1M, 1, SINK, WINDOW))
    ab = accept_bytes(1, CHAIN, VOCAB)
    step_bytes = n * (vb + cb + CHAIN * fb) + ab
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    v_avg_ms = sum(t_verify) / len(t_verify)
    v_gbs = vb / (v_avg_ms * 1e-3) / 1e9
    ctx_gbs = cb / (sum(t_ctx) / len(t_ctx) * 1e-3) / 1e9
    fwd_gbs = fb / (sum(t_fwd) / len(t_fwd) * 1e-3) / 1e9
    res = dict(
        ms_step=ms_step, gbs=gbs, steps_per_s=1e3 / ms_step, step_bytes=step_bytes,
        wall_ms_per_step=t_wall * 1e3 / args.steps, ms_step_with_call_marks=ms_step_marked,
        components_ms=dict(t_verify=per_step_verify, t_ctx_draft=per_step_ctx,
                           t_fwd_draft=per_step_fwd, t_accept_and_gaps=t_acc,
                           verify_per_layer=v_avg_ms,
                           ctx_draft_per_call=sum(t_ctx) / len(t_ctx),
                           fwd_draft_per_call=sum(t_fwd) / len(t_fwd)),
        call_gbs=dict(verify=v_gbs, ctx_draft=ctx_gbs, fwd_draft=fwd_gbs),
        call_ms_percentiles={name: dict(zip(("p10", "p50", "p90"), _percentiles(vals)))
                             for name, vals in (("verify", t_verify), ("ctx_draft", t_ctx),
                                                ("fwd_draft", t_fwd))},
        verify_bytes_per_launch=vb, verify_avg_ms=v_avg_ms,
        graph=dict(ms_step=graph_ms, steps_per_s=1e3 / graph_ms,
                   gbs=step_bytes / (graph_ms * 1e-3) / 1e9,
                   replay_int_outputs_equal=graph_ints_equal,
                   replay_attn_max_abs_diff=graph_att_diff),
        verify_modes=verify_modes,
    )
    return res, layers


def synth_seed(c):
    import synth
    return synth.SEEDS[c]


# ------------------------------------------------------------ 8K and 16K workloads

def run_ctx(args, torch, skg, L, seed):
    """Batch 8 x L context (16,384, or the 8,192 point of BudgetDraft's
    4K / 8K / 16K sweep); per draft budget B: t_verify(64-node tree) +
    4 t_draft(B) + t_accept.  The KV is rotated over 16 copies (8 GiB at
    16K, 4 GiB at 8K) so the 256 MB Infinity Cache does not serve the timed
    reads."""
    import numpy as np
    import synth
    dev = torch.device("cuda:0")
    Bsz, ROT = 8, 16
    s = 1.0 / math.sqrt(D)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed + 500)
    kvs = []
    for _ in range(ROT):
        k = (torch.randn((Bsz, HKV, L, D), generator=gen, device=dev) * s).to(torch.bfloat16)
        v = (torch.randn((Bsz, HKV, L, D), generator=gen, device=dev) * s).to(torch.bfloat16)
        kvs.append((k, v))
    tree = synth.layered_tree(np.random.default_rng(seed), (10, 18, 18, 18))
    N = tree.n
    parents = torch.from_numpy(tree.parents).to(dev)
    vq = (torch.randn((Bsz, N, HQ, D), generator=gen, device=dev) * s).to(torch.bfloat16)
    tk = (torch.randn((Bsz, HKV, N, D), generator=gen, device=dev) * s).to(torch.bfloat16)
    tv = (torch.randn((Bsz, HKV, N, D), generator=gen, device=dev) * s).to(torch.bfloat16)
    dq = (torch.randn((Bsz, 1, HQ, D), generator=gen, device=dev) * s).to(torch.bfloat16)
    cache_len = torch.full((Bsz,), L, dtype=torch.int32, device=dev)
    logits = torch.randn((Bsz, N + 1, VOCAB), generator=gen, device=dev)
    tokens = torch.randint(0, VOCAB, (Bsz, N), generator=gen, device=dev, dtype=torch.int32)
    rng = np.random.default_rng(seed + 1)
    dims = skg.make_dims(Bsz, HQ, HKV, D, skg.SPEC_BF16)
    ws_v = skg.new_workspace(skg.verify_workspace_bytes(dims, N, L), dev)
    ws_a = skg.new_workspace(skg.accept_workspace_bytes(Bsz, N, VOCAB), dev)
    out = {}
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    reps = max(args.steps, 4)
    for bud in (256, 512, 1024, 2048):
        idx = torch.from_numpy(np.stack([synth.budget_indices(rng, L, bud) for _ in range(Bsz)])
                               [:, None, :]).to(dev)
        ws_d = skg.new_workspace(skg.draft_workspace_bytes(dims, 1, bud), dev)

        def step(i, marks=None):
            k, v = kvs[i % ROT]
            if marks: marks[0].record()
            skg.spec_attn_verify_tree(vq, k, v, cache_len, tk, tv, parents, workspace=ws_v)
            if marks: marks[1].record()
            for j in range(4):
                k2, v2 = kvs[(i + 1 + j) % ROT]
                skg.spec_attn_draft_sparse(dq, k2, v2, cache_len, idx=idx, workspace=ws_d)
            if marks: marks[2].record()
            skg.spec_accept_greedy(logits, tokens, parents, 4, workspace=ws_a)
            if marks: marks[3].record()

        for i in range(2):
            step(i)
        torch.cuda.synchronize()
        n_steps = reps * ROT // 4
        a, b = ev(), ev()
        a.record()
        for i in range(n_steps):
            step(i * 5)
        b.record()
        torch.cuda.synchronize()
        ms_step = a.elapsed_time(b) / n_steps
        # per-call breakdown from an instrumented pass (events between kernels
        # idle the GPU for a few microseconds each)
        marks = [[ev() for _ in range(4)] for _ in range(n_steps)]
        prerecord([e for m in marks for e in m], torch)
        for i, m in enumerate(marks):
            step(i * 5, m)
        torch.cuda.synchronize()
        tv_ms = sum(m[0].elapsed_time(m[1]) for m in marks) / len(marks)
        td_ms = sum(m[1].elapsed_time(m[2]) for m in marks) / len(marks) / 4
        ta_ms = sum(m[2].elapsed_time(m[3]) for m in marks) / len(marks)
        # HIP graph of 16 consecutive steps (one rotation cycle), replayed
        g_ms, graph = graph_replay_ms(torch, lambda: [step(i * 5) for i in range(ROT)], max(reps // 4, 2))
        del graph
        g_ms /= ROT
        vb = verify_bytes(Bsz, Bsz * L, N)
        db = draft_bytes(Bsz, L, 1, bud) + Bsz * bud * 4
        ab = accept_bytes(Bsz, N, VOCAB)
        out[str(bud)] = dict(
            context=L, graph_ms_step=g_ms, graph_steps_per_s=1e3 / g_ms,
            ms_step=ms_step, steps_per_s=1e3 / ms_step,
            gbs=(vb + 4 * db + ab) / (ms_step * 1e-3) / 1e9,
            t_verify_ms=tv_ms, t_draft_ms=td_ms, t_accept_ms=ta_ms,
            verify_gbs=vb / (tv_ms * 1e-3) / 1e9, draft_gbs=db / (td_ms * 1e-3) / 1e9,
            accept_gbs=ab / (ta_ms * 1e-3) / 1e9,
            verify_tflops=4 * D * HQ * N * Bsz * L / (tv_ms * 1e-3) / 1e12,
        )
    for w in (ws_v, ws_a):
        assert skg.spec_device_status(w) == 0
    del kvs
    torch.cuda.empty_cache()
    return out


def run_16k(args, torch, skg):
    import synth
    return run_ctx(args, torch, skg, 16384, synth.SEEDS[3])


def run_8k(args, torch, skg):
    import synth
    return run_ctx(args, torch, skg, 8192, synth.SEEDS["8k"])


# ------------------------------------------------------------ machine probes

def run_probes(torch):
    """What this GPU delivers, measured with the probe kernels: the HBM read
    rate of a plain streaming read of 4 GiB through each load path of the
    attention kernels (best over a few launch shapes), and the floor of a
    short call: an empty launch and a one-pass read of a draft call's 16.8 MB
    (the 1M window draft's K/V), both as HIP-graph replays of back-to-back
    launches, the reads rotating over 32 buffers (537 MB) so the Infinity
    Cache does not serve them."""
    import sparse_kv_attention_sink_amd._probe as pr
    pr.load()
    dev = torch.device("cuda:0")
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    sink = torch.zeros(1 << 16, dtype=torch.int32, device=dev)
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev)

    def timed(fn, reps=6):
        fn()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    shapes = {}
    for wg in (2048, 4096, 8192, 16384, 32768, 65536):
        for inf in (8, 16):
            ms = timed(lambda: pr.read(buf, wg, inf, sink))
            shapes[f"regs_wg{wg}_inflight{inf}"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    for wg in (256, 512):
        for st in (4, 6, 8):
            if wg == 512 and st > 4:
                continue   # two workgroups of more than 4 stages exceed the LDS of a CU
            ms = timed(lambda: pr.read_lds(buf, wg, st, sink))
            shapes[f"lds_wg{wg}_stages{st}"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    del buf
    best_regs = max(v for k, v in shapes.items() if k.startswith("regs"))
    best_lds = max(v for k, v in shapes.items() if k.startswith("lds"))

    g_ms, graph = graph_replay_ms(torch, lambda: [pr.empty(1, sink) for _ in range(100)], 10)
    del graph
    empty1 = g_ms / 100 * 1e3
    g_ms, graph = graph_replay_ms(torch, lambda: [pr.empty(256, sink) for _ in range(100)], 10)
    del graph
    empty256 = g_ms / 100 * 1e3
    small = 4100 * 4096   # the 1M window draft's K and V over 8 KV heads: 16,793,600 bytes
    bufs = [torch.ones(small // 2, dtype=torch.bfloat16, device=dev) for _ in range(32)]
    reads = {}
    for wg in (256, 512, 1024):
        g_ms, graph = graph_replay_ms(torch, lambda: [pr.read(b, wg, 4, sink) for b in bufs], 4)
        del graph
        reads[f"wg{wg}"] = round(g_ms / len(bufs) * 1e3, 2)
    del bufs
    # a one-pass read of the acceptance's logits at 16K (8 x 65 x 128,256
    # fp32), rotating over 4 buffers (1.07 GB): what a read of that size
    # reaches, ramp-up and tail included
    mid = ACCEPT_16K_BYTES
    mbufs = [torch.ones(mid // 2, dtype=torch.bfloat16, device=dev) for _ in range(4)]
    mids = {}
    for wg in (2048, 8192, 32768):
        for inf in (8, 16):
            g_ms, graph = graph_replay_ms(torch, lambda: [pr.read(b, wg, inf, sink) for b in mbufs], 4)
            del graph
            mids[f"regs_wg{wg}_inflight{inf}"] = round(mid / (g_ms / len(mbufs) * 1e-3) / 1e9, 1)
    del mbufs
    torch.cuda.empty_cache()
    return {"stream_read_gbs": max(best_regs, best_lds), "stream_read_regs_gbs": best_regs,
            "stream_read_lds_gbs": best_lds, "stream_read_bytes": nbytes, "shapes": shapes,
            "empty_launch_us": {"1_workgroup": round(empty1, 2), "256_workgroups": round(empty256, 2)},
            "read_16_8mb_us": reads, "read_16_8mb_floor_us": min(reads.values()),
            "read_267mb_gbs": mids, "read_267mb_best_gbs": max(mids.values())}


def tree_verify_roofline(r16):
    """Position of the 16K batch-8 64-node tree verify against both of its
    rooflines: its intensity (about 251 flop per byte) sits just below the
    ridge of 2.5 PFLOP/s dense bf16 over 8 TB/s (312), so HBM is the roof
    that bounds it, with the matrix cores close behind.  Per-call time from
    the budget-256 sweep's instrumented pass (events on the launch stream)."""
    if not r16:
        return None
    r = r16["256"]
    tf = r["verify_tflops"]
    return {"kernel": f"tree verify (64 nodes x GQA 4, batch 8 x {r['context']:,} keys)", "bound": "hbm",
            "achieved": round(r["verify_gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(r["verify_gbs"] / HBM_PEAK_GBS, 4),
            "mfma_tflops": round(tf, 1), "mfma_peak_tflops": 2500.0, "mfma_frac": round(tf / 2500.0, 4),
            "avg_launch_ms": round(r["t_verify_ms"], 4)}


# ------------------------------------------------------------ 4K and ragged workloads

def _timed_steps(torch, step, n_steps, n_marks):
    """Time n_steps calls of step(i) back to back (two events around the
    loop), then an instrumented pass whose n_marks events per step give the
    per-call breakdown (events between kernels idle the GPU for a few
    microseconds each, so the two are kept apart)."""
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    for i in range(2):
        step(i)
    torch.cuda.synchronize()
    a, b = ev(), ev()
    a.record()
    for i in range(n_steps):
        step(i)
    b.record()
    torch.cuda.synchronize()
    ms_step = a.elapsed_time(b) / n_steps
    marks = [[ev() for _ in range(n_marks)] for _ in range(n_steps)]
    prerecord([e for m in marks for e in m], torch)
    for i, m in enumerate(marks):
        step(i, m)
    torch.cuda.synchronize()
    parts = [sum(m[k].elapsed_time(m[k + 1]) for m in marks) / n_steps for k in range(n_marks - 1)]
    return ms_step, parts


def run_4k(args, torch, skg):
    """Llama-3-8B-shaped layer at 4K context, batch 1: t_verify(chain of 5) +
    5 t_draft(budget 256) + t_accept over 6 x 128256 logits.  The KV of one
    layer is 16.8 MB, so the step rotates over 64 layers' KV (1.07 GB) and the
    Infinity Cache does not serve the reads."""
    import numpy as np
    import synth
    dev = torch.device("cuda:0")
    Bsz, L, ROT, GAMMA, BUD = 1, 4096, 64, 5, 256
    s = 1.0 / math.sqrt(D)
    gen = torch.Generator(device=dev)
    gen.manual_seed(synth.SEEDS[2] + 500)
    kvs = [tuple((torch.randn((Bsz, HKV, L, D), generator=gen, device=dev) * s).to(torch.bfloat16)
                 for _ in range(2)) for _ in range(ROT)]
    tree = synth.chain_tree(GAMMA)
    parents = torch.from_numpy(tree.parents).to(dev)
    vq = (torch.randn((Bsz, GAMMA, HQ, D), generator=gen, device=dev) * s).to(torch.bfloat16)
    tk = (torch.randn((Bsz, HKV, GAMMA, D), generator=gen, device=dev) * s).to(torch.bfloat16)
    tv = (torch.randn((Bsz, HKV, GAMMA, D), generator=gen, device=dev) * s).to(torch.bfloat16)
    dq = (torch.randn((Bsz, 1, HQ, D), generator=gen, device=dev) * s).to(torch.bfloat16)
    cache_len = torch.full((Bsz,), L, dtype=torch.int32, device=dev)
    logits = torch.randn((Bsz, GAMMA + 1, VOCAB), generator=gen, device=dev)
    tokens = torch.randint(0, VOCAB, (Bsz, GAMMA), generator=gen, device=dev, dtype=torch.int32)
    idx = torch.from_numpy(synth.budget_indices(np.random.default_rng(synth.SEEDS[2] + 1), L, BUD)
                           [None, None, :]).to(dev)
    dims = skg.make_dims(Bsz, HQ, HKV, D, skg.SPEC_BF16)
    ws_v = skg.new_workspace(skg.verify_workspace_bytes(dims, GAMMA, L), dev)
    ws_d = skg.new_workspace(skg.draft_workspace_bytes(dims, 1, BUD), dev)
    ws_a = skg.new_workspace(skg.accept_workspace_bytes(Bsz, GAMMA, VOCAB), dev)

    def step(i, marks=None):
        k, v = kvs[(i * 6) % ROT]
        if marks: marks[0].record()
        skg.spec_attn_verify_tree(vq, k, v, cache_len, tk, tv, parents, workspace=ws_v)
        if marks: marks[1].record()
        for j in range(GAMMA):
            k2, v2 = kvs[(i * 6 + 1 + j) % ROT]
            skg.spec_attn_draft_sparse(dq, k2, v2, cache_len, idx=idx, workspace=ws_d)
        if marks: marks[2].record()
        skg.spec_accept_greedy(logits, tokens, parents, GAMMA, workspace=ws_a)
        if marks: marks[3].record()

    n_steps = max(args.steps, 4) * 8
    ms_step, (tv_ms, td5_ms, ta_ms) = _timed_steps(torch, step, n_steps, 4)
    # HIP graph of 32 consecutive steps (three rotation cycles), replayed
    g_ms, graph = graph_replay_ms(torch, lambda: [step(i) for i in range(32)], max(args.steps, 4))
    del graph
    g_ms /= 32
    vb = verify_bytes(Bsz, L, GAMMA)
    db = draft_bytes(Bsz, L, 1, BUD) + BUD * 4
    ab = accept_bytes(Bsz, GAMMA, VOCAB)
    for w in (ws_v, ws_d, ws_a):
        assert skg.spec_device_status(w) == 0
    del kvs
    torch.cuda.empty_cache()
    return dict(context=L, batch=Bsz, verify=f"chain of {GAMMA}", draft_budget=BUD,
                ms_step=round(ms_step, 4), steps_per_s=round(1e3 / ms_step, 1),
                gbs=round((vb + GAMMA * db + ab) / (ms_step * 1e-3) / 1e9, 1),
                graph_ms_step=round(g_ms, 4), graph_steps_per_s=round(1e3 / g_ms, 1),
                t_verify_us=round(tv_ms * 1e3, 2), t_draft_us=round(td5_ms * 1e3 / GAMMA, 2),
                t_accept_us=round(ta_ms * 1e3, 2),
                verify_gbs=round(vb / (tv_ms * 1e-3) / 1e9, 1),
                draft_gbs=round(db * GAMMA / (td5_ms * 1e-3) / 1e9, 1),
                accept_gbs=round(ab / (ta_ms * 1e-3) / 1e9, 1))


def run_ragged(args, torch, skg):
    """Batch of 16 with contexts drawn from U{2048..32768} and the tail pad
    pattern (the last 32 verify steps of 5 slots each, part of each group
    padding), for the 44-node (widths 10/14/12/8) and the 64-node
    (10/18/18/18) trees: t_verify + t_accept over 16 x (N+1) x 128256 logits.
    The KV (about 1.2 GB read per verify) rotates over 4 copies."""
    import numpy as np
    import synth
    dev = torch.device("cuda:0")
    Bsz, HI, ROT = 16, 32768, 4
    s = 1.0 / math.sqrt(D)
    rng = np.random.default_rng(synth.SEEDS[5])
    lens = rng.integers(2048, HI + 1, size=Bsz).astype(np.int32)
    pad_np = np.zeros((Bsz, HI), dtype=np.uint8)
    for b in range(Bsz):
        pad_np[b, :lens[b]] = synth.pad_groups(rng, int(lens[b]))
    gen = torch.Generator(device=dev)
    gen.manual_seed(synth.SEEDS[5] + 500)
    kvs = [tuple((torch.randn((Bsz, HKV, HI, D), generator=gen, device=dev) * s).to(torch.bfloat16)
                 for _ in range(2)) for _ in range(ROT)]
    cache_len = torch.from_numpy(lens).to(dev)
    pad = torch.from_numpy(pad_np).to(dev)
    dims = skg.make_dims(Bsz, HQ, HKV, D, skg.SPEC_BF16)
    L_sum = int(lens.sum())
    out = {"batch": Bsz, "context_sum": L_sum, "pad_slots": int(pad_np.sum())}
    for name, widths in (("tree44", (10, 14, 12, 8)), ("tree64", (10, 18, 18, 18))):
        tree = synth.layered_tree(rng, widths)
        N = tree.n
        parents = torch.from_numpy(tree.parents).to(dev)
        vq = (torch.randn((Bsz, N, HQ, D), generator=gen, device=dev) * s).to(torch.bfloat16)
        tk = (torch.randn((Bsz, HKV, N, D), generator=gen, device=dev) * s).to(torch.bfloat16)
        tv = (torch.randn((Bsz, HKV, N, D), generator=gen, device=dev) * s).to(torch.bfloat16)
        logits = torch.randn((Bsz, N + 1, VOCAB), generator=gen, device=dev)
        tokens = torch.randint(0, VOCAB, (Bsz, N), generator=gen, device=dev, dtype=torch.int32)
        ws_v = skg.new_workspace(skg.verify_workspace_bytes(dims, N, HI), dev)
        ws_a = skg.new_workspace(skg.accept_workspace_bytes(Bsz, N, VOCAB), dev)

        def step(i, marks=None):
            k, v = kvs[i % ROT]
            if marks: marks[0].record()
            skg.spec_attn_verify_tree(vq, k, v, cache_len, tk, tv, parents, pad=pad, workspace=ws_v)
            if marks: marks[1].record()
            skg.spec_accept_greedy(logits, tokens, parents, 4, workspace=ws_a)
            if marks: marks[2].record()

        n_steps = max(args.steps, 4) * 2
        ms_step, (tv_ms, ta_ms) = _timed_steps(torch, step, n_steps, 3)
        g_ms, graph = graph_replay_ms(torch, lambda: [step(i) for i in range(ROT)], max(args.steps // 2, 2))
        del graph
        g_ms /= ROT
        vb = verify_bytes(Bsz, L_sum, N, pad=True)
        ab = accept_bytes(Bsz, N, VOCAB)
        for w in (ws_v, ws_a):
            assert skg.spec_device_status(w) == 0
        out[name] = dict(nodes=N, ms_step=round(ms_step, 4), steps_per_s=round(1e3 / ms_step, 1),
                         graph_ms_step=round(g_ms, 4), graph_steps_per_s=round(1e3 / g_ms, 1),
                         gbs=round((vb + ab) / (ms_step * 1e-3) / 1e9, 1),
                         t_verify_us=round(tv_ms * 1e3, 2), t_accept_us=round(ta_ms * 1e3, 2),
                         verify_gbs=round(vb / (tv_ms * 1e-3) / 1e9, 1),
                         verify_tflops=round(4 * D * HQ * N * L_sum / (tv_ms * 1e-3) / 1e12, 1),
                         accept_gbs=round(ab / (ta_ms * 1e-3) / 1e9, 1))
        del logits
    del kvs
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------ compaction

def run_compact(torch, skg, reps=20):
    """Compaction of pad slots, in place, on the ragged batch of 16 (contexts
    2K-32K with the tail pad pattern of the last 32 verify steps) and on the
    1M-token sequence with the same tail pattern.  Every timed call starts
    from the padded state again (cache_len and pad restored outside the timed
    events; the rows it moves are the same each time)."""
    import numpy as np
    import synth
    dev = torch.device("cuda:0")
    out = {}
    for name, B, cap, lens in (("ragged_batch16", 16, 32768, None), ("1m", 1, L1M, [L1M])):
        rng = np.random.default_rng(synth.SEEDS[5] + 77)
        lens = rng.integers(2048, cap + 1, size=B).astype(np.int32) if lens is None \
            else np.asarray(lens, np.int32)
        pad_np = np.zeros((B, cap), dtype=np.uint8)
        for b in range(B):
            pad_np[b, :lens[b]] = synth.pad_groups(rng, int(lens[b]))
        k = torch.zeros((B, HKV, cap, D), dtype=torch.bfloat16, device=dev)
        v = torch.zeros_like(k)
        cl0 = torch.from_numpy(lens).to(dev)
        pad0 = torch.from_numpy(pad_np).to(dev)
        cl, pad = cl0.clone(), pad0.clone()
        ws = skg.new_workspace(skg.compact_workspace_bytes(B), dev)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        prerecord([e for p in ev for e in p], torch)
        for i in range(reps + 2):
            cl.copy_(cl0)
            pad.copy_(pad0)
            if i >= 2: ev[i - 2][0].record()
            skg.spec_kv_compact(k, v, cl, pad, workspace=ws)
            if i >= 2: ev[i - 2][1].record()
        torch.cuda.synchronize()
        assert skg.spec_device_status(ws) == 0
        assert cl.cpu().numpy().tolist() == [int(lens[b] - pad_np[b, :lens[b]].sum()) for b in range(B)]
        us = sum(a.elapsed_time(b) for a, b in ev) / reps * 1e3
        moved = 0
        for b in range(B):
            row = pad_np[b, :lens[b]]
            f = int(np.argmax(row)) if row.any() else int(lens[b])
            moved += int((row[f:] == 0).sum())
        out[name] = dict(batch=B, context_sum=int(lens.sum()), pad_slots=int(pad_np.sum()),
                         rows_moved_per_head=moved, us_per_call=round(us, 2),
                         bytes_moved=moved * HKV * 2 * D * ESZ * 2, pad_bytes_scanned=int(lens.sum()))
        del k, v
        torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------ KV commit

def run_commit(torch, skg, *, B, L, widths, depths, seed, reps=60):
    """Time the commit of accepted paths (the step after acceptance) on a
    batch of B caches holding L tokens each: a tree of the given widths, one
    accepted root path per sequence of the given depth, back-to-back calls
    (each appends P = 1 + max depth slots, so the capacity leaves room for
    all of them)."""
    import numpy as np
    import synth
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(seed)
    tree = synth.layered_tree(rng, widths)
    N, P = tree.n, 1 + max(depths)
    cap = L + (reps + 8) * P
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    k = torch.randn((B, HKV, cap, D), generator=g, device=dev).to(torch.bfloat16)
    v = torch.randn((B, HKV, cap, D), generator=g, device=dev).to(torch.bfloat16)
    tk = torch.randn((B, HKV, N, D), generator=g, device=dev).to(torch.bfloat16)
    tv = torch.randn((B, HKV, N, D), generator=g, device=dev).to(torch.bfloat16)
    maxd = int(tree.depth.max()) + 1
    path = np.full((B, maxd), -1, dtype=np.int32)
    for b, d in enumerate(depths):
        if d:
            node = int(rng.choice(np.nonzero(tree.depth == d - 1)[0]))
            p = []
            while node >= 0:
                p.append(node)
                node = int(tree.parents[node])
            path[b, :d] = p[::-1]
    alen = torch.tensor(depths, dtype=torch.int32, device=dev)
    apath = torch.from_numpy(path).to(dev)
    cl = torch.full((B,), L, dtype=torch.int32, device=dev)
    pad = torch.zeros((B, cap), dtype=torch.uint8, device=dev)
    ws = skg.new_workspace(skg.commit_workspace_bytes(), dev)
    n_out = torch.empty(1, dtype=torch.int32, device=dev)
    call = lambda: skg.spec_kv_commit(k, v, cl, pad, tk, tv, alen, apath, n_appended=n_out,  # noqa: E731
                                      workspace=ws)
    for _ in range(4):
        call()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    prerecord([a, b], torch)
    # A few-kernel call costs the host more than the device: park the stream
    # on a spin long enough for the host to queue every timed call, so the
    # events measure the device's back-to-back time.
    torch.cuda._sleep(int(2.5e6 + reps * 1.5e5))
    a.record()
    for _ in range(reps):
        call()
    b.record()
    torch.cuda.synchronize()
    assert skg.spec_device_status(ws) == 0
    us = a.elapsed_time(b) / reps * 1e3
    moved = 2 * sum(depths) * HKV * 2 * D * 2 + B * P
    return dict(us_per_call=round(us, 2), batch=B, context=L, tree_nodes=N,
                accept_len=list(depths), appended_slots=P, bytes_moved_per_call=moved,
                gbs=round(moved / (us * 1e-6) / 1e9, 1))


# ------------------------------------------------------------ partial verification

def run_partial_1m(torch, skg, layers, *, block=128, budget=4096, buffer=64, window=2048,
                   reps=3):
    """Partial verification at the 1M layer: per layer a block-mean table
    (blocks of 128), a shared selection (sink 4, window 2048, the rest in
    blocks), a partial cache of `budget` slots plus a buffer; then the
    chain-3 verify over each layer's partial cache, timed as a pass over the
    32 layers (as the step runs them), against the full-cache verify."""
    dev = torch.device("cuda:0")
    cl = torch.tensor([L1M], dtype=torch.int32, device=dev)
    parents = torch.tensor([-1, 0, 1], dtype=torch.int32, device=dev)
    n_select = (budget - 4 - window) // block
    nb = L1M // block
    dims = skg.make_dims(1, HQ, HKV, D, skg.SPEC_BF16)
    ws_s = skg.new_workspace(skg.select_workspace_bytes(dims, nb), dev)
    ws_v = skg.new_workspace(skg.verify_workspace_bytes(dims, CHAIN, budget + buffer), dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    # outputs allocated up front, so that the timed passes run kernels only
    means = torch.empty((1, HKV, nb, D), dtype=torch.float32, device=dev)
    idxs = [torch.empty((1, 1, budget), dtype=torch.int32, device=dev) for _ in layers]
    parts = []
    for _ in layers:
        pk = torch.zeros((1, HKV, budget + buffer, D), dtype=torch.bfloat16, device=dev)
        parts.append((pk, torch.zeros_like(pk), torch.empty(1, dtype=torch.int32, device=dev),
                      torch.zeros((1, budget + buffer), dtype=torch.uint8, device=dev)))

    def refresh(phase):
        for lay, idx, (pk, pv, plen, ppad) in zip(layers, idxs, parts):
            if phase in ("means", "all"):
                skg.spec_block_means(lay["k"], cl, block, means=means, workspace=ws_s)
            if phase in ("select", "all"):
                skg.spec_select_blocks(lay["verify_q"], means, cl, block=block, capacity=L1M,
                                       n_sink=4, window=window, n_select=n_select, budget=budget,
                                       shared=True, idx=idx, workspace=ws_s)
            if phase in ("gather", "all"):
                skg.spec_kv_gather(lay["k"], lay["v"], cl, idx, partial_k=pk, partial_v=pv,
                                   partial_len=plen, partial_pad=ppad, workspace=ws_s)
    refresh("all")
    torch.cuda.synchronize()
    t_phase = {}
    for phase in ("means", "select", "gather"):
        a, b = ev(), ev()
        prerecord([a, b], torch)
        torch.cuda._sleep(int(3e7))      # the host queues the whole pass first
        a.record()
        refresh(phase)
        b.record()
        torch.cuda.synchronize()
        t_phase[phase] = a.elapsed_time(b) / len(layers) * 1e3
    assert skg.spec_device_status(ws_s) == 0
    out = torch.empty((1, CHAIN, HQ, D), dtype=torch.bfloat16, device=dev)

    def pass_(pad=True):
        for lay, (pk, pv, plen, ppad) in zip(layers, parts):
            skg.spec_attn_verify_tree(lay["verify_q"], pk, pv, plen, lay["tree_k"], lay["tree_v"],
                                      parents, pad=ppad, out=out, want_lse=False,
                                      want_pos_ids=False, workspace=ws_v)
    pass_()
    torch.cuda.synchronize()
    a, b = ev(), ev()
    prerecord([a, b], torch)
    a.record()
    for _ in range(reps):
        pass_()
    b.record()
    torch.cuda.synchronize()
    assert skg.spec_device_status(ws_v) == 0
    per_layer_us = a.elapsed_time(b) / (reps * len(layers)) * 1e3
    part_bytes = HKV * (budget + buffer) * 2 * D * 2 + (budget + buffer)
    del parts, idxs, means
    torch.cuda.empty_cache()
    return dict(block=block, budget=budget, buffer=buffer, window=window, n_select=n_select,
                verify_partial_us_per_layer=round(per_layer_us, 2),
                verify_partial_gbs=round(part_bytes / (per_layer_us * 1e-6) / 1e9, 1),
                refresh_us_per_layer={k: round(v, 2) for k, v in t_phase.items()},
                refresh_note="per layer, at a full verification: the whole mean table (in a "
                             "decode loop only the blocks an append changed), the selection and "
                             "the gather of the partial cache")


# ------------------------------------------------------------ draft ring buffer

def run_ring_1m(torch, skg, layers, *, reps=3):
    """The 1M step's drafts (per layer one 3-query context call and three
    single-query calls, sink 4 + window 4096) over per-layer ring caches of
    4 + 4,098 slots, against the same calls over the full caches; each timed
    as a pass over the 32 layers with only its bracketing events."""
    dev = torch.device("cuda:0")
    cl = torch.tensor([L1M], dtype=torch.int32, device=dev)
    ring = WINDOW + CHAIN - 1
    pos = torch.arange(L1M - ring, L1M, device=dev)
    slots = SINK + (pos - SINK) % ring
    rings = []
    for lay in layers:
        kr = torch.empty((1, HKV, SINK + ring, D), dtype=torch.bfloat16, device=dev)
        vr = torch.empty_like(kr)
        kr[:, :, :SINK] = lay["k"][:, :, :SINK]
        vr[:, :, :SINK] = lay["v"][:, :, :SINK]
        kr[:, :, slots] = lay["k"][:, :, pos]
        vr[:, :, slots] = lay["v"][:, :, pos]
        rings.append((kr, vr))
    dims = skg.make_dims(1, HQ, HKV, D, skg.SPEC_BF16)
    ws_c = skg.new_workspace(skg.draft_workspace_bytes(dims, CHAIN, SINK + WINDOW + CHAIN - 1), dev)
    ws_f = skg.new_workspace(skg.draft_workspace_bytes(dims, 1, SINK + WINDOW), dev)
    out_c = torch.empty((1, CHAIN, HQ, D), dtype=torch.bfloat16, device=dev)
    out_f = torch.empty((1, 1, HQ, D), dtype=torch.bfloat16, device=dev)

    def ring_pass():
        for lay, (kr, vr) in zip(layers, rings):
            skg.spec_attn_draft_ring(lay["ctx_q"], kr, vr, cl, n_sink=SINK, window=WINDOW,
                                     ring=ring, out=out_c, want_lse=False, workspace=ws_c)
            for fq in lay["fwd_q"]:
                skg.spec_attn_draft_ring(fq, kr, vr, cl, n_sink=SINK, window=WINDOW, ring=ring,
                                         out=out_f, want_lse=False, workspace=ws_f)

    def full_pass():
        for lay in layers:
            skg.spec_attn_draft_sparse(lay["ctx_q"], lay["k"], lay["v"], cl, n_sink=SINK,
                                       window=WINDOW, out=out_c, want_lse=False, workspace=ws_c)
            for fq in lay["fwd_q"]:
                skg.spec_attn_draft_sparse(fq, lay["k"], lay["v"], cl, n_sink=SINK, window=WINDOW,
                                           out=out_f, want_lse=False, workspace=ws_f)

    res = {}
    for name, fn in (("ring", ring_pass), ("full_cache", full_pass)):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        prerecord([a, b], torch)
        torch.cuda._sleep(int(3e7))
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        res[name] = a.elapsed_time(b) / reps * 1e3 / len(layers)
    for w in (ws_c, ws_f):
        assert skg.spec_device_status(w) == 0
    del rings
    torch.cuda.empty_cache()
    row = 2 * D * 2 * HKV
    return dict(ring_slots=SINK + ring, draft_us_per_layer_ring=round(res["ring"], 2),
                draft_us_per_layer_full_cache=round(res["full_cache"], 2),
                draft_kv_bytes_per_layer_ring=(SINK + ring) * row,
                draft_kv_bytes_per_layer_full=L1M * row,
                note="per layer: one 3-query context call and three single-query calls")


# ------------------------------------------------------------ one GPU's shard

def run_shard_1m(torch, skg, layers, *, reps=3):
    """One GPU's share of the 1M step under 8-way sharding over KV heads:
    per layer one KV head (Hkv 1, its 4 query heads) over the same 1,048,576
    keys, taken as a strided view of the resident layer (layer i uses KV head
    i mod 8, so the 32 layers' shares do not fit the Infinity Cache): the
    chain-3 verify and the four draft calls, each timed as a pass over the 32
    layers with only its bracketing events."""
    dev = torch.device("cuda:0")
    G = HQ // HKV
    cl = torch.tensor([L1M], dtype=torch.int32, device=dev)
    par = torch.tensor([-1, 0, 1], dtype=torch.int32, device=dev)
    shards = []
    for li, lay in enumerate(layers):
        h = li % HKV
        sl = slice(h * G, (h + 1) * G)
        shards.append(dict(
            k=lay["k"][:, h:h + 1], v=lay["v"][:, h:h + 1],
            tree_k=lay["tree_k"][:, h:h + 1], tree_v=lay["tree_v"][:, h:h + 1],
            verify_q=lay["verify_q"][:, :, sl].contiguous(), ctx_q=lay["ctx_q"][:, :, sl].contiguous(),
            fwd_q=[f[:, :, sl].contiguous() for f in lay["fwd_q"]]))
    dims = skg.make_dims(1, G, 1, D, skg.SPEC_BF16)
    ws_v = skg.new_workspace(skg.verify_workspace_bytes(dims, CHAIN, L1M), dev)
    ws_c = skg.new_workspace(skg.draft_workspace_bytes(dims, CHAIN, SINK + WINDOW + CHAIN - 1), dev)
    ws_f = skg.new_workspace(skg.draft_workspace_bytes(dims, 1, SINK + WINDOW), dev)
    v_out = torch.empty((1, CHAIN, G, D), dtype=torch.bfloat16, device=dev)
    c_out = torch.empty_like(v_out)
    f_out = torch.empty((1, 1, G, D), dtype=torch.bfloat16, device=dev)

    def verify_pass():
        for s in shards:
            skg.spec_attn_verify_tree(s["verify_q"], s["k"], s["v"], cl, s["tree_k"], s["tree_v"],
                                      par, out=v_out, want_lse=False, want_pos_ids=False,
                                      workspace=ws_v)

    def draft_pass():
        for s in shards:
            skg.spec_attn_draft_sparse(s["ctx_q"], s["k"], s["v"], cl, n_sink=SINK, window=WINDOW,
                                       out=c_out, want_lse=False, workspace=ws_c)
            for fq in s["fwd_q"]:
                skg.spec_attn_draft_sparse(fq, s["k"], s["v"], cl, n_sink=SINK, window=WINDOW,
                                           out=f_out, want_lse=False, workspace=ws_f)

    res = {}
    for name, fn in (("verify", verify_pass), ("drafts", draft_pass)):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        prerecord([a, b], torch)
        torch.cuda._sleep(int(3e7))
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        res[name] = a.elapsed_time(b) / reps * 1e3 / len(shards)
    for w in (ws_v, ws_c, ws_f):
        assert skg.spec_device_status(w) == 0
    vbytes = verify_bytes(1, L1M, CHAIN) // HKV
    view = window_view_len(L1M, CHAIN, SINK, WINDOW)
    return dict(kv_heads=1, q_heads=G, context=L1M,
                verify_us_per_layer=round(res["verify"], 2),
                verify_gbs=round(vbytes / (res["verify"] * 1e-6) / 1e9, 1),
                drafts_us_per_layer=round(res["drafts"], 2),
                attention_ms_per_step=round((res["verify"] + res["drafts"]) * len(shards) * 1e-3, 3),
                note="one KV head per layer of the 32, as under 8-way KV-head sharding; "
                     "drafts = one 3-query and three single-query calls")


# ------------------------------------------------------------ budget selection

def run_select(torch, skg, *, B=8, L=16384, block=16, reps=24, seed=8400):
    """Time the block-mean table build (every block of a batch of B caches
    of L tokens) and the block selection per draft budget (window B/2, sink
    4, as many blocks as the rest holds).  Keys and tables are rotated over
    enough copies that the Infinity Cache does not serve them."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    s = 1.0 / math.sqrt(D)
    ROTK, ROTM = 4, 16
    ks = [(torch.randn((B, HKV, L, D), generator=g, device=dev) * s).to(torch.bfloat16)
          for _ in range(ROTK)]
    q = (torch.randn((B, 1, HQ, D), generator=g, device=dev) * s).to(torch.bfloat16)
    cl = torch.full((B,), L, dtype=torch.int32, device=dev)
    nb = L // block
    tables = [torch.empty((B, HKV, nb, D), dtype=torch.float32, device=dev) for _ in range(ROTM)]
    ws = skg.new_workspace(skg.select_workspace_bytes(skg.make_dims(B, HQ, HKV, D, skg.SPEC_BF16),
                                                      nb), dev)
    for i, t in enumerate(tables):
        skg.spec_block_means(ks[i % ROTK], cl, block, means=t, workspace=ws)
    torch.cuda.synchronize()

    def timed(fn, n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        prerecord([a, b], torch)
        torch.cuda._sleep(int(2.5e6 + n * 3e5))      # let the host queue every call first
        a.record()
        for i in range(n):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n * 1e3

    means_us = timed(lambda i: skg.spec_block_means(ks[i % ROTK], cl, block,
                                                    means=tables[i % ROTM], workspace=ws), reps)
    means_bytes = B * HKV * L * D * 2 + B * HKV * nb * D * 4
    out = dict(block=block, batch=B, context=L,
               means_table_us=round(means_us, 2),
               means_table_gbs=round(means_bytes / (means_us * 1e-6) / 1e9, 1),
               means_bytes=means_bytes, select={})
    for bud in (256, 512, 1024, 2048):
        win = bud // 2
        nsel = (bud - 4 - win) // block
        idx = torch.empty((B, HKV, bud), dtype=torch.int32, device=dev)
        fn = lambda i: skg.spec_select_blocks(q, tables[i % ROTM], cl, block=block,  # noqa: E731
                                              capacity=L, n_sink=4, window=win, n_select=nsel,
                                              budget=bud, idx=idx, workspace=ws)
        fn(0)
        us = timed(fn, reps)
        cand = (L - win - 4 + block - 1) // block
        sel_bytes = B * HKV * cand * D * 4 + B * HKV * bud * 4
        out["select"][str(bud)] = dict(n_select=nsel, us_per_call=round(us, 2),
                                       bytes_per_call=sel_bytes,
                                       gbs=round(sel_bytes / (us * 1e-6) / 1e9, 1))
    assert skg.spec_device_status(ws) == 0
    del ks, tables
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------ CPU baseline

def cpu_baseline(layers, torch, budget_s=12.0):
    """The fp64 oracle on a bounded sample of the 1M step: for layer 0, one KV
    head at a time, the verify of the 3-token chain over all 1,048,576 keys
    plus the context and single-query draft calls of that head's 4 query
    heads, until the time budget is spent."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    lay = layers[0]
    G = HQ // HKV

    def bits(t):
        return t.view(torch.int16).cpu().numpy().view(np.uint16)

    vq, tkk, tvv, cq = (bits(lay[n]) for n in ("verify_q", "tree_k", "tree_v", "ctx_q"))
    fq = [bits(x) for x in lay["fwd_q"]]
    par = np.array([-1, 0, 1], dtype=np.int32)
    cl = np.array([L1M], dtype=np.int32)
    done_bytes, heads = 0, 0
    t0 = time.perf_counter()
    elapsed = 0.0
    for g in range(HKV):
        kb = bits(lay["k"][:, g:g + 1])
        vb = bits(lay["v"][:, g:g + 1])
        t1 = time.perf_counter()
        hs = slice(g * G, (g + 1) * G)
        oracle.verify_attn_ref(vq[:, :, hs], kb, vb, cl, tkk[:, g:g + 1], tvv[:, g:g + 1], par,
                               scale=1 / math.sqrt(D))
        oracle.draft_attn_ref(cq[:, :, hs], kb, vb, cl, scale=1 / math.sqrt(D), n_sink=SINK,
                              window=WINDOW)
        for f in fq:
            oracle.draft_attn_ref(f[:, :, hs], kb, vb, cl, scale=1 / math.sqrt(D), n_sink=SINK,
                                  window=WINDOW)
        elapsed += time.perf_counter() - t1
        heads += 1
        done_bytes += (verify_bytes(1, L1M, CHAIN)
                       + draft_bytes(1, L1M, CHAIN, window_view_len(L1M, CHAIN, SINK, WINDOW))
                       + CHAIN * draft_bytes(1, L1M, 1, window_view_len(L1M, 1, SINK, WINDOW))) / HKV
        if elapsed >= budget_s:
            break
    return dict(value=done_bytes / elapsed / 1e9, unit="GB/s", cores=threads, kind="oracle",
                sample=f"1M step, layer 0, {heads} of 8 KV heads: chain-3 verify over 1,048,576 "
                       f"keys + 1 context and 3 single-query window draft calls per head "
                       f"(fp64 NumPy oracle, {elapsed:.1f}s; host cores visible: {os.cpu_count()})",
                seconds=elapsed)


# ------------------------------------------------------------ HBM traffic

PROFILE_DIR = os.path.join(ROOT, "profiles")
TRAFFIC_PROFILE = os.path.join(PROFILE_DIR, "verify_chain3_1m_hbm_traffic.md")


TRAFFIC_SOURCES = ("attn.hip", "api.hip", "dev_common.h", "spec_internal.h")


def source_digest():
    """sha256 over the sources of the verify kernel and of its launch plan,
    so that counter figures taken on other kernel code are never reported."""
    import hashlib
    h = hashlib.sha256()
    for name in TRAFFIC_SOURCES:
        h.update(name.encode())
        with open(os.path.join(ROOT, "sparse_kv_attention_sink_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per verify launch from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by the same counter's reading for a
    plain copy of known size), or None if it is missing or was taken on other
    kernel sources."""
    try:
        with open(TRAFFIC_PROFILE) as f:
            text = f.read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        line = line.strip().lstrip("-").strip()
        if ":" in line and line.split(":", 1)[0] in ("source_sha256", "traffic_bytes_per_launch"):
            k, v = line.split(":", 1)
            fields[k] = v.strip().strip("`")
    if fields.get("source_sha256") != source_digest() or "traffic_bytes_per_launch" not in fields:
        return None
    return int(fields["traffic_bytes_per_launch"])


def copy_probe(torch, gib=1, reps=4):
    """A plain device copy of known size, the calibration of the HBM byte
    counters: FETCH_SIZE and WRITE_SIZE of one dispatch of it should read
    gib GiB each."""
    n = gib << 30
    x = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "dispatches": reps}))


# ------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--layers", type=int, default=LAYERS)
    ap.add_argument("--skip-16k", action="store_true")
    ap.add_argument("--skip-1m", action="store_true",
                    help="only the 16K batch-8 sweep (for profiling it alone)")
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--ragged-only", action="store_true",
                    help="only the ragged batch of 16 (for profiling it alone)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a 1 GiB device copy (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the hot path needs no "
                                   "collectives, and --gpus above 1 is not supported"}))
        sys.exit(2)
    import torch
    import sparse_kv_attention_sink_amd as skg
    skg.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_probe:
        copy_probe(torch)
        return

    if args.ragged_only:
        print(json.dumps({"ragged": run_ragged(args, torch, skg)}), flush=True)
        return
    if args.skip_1m:
        print(json.dumps({"ctx16k": run_16k(args, torch, skg),
                          "ctx8k": run_8k(args, torch, skg)}), flush=True)
        return
    probes = run_probes(torch)
    log(f"[bench] stream read {probes['stream_read_gbs']} GB/s (registers "
        f"{probes['stream_read_regs_gbs']}, LDS copies {probes['stream_read_lds_gbs']}); empty "
        f"launch {probes['empty_launch_us']} us; 16.8 MB read {probes['read_16_8mb_floor_us']} us; "
        f"267 MB read {probes['read_267mb_best_gbs']} GB/s")
    r1m, layers = run_1m(args, torch, skg)
    log(f"[bench] 1M step: {r1m['ms_step']:.3f} ms, {r1m['gbs']:.1f} GB/s")
    cpu = None
    if not args.skip_cpu:
        cpu = cpu_baseline(layers, torch)
        log(f"[bench] cpu oracle: {cpu['value']:.3f} GB/s")
    ring = run_ring_1m(torch, skg, layers)
    log(f"[bench] ring drafts: {ring['draft_us_per_layer_ring']} us per layer "
        f"(full cache {ring['draft_us_per_layer_full_cache']} us)")
    shard = run_shard_1m(torch, skg, layers)
    log(f"[bench] 8-way KV-head shard of the 1M step: verify {shard['verify_us_per_layer']} us "
        f"per layer ({shard['verify_gbs']} GB/s), drafts {shard['drafts_us_per_layer']} us")
    partial = run_partial_1m(torch, skg, layers)
    partial["verify_full_us_per_layer"] = round(r1m["verify_avg_ms"] * 1e3, 2)
    log(f"[bench] partial verify: {partial['verify_partial_us_per_layer']} us per layer "
        f"(full {partial['verify_full_us_per_layer']} us)")
    del layers
    torch.cuda.empty_cache()
    r16 = None if args.skip_16k else run_16k(args, torch, skg)
    r8k = None if args.skip_16k else run_8k(args, torch, skg)
    r4k = run_4k(args, torch, skg)
    log(f"[bench] 4K step: {r4k['ms_step']} ms ({r4k['steps_per_s']} steps/s)")
    rrag = run_ragged(args, torch, skg)
    log(f"[bench] ragged batch: tree44 {rrag['tree44']['ms_step']} ms, "
        f"tree64 {rrag['tree64']['ms_step']} ms")
    commit = {
        "16k_batch8_tree64": run_commit(torch, skg, B=8, L=16384, widths=(10, 18, 18, 18),
                                        depths=[4, 3, 2, 1, 0, 4, 2, 3], seed=8300),
        "1m_chain3": run_commit(torch, skg, B=1, L=L1M, widths=(1, 1, 1), depths=[3], seed=8301),
    }
    log(f"[bench] kv commit: {commit['16k_batch8_tree64']['us_per_call']} us (16K batch 8), "
        f"{commit['1m_chain3']['us_per_call']} us (1M chain 3)")
    compact = run_compact(torch, skg)
    log(f"[bench] compaction: {compact['ragged_batch16']['us_per_call']} us (ragged batch 16), "
        f"{compact['1m']['us_per_call']} us (1M)")
    select = run_select(torch, skg)
    log(f"[bench] block means table: {select['means_table_us']} us; selection: "
        + ", ".join(f"{k} {v['us_per_call']} us" for k, v in select["select"].items()))

    v_ms = r1m["verify_avg_ms"]
    achieved = r1m["verify_bytes_per_launch"] / (v_ms * 1e-3) / 1e9
    ceil = probes["stream_read_gbs"]
    # every kernel's rate as a fraction of the measured stream-read ceiling
    vs_stream = {"verify_1m": round(achieved / ceil, 4),
                 "ctx_draft_1m": round(r1m["call_gbs"]["ctx_draft"] / ceil, 4),
                 "fwd_draft_1m": round(r1m["call_gbs"]["fwd_draft"] / ceil, 4)}
    for tag, r in (("16k", r16), ("8k", r8k)):
        if r:
            for bud, x in r.items():
                vs_stream[f"draft_{tag}_budget{bud}"] = round(x["draft_gbs"] / ceil, 4)
            vs_stream[f"tree_verify_{tag}"] = round(r["256"]["verify_gbs"] / ceil, 4)
            vs_stream[f"accept_{tag}"] = round(r["256"]["accept_gbs"] / ceil, 4)
    for tree_name in ("tree44", "tree64"):
        vs_stream[f"ragged_verify_{tree_name}"] = round(rrag[tree_name]["verify_gbs"] / ceil, 4)
    if r16:
        # the acceptance against a plain read of its own size (the 4 GiB
        # ceiling leaves out a 267 MB read's ramp-up and tail)
        vs_stream["accept_16k_vs_same_size_read"] = round(r16["256"]["accept_gbs"] / probes["read_267mb_best_gbs"], 4)
    floor = probes["read_16_8mb_floor_us"]
    draft_floor = {"read_16_8mb_floor_us": floor,
                   "empty_launch_us": probes["empty_launch_us"]["256_workgroups"],
                   "ctx_draft_1m_us": round(r1m["components_ms"]["ctx_draft_per_call"] * 1e3, 2),
                   "fwd_draft_1m_us": round(r1m["components_ms"]["fwd_draft_per_call"] * 1e3, 2)}
    line = {
        "metric": METRIC,
        "value": round(r1m["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r1m["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1)/sqrt(128) bf16 KV and queries drawn on the GPU "
                "(no datasets, no trained weights)",
        "config": {"workload": "1M-token windowed draft + chain-3 verify step",
                   "batch": 1, "context": L1M, "layers": args.layers, "q_heads": HQ,
                   "kv_heads": HKV, "head_dim": D, "draft": "sink 4 + window 4096; per layer "
                   "1 context call (3 chained queries) + 3 single-query calls",
                   "verify": "3-token chain over the full cache per layer", "vocab": VOCAB},
        "pct_of_hbm_peak": round(100 * r1m["gbs"] / HBM_PEAK_GBS, 2),
        "steps_per_s": round(r1m["steps_per_s"], 3),
        "graph": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r1m["graph"].items()},
        "components_ms": {k: round(v, 4) for k, v in r1m["components_ms"].items()},
        "call_gbs": {k: round(v, 1) for k, v in r1m["call_gbs"].items()},
        "call_ms_percentiles": r1m["call_ms_percentiles"],
        "roofline": {"kernel": "verify (chain 3 over 1,048,576 keys, 8 KV heads)",
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "bytes_per_launch": r1m["verify_bytes_per_launch"],
                     "avg_launch_ms": round(v_ms, 4)},
        "cpu_baseline": cpu,
        "roofline_tree_verify_16k": tree_verify_roofline(r16),
        "roofline_tree_verify_8k": tree_verify_roofline(r8k),
        "machine": probes,
        "vs_stream_read": vs_stream,
        "draft_floor": draft_floor,
        "verify_modes_1m": r1m["verify_modes"],
        "ctx16k": r16,
        "ctx8k": r8k,
        "ctx4k": r4k,
        "ragged": rrag,
        "kv_commit": commit,
        "kv_compact": compact,
        "budget_select": select,
        "partial_verify_1m": partial,
        "ring_draft_1m": ring,
        "shard_1m_kv1": shard,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
