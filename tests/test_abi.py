"""The C ABI on the CPU: the library loads, exports every function the header
declares, sizes workspaces without a device, and rejects bad arguments before
launching anything (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import sparse_kv_attention_sink_amd as skg
from sparse_kv_attention_sink_amd import SpecDims, SpecKV

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_attn.h")


@pytest.fixture(scope="module")
def lib():
    import torch
    if torch.cuda.is_available():
        # the validation cases below pass fake device pointers: a case that
        # slipped through validation would launch a kernel on them
        pytest.skip("argument checks with fake pointers run only where no GPU is visible")
    if not os.path.exists(skg.LIB_PATH):
        pytest.fail("libspecattn.so is not built (python -m sparse_kv_attention_sink_amd.build)")
    return skg.load()


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:spec_status|size_t|const char\*|int32_t)\s+(spec_\w+)\(",
                                 text, flags=re.M)))


def test_header_declares_the_four_operations():
    fns = header_functions()
    for name in ("spec_attn_draft_sparse", "spec_attn_verify_tree", "spec_accept_greedy",
                 "spec_kv_commit"):
        assert name in fns


def test_every_declared_function_is_exported(lib):
    fns = header_functions()
    assert fns == sorted(skg.EXPORTED)
    for name in fns:
        assert hasattr(lib, name), name


def test_abi_version(lib):
    assert lib.spec_abi_version() == 2
    assert lib.spec_status_string(skg.SPEC_E_WORKSPACE) == b"SPEC_E_WORKSPACE"


def dims(B=1, Hq=32, Hkv=8, D=128, dtype=skg.SPEC_BF16, scale=0.088, flags=0):
    return SpecDims(B, Hq, Hkv, D, dtype, scale, flags)


# Every workspace: a 256-byte header, the 1 MiB counter region, then scratch.
SCRATCH = 256 + (1 << 20)


def test_every_scratch_region_starts_after_the_counter_region(lib):
    """No call's scratch may overlap the counter region, whatever its shape,
    so that one workspace serves calls of every kind and shape."""
    for B in (1, 8, 16, 300):
        d = dims(B=B)
        for T, view in ((1, 256), (3, 4100), (1, 1 << 19), (8, 64)):
            assert skg.draft_workspace_bytes(d, T, view) >= SCRATCH
        for N, cap in ((3, 1 << 20), (64, 16384), (44, 32768), (5, 4096)):
            assert skg.verify_workspace_bytes(d, N, cap) >= SCRATCH
        assert skg.accept_workspace_bytes(B, 64, 128256) >= SCRATCH + B * 65 * 8
        assert lib.spec_compact_workspace_bytes(B) >= SCRATCH
        assert lib.spec_select_workspace_bytes(ctypes.byref(d), 16) >= SCRATCH
        dd = dims(B=B, dtype=skg.SPEC_F32, D=64, Hq=2, Hkv=1)
        assert skg.verify_workspace_bytes(dd, 15, 512) >= SCRATCH
        assert skg.draft_workspace_bytes(dd, 1, 68) >= SCRATCH


def test_unknown_flag_bits_are_rejected(lib):
    assert skg.draft_workspace_bytes(dims(flags=skg.SPEC_FLAG_DETERMINISTIC), 1, 256) > 0
    assert skg.draft_workspace_bytes(dims(flags=2), 1, 256) == 0
    assert b"flag" in lib.spec_last_error()


def test_workspace_sizes_are_device_free_and_monotone(lib):
    d = dims(B=8)
    a = skg.draft_workspace_bytes(d, 1, 256)
    b = skg.draft_workspace_bytes(d, 1, 2048)
    assert 256 <= a <= b and a % 256 == 0
    v = skg.verify_workspace_bytes(d, 64, 16384)
    assert v >= 256 + 8 * 64 * 8
    assert skg.accept_workspace_bytes(8, 64, 128256) >= 256 + 8 * 65 * 8
    assert skg.draft_workspace_bytes(d, 1, 256) == a          # deterministic
    assert skg.verify_workspace_bytes(dims(), 65, 100) == 0     # > 64 nodes
    assert b"n_nodes" in lib.spec_last_error()


FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def kv(cap=4096, stride_t=128, ptr=FAKE):
    return SpecKV(ptr, ptr, 8 * cap * 128, cap * 128, stride_t, cap)


def draft(lib, d, *, q=FAKE, tq=1, cache=None, sink=4, win=64, idx=None, budget=0, ws=FAKE,
          wsb=1 << 30, out=FAKE):
    cache = cache or kv()
    return lib.spec_attn_draft_sparse(ctypes.byref(d), q, tq, ctypes.byref(cache), FAKE, sink, win,
                                      idx, budget, 0, 0, out, None, ws, wsb, None)


@pytest.mark.parametrize("bad,status", [
    (dict(d=dims(Hq=30, Hkv=8)), skg.SPEC_E_INVALID),
    (dict(d=dims(D=96)), skg.SPEC_E_UNSUPPORTED),
    (dict(d=dims(dtype=7)), skg.SPEC_E_UNSUPPORTED),
    (dict(d=dims(scale=0.0)), skg.SPEC_E_INVALID),
    (dict(d=dims(scale=float("inf"))), skg.SPEC_E_INVALID),
    (dict(d=dims(B=-1)), skg.SPEC_E_INVALID),
    (dict(tq=0), skg.SPEC_E_INVALID),
    (dict(q=None), skg.SPEC_E_INVALID),
    (dict(q=FAKE + 2), skg.SPEC_E_INVALID),
    (dict(out=None), skg.SPEC_E_INVALID),
    (dict(cache=kv(stride_t=64)), skg.SPEC_E_INVALID),
    (dict(cache=kv(stride_t=132)), skg.SPEC_E_INVALID),
    (dict(cache=kv(ptr=FAKE + 8)), skg.SPEC_E_INVALID),
    (dict(cache=kv(cap=-1)), skg.SPEC_E_INVALID),
    (dict(win=0), skg.SPEC_E_INVALID),
    (dict(sink=-1), skg.SPEC_E_INVALID),
    (dict(idx=FAKE, budget=0), skg.SPEC_E_INVALID),
    (dict(idx=FAKE + 2, budget=16), skg.SPEC_E_INVALID),
    (dict(ws=None), skg.SPEC_E_WORKSPACE),
    (dict(wsb=16), skg.SPEC_E_WORKSPACE),
    (dict(ws=FAKE + 16), skg.SPEC_E_INVALID),
])
def test_draft_rejects_bad_arguments(lib, bad, status):
    d = bad.pop("d", dims())
    assert draft(lib, d, **bad) == status
    assert lib.spec_last_error()


def verify(lib, d, *, n=5, cache=None, tree=None, parents=FAKE, psb=0, pad=None, pad_sb=0,
           ws=FAKE, wsb=1 << 30):
    cache = cache or kv()
    tree = tree or kv(cap=n)
    return lib.spec_attn_verify_tree(ctypes.byref(d), FAKE, n, ctypes.byref(cache), FAKE, pad,
                                     pad_sb, ctypes.byref(tree), parents, psb, FAKE, None, None,
                                     ws, wsb, None)


@pytest.mark.parametrize("bad,status", [
    (dict(n=0), skg.SPEC_E_INVALID),
    (dict(n=65), skg.SPEC_E_UNSUPPORTED),
    (dict(parents=None), skg.SPEC_E_INVALID),
    (dict(psb=3), skg.SPEC_E_INVALID),
    (dict(pad=FAKE, pad_sb=4095), skg.SPEC_E_INVALID),
    (dict(pad=FAKE, pad_sb=1024), skg.SPEC_E_INVALID),
    (dict(pad=FAKE + 1, pad_sb=4096), skg.SPEC_E_INVALID),
    (dict(tree=kv(cap=5, ptr=FAKE + 4)), skg.SPEC_E_INVALID),
    (dict(wsb=1024), skg.SPEC_E_WORKSPACE),
])
def test_verify_rejects_bad_arguments(lib, bad, status):
    assert verify(lib, dims(), **bad) == status


@pytest.mark.parametrize("args,status", [
    ((1, 0, 100), skg.SPEC_E_INVALID),
    ((1, 65, 100), skg.SPEC_E_UNSUPPORTED),
    ((1, 4, 0), skg.SPEC_E_INVALID),
    ((-1, 4, 100), skg.SPEC_E_INVALID),
])
def test_accept_rejects_bad_arguments(lib, args, status):
    B, N, V = args
    st = lib.spec_accept_greedy(B, N, V, FAKE, FAKE, FAKE, 0, 4, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == status


def test_accept_rejects_bad_pointers(lib):
    assert lib.spec_accept_greedy(1, 4, 100, FAKE + 4, FAKE, FAKE, 0, 4, FAKE, FAKE, FAKE, FAKE,
                                  1 << 30, None) == skg.SPEC_E_INVALID
    assert lib.spec_accept_greedy(1, 4, 100, FAKE, FAKE, FAKE, 0, 0, FAKE, FAKE, FAKE, FAKE,
                                  1 << 30, None) == skg.SPEC_E_INVALID
    assert lib.spec_accept_greedy(1, 4, 100, FAKE, FAKE, FAKE, 0, 4, FAKE, FAKE, FAKE, FAKE,
                                  8, None) == skg.SPEC_E_WORKSPACE


def commit(lib, *, B=2, hkv=8, D=128, dtype=skg.SPEC_BF16, cache=None, tree=None, n=5, cl=FAKE,
           pad=FAKE, pad_sb=4096, al=FAKE, ap=FAKE, md=4, na=None, ws=FAKE, wsb=256):
    cache = cache or kv()
    tree = tree or kv(cap=n)
    return lib.spec_kv_commit(B, hkv, D, dtype, ctypes.byref(cache), cl, pad, pad_sb,
                              ctypes.byref(tree), n, al, ap, md, na, ws, wsb, None)


@pytest.mark.parametrize("bad,status", [
    (dict(B=-1), skg.SPEC_E_INVALID),
    (dict(hkv=0), skg.SPEC_E_INVALID),
    (dict(D=96), skg.SPEC_E_UNSUPPORTED),
    (dict(dtype=7), skg.SPEC_E_UNSUPPORTED),
    (dict(n=0), skg.SPEC_E_INVALID),
    (dict(n=65), skg.SPEC_E_UNSUPPORTED),
    (dict(md=0), skg.SPEC_E_INVALID),
    (dict(cl=None), skg.SPEC_E_INVALID),
    (dict(pad=None), skg.SPEC_E_INVALID),
    (dict(al=None), skg.SPEC_E_INVALID),
    (dict(ap=None), skg.SPEC_E_INVALID),
    (dict(cl=FAKE + 2), skg.SPEC_E_INVALID),
    (dict(na=FAKE + 2), skg.SPEC_E_INVALID),
    (dict(pad_sb=4095), skg.SPEC_E_INVALID),
    (dict(cache=kv(stride_t=64)), skg.SPEC_E_INVALID),
    (dict(cache=kv(ptr=FAKE + 8)), skg.SPEC_E_INVALID),
    (dict(tree=kv(cap=5, ptr=FAKE + 4)), skg.SPEC_E_INVALID),
    (dict(ws=None), skg.SPEC_E_WORKSPACE),
    (dict(wsb=16), skg.SPEC_E_WORKSPACE),
    (dict(ws=FAKE + 16), skg.SPEC_E_INVALID),
])
def test_commit_rejects_bad_arguments(lib, bad, status):
    assert commit(lib, **bad) == status
    assert lib.spec_last_error()


def test_commit_workspace_is_the_error_word(lib):
    assert lib.spec_commit_workspace_bytes() == 256


def means_call(lib, d, *, cache=None, block=16, first=0, n=4, means=FAKE, max_blocks=256,
               cl=FAKE, pad=None, pad_sb=0, ws=FAKE, wsb=256):
    cache = cache or kv()
    return lib.spec_block_means(ctypes.byref(d), ctypes.byref(cache), cl, pad, pad_sb, block,
                                first, n, means, max_blocks, ws, wsb, None)


@pytest.mark.parametrize("bad,status", [
    (dict(block=0), skg.SPEC_E_INVALID),
    (dict(first=-1), skg.SPEC_E_INVALID),
    (dict(first=250, n=7), skg.SPEC_E_INVALID),
    (dict(means=None), skg.SPEC_E_INVALID),
    (dict(means=FAKE + 4), skg.SPEC_E_INVALID),
    (dict(cl=None), skg.SPEC_E_INVALID),
    (dict(pad=FAKE, pad_sb=100), skg.SPEC_E_INVALID),
    (dict(cache=kv(stride_t=64)), skg.SPEC_E_INVALID),
    (dict(ws=None), skg.SPEC_E_WORKSPACE),
    (dict(ws=FAKE + 8), skg.SPEC_E_INVALID),
])
def test_block_means_rejects_bad_arguments(lib, bad, status):
    assert means_call(lib, dims(), **bad) == status


def select_call(lib, d, *, q=FAKE, tq=1, means=FAKE, max_blocks=256, block=16, cl=FAKE, cap=4096,
                pad=None, pad_sb=0, sink=4, win=64, nsel=8, shared=0, idx=FAKE, budget=196,
                scores=None, ws=FAKE, wsb=1 << 30):
    return lib.spec_select_blocks(ctypes.byref(d), q, tq, means, max_blocks, block, cl, cap, pad,
                                  pad_sb, sink, win, nsel, shared, idx, budget, scores, ws, wsb,
                                  None)


@pytest.mark.parametrize("bad,status", [
    (dict(tq=0), skg.SPEC_E_INVALID),
    (dict(block=0), skg.SPEC_E_INVALID),
    (dict(max_blocks=255), skg.SPEC_E_INVALID),          # 255 x 16 < 4096
    (dict(max_blocks=8193, cap=16), skg.SPEC_E_UNSUPPORTED),
    (dict(nsel=2049, budget=1 << 20), skg.SPEC_E_UNSUPPORTED),
    (dict(budget=195), skg.SPEC_E_INVALID),              # 4 + 64 + 8 x 16 = 196
    (dict(sink=-1), skg.SPEC_E_INVALID),
    (dict(q=None), skg.SPEC_E_INVALID),
    (dict(q=FAKE + 2), skg.SPEC_E_INVALID),
    (dict(idx=None), skg.SPEC_E_INVALID),
    (dict(scores=FAKE + 2), skg.SPEC_E_INVALID),
    (dict(pad=FAKE, pad_sb=4000), skg.SPEC_E_INVALID),
    (dict(wsb=4), skg.SPEC_E_WORKSPACE),
    (dict(wsb=256 + 8 * 256 * 4 - 4), skg.SPEC_E_WORKSPACE),    # one score short
])
def test_select_blocks_rejects_bad_arguments(lib, bad, status):
    assert select_call(lib, dims(), **bad) == status


def gather_call(lib, *, B=2, hkv=8, D=128, dtype=skg.SPEC_BF16, cache=None, cl=FAKE, idx=FAKE,
                budget=64, isb=64, partial=None, plen=FAKE, ppad=FAKE, ppsb=64, ws=FAKE, wsb=256):
    cache = cache or kv()
    partial = partial or kv(cap=64)
    return lib.spec_kv_gather(B, hkv, D, dtype, ctypes.byref(cache), cl, idx, budget, isb,
                              ctypes.byref(partial), plen, ppad, ppsb, ws, wsb, None)


@pytest.mark.parametrize("bad,status", [
    (dict(budget=0), skg.SPEC_E_INVALID),
    (dict(B=-1), skg.SPEC_E_INVALID),
    (dict(D=96), skg.SPEC_E_UNSUPPORTED),
    (dict(budget=65, isb=65), skg.SPEC_E_INVALID),           # partial capacity 64 < budget
    (dict(isb=63), skg.SPEC_E_INVALID),
    (dict(idx=None), skg.SPEC_E_INVALID),
    (dict(idx=FAKE + 2), skg.SPEC_E_INVALID),
    (dict(plen=None), skg.SPEC_E_INVALID),
    (dict(ppad=None), skg.SPEC_E_INVALID),
    (dict(ppsb=63), skg.SPEC_E_INVALID),
    (dict(partial=kv(cap=64, ptr=FAKE + 8)), skg.SPEC_E_INVALID),
    (dict(cache=kv(stride_t=64)), skg.SPEC_E_INVALID),
    (dict(wsb=8), skg.SPEC_E_WORKSPACE),
])
def test_gather_rejects_bad_arguments(lib, bad, status):
    assert gather_call(lib, **bad) == status


def test_verify_mode_follows_the_schedule_table(lib):
    """The host-side schedule against the hand-enumerated table of SpecPV
    section 3.3 (the same fixture pins the oracle)."""
    import json
    with open(os.path.join(ROOT, "tests", "golden", "verify_mode_specpv.json")) as f:
        fx = json.load(f)
    for case in fx["cases"]:
        *args, mode = case
        assert lib.spec_verify_mode(*args) == mode, case
    assert lib.spec_verify_mode(-1, 4096, 0, 3, 64) == skg.SPEC_E_INVALID
    assert lib.spec_verify_mode(100, 4096, 0, 0, 64) == skg.SPEC_E_INVALID


def ring_call(lib, d, *, tq=1, cache=None, sink=4, win=64, ring=64, ws=FAKE, wsb=1 << 30):
    cache = cache or kv(cap=68)
    return lib.spec_attn_draft_ring(ctypes.byref(d), FAKE, tq, ctypes.byref(cache), FAKE, sink,
                                    win, ring, FAKE, None, ws, wsb, None)


@pytest.mark.parametrize("bad,status", [
    (dict(ring=63), skg.SPEC_E_INVALID),                      # < window + Tq - 1
    (dict(tq=3, ring=65), skg.SPEC_E_INVALID),
    (dict(cache=kv(cap=67)), skg.SPEC_E_INVALID),             # < n_sink + ring
    (dict(win=0), skg.SPEC_E_INVALID),
    (dict(sink=-1), skg.SPEC_E_INVALID),
    (dict(tq=0), skg.SPEC_E_INVALID),
    (dict(ws=None), skg.SPEC_E_WORKSPACE),
])
def test_ring_draft_rejects_bad_arguments(lib, bad, status):
    assert ring_call(lib, dims(), **bad) == status


def test_device_status_rejects_null(lib):
    assert lib.spec_device_status(None, None, None) == skg.SPEC_E_INVALID


def test_empty_batch_is_a_no_op(lib):
    """batch = 0 passes validation and launches nothing."""
    assert draft(lib, dims(B=0)) == skg.SPEC_OK
    assert verify(lib, dims(B=0)) == skg.SPEC_OK
    assert lib.spec_accept_greedy(0, 4, 100, FAKE, FAKE, FAKE, 0, 4, FAKE, FAKE, FAKE, FAKE,
                                  1 << 30, None) == skg.SPEC_OK
    assert commit(lib, B=0) == skg.SPEC_OK
    assert means_call(lib, dims(B=0)) == skg.SPEC_OK
    assert select_call(lib, dims(B=0)) == skg.SPEC_OK
    assert gather_call(lib, B=0) == skg.SPEC_OK
    d = dims(B=8)
    assert lib.spec_select_workspace_bytes(ctypes.byref(d), 0) == SCRATCH
    assert lib.spec_select_workspace_bytes(ctypes.byref(d), 1024) == SCRATCH + 8 * 8 * 1024 * 4


def test_binding_fails_loudly_without_library(tmp_path):
    """No silent fallback: a missing library is an error."""
    saved = skg._lib._lib
    skg._lib._lib = None
    try:
        with pytest.raises(RuntimeError):
            skg._lib.load(str(tmp_path / "missing.so"))
    finally:
        skg._lib._lib = saved


PROBE_HEADER = os.path.join(ROOT, "include", "spec_probe.h")


def test_probe_library_exports_its_header():
    """The measurement library loads and exports every function of
    spec_probe.h; its argument checks reject bad shapes before a launch."""
    import torch
    import sparse_kv_attention_sink_amd._probe as pr
    text = open(PROBE_HEADER).read()
    fns = sorted(set(re.findall(r"^\s*int32_t\s+(spec_\w+)\(", text, flags=re.M)))
    assert fns == sorted(pr.EXPORTED)
    plib = pr.load()
    for name in fns:
        assert hasattr(plib, name), name
    if torch.cuda.is_available():
        return
    fake = ctypes.c_void_p(1 << 20)
    assert plib.spec_probe_read(fake, 4096 * 3 + 1, 8, 8, fake, None) == -1   # not whole blocks
    assert plib.spec_probe_read(fake, 4096, 8, 5, fake, None) == -1           # in_flight
    assert plib.spec_probe_read(None, 4096, 8, 8, fake, None) == -1
    assert plib.spec_probe_read_lds(fake, 16384, 8, 3, fake, None) == -1      # stages
    assert plib.spec_probe_read_lds(fake, 4096, 8, 4, fake, None) == -1      # not whole stages
    assert plib.spec_probe_empty(0, fake, None) == -1


def test_noalloc_verify_refuses_shapes_beyond_its_static_scratch(lib):
    """The static scratch holds 64 MiB: a shape needing more is refused
    before anything is launched; invalid arguments fail as in the workspace
    variant; batch 0 is a no-op."""
    d = dims(B=256)
    assert skg.verify_workspace_bytes(d, 64, 1 << 17) > 64 << 20
    fake = 1 << 20
    kv = SpecKV(fake, fake, 8 * (1 << 17) * 128, (1 << 17) * 128, 128, 1 << 17)
    tr = SpecKV(fake, fake, 8 * 64 * 128, 64 * 128, 128, 64)
    P = ctypes.c_void_p
    st = lib.spec_attn_verify_tree_noalloc(ctypes.byref(d), P(fake), 64, ctypes.byref(kv), P(fake),
                                           None, 0, ctypes.byref(tr), P(fake), 0, P(fake), None, None,
                                           None)
    assert st == skg.SPEC_E_UNSUPPORTED
    assert b"static array" in lib.spec_last_error()
    st = lib.spec_attn_verify_tree_noalloc(ctypes.byref(d), P(fake), 65, ctypes.byref(kv), P(fake),
                                           None, 0, ctypes.byref(tr), P(fake), 0, P(fake), None, None,
                                           None)
    assert st == skg.SPEC_E_UNSUPPORTED          # more than 64 nodes
    st = lib.spec_attn_verify_tree_noalloc(ctypes.byref(d), None, 64, ctypes.byref(kv), P(fake),
                                           None, 0, ctypes.byref(tr), P(fake), 0, P(fake), None, None,
                                           None)
    assert st == skg.SPEC_E_INVALID              # null q
    z = dims(B=0)
    assert lib.spec_attn_verify_tree_noalloc(ctypes.byref(z), None, 5, None, None, None, 0, None,
                                             None, 0, None, None, None, None) == skg.SPEC_OK
