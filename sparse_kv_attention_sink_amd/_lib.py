"""ctypes binding of libspecattn (argument marshalling only).

Every function takes torch tensors that already live on the GPU, checks that
their shapes agree with each other, and passes raw device pointers, strides
and the current HIP stream to the C ABI in ``include/spec_attn.h``.  All
arithmetic happens in the library's HIP kernels; there is no fallback path:
if the library is missing or no GPU tensor is given, the call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libspecattn.so")

SPEC_OK = 0
SPEC_E_INVALID = -1
SPEC_E_UNSUPPORTED = -2
SPEC_E_WORKSPACE = -3
SPEC_E_HIP = -4
SPEC_E_DEVICE_RANGE = -5
SPEC_F32 = 0
SPEC_BF16 = 1
SPEC_FLAG_DETERMINISTIC = 1
SPEC_DEV_CACHE_LEN = 1
SPEC_DEV_INDEX = 2
SPEC_DEV_PARENT = 4
SPEC_DEV_DEPTH = 8
SPEC_DEV_COMMIT = 16
SPEC_VERIFY_FULL = 0
SPEC_VERIFY_PARTIAL = 1

EXPORTED = [
    "spec_attn_draft_sparse", "spec_attn_draft_ring", "spec_attn_verify_tree",
    "spec_accept_greedy", "spec_kv_commit", "spec_kv_compact", "spec_compact_workspace_bytes",
    "spec_draft_workspace_bytes", "spec_verify_workspace_bytes", "spec_accept_workspace_bytes",
    "spec_attn_verify_tree_noalloc",
    "spec_commit_workspace_bytes", "spec_block_means", "spec_select_blocks",
    "spec_select_workspace_bytes", "spec_kv_gather", "spec_verify_mode",
    "spec_device_status", "spec_status_string", "spec_last_error", "spec_abi_version",
]


class SpecDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("flags", ctypes.c_uint32)]


class SpecKV(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("stride_b", ctypes.c_int64),
                ("stride_h", ctypes.c_int64), ("stride_t", ctypes.c_int64),
                ("capacity", ctypes.c_int32)]


class SpecError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libspecattn.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m sparse_kv_attention_sink_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.spec_attn_draft_sparse.argtypes = [P, P, I32, P, P, I32, I32, P, I32, I64, I64, P, P, P, SZ, P]
    lib.spec_attn_draft_sparse.restype = I32
    lib.spec_attn_draft_ring.argtypes = [P, P, I32, P, P, I32, I32, I32, P, P, P, SZ, P]
    lib.spec_attn_draft_ring.restype = I32
    lib.spec_attn_verify_tree.argtypes = [P, P, I32, P, P, P, I64, P, P, I64, P, P, P, P, SZ, P]
    lib.spec_attn_verify_tree.restype = I32
    lib.spec_attn_verify_tree_noalloc.argtypes = [P, P, I32, P, P, P, I64, P, P, I64, P, P, P, P]
    lib.spec_attn_verify_tree_noalloc.restype = I32
    lib.spec_accept_greedy.argtypes = [I32, I32, I32, P, P, P, I64, I32, P, P, P, P, SZ, P]
    lib.spec_accept_greedy.restype = I32
    lib.spec_kv_commit.argtypes = [I32, I32, I32, I32, P, P, P, I64, P, I32, P, P, I32, P, P, SZ, P]
    lib.spec_kv_commit.restype = I32
    lib.spec_commit_workspace_bytes.argtypes = []
    lib.spec_commit_workspace_bytes.restype = SZ
    lib.spec_kv_compact.argtypes = [I32, I32, I32, I32, P, P, P, I64, P, SZ, P]
    lib.spec_kv_compact.restype = I32
    lib.spec_compact_workspace_bytes.argtypes = [I32]
    lib.spec_compact_workspace_bytes.restype = SZ
    lib.spec_block_means.argtypes = [P, P, P, P, I64, I32, I32, I32, P, I32, P, SZ, P]
    lib.spec_block_means.restype = I32
    lib.spec_select_blocks.argtypes = [P, P, I32, P, I32, I32, P, I32, P, I64, I32, I32, I32, I32,
                                       P, I32, P, P, SZ, P]
    lib.spec_select_blocks.restype = I32
    lib.spec_select_workspace_bytes.argtypes = [P, I32]
    lib.spec_kv_gather.argtypes = [I32, I32, I32, I32, P, P, P, I32, I64, P, P, P, I64, P, SZ, P]
    lib.spec_kv_gather.restype = I32
    lib.spec_verify_mode.argtypes = [I64, I32, I32, I32, I32]
    lib.spec_verify_mode.restype = I32
    lib.spec_select_workspace_bytes.restype = SZ
    lib.spec_draft_workspace_bytes.argtypes = [P, I32, I32]
    lib.spec_draft_workspace_bytes.restype = SZ
    lib.spec_verify_workspace_bytes.argtypes = [P, I32, I32]
    lib.spec_verify_workspace_bytes.restype = SZ
    lib.spec_accept_workspace_bytes.argtypes = [I32, I32, I32]
    lib.spec_accept_workspace_bytes.restype = SZ
    lib.spec_device_status.argtypes = [P, P, ctypes.POINTER(ctypes.c_uint32)]
    lib.spec_device_status.restype = I32
    lib.spec_status_string.argtypes = [I32]
    lib.spec_status_string.restype = ctypes.c_char_p
    lib.spec_last_error.argtypes = []
    lib.spec_last_error.restype = ctypes.c_char_p
    lib.spec_abi_version.argtypes = []
    lib.spec_abi_version.restype = I32
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != SPEC_OK:
        lib = load()
        raise SpecError(status, f"{lib.spec_status_string(status).decode()}: "
                                f"{lib.spec_last_error().decode()}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SPEC_BF16
    if t.dtype == torch.float32:
        return SPEC_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _on_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")


def make_dims(B, Hq, Hkv, D, dtype_code, scale=None, deterministic=False) -> SpecDims:
    return SpecDims(B, Hq, Hkv, D, dtype_code, 1.0 / math.sqrt(D) if scale is None else scale,
                    SPEC_FLAG_DETERMINISTIC if deterministic else 0)


def _kv(k: torch.Tensor, v: torch.Tensor) -> SpecKV:
    if k.dim() != 4 or k.shape != v.shape:
        raise ValueError("K and V must be 4-D [B, Hkv, L, D] with equal shapes")
    if k.stride() != v.stride() or k.stride(3) != 1:
        raise ValueError("K and V must share strides with a contiguous last dimension")
    return SpecKV(k.data_ptr(), v.data_ptr(), k.stride(0), k.stride(1), k.stride(2), k.shape[2])


def draft_workspace_bytes(dims: SpecDims, n_q_tokens: int, max_view_len: int) -> int:
    return int(load().spec_draft_workspace_bytes(ctypes.byref(dims), n_q_tokens, max_view_len))


def verify_workspace_bytes(dims: SpecDims, n_nodes: int, capacity: int) -> int:
    return int(load().spec_verify_workspace_bytes(ctypes.byref(dims), n_nodes, capacity))


def accept_workspace_bytes(batch: int, n_nodes: int, vocab: int) -> int:
    return int(load().spec_accept_workspace_bytes(batch, n_nodes, vocab))


def new_workspace(nbytes: int, device) -> torch.Tensor:
    """Zero-filled workspace (the library requires zeros before first use)."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def spec_attn_draft_sparse(q, k_cache, v_cache, cache_len, *, n_sink=0, window=0, idx=None,
                           scale=None, out=None, lse=None, workspace=None, want_lse=True,
                           deterministic=False):
    """Draft attention over sink + window (idx None) or a budget list idx
    ``[B, 1 or Hkv, budget]`` int32.  ``deterministic`` sets
    SPEC_FLAG_DETERMINISTIC.  Returns (out, lse)."""
    lib = load()
    _on_gpu(q, k_cache, v_cache, cache_len, idx)
    if q.dim() != 4 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, Tq, Hq, D] tensor")
    B, Tq, Hq, D = q.shape
    if k_cache.shape[0] != B or k_cache.shape[3] != D or q.dtype != k_cache.dtype:
        raise ValueError("q and the cache disagree on batch, head_dim or dtype")
    if cache_len.dtype != torch.int32 or cache_len.numel() != B or not cache_len.is_contiguous():
        raise ValueError("cache_len must be a contiguous int32 [B] tensor")
    kv = _kv(k_cache, v_cache)
    dims = make_dims(B, Hq, k_cache.shape[1], D, _dtype_code(q), scale, deterministic)
    budget, isb, ish = 0, 0, 0
    if idx is not None:
        if idx.dtype != torch.int32 or idx.dim() != 3 or idx.shape[0] != B or idx.stride(2) != 1:
            raise ValueError("idx must be int32 [B, 1 or Hkv, budget] with a contiguous last dim")
        if idx.shape[1] not in (1, k_cache.shape[1]):
            raise ValueError("idx must have 1 or Hkv rows per sequence")
        budget, isb = idx.shape[2], idx.stride(0)
        ish = 0 if idx.shape[1] == 1 else idx.stride(1)
        view = budget
    else:
        view = min(k_cache.shape[2], n_sink + window + Tq - 1)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Tq, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = new_workspace(draft_workspace_bytes(dims, Tq, view), q.device)
    st = lib.spec_attn_draft_sparse(ctypes.byref(dims), _ptr(q), Tq, ctypes.byref(kv),
                                    _ptr(cache_len), n_sink, window, _ptr(idx), budget, isb, ish,
                                    _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                                    _stream(q))
    _check(st)
    return out, lse


def spec_attn_draft_ring(q, k_ring, v_ring, cache_len, *, n_sink, window, ring, scale=None,
                         out=None, lse=None, workspace=None, want_lse=True, deterministic=False):
    """Window draft over a ring cache ``[B, Hkv, >= n_sink + ring, D]``
    (position p >= n_sink at slot n_sink + (p - n_sink) % ring); ``cache_len``
    holds the logical lengths.  Returns (out, lse)."""
    lib = load()
    _on_gpu(q, k_ring, v_ring, cache_len)
    if q.dim() != 4 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, Tq, Hq, D] tensor")
    B, Tq, Hq, D = q.shape
    if k_ring.shape[0] != B or k_ring.shape[3] != D or q.dtype != k_ring.dtype:
        raise ValueError("q and the ring cache disagree on batch, head_dim or dtype")
    if cache_len.dtype != torch.int32 or cache_len.numel() != B or not cache_len.is_contiguous():
        raise ValueError("cache_len must be a contiguous int32 [B] tensor")
    kv = _kv(k_ring, v_ring)
    dims = make_dims(B, Hq, k_ring.shape[1], D, _dtype_code(q), scale, deterministic)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Tq, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = new_workspace(draft_workspace_bytes(dims, Tq, n_sink + window + Tq - 1),
                                  q.device)
    st = lib.spec_attn_draft_ring(ctypes.byref(dims), _ptr(q), Tq, ctypes.byref(kv),
                                  _ptr(cache_len), n_sink, window, ring, _ptr(out), _ptr(lse),
                                  _ptr(workspace), workspace.numel(), _stream(q))
    _check(st)
    return out, lse


def spec_attn_verify_tree(q, k_cache, v_cache, cache_len, tree_k, tree_v, parents, *, pad=None,
                          scale=None, out=None, lse=None, pos_ids=None, want_lse=True,
                          want_pos_ids=True, workspace=None, deterministic=False):
    """Tree-masked verify attention.  q ``[B, N, Hq, D]``; tree K/V
    ``[B, Hkv, N, D]``; parents int32 ``[N]`` or ``[B, N]``; pad uint8
    ``[B, >= L_cap]`` or None; ``deterministic`` sets
    SPEC_FLAG_DETERMINISTIC.  Returns (out, lse, pos_ids)."""
    lib = load()
    _on_gpu(q, k_cache, v_cache, cache_len, tree_k, tree_v, parents, pad)
    if q.dim() != 4 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, N, Hq, D] tensor")
    B, N, Hq, D = q.shape
    if k_cache.shape[0] != B or k_cache.shape[3] != D or q.dtype != k_cache.dtype:
        raise ValueError("q and the cache disagree on batch, head_dim or dtype")
    if tree_k.shape[0] != B or tree_k.shape[1] != k_cache.shape[1] or tree_k.shape[2] < N:
        raise ValueError("tree K/V must be [B, Hkv, >= N, D]")
    if cache_len.dtype != torch.int32 or cache_len.numel() != B or not cache_len.is_contiguous():
        raise ValueError("cache_len must be a contiguous int32 [B] tensor")
    if parents.dtype != torch.int32 or parents.shape[-1] != N or parents.stride(-1) != 1:
        raise ValueError("parents must be int32 [N] or [B, N]")
    psb = 0 if parents.dim() == 1 else parents.stride(0)
    if parents.dim() == 2 and parents.shape[0] != B:
        raise ValueError("parents must be [N] or [B, N]")
    kv = _kv(k_cache, v_cache)
    tkv = _kv(tree_k, tree_v)
    dims = make_dims(B, Hq, k_cache.shape[1], D, _dtype_code(q), scale, deterministic)
    pad_sb = 0
    if pad is not None:
        if pad.dtype != torch.uint8 or pad.dim() != 2 or pad.shape[0] != B or pad.stride(1) != 1:
            raise ValueError("pad must be uint8 [B, >= L_cap]")
        if pad.shape[1] < (k_cache.shape[2] + 3) // 4 * 4 or pad.stride(0) % 4:
            raise ValueError("pad rows must hold L_cap rounded up to a multiple of 4 bytes, "
                             "with a row stride that is a multiple of 4")
        pad_sb = pad.stride(0)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, N, Hq), dtype=torch.float32, device=q.device)
    if pos_ids is None and want_pos_ids:
        pos_ids = torch.empty((B, N), dtype=torch.int32, device=q.device)
    if workspace is None:
        workspace = new_workspace(verify_workspace_bytes(dims, N, k_cache.shape[2]), q.device)
    st = lib.spec_attn_verify_tree(ctypes.byref(dims), _ptr(q), N, ctypes.byref(kv),
                                   _ptr(cache_len), _ptr(pad), pad_sb, ctypes.byref(tkv),
                                   _ptr(parents), psb, _ptr(out), _ptr(lse), _ptr(pos_ids),
                                   _ptr(workspace), workspace.numel(), _stream(q))
    _check(st)
    return out, lse, pos_ids


def spec_attn_verify_tree_noalloc(q, k_cache, v_cache, cache_len, tree_k, tree_v, parents, *,
                                  out, pos_ids=None, lse=None, pad=None, scale=None,
                                  deterministic=False):
    """spec_attn_verify_tree on the library's static scratch: no workspace,
    and the caller passes every output it wants (``out`` is required), so the
    call allocates nothing.  Returns (out, lse, pos_ids)."""
    lib = load()
    _on_gpu(q, k_cache, v_cache, cache_len, tree_k, tree_v, parents, pad, out, lse, pos_ids)
    if q.dim() != 4 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, N, Hq, D] tensor")
    B, N, Hq, D = q.shape
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    if parents.dtype != torch.int32 or parents.shape[-1] != N or parents.stride(-1) != 1:
        raise ValueError("parents must be int32 [N] or [B, N]")
    psb = 0 if parents.dim() == 1 else parents.stride(0)
    kv = _kv(k_cache, v_cache)
    tkv = _kv(tree_k, tree_v)
    dims = make_dims(B, Hq, k_cache.shape[1], D, _dtype_code(q), scale, deterministic)
    pad_sb = 0 if pad is None else pad.stride(0)
    st = lib.spec_attn_verify_tree_noalloc(ctypes.byref(dims), _ptr(q), N, ctypes.byref(kv),
                                           _ptr(cache_len), _ptr(pad), pad_sb, ctypes.byref(tkv),
                                           _ptr(parents), psb, _ptr(out), _ptr(lse), _ptr(pos_ids),
                                           _stream(q))
    _check(st)
    return out, lse, pos_ids


def spec_accept_greedy(logits, draft_tokens, parents, max_depth, *, accept_len=None,
                       accept_path=None, bonus=None, workspace=None):
    """Greedy tree acceptance.  logits fp32 ``[B, N+1, V]``; draft_tokens
    int32 ``[B, N]``; parents int32 ``[N]`` or ``[B, N]``.  Returns
    (accept_len [B], accept_path [B, max_depth], bonus [B])."""
    lib = load()
    _on_gpu(logits, draft_tokens, parents)
    if logits.dtype != torch.float32 or logits.dim() != 3 or not logits.is_contiguous():
        raise ValueError("logits must be contiguous fp32 [B, N+1, V]")
    B, N1, V = logits.shape
    N = N1 - 1
    if draft_tokens.dtype != torch.int32 or tuple(draft_tokens.shape) != (B, N) or \
            not draft_tokens.is_contiguous():
        raise ValueError("draft_tokens must be contiguous int32 [B, N]")
    if parents.dtype != torch.int32 or parents.shape[-1] != N or parents.stride(-1) != 1:
        raise ValueError("parents must be int32 [N] or [B, N]")
    psb = 0 if parents.dim() == 1 else parents.stride(0)
    dev = logits.device
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if accept_path is None:
        accept_path = torch.empty((B, max_depth), dtype=torch.int32, device=dev)
    if bonus is None:
        bonus = torch.empty(B, dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = new_workspace(accept_workspace_bytes(B, N, V), dev)
    st = lib.spec_accept_greedy(B, N, V, _ptr(logits), _ptr(draft_tokens), _ptr(parents), psb,
                                max_depth, _ptr(accept_len), _ptr(accept_path), _ptr(bonus),
                                _ptr(workspace), workspace.numel(), _stream(logits))
    _check(st)
    return accept_len, accept_path, bonus


def commit_workspace_bytes() -> int:
    return int(load().spec_commit_workspace_bytes())


def spec_kv_commit(k_cache, v_cache, cache_len, pad, tree_k, tree_v, accept_len, accept_path, *,
                   n_appended=None, workspace=None):
    """Append each sequence's accepted path (the K/V rows of
    ``accept_path[b, :accept_len[b]]`` in ``tree_k``/``tree_v``) to its cache
    after ``cache_len[b]``, pad the batch to one uniform length P, and advance
    ``cache_len`` and ``pad`` in place.  Returns ``n_appended`` (int32 [1] = P)."""
    lib = load()
    _on_gpu(k_cache, v_cache, cache_len, pad, tree_k, tree_v, accept_len, accept_path)
    B, Hkv, _, D = k_cache.shape
    if tree_k.shape[0] != B or tree_k.shape[1] != Hkv or tree_k.shape[3] != D or \
            tree_k.dtype != k_cache.dtype:
        raise ValueError("tree K/V must be [B, Hkv, N, D] of the cache's dtype")
    if cache_len.dtype != torch.int32 or cache_len.numel() != B or not cache_len.is_contiguous():
        raise ValueError("cache_len must be a contiguous int32 [B] tensor")
    if pad.dtype != torch.uint8 or pad.dim() != 2 or pad.shape[0] != B or pad.stride(1) != 1 or \
            pad.shape[1] < k_cache.shape[2]:
        raise ValueError("pad must be uint8 [B, >= L_cap]")
    if accept_len.dtype != torch.int32 or accept_len.numel() != B or not accept_len.is_contiguous():
        raise ValueError("accept_len must be a contiguous int32 [B] tensor")
    if accept_path.dtype != torch.int32 or accept_path.dim() != 2 or accept_path.shape[0] != B or \
            not accept_path.is_contiguous():
        raise ValueError("accept_path must be a contiguous int32 [B, max_depth] tensor")
    kv = _kv(k_cache, v_cache)
    tkv = _kv(tree_k, tree_v)
    if n_appended is None:
        n_appended = torch.empty(1, dtype=torch.int32, device=k_cache.device)
    if workspace is None:
        workspace = new_workspace(commit_workspace_bytes(), k_cache.device)
    st = lib.spec_kv_commit(B, Hkv, D, _dtype_code(k_cache), ctypes.byref(kv), _ptr(cache_len),
                            _ptr(pad), pad.stride(0), ctypes.byref(tkv), tree_k.shape[2],
                            _ptr(accept_len), _ptr(accept_path), accept_path.shape[1],
                            _ptr(n_appended), _ptr(workspace), workspace.numel(), _stream(k_cache))
    _check(st)
    return n_appended


def compact_workspace_bytes(batch: int) -> int:
    return int(load().spec_compact_workspace_bytes(batch))


def spec_kv_compact(k_cache, v_cache, cache_len, pad, *, workspace=None):
    """Drop each sequence's padding slots in place: the valid slots below
    ``cache_len[b]`` move to the front in order, ``cache_len`` becomes their
    count and the pad bytes below the old length are cleared."""
    lib = load()
    _on_gpu(k_cache, v_cache, cache_len, pad)
    B, Hkv, _, D = k_cache.shape
    if cache_len.dtype != torch.int32 or cache_len.numel() != B or not cache_len.is_contiguous():
        raise ValueError("cache_len must be a contiguous int32 [B] tensor")
    if pad.dtype != torch.uint8 or pad.dim() != 2 or pad.shape[0] != B or pad.stride(1) != 1 or \
            pad.shape[1] < k_cache.shape[2]:
        raise ValueError("pad must be uint8 [B, >= L_cap]")
    kv = _kv(k_cache, v_cache)
    if workspace is None:
        workspace = new_workspace(compact_workspace_bytes(B), k_cache.device)
    st = lib.spec_kv_compact(B, Hkv, D, _dtype_code(k_cache), ctypes.byref(kv), _ptr(cache_len),
                             _ptr(pad), pad.stride(0), _ptr(workspace), workspace.numel(),
                             _stream(k_cache))
    _check(st)


def select_workspace_bytes(dims: SpecDims, max_blocks: int = 0) -> int:
    return int(load().spec_select_workspace_bytes(ctypes.byref(dims), max_blocks))


def _pad_arg(pad, B, capacity):
    if pad is None:
        return None, 0
    if pad.dtype != torch.uint8 or pad.dim() != 2 or pad.shape[0] != B or pad.stride(1) != 1 or \
            pad.shape[1] < capacity:
        raise ValueError("pad must be uint8 [B, >= L_cap]")
    return pad, pad.stride(0)


def spec_block_means(k_cache, cache_len, block, *, pad=None, first_block=0, n_blocks=None,
                     means=None, workspace=None):
    """Mean key of the cache blocks [first_block, first_block + n_blocks)
    into ``means`` (fp32 ``[B, Hkv, max_blocks, D]``; allocated for the
    whole capacity when None).  Returns ``means``."""
    lib = load()
    _on_gpu(k_cache, cache_len, pad, means)
    B, Hkv, cap, D = k_cache.shape
    if cache_len.dtype != torch.int32 or cache_len.numel() != B or not cache_len.is_contiguous():
        raise ValueError("cache_len must be a contiguous int32 [B] tensor")
    if means is None:
        means = torch.full((B, Hkv, -(-cap // block), D), float("nan"), dtype=torch.float32,
                           device=k_cache.device)
    if means.dtype != torch.float32 or means.dim() != 4 or not means.is_contiguous() or \
            tuple(means.shape[:2]) != (B, Hkv) or means.shape[3] != D:
        raise ValueError("means must be contiguous fp32 [B, Hkv, max_blocks, D]")
    if n_blocks is None:
        n_blocks = means.shape[2] - first_block
    kv = _kv(k_cache, k_cache)
    pad_t, psb = _pad_arg(pad, B, cap)
    dims = make_dims(B, Hkv, Hkv, D, _dtype_code(k_cache))
    if workspace is None:
        workspace = new_workspace(select_workspace_bytes(dims), k_cache.device)
    st = lib.spec_block_means(ctypes.byref(dims), ctypes.byref(kv), _ptr(cache_len), _ptr(pad_t),
                              psb, block, first_block, n_blocks, _ptr(means), means.shape[2],
                              _ptr(workspace), workspace.numel(), _stream(k_cache))
    _check(st)
    return means


def spec_select_blocks(q, means, cache_len, *, block, capacity, n_sink, window, n_select, budget,
                       pad=None, shared=False, idx=None, scores=None, want_scores=False,
                       workspace=None):
    """Budget lists ``[B, Hkv, budget]`` (``[B, 1, budget]`` when shared)
    int32 (sink, best-scoring blocks, window; -1 padded) from block means.
    Returns (idx, scores or None)."""
    lib = load()
    _on_gpu(q, means, cache_len, pad, idx, scores)
    if q.dim() != 4 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, Tq, Hq, D] tensor")
    B, T, Hq, D = q.shape
    if means.dtype != torch.float32 or means.dim() != 4 or not means.is_contiguous() or \
            means.shape[0] != B or means.shape[3] != D:
        raise ValueError("means must be contiguous fp32 [B, Hkv, max_blocks, D]")
    Hkv, max_blocks = means.shape[1], means.shape[2]
    if cache_len.dtype != torch.int32 or cache_len.numel() != B or not cache_len.is_contiguous():
        raise ValueError("cache_len must be a contiguous int32 [B] tensor")
    pad_t, psb = _pad_arg(pad, B, capacity)
    n_lists = 1 if shared else Hkv
    if idx is None:
        idx = torch.empty((B, n_lists, budget), dtype=torch.int32, device=q.device)
    if scores is None and want_scores:
        scores = torch.empty((B, n_lists, max_blocks), dtype=torch.float32, device=q.device)
    if tuple(idx.shape) != (B, n_lists, budget) or idx.dtype != torch.int32 or not idx.is_contiguous():
        raise ValueError("idx must be a contiguous int32 [B, 1 or Hkv, budget] tensor")
    dims = make_dims(B, Hq, Hkv, D, _dtype_code(q))
    if workspace is None:
        workspace = new_workspace(select_workspace_bytes(dims, max_blocks), q.device)
    st = lib.spec_select_blocks(ctypes.byref(dims), _ptr(q), T, _ptr(means), max_blocks, block,
                                _ptr(cache_len), capacity, _ptr(pad_t), psb, n_sink, window,
                                n_select, int(bool(shared)), _ptr(idx), budget, _ptr(scores),
                                _ptr(workspace), workspace.numel(), _stream(q))
    _check(st)
    return idx, scores


def spec_kv_gather(k_cache, v_cache, cache_len, idx, *, partial_k=None, partial_v=None,
                   partial_len=None, partial_pad=None, capacity=None, workspace=None):
    """Build the partial cache from one budget list per sequence (``idx``
    int32 ``[B, 1, budget]`` or ``[B, budget]``).  Returns (partial_k,
    partial_v, partial_len, partial_pad); the partial tensors are allocated
    (zero-filled) with ``capacity`` slots (default: the budget) when None."""
    lib = load()
    _on_gpu(k_cache, v_cache, cache_len, idx, partial_k, partial_v, partial_len, partial_pad)
    B, Hkv, _, D = k_cache.shape
    if idx.dtype != torch.int32 or idx.shape[0] != B or idx.stride(-1) != 1 or \
            (idx.dim() == 3 and idx.shape[1] != 1) or idx.dim() not in (2, 3):
        raise ValueError("idx must be int32 [B, 1, budget] or [B, budget]")
    budget = idx.shape[-1]
    if cache_len.dtype != torch.int32 or cache_len.numel() != B or not cache_len.is_contiguous():
        raise ValueError("cache_len must be a contiguous int32 [B] tensor")
    dev = k_cache.device
    cap = budget if capacity is None else capacity
    if partial_k is None:
        partial_k = torch.zeros((B, Hkv, cap, D), dtype=k_cache.dtype, device=dev)
        partial_v = torch.zeros_like(partial_k)
    if partial_len is None:
        partial_len = torch.empty(B, dtype=torch.int32, device=dev)
    if partial_pad is None:
        partial_pad = torch.zeros((B, (partial_k.shape[2] + 3) // 4 * 4), dtype=torch.uint8, device=dev)
    kv = _kv(k_cache, v_cache)
    pkv = _kv(partial_k, partial_v)
    if workspace is None:
        workspace = new_workspace(256, dev)
    st = lib.spec_kv_gather(B, Hkv, D, _dtype_code(k_cache), ctypes.byref(kv), _ptr(cache_len),
                            _ptr(idx), budget, idx.stride(0), ctypes.byref(pkv), _ptr(partial_len),
                            _ptr(partial_pad), partial_pad.stride(0), _ptr(workspace),
                            workspace.numel(), _stream(k_cache))
    _check(st)
    return partial_k, partial_v, partial_len, partial_pad


def spec_verify_mode(seq_len: int, budget: int, buffered: int, n_nodes: int,
                     buffer_capacity: int) -> int:
    """SPEC_VERIFY_FULL or SPEC_VERIFY_PARTIAL for the next step (host only)."""
    r = load().spec_verify_mode(seq_len, budget, buffered, n_nodes, buffer_capacity)
    if r < 0:
        _check(r)
    return int(r)


def spec_device_status(workspace: torch.Tensor) -> int:
    """Synchronise the current stream and return (and clear) the device error
    bits kept in ``workspace`` (0 = no error)."""
    lib = load()
    bits = ctypes.c_uint32(0)
    st = lib.spec_device_status(_ptr(workspace), _stream(workspace), ctypes.byref(bits))
    if st not in (SPEC_OK, SPEC_E_DEVICE_RANGE):
        _check(st)
    return int(bits.value)
