"""Partial verification, plain definitions (test infrastructure only).

SpecPV (section 3.2 "Partial Verification"): verification attends to a
partial KV cache of a sink, retrieved blocks, a local window and a buffer of
the tokens verified since, kept contiguous in token order and handled as one
KV segment in the attention pass.  Section 3.3 "Rectified with Full
Verification": a full verification over the whole cache refreshes the partial
cache; partial verification is disabled while the sequence is shorter than
the partial budget, and a full verification replaces it whenever the
partially verified tokens plus the new candidates would exceed the buffer.

Reading of what the pages leave open:

* The partial cache is built from a budget list (the sink / blocks / window
  list of the block-mean selection): slot j holds the key and value of the
  listed position; a -1 entry gives a padding slot (pad byte 1, zeros).  Its
  length is the list length, and the buffer's tokens are appended after it
  by the KV commit, like any cache.
* A listed position outside [0, cache_len) other than -1 is an input error:
  its slot becomes padding and the error is reported.
* Partial verification is the tree verify over the partial cache.
"""
from __future__ import annotations

import numpy as np

ERR_INDEX = 2
FULL, PARTIAL = 0, 1


def gather_ref(k, v, cache_len, idx, capacity: int):
    """Partial cache from one budget list per sequence, ``idx`` ``[B, 1,
    budget]``: returns ``(pk, pv, pad, length, err)`` with ``pk``/``pv``
    ``[B, Hkv, capacity, D]`` (slot j = listed position j; zero for padding
    slots and past the list), ``pad`` ``[B, capacity]`` uint8 (1 for -1 and
    bad entries, 0 elsewhere), ``length`` ``[B]`` = budget."""
    k = np.asarray(k)
    B, Hkv, _, D = k.shape
    idx = np.asarray(idx)
    if idx.shape[1] != 1:
        raise ValueError("a partial cache takes one list per sequence")
    pk = np.zeros((B, Hkv, capacity, D), dtype=k.dtype)
    pv = np.zeros((B, Hkv, capacity, D), dtype=k.dtype)
    pad = np.zeros((B, capacity), dtype=np.uint8)
    err = 0
    for b in range(B):
        L = int(cache_len[b])
        for j, p in enumerate(idx[b, 0]):
            p = int(p)
            if 0 <= p < L:
                pk[b, :, j] = k[b, :, p]
                pv[b, :, j] = v[b, :, p]
            else:
                if p != -1:
                    err |= ERR_INDEX
                pad[b, j] = 1
    return pk, pv, pad, np.full(B, idx.shape[2], dtype=np.int32), err


def verify_mode_ref(seq_len: int, budget: int, buffered: int, n_nodes: int,
                    buffer_capacity: int) -> int:
    """FULL while the sequence is shorter than the partial budget, or when
    the buffered (partially verified) tokens plus the new candidates would
    not fit the buffer; PARTIAL otherwise."""
    if seq_len < budget:
        return FULL
    if buffered + n_nodes > buffer_capacity:
        return FULL
    return PARTIAL
