"""KV commit of the accepted path, plain definition (test infrastructure only).

After acceptance, a batched verifier keeps each sequence's accepted tokens
and pads the batch to one uniform number of new slots; the pad slots are then
scored -inf by later attention and ignored by the position remap (SpecMemo
review, "What carries the argument" and Figure 9: the four sequences accept
2, 4, 1 and 2 tokens and are padded to one shape).  Candidates that were not
accepted are removed from the cache once verification is done (SpecPV,
section 3.3 "Rectified with Full Verification").

Reading of what the pages leave open:

* A sequence that accepted tau draft nodes appends tau + 1 slots: the
  accepted nodes' keys and values, copied from the tree K/V in path order,
  then one slot for the bonus token (the verifier's target after the last
  accepted node).  The bonus token becomes the next anchor; its K/V comes
  from the caller's next forward pass, so the commit marks the slot valid
  and writes no K/V into it.
* Every sequence of the batch appends the same P = 1 + max_b tau_b slots;
  slots past a sequence's bonus slot are padding (pad byte 1), and
  cache_len grows by P.
* A sequence whose accept length lies outside [0, min(max_depth, N)] (a root
  path has at most N nodes), or whose path names a node outside [0, N),
  contributes tau = 0 to P and appends P padding slots (nothing of it is
  committed); the error is reported.
* A sequence whose cache_len lies outside [0, capacity - P] is left as it
  is (no slot written, cache_len unchanged); the error is reported.
"""
from __future__ import annotations

import numpy as np

ERR_CACHE_LEN = 1
ERR_COMMIT = 16


def _valid(tau: int, path_b, n_nodes: int, max_depth: int) -> bool:
    if tau < 0 or tau > min(max_depth, n_nodes):
        return False
    return all(0 <= int(path_b[j]) < n_nodes for j in range(tau))


def commit_ref(k, v, cache_len, pad, tree_k, tree_v, accept_len, accept_path, max_depth: int):
    """Commit the accepted paths of a batch.

    ``k``, ``v``: cache ``[B, Hkv, L_cap, D]`` (any element type: the commit
    copies elements); ``cache_len`` ``[B]``; ``pad`` ``[B, >= L_cap]`` uint8
    (nonzero = padding); ``tree_k``, ``tree_v``: ``[B, Hkv, N, D]``, the K/V
    of the speculated nodes; ``accept_len`` ``[B]`` and ``accept_path``
    ``[B, max_depth]`` as produced by greedy acceptance.

    Returns ``(k, v, cache_len, pad, P, err)``: new arrays (the inputs are
    not modified), the number of slots appended per sequence and the error
    bits (1: a cache_len out of range; 16: a bad accept length or path).
    """
    k = np.array(k, copy=True)
    v = np.array(v, copy=True)
    pad = np.array(pad, copy=True)
    cache_len = np.array(cache_len, dtype=np.int64, copy=True)
    tree_k = np.asarray(tree_k)
    tree_v = np.asarray(tree_v)
    accept_len = np.asarray(accept_len)
    accept_path = np.asarray(accept_path)
    B = len(cache_len)
    cap = k.shape[2]
    N = tree_k.shape[2]
    err = 0
    valid = [_valid(int(accept_len[b]), accept_path[b], N, max_depth) for b in range(B)]
    P = 1 + max([int(accept_len[b]) if valid[b] else 0 for b in range(B)], default=0)
    for b in range(B):
        if not valid[b]:
            err |= ERR_COMMIT
        L = int(cache_len[b])
        if L < 0 or L + P > cap:
            err |= ERR_CACHE_LEN
            continue
        tau = int(accept_len[b]) if valid[b] else -1
        for j in range(tau if tau > 0 else 0):
            node = int(accept_path[b, j])
            k[b, :, L + j, :] = tree_k[b, :, node, :]
            v[b, :, L + j, :] = tree_v[b, :, node, :]
        for j in range(P):
            pad[b, L + j] = 0 if j <= tau else 1
        cache_len[b] = L + P
    return k, v, cache_len, pad, P, err


def compact_ref(k, v, cache_len, pad):
    """Drop the padding slots of each sequence's cache (the pads that batched
    commits leave behind; SpecPV section 3.3 removes the tokens that were not
    accepted once verification is done, SpecMemo Figure 9 pads per step).

    Reading of what the pages leave open: the valid slots j < cache_len[b]
    (pad byte 0) keep their order and move to slots 0, 1, ...; cache_len[b]
    becomes their count; every pad byte below the old cache_len is cleared.
    The contents of the slots from the new cache_len on are left unspecified
    (here: as they were).  A sequence whose cache_len lies outside
    [0, capacity] is left as it is and the error is reported (bit 1).

    ``k``, ``v``: ``[B, Hkv, L_cap, D]``; ``cache_len`` ``[B]``; ``pad``
    ``[B, >= L_cap]`` uint8.  Returns new arrays ``(k, v, cache_len, pad,
    err)``.
    """
    k = np.array(k, copy=True)
    v = np.array(v, copy=True)
    pad = np.array(pad, copy=True)
    cache_len = np.array(cache_len, dtype=np.int64, copy=True)
    cap = k.shape[2]
    err = 0
    for b in range(len(cache_len)):
        L = int(cache_len[b])
        if L < 0 or L > cap:
            err |= ERR_CACHE_LEN
            continue
        keep = np.nonzero(pad[b, :L] == 0)[0]
        n = len(keep)
        k[b][:, :n] = k[b][:, keep]
        v[b][:, :n] = v[b][:, keep]
        pad[b, :L] = 0
        cache_len[b] = n
    return k, v, cache_len, pad, err
