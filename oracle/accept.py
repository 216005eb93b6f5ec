"""Greedy tree acceptance, plain definitions (test infrastructure only).

Logits are ``[B, N+1, V]`` float32: row 0 is the verifier's output at the
anchor (the last committed token) and row i+1 its output at tree node i.  The
verifier's greedy target after a position is the argmax of that row
(BudgetDraft review, Figure 2: the full-cache verifier produces greedy
targets).  A draft node is accepted when its token equals its parent's
greedy target and its parent is accepted; the target alone decides every
accepted token (Windowed-MTP review, losslessness).  The accept length counts
accepted draft tokens and may be 0 (SpecPV, section 4.1 "Metrics").
"""
from __future__ import annotations

import numpy as np

from .attention import tree_depths


def argmax_ref(row: np.ndarray) -> int:
    """Index of the maximum of one row.  Ties go to the smallest index; a NaN
    counts as larger than every number, so the first NaN wins."""
    row = np.asarray(row)
    nan = np.isnan(row)
    if nan.any():
        return int(np.nonzero(nan)[0][0])
    return int(np.nonzero(row == row.max())[0][0])


def _one(logits_b, tok_b, par_b, max_depth):
    N = len(par_b)
    am = [argmax_ref(logits_b[r]) for r in range(N + 1)]
    depth = tree_depths(par_b)
    acc = np.zeros(N, dtype=bool)
    for i in range(N):                      # parents precede children
        p = int(par_b[i])
        parent_ok = True if p < 0 else acc[p]
        acc[i] = parent_ok and int(tok_b[i]) == am[p + 1]
    best = -1
    for i in range(N):                      # deepest accepted, then lowest index
        if acc[i] and (best < 0 or depth[i] > depth[best]):
            best = i
    if best < 0:
        return 0, [], am[0], am
    path = []
    j = best
    while j >= 0:
        path.append(j)
        j = int(par_b[j])
    path.reverse()
    if len(path) > max_depth:
        raise ValueError("accepted path longer than max_depth")
    return len(path), path, am[best + 1], am


def accept_ref(logits, tokens, parents, max_depth: int):
    """Per sequence: accept length, accepted path (root first, -1 padded to
    ``max_depth``) and the bonus token (the verifier's greedy target after the
    last accepted position, i.e. after the anchor when nothing is accepted).
    ``parents`` is ``[N]`` (shared) or ``[B, N]``."""
    logits = np.asarray(logits)
    B = logits.shape[0]
    par = np.asarray(parents)
    lens = np.zeros(B, dtype=np.int32)
    paths = np.full((B, max_depth), -1, dtype=np.int32)
    bonus = np.zeros(B, dtype=np.int32)
    for b in range(B):
        pb = par if par.ndim == 1 else par[b]
        n, path, bon, _ = _one(logits[b], tokens[b], pb, max_depth)
        lens[b] = n
        paths[b, :n] = path
        bonus[b] = bon
    return lens, paths, bonus


def accept_bruteforce(logits, tokens, parents, max_depth: int):
    """Same result by enumeration: list every root-to-node path, keep those
    whose every node carries its predecessor's greedy target, take the longest
    (ties: smallest end node).  Independent of the flag propagation above."""
    logits = np.asarray(logits)
    B = logits.shape[0]
    par = np.asarray(parents)
    lens = np.zeros(B, dtype=np.int32)
    paths = np.full((B, max_depth), -1, dtype=np.int32)
    bonus = np.zeros(B, dtype=np.int32)
    for b in range(B):
        pb = par if par.ndim == 1 else par[b]
        N = len(pb)
        target = [int(np.argmax(logits[b, r])) for r in range(N + 1)]
        best_path, best_end = [], -1
        for end in range(N):
            path = []
            j = end
            while j >= 0:
                path.append(j)
                j = int(pb[j])
            path.reverse()
            prev_row = 0
            ok = True
            for node in path:
                if int(tokens[b, node]) != target[prev_row]:
                    ok = False
                    break
                prev_row = node + 1
            if ok and len(path) > len(best_path):
                best_path, best_end = path, end
        lens[b] = len(best_path)
        paths[b, :len(best_path)] = best_path
        bonus[b] = target[best_end + 1] if best_end >= 0 else target[0]
    return lens, paths, bonus
