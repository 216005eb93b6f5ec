"""Shared test helpers: moving generator arrays to the GPU and comparing the
library's outputs with the oracle's."""
from __future__ import annotations

import numpy as np
import torch

import oracle

ATOL = {"bf16": 1e-2, "f32": 2e-5}      # max-abs bar against the fp64 oracle
RTOL_L2 = {"bf16": 1e-2, "f32": 1e-5}   # relative L2 guard (a near-uniform softmax has tiny outputs)


def dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    """Generator array -> GPU tensor (uint16 bit patterns become bfloat16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def host64(t: torch.Tensor) -> np.ndarray:
    """GPU output -> float64 numpy (bf16 widened exactly)."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
        return oracle.decode_bf16(bits)
    return t.cpu().numpy().astype(np.float64)


# Per-element bar for bf16: |got - ref| <= 1e-2 + 2^-7 |ref|.  The relative
# term covers the two roundings whose error grows with the output itself:
# the bf16 output (half an ulp, 2^-8 |o|) and the bf16 probabilities of the
# P.V product (2^-8 of each term, i.e. up to 2^-8 |o| when one key dominates
# the row).  The absolute 1e-2 is the bar the workloads state for bf16;
# fp32 stays absolute.
RTOL_ELEM = {"bf16": 2.0 ** -7, "f32": 0.0}

# (label, max |err|, fraction of the per-element bar used) of every
# assert_close call of the session; conftest prints them at the end.
ERROR_LOG: list = []


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    """Every element within its bar, atol + rtol_elem |ref|, plus a relative
    L2 guard, on the rows the oracle computed (NaN rows in ``ref`` are rows
    it skipped).  Returns the max abs error and logs it with the fraction of
    the bar it used."""
    mask = ~np.isnan(ref)
    assert mask.any(), "oracle computed nothing"
    g, r = got[mask], ref[mask]
    assert np.all(np.isfinite(g)), f"{what}: non-finite outputs"
    d = np.abs(g - r)
    bar = ATOL[dtype] + RTOL_ELEM[dtype] * np.abs(r)
    used = float((d / bar).max())
    err = float(d.max())
    ERROR_LOG.append((what, dtype, err, used))
    if used > 1.0:
        i = int(np.argmax(d / bar))
        raise AssertionError(f"{what}: |err| {d[i]:.3e} > bar {bar[i]:.3e} at ref {r[i]:.4g} "
                             f"(max abs error {err:.3e}, {used:.2f}x the bar)")
    nr = np.linalg.norm(r)
    if nr > 0:
        rel = np.linalg.norm(g - r) / nr
        assert rel <= RTOL_L2[dtype], f"{what}: relative L2 error {rel:.3e} > {RTOL_L2[dtype]}"
    return err


def assert_lse_close(got: np.ndarray, ref: np.ndarray, tol: float, what: str = ""):
    mask = ~np.isnan(ref)
    g, r = got[mask], ref[mask]
    inf = np.isinf(r)
    assert np.array_equal(np.isinf(g), inf), f"{what}: -inf pattern differs"
    if (~inf).any():
        err = np.abs(g[~inf] - r[~inf]).max()
        assert err <= tol, f"{what}: lse error {err:.3e} > {tol}"
