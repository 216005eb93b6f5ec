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


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "",
                 magnitude: float = 1.0):
    """Max-abs error within the bar, plus a relative L2 guard, on the rows
    the oracle computed (NaN rows in ``ref`` are rows it skipped).

    ``magnitude`` scales the absolute bar for inputs whose outputs exceed 1:
    a bf16 output near x carries a rounding error of up to |x| 2^-9, and the
    bf16 probabilities of P.V up to another |x| 2^-9, so the bar of outputs
    of order 1 becomes a relative one above it."""
    mask = ~np.isnan(ref)
    assert mask.any(), "oracle computed nothing"
    g, r = got[mask], ref[mask]
    assert np.all(np.isfinite(g)), f"{what}: non-finite outputs"
    err = np.abs(g - r).max()
    bar = ATOL[dtype] * max(1.0, magnitude)
    assert err <= bar, f"{what}: max abs error {err:.3e} > {bar:.3e}"
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
