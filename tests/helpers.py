"""Shared test utilities: comparisons and host<->device conversions.

Only plumbing lives here (no arithmetic of the method): the oracle computes the
expected values, the library computes the results, and these helpers move and
compare bits.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

REL_L2_TOL = 2e-3   # floats: relative L2 per (request, head) unit, in the stored dtype


def bf16_np(t: torch.Tensor) -> np.ndarray:
    """Bits of a bf16 tensor (any device) as numpy uint16."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def widen(bits: np.ndarray) -> np.ndarray:
    return oracle.bf16_widen(bits)


def rel_l2(got: np.ndarray, want: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(want)
    num = np.linalg.norm(got - want)
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


def worst_unit_rel_l2(got: np.ndarray, want: np.ndarray, unit_axes: int) -> float:
    """Largest relative L2 over units formed by the leading ``unit_axes`` axes."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    lead = got.shape[:unit_axes]
    g = got.reshape(int(np.prod(lead)), -1)
    w = want.reshape(int(np.prod(lead)), -1)
    worst = 0.0
    for i in range(g.shape[0]):
        if np.linalg.norm(w[i]) == 0.0 and np.linalg.norm(g[i]) == 0.0:
            continue
        worst = max(worst, rel_l2(g[i], w[i]))
    return worst


def unit_rel_l2(got: np.ndarray, want: np.ndarray, unit_axes: int, chunk: int = 2048) -> np.ndarray:
    """Relative L2 of every unit formed by the leading ``unit_axes`` axes, as an
    array of that shape.  uint16 inputs are bf16 bits and are widened first; the
    work goes in blocks of ``chunk`` units to bound the host memory.  A unit whose
    reference and result are both zero scores 0."""
    lead = got.shape[:unit_axes]
    n = int(np.prod(lead))
    g = got.reshape(n, -1)
    w = want.reshape(n, -1)
    res = np.zeros(n, dtype=np.float64)
    for i in range(0, n, chunk):
        gi = widen(g[i:i + chunk]) if g.dtype == np.uint16 else g[i:i + chunk].astype(np.float64)
        wi = widen(w[i:i + chunk]) if w.dtype == np.uint16 else w[i:i + chunk].astype(np.float64)
        num = np.linalg.norm(gi - wi, axis=1)
        den = np.linalg.norm(wi, axis=1)
        with np.errstate(divide="ignore", invalid="ignore"):
            r = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num > 0, np.inf, 0.0))
        res[i:i + chunk] = r
    return res.reshape(lead)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x| (8 significant bits; the smallest normal's
    spacing below it)."""
    ax = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def output_unit_ok(got_bits: np.ndarray, want_bits: np.ndarray, exact: np.ndarray, tol: float = REL_L2_TOL):
    """Output comparison of one unit, for units small enough that one rounding
    decision matters.  First the stated rule: relative L2 of the GPU's bf16
    outputs against the oracle's bf16-rounded ones.  Where that exceeds tol, the
    two sides have rounded values that lie next to a bf16 rounding midpoint to
    neighbouring bf16 values, and both results are correct roundings: then every
    GPU output must be within one bf16 spacing of the oracle's exact value, and
    the GPU's error beyond the error of rounding the exact values, sqrt(e^2 -
    r^2) with e = |gpu - exact| and r = |bf16(exact) - exact| in relative L2,
    must be within tol.  The spacing is taken at no less than 1/16 of the unit's
    RMS exact output: an fp32-accumulated output carries an absolute error that
    scales with the unit's magnitude, which can exceed the spacing at an output
    near zero.  Returns (ok, stated rel-L2, excess)."""
    got = widen(got_bits)
    want = widen(want_bits)
    ex = np.asarray(exact, dtype=np.float64)
    e_stated = rel_l2(got, want)
    if e_stated <= tol:
        return True, e_stated, 0.0
    floor = np.sqrt(np.mean(ex * ex)) / 16.0
    valid = bool(np.all(np.abs(got - ex) <= bf16_ulp(np.maximum(np.abs(ex), floor))))
    e = rel_l2(got, ex)
    r = rel_l2(want, ex)
    excess = float(np.sqrt(max(e * e - r * r, 0.0)))
    return valid and excess <= tol, e_stated, excess


def pool_to_oracle(ssm: torch.Tensor, conv: torch.Tensor) -> oracle.Pool:
    """Copy a device (or host) pool into an oracle host pool, byte for byte."""
    L, N, H, V, K = ssm.shape
    dt = oracle.SSM_F32 if ssm.dtype == torch.float32 else oracle.SSM_BF16
    p = oracle.Pool(L, N, H, K, V, dt)
    if dt == oracle.SSM_F32:
        p.ssm()[:] = ssm.detach().cpu().numpy()
    else:
        p.ssm()[:] = bf16_np(ssm)
    p.conv()[:] = bf16_np(conv)
    return p


def ssm_values(p: oracle.Pool) -> np.ndarray:
    """Pool ssm as float64 values [L,N,H,V,K]."""
    s = p.ssm()
    return s.astype(np.float64) if p.ssm_dtype == oracle.SSM_F32 else widen(s)


def device_ssm_values(ssm: torch.Tensor) -> np.ndarray:
    return ssm.detach().cpu().to(torch.float64).numpy()


def pool_bytes_equal(ssm: torch.Tensor, conv: torch.Tensor, p: oracle.Pool) -> bool:
    a = ssm.detach().cpu().contiguous().view(torch.uint8).numpy().ravel()
    b = conv.detach().cpu().contiguous().view(torch.uint8).numpy().ravel()
    return np.array_equal(a, p.ssm_bytes) and np.array_equal(b, p.conv_bytes)
