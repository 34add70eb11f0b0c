"""Parity helpers shared by the GPU tests (test infrastructure).

The tolerance is the one the hot path is held to: per token, relative L2
error <= 2e-3; over the whole call, max elementwise error <= 1e-2 * max|y_ref|.
Integer / bit-level results (unpacking, exact dequantisation, skip-zero
zeros) are compared bit for bit instead.
"""
import numpy as np
import torch

REL_L2 = 2e-3
MAX_ABS_FRAC = 1e-2


def x_to_torch(x: np.ndarray, device="cuda") -> torch.Tensor:
    """float32 values or bf16 bit patterns (uint16) -> device tensor."""
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def check_close(y_gpu, y_ref, what=""):
    y = np.asarray(y_gpu, dtype=np.float64)
    r = np.asarray(y_ref, dtype=np.float64)
    assert y.shape == r.shape, (y.shape, r.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    if y.ndim == 1:
        y, r = y[None], r[None]
    err = np.linalg.norm(y - r, axis=1)
    nrm = np.linalg.norm(r, axis=1)
    rel = np.where(nrm > 0, err / np.maximum(nrm, 1e-300), err)
    mx = np.abs(y - r).max() if y.size else 0.0
    ref_max = np.abs(r).max() if r.size else 0.0
    assert rel.max() <= REL_L2, f"{what}: per-token rel-L2 {rel.max():.3e} > {REL_L2}"
    assert mx <= MAX_ABS_FRAC * ref_max + 1e-30, \
        f"{what}: max abs err {mx:.3e} > {MAX_ABS_FRAC} * {ref_max:.3e}"
    return float(rel.max()), float(mx / ref_max) if ref_max > 0 else 0.0


def dead_rows(T, e):
    """Logical rows of expert e that are skip-zero."""
    if T.row_map is None:
        return np.zeros(T.rows, dtype=bool)
    return T.row_map[e * T.rows:(e + 1) * T.rows] < 0


def check_close_terms(y_gpu, y_ref, y_terms, what="", well_conditioned=0.25):
    """Per-token error against the size of the terms that make up the token.

    y_terms[t] is the token's output recomputed with every product replaced
    by its magnitude (|w| |W| |h|), so ||y_ref[t]|| << ||y_terms[t]|| means
    the terms cancel.  Each token's error must stay within REL_L2 of
    ||y_terms[t]||; a token whose terms do not cancel much
    (||y_ref|| >= well_conditioned * ||y_terms||) must also meet the plain
    per-token bar, and the call the max-abs bar."""
    y = np.asarray(y_gpu, dtype=np.float64)
    r = np.asarray(y_ref, dtype=np.float64)
    m = np.asarray(y_terms, dtype=np.float64)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    err = np.linalg.norm(y - r, axis=1)
    nrm = np.linalg.norm(r, axis=1)
    mag = np.linalg.norm(m, axis=1)
    worst = (err / np.maximum(mag, 1e-300)).max()
    assert worst <= REL_L2, f"{what}: error {worst:.3e} of the terms' size > {REL_L2}"
    good = nrm >= well_conditioned * mag
    assert good.mean() >= 0.5, f"{what}: only {good.mean():.2f} of the tokens well conditioned"
    rel = err[good] / nrm[good]
    assert rel.max() <= REL_L2, f"{what}: per-token rel-L2 {rel.max():.3e} > {REL_L2}"
    mx = np.abs(y - r).max()
    assert mx <= MAX_ABS_FRAC * np.abs(r).max(), f"{what}: max abs err {mx:.3e}"
    return float(worst)
