"""Comparison rules shared by the GPU parity tests.

Index rule (floating point decides an integer): indices agree on >= 99.99% of
coordinates and every disagreement is one step apart with the oracle's
rotated unit-vector coordinate within 1e-5 of a decision boundary.
Reconstructions and logits: per-row relative L2 error <= 1e-3 and every
element within 1e-3 of the row's RMS (float32 accumulation).
Sign rule (QJL bits, silent in the stated bars; derived from the split-bf16
arithmetic of the projection): on vectors whose indices all agree, >= 99.9%
of bits agree and every disagreement has |(S r)_i| <= 2e-4 * ||r||.
"""
import numpy as np

IDX_AGREE = 0.9999
IDX_BOUNDARY_TOL = 1e-5
REL_TOL = 1e-3
SIGN_AGREE = 0.999
SIGN_TOL = 2e-4


def check_indices(gpu_idx, ora_idx, ora_y, boundaries, what=""):
    gpu_idx = np.asarray(gpu_idx).astype(np.int64)
    ora_idx = np.asarray(ora_idx).astype(np.int64)
    mism = gpu_idx != ora_idx
    frac = 1.0 - mism.mean()
    assert frac >= IDX_AGREE, f"{what}: index agreement {frac:.6f}"
    if mism.any():
        assert np.all(np.abs(gpu_idx[mism] - ora_idx[mism]) == 1), f"{what}: a mismatch is more than one step"
        yv = np.asarray(ora_y)[mism]
        dist = np.min(np.abs(yv[:, None] - np.asarray(boundaries)[None, :]), axis=1)
        assert dist.max() <= IDX_BOUNDARY_TOL, f"{what}: mismatch {dist.max():.3g} from a boundary"
    return frac, int(mism.sum())


def check_rows(got, ref, what="", tol=REL_TOL):
    got = np.asarray(got, dtype=np.float64).reshape(-1, np.asarray(got).shape[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(got.shape)
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    rms = den / np.sqrt(ref.shape[1])
    ok = den > 0
    rel = np.where(ok, num / np.where(ok, den, 1.0), num)
    assert rel.max() <= tol, f"{what}: worst row relative error {rel.max():.3g}"
    el = np.max(np.abs(got - ref), axis=1)
    assert np.all(el <= tol * np.maximum(rms, 1e-30) + (0 if ok.all() else 1e-30)), f"{what}: element error"
    return float(rel.max())


def check_signs(gpu_bits, ora_bits, ora_proj, ora_rnorm, what=""):
    gpu_bits = np.asarray(gpu_bits).astype(np.int64)
    ora_bits = np.asarray(ora_bits).astype(np.int64)
    mism = gpu_bits != ora_bits
    frac = 1.0 - mism.mean()
    assert frac >= SIGN_AGREE, f"{what}: sign agreement {frac:.6f}"
    if mism.any():
        r = np.broadcast_to(np.asarray(ora_rnorm)[:, None], mism.shape)[mism]
        p = np.abs(np.asarray(ora_proj)[mism])
        assert np.all(p <= SIGN_TOL * r + 1e-30), f"{what}: sign mismatch at |Sr| = {(p / r).max():.3g} ||r||"
    return frac, int(mism.sum())
