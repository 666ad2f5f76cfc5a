"""Comparison rules shared by the GPU parity tests.

Index rule (floating point decides an integer): indices agree on >= 99.99% of
coordinates and every disagreement is one step apart with the oracle's
rotated unit-vector coordinate within 1e-5 of a decision boundary.
Reconstructions and logits: per-row relative L2 error <= 1e-3 and every
element within 1e-3 of the row's RMS (float32 accumulation).
Sign rule (QJL bits): the oracle re-derives the residual, its norm and the
projection S r from the GPU's own indices (prod_signs_from_indices), so every
vector is checked, index flips included.  >= 99.99% of bits agree and every
disagreement has |(S r)_i| <= SIGN_TOL in unit-vector units (the units of the
index rule).  The bound comes from the split-bf16 arithmetic: each product of
a hi/lo-split operand pair carries a relative error of about 2^-17 (RMS), so
the decided value (S r)_i = (M r~)_i carries an error of RMS about
2^-17 sqrt(1 + ||r||^2) (rotation error pushed through M, plus the second
product); the tiled path, which forms S u - M c[idx], about sqrt(2) 2^-17.
SIGN_TOL is about 4.6 of those standard deviations.  The residual norm
agrees to RNORM_RTOL (its error is the projection of the rotation error on
r, about 2^-17 / sqrt(d) in absolute terms).
"""
import numpy as np

IDX_AGREE = 0.9999
IDX_BOUNDARY_TOL = 1e-5
REL_TOL = 1e-3
SIGN_AGREE = 0.9999
SIGN_TOL = 5e-5
RNORM_RTOL = 1e-4


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


def check_signs(gpu_bits, ora_bits, ora_proj, what=""):
    gpu_bits = np.asarray(gpu_bits).astype(np.int64)
    ora_bits = np.asarray(ora_bits).astype(np.int64)
    mism = gpu_bits != ora_bits
    frac = 1.0 - mism.mean()
    assert frac >= SIGN_AGREE, f"{what}: sign agreement {frac:.7f}"
    worst = 0.0
    if mism.any():
        worst = float(np.abs(np.asarray(ora_proj)[mism]).max())
        assert worst <= SIGN_TOL, f"{what}: sign mismatch at |Sr| = {worst:.3g}"
    return frac, int(mism.sum()), worst


class QJLCheck:
    """Collects the GPU's QJL signs and residual norms of several batches
    beside the oracle's QJL stage taken on the GPU's own indices
    (prod_signs_from_indices), then applies the sign rule to all of them at
    once (the agreement share is a statistic of the whole test)."""

    def __init__(self):
        self.gpu, self.ora, self.proj, self.grn, self.orn = [], [], [], [], []

    def add(self, cd, x, gpu_idx, gpu_bits, gpu_rnorms, group=0):
        from oracle import tq_oracle as O

        x = np.asarray(x, dtype=np.float64).reshape(-1, cd.d)
        ref = O.prod_signs_from_indices(cd, x, gpu_idx, group)
        self.gpu.append(np.asarray(gpu_bits).reshape(ref["proj"].shape))
        self.ora.append(O.signs_to_bits(ref["signs"]))
        self.proj.append(ref["proj"])
        self.grn.append(np.asarray(gpu_rnorms, dtype=np.float64).reshape(-1))
        self.orn.append(ref["rnorms"])
        return self

    def check(self, what=""):
        out = check_signs(np.concatenate(self.gpu), np.concatenate(self.ora), np.concatenate(self.proj), what)
        got, ref = np.concatenate(self.grn), np.concatenate(self.orn)
        bad = np.abs(got - ref) > RNORM_RTOL * np.abs(ref) + 1e-6
        assert not bad.any(), f"{what}: residual norm off by {np.max(np.abs(got - ref) / np.maximum(ref, 1e-30)):.3g}"
        return out


def check_qjl(cd, x, gpu_idx, gpu_bits, gpu_rnorms, group=0, what=""):
    """QJL signs and residual norms of every vector of x ([n, d]) against the
    oracle's QJL stage taken on the GPU's own indices (None without mse
    bits): sign rule above, residual norms to RNORM_RTOL."""
    return QJLCheck().add(cd, x, gpu_idx, gpu_bits, gpu_rnorms, group).check(what)
