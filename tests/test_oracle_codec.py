"""Pins for the oracle's packing, quantizers and estimators (CPU only)."""
import math
import os

import numpy as np
import pytest

import workloads
from oracle import tq_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- packing ---
def _pack_by_hand(idx, bits, rbytes):
    stream = []
    for v in idx:
        for k in range(bits):
            stream.append((int(v) >> k) & 1)
    stream += [0] * (rbytes * 8 - len(stream))
    return [sum(stream[8 * i + k] << k for k in range(8)) for i in range(rbytes)]


def test_pack_golden_example():
    with open(os.path.join(GOLDEN, "pack_b3.txt")) as f:
        rows = {l.split()[0]: [int(v) for v in l.split()[1:]] for l in f if l.strip() and not l.startswith("#")}
    bits = rows["bits"][0]
    out = O.pack(np.array(rows["idx"]), bits)
    assert out.tolist() == rows["bytes"]


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("count", [1, 2, 3, 127, 128, 200])
def test_pack_matches_bit_by_bit_and_roundtrips(bits, count):
    rng = np.random.default_rng(bits * 1000 + count)
    idx = rng.integers(0, 1 << bits, (3, count))
    rb = O.row_bytes(count, bits)
    assert rb % 16 == 0 and rb * 8 >= count * bits and (rb - 16) * 8 < count * bits
    p = O.pack(idx, bits)
    assert p.shape == (3, rb)
    for r in range(3):
        assert p[r].tolist() == _pack_by_hand(idx[r], bits, rb)
    assert np.array_equal(O.unpack(p, bits, count), idx)


# ---------------------------------------------------------------- mse ------
@pytest.fixture(scope="module")
def parity_x():
    return workloads.parity_vectors().astype(np.float64)


@pytest.fixture(scope="module")
def parity_q():
    return workloads.parity_queries().astype(np.float64)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_mse_distortion_matches_codebook_distortion(parity_x, bits):
    # For u uniform on the sphere and any fixed Pi, E||u - u_hat||^2 = D_b.
    cd = O.make_codec(128, bits, O.MSE, 0)
    idx, nu, _ = O.quantize_mse(cd, parity_x)
    xh = O.dequantize_mse(cd, idx, nu)
    u = parity_x / nu[:, None]
    err = np.sum((u - xh / nu[:, None]) ** 2, axis=1)
    se = err.std() / math.sqrt(err.size)
    assert abs(err.mean() - cd.distortion) < 4 * se
    assert cd.distortion * 4 ** bits < math.sqrt(3) * math.pi / 2


@pytest.mark.parametrize("bits", [1, 2, 4])
def test_mse_inner_product_shrinkage(parity_x, parity_q, bits):
    # slope of <q, x_hat> against <q, x> is 1 - D_b; b = 1 gives ~0.64 (36% low)
    cd = O.make_codec(128, bits, O.MSE, 0)
    idx, nu, _ = O.quantize_mse(cd, parity_x)
    xh = O.dequantize_mse(cd, idx, nu)
    a = (parity_q @ xh.T).ravel()
    b = (parity_q @ parity_x.T).ravel()
    slope = float(a @ b / (b @ b))
    assert slope == pytest.approx(1.0 - cd.distortion, rel=0.015)
    if bits == 1:
        assert slope == pytest.approx(2 / math.pi, abs=0.02)


def test_norm_and_reconstruction_scale(parity_x):
    cd = O.make_codec(128, 4, O.MSE, 0)
    idx, nu, y = O.quantize_mse(cd, parity_x)
    assert np.allclose(nu, np.linalg.norm(parity_x, axis=1), rtol=1e-14)
    # y is Pi u, unit norm
    assert np.allclose(np.linalg.norm(y, axis=1), 1.0, atol=1e-12)
    assert idx.min() >= 0 and idx.max() < 16


def test_zero_vector_and_scale_invariance():
    cd = O.make_codec(128, 3, O.PROD, 0)
    x = np.zeros((2, 128))
    x[1, 5] = 3.0
    res = O.quantize_prod(cd, x)
    assert res["norms"][0] == 0.0 and res["rnorms"][0] == 0.0
    assert np.all(res["signs"][0] == 1)
    # y = 0 maps to #{t_k < 0} = L/2 - 1 for every coordinate
    assert np.all(res["idx"][0] == 1)
    assert np.all(O.dequantize_prod(cd, res["idx"], res["signs"], res["norms"], res["rnorms"])[0] == 0.0)
    # codes do not depend on the scale of x
    r2 = O.quantize_prod(cd, x * 7.25)
    assert np.array_equal(r2["idx"], res["idx"]) and np.array_equal(r2["signs"], res["signs"])
    assert np.allclose(r2["rnorms"], res["rnorms"], rtol=1e-13)


# ---------------------------------------------------------------- prod -----
def _prod_trials(d, bits, trials, seed=5):
    """Estimator <y, x_tilde> over `trials` independent S draws (group index =
    trial), for one fixed x and y and a fixed Pi."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((1, d))
    y = rng.standard_normal(d)
    cd = O.make_codec(d, bits, O.PROD, 123, groups=1)
    est = np.empty(trials)
    r_norm = None
    for g in range(trials):
        cd.ss = [O.qjl_matrix(d, 123, g + 1)]
        res = O.quantize_prod(cd, x)
        xt = O.dequantize_prod(cd, res["idx"], res["signs"], res["norms"], res["rnorms"])
        est[g] = float(xt[0] @ y)
        r_norm = res["rnorms"][0]
    # fixed quantities for the variance law
    nu = float(np.linalg.norm(x))
    u = x[0] / nu
    if cd.mse_bits:
        u_hat = cd.centroids[O.quantize_mse(cd, x)[0][0]] @ cd.pis[0]
    else:
        u_hat = np.zeros(d)
    r = u - u_hat
    return est, float(x[0] @ y), nu, r, y, r_norm


@pytest.mark.slow
@pytest.mark.parametrize("d,bits,trials", [(32, 3, 100000), (128, 4, 10000)])
def test_prod_estimator_is_unbiased_with_the_predicted_variance(d, bits, trials):
    est, truth, nu, r, y, gamma = _prod_trials(d, bits, trials)
    err = est - truth
    sigma = err.std()
    assert abs(err.mean()) < 3.0 * sigma / math.sqrt(trials)
    # conditional on r, Var = nu^2 gamma^2/m ((pi/2)||y||^2 - <r/gamma, y>^2)
    assert gamma == pytest.approx(np.linalg.norm(r), rel=1e-12)
    var = nu ** 2 * gamma ** 2 / d * (math.pi / 2 * (y @ y) - (r / gamma @ y) ** 2)
    assert err.var() == pytest.approx(var, rel=6.0 * math.sqrt(2.0 / trials) + 0.01)


def test_prod_error_variance_scales_as_one_over_d():
    # "error decays with d": for unit x, y and fixed b, Var * d is about constant
    vals = []
    for d in (64, 256):
        est, truth, nu, r, y, gamma = _prod_trials(d, 2, 1500, seed=9)
        vals.append(np.var(est - truth) * d / (nu * np.linalg.norm(y)) ** 2)
    assert 0.6 < vals[0] / vals[1] < 1.6


def test_prod_one_bit_is_pure_qjl():
    cd = O.make_codec(64, 1, O.PROD, 4)
    x = np.random.default_rng(1).standard_normal((5, 64))
    res = O.quantize_prod(cd, x)
    assert res["idx"] is None
    assert np.allclose(res["rnorms"], 1.0)
    assert np.array_equal(res["signs"], np.where(x @ cd.ss[0].T >= 0, 1, -1))


# ---------------------------------------------------------------- logits ---
@pytest.mark.parametrize("variant,bits", [(O.MSE, 2), (O.MSE, 4), (O.PROD, 2), (O.PROD, 4), (O.PROD, 1)])
def test_fast_logits_equal_plain_logits(parity_x, parity_q, variant, bits):
    cd = O.make_codec(128, bits, variant, 0)
    x = parity_x[:300]
    if variant == O.MSE:
        idx, nu, _ = O.quantize_mse(cd, x)
        keys = dict(idx=idx, norms=nu)
    else:
        keys = O.quantize_prod(cd, x)
    q = parity_q[:17]
    plain = O.logits_plain(cd, q, keys)
    fast = O.logits_fast(cd, q, keys)
    assert np.max(np.abs(plain - fast)) < 1e-12 * np.max(np.abs(plain))


def test_unit_queries_reproduce_reconstruction(parity_x):
    cd = O.make_codec(128, 3, O.PROD, 0)
    keys = O.quantize_prod(cd, parity_x[:50])
    xt = O.dequantize_prod(cd, keys["idx"], keys["signs"], keys["norms"], keys["rnorms"])
    eye = np.eye(128)
    assert np.allclose(O.logits_fast(cd, eye, keys), xt.T, atol=1e-12)


def test_eight_bit_mse_logits_are_nearly_exact(parity_x, parity_q):
    cd = O.make_codec(128, 8, O.MSE, 0)
    idx, nu, _ = O.quantize_mse(cd, parity_x[:200])
    got = O.logits_fast(cd, parity_q[:20], dict(idx=idx, norms=nu))
    ref = parity_q[:20] @ parity_x[:200].T
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert rel < 3.0 * math.sqrt(cd.distortion)
    assert cd.distortion < 1e-4


# ------------------------------------------- QJL stage from given indices ---
def _hand_codec(mse_bits):
    """d = 4 codec with hand-chosen tables.  Pi is the cyclic shift
    y_i = u_{(i+1) % 4} (not symmetric, so a transposed Pi changes the
    answer); S is not symmetric either; the centroids are dyadic, so every
    step below is exact in float64."""
    pi = np.zeros((4, 4))
    for i in range(4):
        pi[i, (i + 1) % 4] = 1.0
    s = np.array([[1.0, 0.0, 0.0, 0.0],
                  [0.0, 1.0, 0.0, 0.0],
                  [0.0, 0.0, -1.0, 3.0],
                  [0.0, 1.0, -1.0, 0.0]])
    cd = O.Codec(4, mse_bits + 1, O.PROD, 0, 1, mse_bits, pis=[pi], ss=[s])
    if mse_bits:
        cd.centroids = np.array([-0.75, -0.25, 0.25, 0.75])
    return cd


def test_prod_signs_from_indices_by_hand():
    cd = _hand_codec(2)
    # u = (1/2, 1/2, 1/2, 1/2) for the first two rows; the third is zero
    x = np.array([[2.0, 2.0, 2.0, 2.0], [1e-3, 1e-3, 1e-3, 1e-3], [0.0, 0.0, 0.0, 0.0]])
    idx = np.array([[3, 1, 2, 0], [3, 1, 2, 0], [0, 3, 0, 3]])
    out = O.prod_signs_from_indices(cd, x, idx)
    # c[idx] = (3/4, -1/4, 1/4, -3/4); Pi^T c[idx] = (-3/4, 3/4, -1/4, 1/4)
    # r = u - Pi^T c[idx] = (5/4, -1/4, 3/4, 1/4), ||r||^2 = 9/4
    # S r = (5/4, -1/4, -3/4 + 3/4 = 0, -1/4 - 3/4 = -1); sign(0) = +1
    for row in (0, 1):
        assert out["rnorms"][row] == 1.5
        assert out["proj"][row].tolist() == [1.25, -0.25, 0.0, -1.0]
        assert out["signs"][row].tolist() == [1, -1, 1, -1]
    assert out["rnorms"][2] == 0.0
    assert out["proj"][2].tolist() == [0.0] * 4 and out["signs"][2].tolist() == [1] * 4


def test_prod_signs_from_indices_without_mse_bits_by_hand():
    # b = 1: r = u, gamma = 1, signs of S u
    cd = _hand_codec(0)
    out = O.prod_signs_from_indices(cd, np.array([[3.0, 3.0, 3.0, 3.0]]), None)
    assert out["rnorms"][0] == 1.0
    assert out["proj"][0].tolist() == [0.5, 0.5, 1.0, 0.0]
    assert out["signs"][0].tolist() == [1, 1, 1, 1]


@pytest.mark.parametrize("d,bits", [(128, 4), (128, 2), (200, 3), (64, 1)])
def test_prod_signs_from_own_indices_equal_quantize_prod(d, bits):
    cd = O.make_codec(d, bits, O.PROD, 6)
    x = np.random.default_rng(d + bits).standard_normal((300, d))
    x[7] = 0.0
    res = O.quantize_prod(cd, x)
    got = O.prod_signs_from_indices(cd, x, res["idx"])
    assert np.array_equal(got["signs"], res["signs"])
    assert np.allclose(got["rnorms"], res["rnorms"], rtol=1e-13, atol=0)
    assert np.allclose(got["proj"], res["proj"], rtol=0, atol=1e-12)


def test_prod_residual_norm_moves_by_the_flipped_coordinate():
    """Moving index j one step changes the rotated-domain residual only in
    coordinate j: ||r'||^2 = ||r||^2 - (y_j - c[i])^2 + (y_j - c[i'])^2,
    with y = Pi u from the quantizer (Pi orthogonal)."""
    cd = O.make_codec(128, 3, O.PROD, 8)
    x = np.random.default_rng(3).standard_normal((64, 128))
    res = O.quantize_prod(cd, x)
    rng = np.random.default_rng(4)
    j = rng.integers(0, 128, 64)
    rows = np.arange(64)
    idx2 = res["idx"].copy()
    up = idx2[rows, j] < 3
    idx2[rows, j] = np.where(up, idx2[rows, j] + 1, idx2[rows, j] - 1)
    got = O.prod_signs_from_indices(cd, x, idx2)
    y = res["y"][rows, j]
    c = cd.centroids
    want = res["rnorms"] ** 2 - (y - c[res["idx"][rows, j]]) ** 2 + (y - c[idx2[rows, j]]) ** 2
    assert np.allclose(got["rnorms"] ** 2, want, rtol=1e-12)
    # and the projection moves by -(c[i'] - c[i]) S Pi^T e_j
    delta = (c[idx2[rows, j]] - c[res["idx"][rows, j]])[:, None] * (cd.pis[0][j] @ cd.ss[0].T)
    assert np.allclose(got["proj"], res["proj"] - delta, atol=1e-12)
