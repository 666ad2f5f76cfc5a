"""Pins of the oracle's outlier-channel mixed precision (CPU): reductions to
the plain codec, the bit budget of the 2.5- / 3.5-bit configurations, the
distortion predicted by the two parts' Lloyd-Max constants, unbiased prod
inner products, and the decomposition of logits over the parts."""
import math

import numpy as np
import pytest

from oracle import tq_oracle as O


def _outlier_data(d, n, groups, seed, n_big=4):
    """Per group: n_big channels scaled x10 (the KV workload's outliers)
    among the first listed outlier channels."""
    rng = np.random.default_rng(seed)
    chans, xs = [], []
    for g in range(groups):
        big = rng.choice(d, n_big, replace=False)
        rest = rng.choice(np.setdiff1d(np.arange(d), big), d // 2 - n_big, replace=False)
        chans.append(np.concatenate([big, rest]))
        x = rng.standard_normal((n, d))
        x[:, big] *= 10.0
        xs.append(x)
    return np.array(chans), xs


def test_empty_outlier_part_is_the_plain_codec_at_seed_plus_one():
    d, b = 64, 3
    mx = O.make_mixed(d, b, O.MSE, 5, np.zeros((1, 0), dtype=np.int64))
    plain = O.make_codec(d, b, O.MSE, 6)
    x = np.random.default_rng(0).standard_normal((20, d))
    po, pr = O.mixed_quantize(mx, x)
    assert po is None
    idx, nu, _ = O.quantize_mse(plain, x)
    # (norms of a gathered copy may differ from the original's in the last bit)
    assert np.array_equal(pr["idx"], idx) and np.allclose(pr["norms"], nu, rtol=1e-14, atol=0)
    assert np.allclose(O.mixed_dequantize(mx, (po, pr)), O.dequantize_mse(plain, idx, nu), rtol=1e-13, atol=1e-15)


def test_all_channels_outliers_is_the_plain_codec_on_permuted_channels():
    d, b = 48, 2
    perm = np.random.default_rng(1).permutation(d)
    mx = O.make_mixed(d, b, O.PROD, 9, perm[None, :])
    plain = O.make_codec(d, b + 1, O.PROD, 9)
    x = np.random.default_rng(2).standard_normal((10, d))
    po, pr = O.mixed_quantize(mx, x)
    assert pr is None
    ref = O.quantize_prod(plain, x[:, perm])
    assert np.array_equal(po["idx"], ref["idx"]) and np.array_equal(po["signs"], ref["signs"])
    rec = O.mixed_dequantize(mx, (po, pr))
    want = np.empty_like(rec)
    want[:, perm] = O.dequantize_prod(plain, ref["idx"], ref["signs"], ref["norms"], ref["rnorms"])
    assert np.allclose(rec, want, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("b,eff", [(2, 2.5), (3, 3.5)])
def test_half_the_channels_at_one_more_bit_is_the_pages_bit_budget(b, eff):
    d = 128
    mx = O.make_mixed(d, b, O.MSE, 1, np.arange(0, d, 2)[None, :])
    bits = mx.outlier.mse_bits * mx.n_out + mx.regular.mse_bits * (d - mx.n_out)
    assert bits / d == eff
    x = np.random.default_rng(3).standard_normal((4, d))
    po, pr = O.mixed_quantize(mx, x)
    # the packed rows carry exactly those bits (before the 16-byte padding)
    assert (mx.n_out * mx.outlier.mse_bits + 7) // 8 + ((d - mx.n_out) * mx.regular.mse_bits + 7) // 8 == bits // 8
    assert O.pack(po["idx"], mx.outlier.mse_bits).shape[1] == O.row_bytes(mx.n_out, b + 1)


def test_mixed_distortion_is_the_sum_of_the_parts_lloyd_max_distortions():
    d, b, G = 128, 2, 8
    chans, xs = _outlier_data(d, 300, G, seed=3)
    mx = O.make_mixed(d, b, O.MSE, 5, chans, groups=G)
    plain = O.make_codec(d, b, O.MSE, 7, groups=G)
    got, pred, plain_err = [], [], []
    for g in range(G):
        x = xs[g]
        xh = O.mixed_dequantize(mx, O.mixed_quantize(mx, x, g), g)
        got.append(((x - xh) ** 2).sum(1).mean())
        xo, xr = x[:, mx.channels[g][:mx.n_out]], x[:, mx.channels[g][mx.n_out:]]
        pred.append(mx.outlier.distortion * (xo ** 2).sum(1).mean() + mx.regular.distortion * (xr ** 2).sum(1).mean())
        idx, nu, _ = O.quantize_mse(plain, x, g)
        plain_err.append(((x - O.dequantize_mse(plain, idx, nu, g)) ** 2).sum(1).mean())
    ratio = np.array(got) / np.array(pred)
    assert np.all(np.abs(ratio - 1.0) < 0.08), ratio
    assert abs(np.mean(got) / np.mean(pred) - 1.0) < 0.03
    # keeping the outlier channels at one more bit beats the plain b-bit codec
    assert np.mean(plain_err) > 2.0 * np.mean(got)


def test_mixed_prod_inner_products_are_unbiased():
    d, b, trials = 32, 2, 4000
    rng = np.random.default_rng(4)
    x = rng.standard_normal((1, d))
    x[0, :3] *= 10.0
    y = rng.standard_normal(d)
    chans = np.arange(8)[None, :]
    mx = O.make_mixed(d, b, O.PROD, 11, chans)
    est = np.empty(trials)
    for t in range(trials):  # a fresh S for each part and trial
        mx.outlier.ss = [O.qjl_matrix(mx.n_out, 11, t + 1)]
        mx.regular.ss = [O.qjl_matrix(d - mx.n_out, 12, t + 1)]
        est[t] = float(O.mixed_dequantize(mx, O.mixed_quantize(mx, x))[0] @ y)
    err = est - float(x[0] @ y)
    assert abs(err.mean()) < 3.0 * err.std() / math.sqrt(trials)


@pytest.mark.parametrize("variant", [O.MSE, O.PROD])
def test_mixed_logits_are_the_sum_of_the_parts_logits(variant):
    d, b, G = 64, 3, 2
    chans, xs = _outlier_data(d, 50, G, seed=6, n_big=3)
    mx = O.make_mixed(d, b, variant, 3, chans, groups=G)
    q = np.random.default_rng(7).standard_normal((5, d))
    for g in range(G):
        po, pr = O.mixed_quantize(mx, xs[g], g)
        plain = O.mixed_logits_plain(mx, q, (po, pr), g)
        perm = mx.channels[g]
        fast = (O.logits_fast(mx.outlier, q[:, perm[:mx.n_out]], po, g)
                + O.logits_fast(mx.regular, q[:, perm[mx.n_out:]], pr, g))
        assert np.allclose(plain, fast, rtol=1e-10, atol=1e-9)
