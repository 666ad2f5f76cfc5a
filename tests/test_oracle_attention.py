"""Pins of the oracle's decode attention (CPU): closed forms that any
mistake in the softmax axis, the scale, the key/value pairing or the
normalisation breaks."""
import numpy as np
import pytest

from oracle import tq_oracle as O


def _kv(d, n, seed, kbits=4, vbits=3):
    rng = np.random.default_rng(seed)
    ck = O.make_codec(d, kbits, O.PROD, seed)
    cv = O.make_codec(d, vbits, O.MSE, seed + 1)
    k = O.quantize_prod(ck, rng.standard_normal((n, d)))
    idx, nu, _ = O.quantize_mse(cv, rng.standard_normal((n, d)))
    keys = dict(idx=k["idx"], signs=k["signs"], norms=k["norms"], rnorms=k["rnorms"])
    values = dict(idx=idx, norms=nu)
    vh = O.dequantize_mse(cv, idx, nu)
    q = rng.standard_normal((3, d))
    return ck, cv, keys, values, vh, q


def test_single_key_returns_its_value():
    ck, cv, keys, values, vh, q = _kv(16, 1, 3)
    out = O.attention_plain(ck, cv, q, keys, values, 0.7)
    assert np.allclose(out, np.repeat(vh, 3, axis=0), rtol=0, atol=1e-12)


def test_zero_scale_is_the_mean_of_the_values():
    ck, cv, keys, values, vh, q = _kv(24, 37, 4)
    out = O.attention_plain(ck, cv, q, keys, values, 0.0)
    assert np.allclose(out, np.repeat(vh.mean(axis=0, keepdims=True), 3, axis=0), atol=1e-12)


def test_large_scale_selects_the_best_key():
    ck, cv, keys, values, vh, q = _kv(32, 50, 5)
    logit = O.logits_plain(ck, q, keys)
    out = O.attention_plain(ck, cv, q, keys, values, 1e6)
    assert np.allclose(out, vh[np.argmax(logit, axis=1)], atol=1e-9)


def test_permuting_key_value_pairs_changes_nothing():
    ck, cv, keys, values, vh, q = _kv(16, 29, 6)
    perm = np.random.default_rng(0).permutation(29)
    pk = {k: np.asarray(v)[perm] for k, v in keys.items()}
    pv = {k: np.asarray(v)[perm] for k, v in values.items()}
    a = O.attention_plain(ck, cv, q, keys, values, 0.3)
    b = O.attention_plain(ck, cv, q, pk, pv, 0.3)
    assert np.allclose(a, b, atol=1e-12)


@pytest.mark.parametrize("scale", [0.05, 0.5])
def test_two_keys_is_a_logistic_blend(scale):
    ck, cv, keys, values, vh, q = _kv(16, 2, 7)
    logit = O.logits_plain(ck, q, keys)
    lam = 1.0 / (1.0 + np.exp(-scale * (logit[:, 0] - logit[:, 1])))
    want = lam[:, None] * vh[0][None, :] + (1.0 - lam)[:, None] * vh[1][None, :]
    out = O.attention_plain(ck, cv, q, keys, values, scale)
    assert np.allclose(out, want, atol=1e-12)
