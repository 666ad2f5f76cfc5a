"""GPU parity of the fused top-k maximum inner product search against the
oracle's scores.  Several answers can be correct where scores tie within
the logits tolerance, so the test checks what is unique: every returned
score equals the oracle's estimate for that key (1e-3 of the row's RMS),
scores are non-increasing, indices are distinct, and no key left out beats
the k-th returned score by more than the tolerance."""
import numpy as np
import pytest
import torch

import kv_cache_compression_tq_amd as tq
import workloads
from oracle import tq_oracle as O
from parity import REL_TOL

pytestmark = pytest.mark.gpu


def _cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def check_topk(g_sc, g_idx, full, k, what):
    """g_sc, g_idx: [nq][k] from the GPU; full: [nq][n_keys] oracle scores."""
    for i in range(full.shape[0]):
        row = full[i]
        tol = REL_TOL * np.sqrt(np.mean(row ** 2))
        idx = g_idx[i].astype(np.int64)
        assert len(set(idx.tolist())) == k, f"{what} q{i}: repeated indices"
        assert np.all(np.diff(g_sc[i]) <= 0), f"{what} q{i}: scores not sorted"
        assert np.max(np.abs(g_sc[i] - row[idx])) <= tol, f"{what} q{i}: score differs from the oracle"
        rest = np.ones(row.shape[0], bool)
        rest[idx] = False
        if rest.any():
            assert row[rest].max() <= g_sc[i][-1] + 2 * tol, f"{what} q{i}: a better key was left out"


def _stored(cd, keys):
    out = {"norms": _cuda(keys["norms"].astype(np.float32))}
    if cd.mse_bits:
        out["codes"] = _cuda(O.pack(keys["idx"], cd.mse_bits))
    if cd.variant == O.PROD:
        out["signs"] = _cuda(O.pack(O.signs_to_bits(keys["signs"]), 1))
        out["rnorms"] = _cuda(keys["rnorms"].astype(np.float32))
    return out


# d decides the scan's contraction steps: d <= 128 takes 4 (a lane group's codes are whole words), 128 < d
# <= 224 takes 7 (7 mb code bytes and 7 sign bytes per lane group: unaligned runs unless mb = 4), and d > 224
# takes 8
CASES = [(200, 2, O.PROD), (200, 4, O.PROD), (128, 3, O.MSE), (64, 1, O.PROD), (96, 5, O.PROD), (200, 4, O.MSE),
         (208, 3, O.PROD), (150, 2, O.MSE), (256, 3, O.PROD), (240, 2, O.MSE)]


@pytest.mark.parametrize("d,bits,variant", CASES)
@pytest.mark.parametrize("k", [1, 10, 64])
def test_topk_oracle_codes(d, bits, variant, k):
    nq, n = 37, 3001
    rng = np.random.default_rng(d + bits * 7 + k)
    x = rng.standard_normal((n, d))
    x[5] = x[900]  # equal scores: ties go to the lower index
    q = rng.standard_normal((nq, d)).astype(np.float32)
    cd = O.make_codec(d, bits, variant, 19)
    codec = tq.Codec(d, bits, variant, seed=19)
    if variant == O.MSE:
        idx, nu, _ = O.quantize_mse(cd, x)
        keys = dict(idx=idx, norms=nu.astype(np.float32).astype(np.float64))
    else:
        r = O.quantize_prod(cd, x)
        keys = dict(idx=r["idx"], signs=r["signs"], norms=r["norms"].astype(np.float32).astype(np.float64),
                    rnorms=r["rnorms"].astype(np.float32).astype(np.float64))
    sc, ix = codec.topk(_cuda(q), _stored(cd, keys), k)
    full = O.logits_plain(cd, q.astype(np.float64), keys)
    check_topk(sc.cpu().numpy(), ix.cpu().numpy(), full, k, f"d={d} b={bits}")


@pytest.mark.parametrize("d,bits,variant", [(300, 3, O.PROD), (128, 6, O.MSE), (520, 2, O.PROD), (64, 8, O.MSE)])
def test_topk_score_then_select(d, bits, variant):
    """Codecs the fused scan does not take (d > 256, more than 4 mse bits):
    the logits kernels score 65536-key chunks of 64-query blocks and the
    selection keeps each segment's best k.  70 queries (two blocks) over
    70000 keys (two chunks), with equal keys inside a chunk and across the
    chunk boundary (ties go to the lower index)."""
    nq, n = 70, 70000
    rng = np.random.default_rng(d + bits)
    x = rng.standard_normal((n, d))
    x[5] = x[900]
    x[66000] = x[10]
    q = rng.standard_normal((nq, d)).astype(np.float32)
    q[3] = x[66000]  # a query whose best keys are the equal pair 10 and 66000
    cd = O.make_codec(d, bits, variant, 23)
    codec = tq.Codec(d, bits, variant, seed=23)
    if variant == O.MSE:
        idx, nu, _ = O.quantize_mse(cd, x)
        keys = dict(idx=idx, norms=nu.astype(np.float32).astype(np.float64))
    else:
        r = O.quantize_prod(cd, x)
        keys = dict(idx=r["idx"], signs=r["signs"], norms=r["norms"].astype(np.float32).astype(np.float64),
                    rnorms=r["rnorms"].astype(np.float32).astype(np.float64))
    stored = _stored(cd, keys)
    full = O.logits_fast(cd, q.astype(np.float64), keys)
    for k in (1, 10, 64):
        sc, ix = codec.topk(_cuda(q), stored, k)
        check_topk(sc.cpu().numpy(), ix.cpu().numpy(), full, k, f"d={d} b={bits} k={k}")
        if k >= 2:
            assert ix[3, 0].item() == 10 and ix[3, 1].item() == 66000, "equal keys: the lower index first"


def test_topk_small_index_and_single_key_range():
    d, n, k = 200, 64, 64  # k equals the index size: every key, sorted
    rng = np.random.default_rng(3)
    x = rng.standard_normal((n, d))
    cd = O.make_codec(d, 2, O.PROD, 1)
    codec = tq.Codec(d, 2, tq.TQ_PROD, seed=1)
    r = O.quantize_prod(cd, x)
    keys = dict(idx=r["idx"], signs=r["signs"], norms=r["norms"].astype(np.float32).astype(np.float64),
                rnorms=r["rnorms"].astype(np.float32).astype(np.float64))
    q = rng.standard_normal((3, d)).astype(np.float32)
    sc, ix = codec.topk(_cuda(q), _stored(cd, keys), k)
    assert sorted(ix.cpu().numpy()[0].tolist()) == list(range(n))
    check_topk(sc.cpu().numpy(), ix.cpu().numpy(), O.logits_plain(cd, q.astype(np.float64), keys), k, "all keys")


@pytest.mark.parametrize("bits", [2, 4])
def test_topk_nn_index_full_size_sampled(bits):
    """10^6 unit vectors at d = 200 from the 1000-centre mixture, indexed on
    the GPU with prod b; 10^4 queries searched for their top 64; a sample of
    60 queries checked against the oracle's scores over all 10^6 keys."""
    centres = workloads.nn_centres()
    x = workloads.nn_points(workloads.NN_POINTS, 7, centres)
    qs = workloads.nn_points(workloads.NN_QUERIES, 8, centres).astype(np.float32)
    codec = tq.Codec(workloads.NN_D, bits, tq.TQ_PROD, seed=0)
    keys = codec.quantize(_cuda(x).unsqueeze(0))
    sc, ix = codec.topk(_cuda(qs), {k: (None if v is None else v[0]) for k, v in keys.items()}, 64)
    torch.cuda.synchronize()
    cd = O.make_codec(workloads.NN_D, bits, O.PROD, 0)
    sample = np.sort(np.random.default_rng(1).choice(workloads.NN_QUERIES, 60, replace=False))
    mb = bits - 1
    full = np.empty((sample.size, workloads.NN_POINTS))
    step = 100_000
    for a in range(0, workloads.NN_POINTS, step):
        b = min(a + step, workloads.NN_POINTS)
        kd = dict(signs=O.bits_to_signs(O.unpack(keys["signs"][0, a:b].cpu().numpy(), 1, workloads.NN_D)),
                  norms=keys["norms"][0, a:b].cpu().numpy().astype(np.float64),
                  rnorms=keys["rnorms"][0, a:b].cpu().numpy().astype(np.float64))
        kd["idx"] = O.unpack(keys["codes"][0, a:b].cpu().numpy(), mb, workloads.NN_D)
        full[:, a:b] = O.logits_fast(cd, qs[sample].astype(np.float64), kd)
    check_topk(sc.cpu().numpy()[sample], ix.cpu().numpy()[sample], full, 64, f"NN b={bits}")
