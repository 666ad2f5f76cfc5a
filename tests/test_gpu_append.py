"""GPU parity of the online append (one vector per set written into chosen
rows of a cache) against the oracle, and its effect on the rest of the cache
(bit-exact: untouched)."""
import numpy as np
import pytest
import torch

import kv_cache_compression_tq_amd as tq
import workloads
from oracle import tq_oracle as O
from parity import QJLCheck, check_indices

pytestmark = pytest.mark.gpu


def _cache(codec, rows):
    c = codec.empty_codes(1, rows)
    out = {}
    for k, v in c.items():
        if v is None:
            out[k] = None
            continue
        v = v[0]
        if v.dtype == torch.uint8:
            v.fill_(0xA5)
        else:
            v.fill_(-7.0)
        out[k] = v
    return out


def _check_rows(codec, cd, cache, before, rows, x64):
    """Every appended row against the oracle.  The index and sign rules are
    taken over all coordinates of the appended batch, as for a quantized
    batch (a single vector holds only d coordinates); norms row by row."""
    n_sets, d = x64.shape
    n_rows = cache["norms"].shape[0]
    valid = (rows >= 0) & (rows < n_rows)
    written = torch.from_numpy(rows[valid]).cuda()
    gi, oi, oy = [], [], []
    qjl = QJLCheck()
    for s in range(n_sets):
        if not valid[s]:
            continue
        g = s % cd.groups
        r = int(rows[s])
        if cd.variant == O.MSE:
            idx, nu, y = O.quantize_mse(cd, x64[s:s + 1], g)
            gidx = codec.unpack(cache["codes"][r:r + 1].contiguous(), cd.mse_bits).cpu().numpy()
            gi.append(gidx), oi.append(idx), oy.append(y)
            assert np.allclose(cache["norms"][r].item(), nu[0], rtol=1e-5)
        else:
            res = O.quantize_prod(cd, x64[s:s + 1], g)
            gidx = None
            if cd.mse_bits:
                gidx = codec.unpack(cache["codes"][r:r + 1].contiguous(), cd.mse_bits).cpu().numpy()
                gi.append(gidx), oi.append(res["idx"]), oy.append(res["y"])
            qjl.add(cd, x64[s:s + 1], gidx, codec.unpack(cache["signs"][r:r + 1].contiguous(), 1).cpu().numpy(),
                    cache["rnorms"][r:r + 1].cpu().numpy(), g)
            assert np.allclose(cache["norms"][r].item(), res["norms"][0], rtol=1e-5)
    if gi:
        check_indices(np.concatenate(gi), np.concatenate(oi), np.concatenate(oy), cd.boundaries, "appended rows")
    if qjl.gpu:
        qjl.check("appended rows")
    # every other row is untouched
    keep = torch.ones(n_rows, dtype=torch.bool, device="cuda")
    keep[written] = False
    for k, v in cache.items():
        if v is not None:
            assert torch.equal(v[keep], before[k][keep]), k


CASES = [
    (128, 4, O.MSE, torch.float32), (128, 3, O.MSE, torch.bfloat16), (128, 4, O.PROD, torch.float32),
    (128, 1, O.PROD, torch.bfloat16), (128, 5, O.PROD, torch.float32), (200, 2, O.PROD, torch.float32),
    (17, 3, O.MSE, torch.float32), (96, 2, O.PROD, torch.bfloat16), (1536, 3, O.PROD, torch.float32),
]


@pytest.mark.parametrize("d,bits,variant,dtype", CASES)
def test_append_matches_oracle(d, bits, variant, dtype):
    n_sets, cache_rows, groups = 6, 50, 3
    rng = np.random.default_rng(d * 10 + bits)
    x = rng.standard_normal((n_sets, d)).astype(np.float32)
    x[2] = 0.0  # a zero vector
    xt = torch.from_numpy(x).to(dtype).cuda()
    x64 = xt.float().cpu().numpy().astype(np.float64)
    rows = rng.choice(cache_rows, n_sets, replace=False).astype(np.int64)
    codec = tq.Codec(d, bits, variant, seed=13, groups=groups)
    cd = O.make_codec(d, bits, variant, 13, groups=groups)
    cache = _cache(codec, cache_rows)
    before = {k: (None if v is None else v.clone()) for k, v in cache.items()}
    codec.append(xt, torch.from_numpy(rows).cuda(), cache)
    torch.cuda.synchronize()
    _check_rows(codec, cd, cache, before, rows, x64)


@pytest.mark.parametrize("n_sets,groups,variant,bits,dtype", [
    (700, 2, O.PROD, 4, torch.float32),   # 350 vectors per group: 11 tiles over two workgroups
    (333, 5, O.MSE, 2, torch.bfloat16),   # ragged: 67 and 66 vectors per group
    (3, 5, O.PROD, 3, torch.bfloat16),    # more groups than sets
    (97, 4, O.MSE, 4, torch.float32),
])
def test_append_many_vectors_per_group(n_sets, groups, variant, bits, dtype):
    d, cache_rows = 128, 2 * n_sets + 5
    rng = np.random.default_rng(n_sets + groups)
    x = rng.standard_normal((n_sets, d)).astype(np.float32)
    x[n_sets // 2] = 0.0
    xt = torch.from_numpy(x).to(dtype).cuda()
    x64 = xt.float().cpu().numpy().astype(np.float64)
    rows = rng.choice(cache_rows, n_sets, replace=False).astype(np.int64)
    rows[::7] = -1                    # skipped
    rows[3::11] = cache_rows + 4      # skipped
    codec = tq.Codec(d, bits, variant, seed=21, groups=groups)
    cd = O.make_codec(d, bits, variant, 21, groups=groups)
    cache = _cache(codec, cache_rows)
    before = {k: (None if v is None else v.clone()) for k, v in cache.items()}
    codec.append(xt, torch.from_numpy(rows).cuda(), cache)
    torch.cuda.synchronize()
    _check_rows(codec, cd, cache, before, rows, x64)


def test_append_unaligned_input():
    """An input that is not 16-byte aligned takes the one-workgroup-per-set
    kernel; both kernels agree with the oracle."""
    d, n_sets, cache_rows = 128, 9, 20
    rng = np.random.default_rng(5)
    base = torch.from_numpy(rng.standard_normal(n_sets * d + 1).astype(np.float32)).to(torch.bfloat16).cuda()
    xt = base[1:].view(n_sets, d)
    x64 = xt.float().cpu().numpy().astype(np.float64)
    rows = rng.choice(cache_rows, n_sets, replace=False).astype(np.int64)
    codec = tq.Codec(d, 3, O.PROD, seed=4, groups=2)
    cd = O.make_codec(d, 3, O.PROD, 4, groups=2)
    cache = _cache(codec, cache_rows)
    before = {k: (None if v is None else v.clone()) for k, v in cache.items()}
    codec.append(xt, torch.from_numpy(rows).cuda(), cache)
    torch.cuda.synchronize()
    _check_rows(codec, cd, cache, before, rows, x64)


def test_append_skips_rows_outside_the_cache():
    codec = tq.Codec(128, 4, tq.TQ_PROD, seed=2)
    cache = _cache(codec, 10)
    before = {k: (None if v is None else v.clone()) for k, v in cache.items()}
    x = torch.randn(3, 128, device="cuda")
    codec.append(x, torch.tensor([-1, 10, 1 << 40], dtype=torch.int64, device="cuda"), cache)
    torch.cuda.synchronize()
    for k, v in cache.items():
        if v is not None:
            assert torch.equal(v, before[k]), k


def test_append_decode_shape_paged():
    """16 batch x 8 KV heads: one new key (prod b=4) and value (mse b=4) per
    (batch, head) into a paged cache of 128 x 4096 rows at scattered
    positions; every appended row checked against the oracle."""
    sets, d, per = workloads.DEC_BATCH * workloads.DEC_KV_HEADS, 128, 4096
    rng = np.random.default_rng(11)
    pos = rng.integers(0, per, sets)
    rows = (np.arange(sets) * per + pos).astype(np.int64)
    for variant, seed in ((O.PROD, 0), (O.MSE, 1)):
        codec = tq.Codec(d, 4, variant, seed=seed, groups=workloads.DEC_KV_HEADS)
        cd = O.make_codec(d, 4, variant, seed, groups=workloads.DEC_KV_HEADS)
        cache = _cache(codec, sets * per)
        before = {k: (None if v is None else v.clone()) for k, v in cache.items()}
        x = rng.standard_normal((sets, d)).astype(np.float32)
        codec.append(torch.from_numpy(x).cuda(), torch.from_numpy(rows).cuda(), cache)
        torch.cuda.synchronize()
        _check_rows(codec, cd, cache, before, rows, x.astype(np.float64))
