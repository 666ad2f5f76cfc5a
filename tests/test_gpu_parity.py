"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Every expected value comes from oracle/ on the same seeded inputs.  The only
library outputs the oracle reads are codes it is asked to score: the QJL stage
taken on the GPU's own indices, so that the signs of a vector with one index
at a boundary flipped are still checked.  GPU codes are decoded with the
library's own unpack (itself checked bit-exact against the oracle's packing).
"""
import math

import numpy as np
import pytest
import torch

import kv_cache_compression_tq_amd as tq
import workloads
from oracle import tq_oracle as O
from parity import REL_TOL, QJLCheck, check_indices, check_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    torch.cuda.init()


def _cuda(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def _bf16_round(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def _gpu_idx(codec, packed, bits):
    """Decode the library's packed rows with the library's unpack."""
    rows = packed.reshape(-1, packed.shape[-1]).contiguous()
    return codec.unpack(rows, bits).cpu().numpy().astype(np.int64)


def _oracle_sets(cd, x, fn):
    return [fn(cd, x[s].astype(np.float64), s % cd.groups) for s in range(x.shape[0])]


# --------------------------------------------------------------- tables ----
def test_device_tables_equal_host_tables_and_match_oracle():
    codec = tq.Codec(128, 4, tq.TQ_PROD, seed=77, groups=3)
    cd = O.make_codec(128, 4, O.PROD, 77, groups=3)
    for g in range(3):
        dev = codec.tables(g)
        host = tq.host_tables(128, 4, tq.TQ_PROD, 77, g)
        for k in ("Pi", "S", "centroids", "boundaries"):
            assert np.array_equal(dev[k], host[k]), k
        assert np.max(np.abs(dev["Pi"] - cd.pis[g])) < 1e-6
        assert np.max(np.abs(dev["S"] - cd.ss[g])) < 1e-6
        assert np.allclose(dev["centroids"], cd.centroids, rtol=2e-7, atol=0)
        p = dev["Pi"].astype(np.float64)
        assert np.max(np.abs(p @ p.T - np.eye(128))) < 1e-6


# ------------------------------------------------------------- packing -----
@pytest.mark.parametrize("d", [2, 3, 128, 200])
@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 8])
def test_pack_unpack_bit_exact(d, bits):
    codec = tq.Codec(d, 2, tq.TQ_MSE, seed=0)
    rng = np.random.default_rng(d * 10 + bits)
    idx = rng.integers(0, 1 << bits, (257, d)).astype(np.uint8)
    packed = codec.pack(_cuda(idx), bits).cpu().numpy()
    assert np.array_equal(packed, O.pack(idx, bits))
    back = codec.unpack(_cuda(O.pack(idx, bits)), bits).cpu().numpy()
    assert np.array_equal(back, idx)


# ------------------------------------------------------------ quantize -----
MSE_CASES = [
    # d, bits, dtype, n_sets, n, groups
    (128, 2, "f32", 1, 4096, 1),
    (128, 4, "f32", 1, 4096, 1),
    (128, 4, "bf16", 3, 1000, 2),
    (128, 3, "bf16", 2, 777, 2),
    (128, 1, "f32", 1, 95, 1),
    (128, 2, "bf16", 1, 33, 1),
    (200, 2, "f32", 1, 513, 1),
    (200, 4, "bf16", 2, 300, 2),
    (3, 2, "f32", 1, 64, 1),
    (3, 6, "f32", 1, 300, 1),
    (2, 1, "f32", 1, 300, 1),
    (2, 4, "bf16", 2, 257, 2),
    (96, 3, "f32", 2, 100, 2),
    (128, 4, "bf16", 1, 65573, 1),    # several 16-vector stages per wave and a ragged last stage
    (128, 3, "bf16", 2, 40011, 2),
    # 5..8 mse bits: the dimension-generic kernels (float32 arithmetic)
    (128, 5, "f32", 1, 1000, 1),
    (128, 6, "bf16", 2, 300, 2),
    (128, 7, "f32", 1, 257, 1),
    (128, 8, "f32", 2, 200, 2),
    (200, 6, "f32", 1, 301, 1),
    (200, 8, "bf16", 1, 150, 1),
    (128, 5, "bf16", 1, 4096, 1),
    (100, 7, "f32", 1, 200, 1),
    (100, 5, "bf16", 2, 130, 2),
]


def _inputs(d, dtype, n_sets, n, seed):
    if d == 128 and n_sets == 1 and n == 4096:
        x = workloads.parity_vectors()[None]
    else:
        x = np.random.default_rng(seed).standard_normal((n_sets, n, d)).astype(np.float32)
        x[..., 0] *= 10.0  # an outlier channel
    if dtype == "bf16":
        x = _bf16_round(x)
        xt = _cuda(x, torch.bfloat16)
    else:
        xt = _cuda(x)
    return x, xt


@pytest.mark.parametrize("d,bits,dtype,n_sets,n,groups", MSE_CASES)
def test_quantize_mse_matches_oracle(d, bits, dtype, n_sets, n, groups):
    x, xt = _inputs(d, dtype, n_sets, n, seed=bits * 7 + d)
    codec = tq.Codec(d, bits, tq.TQ_MSE, seed=5, groups=groups)
    cd = O.make_codec(d, bits, O.MSE, 5, groups=groups)
    out = codec.quantize(xt)
    torch.cuda.synchronize()
    gidx = _gpu_idx(codec, out["codes"], bits).reshape(n_sets, n, d)
    codes = out["codes"].cpu().numpy()
    used = (d * bits + 7) // 8
    assert not codes[..., used:].any(), "padding bytes must be zero"
    norms = out["norms"].cpu().numpy()
    for s, (idx, nu, y) in enumerate(_oracle_sets(cd, x, O.quantize_mse)):
        check_indices(gidx[s], idx, y, cd.boundaries, f"set {s}")
        assert np.allclose(norms[s], nu, rtol=1e-5)


PROD_CASES = [
    (128, 4, "f32", 1, 4096, 1),
    (128, 2, "f32", 1, 4096, 1),
    (128, 1, "f32", 1, 500, 1),
    (128, 4, "bf16", 2, 600, 2),
    (128, 3, "bf16", 1, 61, 1),
    (128, 2, "bf16", 3, 257, 2),    # bf16 prod, 1..4 mse bits: the register-resident kernel
    (128, 5, "bf16", 1, 1000, 1),
    (128, 4, "bf16", 1, 4096, 1),
    (128, 4, "bf16", 1, 65573, 1),  # several 16-vector stages per wave and a ragged last stage
    (128, 3, "bf16", 2, 40011, 2),
    (128, 5, "f32", 1, 300, 1),
    (200, 3, "f32", 1, 400, 1),
    (3, 2, "f32", 1, 64, 1),
    (2, 3, "f32", 2, 400, 2),
    (2, 1, "f32", 1, 100, 1),
    # d not a multiple of 8: the generic kernels, 8 vectors per workgroup (ragged last group, two sets)
    (100, 3, "f32", 2, 203, 2),
    (100, 5, "bf16", 1, 77, 1),
    (100, 1, "f32", 1, 9, 1),
]


@pytest.mark.parametrize("d,bits,dtype,n_sets,n,groups", PROD_CASES)
def test_quantize_prod_matches_oracle(d, bits, dtype, n_sets, n, groups):
    x, xt = _inputs(d, dtype, n_sets, n, seed=bits * 11 + d)
    codec = tq.Codec(d, bits, tq.TQ_PROD, seed=9, groups=groups)
    cd = O.make_codec(d, bits, O.PROD, 9, groups=groups)
    out = codec.quantize(xt)
    torch.cuda.synchronize()
    mb = bits - 1
    gbits = _gpu_idx(codec, out["signs"], 1).reshape(n_sets, n, d)
    gidx = _gpu_idx(codec, out["codes"], mb).reshape(n_sets, n, d) if mb else None
    norms, rnorms = out["norms"].cpu().numpy(), out["rnorms"].cpu().numpy()
    qjl = QJLCheck()
    for s, res in enumerate(_oracle_sets(cd, x, O.quantize_prod)):
        if mb:
            check_indices(gidx[s], res["idx"], res["y"], cd.boundaries, f"set {s}")
        # signs and residual norms of every vector, on the GPU's own indices
        qjl.add(cd, x[s], gidx[s] if mb else None, gbits[s], rnorms[s], s % groups)
        assert np.allclose(norms[s], res["norms"], rtol=1e-5)
    qjl.check(f"d={d} prod b={bits}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_quantize_zero_and_tiny_vectors(dtype):
    x = np.zeros((1, 40, 128), np.float32)
    x[0, 1, 3] = 1e-30  # representable in bfloat16 too (float32 exponent range)
    x[0, 2, :] = 1.0
    for variant, bits in ((tq.TQ_MSE, 4), (tq.TQ_PROD, 4), (tq.TQ_PROD, 2), (tq.TQ_PROD, 1)):
        codec = tq.Codec(128, bits, variant, seed=3)
        out = codec.quantize(_cuda(x).to(dtype))
        torch.cuda.synchronize()
        mb = codec.mse_bits
        assert out["norms"][0, 0].item() == 0.0
        if mb:
            idx = _gpu_idx(codec, out["codes"], mb)
            assert np.all(idx[0] == (1 << mb) // 2 - 1)
        if variant == tq.TQ_PROD:
            assert out["rnorms"][0, 0].item() == 0.0
            assert np.all(_gpu_idx(codec, out["signs"], 1)[0] == 1)
        rec = codec.dequantize(out)
        assert torch.all(rec[0, 0] == 0)


def test_empty_inputs_are_noops():
    codec = tq.Codec(128, 3, tq.TQ_PROD, seed=1)
    x = torch.zeros((2, 0, 128), device="cuda")
    out = codec.quantize(x)
    assert out["norms"].numel() == 0
    q = torch.zeros((2, 4, 128), device="cuda")
    assert codec.logits(q, out).numel() == 0


def test_quantize_is_deterministic():
    x, xt = _inputs(128, "bf16", 4, 2048, seed=3)
    codec = tq.Codec(128, 4, tq.TQ_PROD, seed=2, groups=4)
    a = codec.quantize(xt)
    b = codec.quantize(xt)
    torch.cuda.synchronize()
    for k in ("codes", "signs", "norms", "rnorms"):
        assert torch.equal(a[k], b[k]), k


# ------------------------------------------------- dequantize / logits -----
def _oracle_keys(cd, x, group):
    """Oracle codes for x, in the stored layout (float32 norms)."""
    if cd.variant == O.MSE:
        idx, nu, _ = O.quantize_mse(cd, x, group)
        res = dict(idx=idx, norms=nu.astype(np.float32).astype(np.float64))
    else:
        r = O.quantize_prod(cd, x, group)
        res = dict(idx=r["idx"], signs=r["signs"], norms=r["norms"].astype(np.float32).astype(np.float64),
                   rnorms=r["rnorms"].astype(np.float32).astype(np.float64))
    return res


def _stored(cd, keys_per_set):
    out = {}
    if cd.mse_bits:
        out["codes"] = _cuda(np.stack([O.pack(k["idx"], cd.mse_bits) for k in keys_per_set]))
    out["norms"] = _cuda(np.stack([k["norms"] for k in keys_per_set]).astype(np.float32))
    if cd.variant == O.PROD:
        out["signs"] = _cuda(np.stack([O.pack(O.signs_to_bits(k["signs"]), 1) for k in keys_per_set]))
        out["rnorms"] = _cuda(np.stack([k["rnorms"] for k in keys_per_set]).astype(np.float32))
    return out


DEQ_CASES = [(128, 4, O.MSE), (128, 2, O.MSE), (128, 1, O.MSE), (128, 3, O.MSE), (128, 4, O.PROD),
             (128, 1, O.PROD), (128, 2, O.PROD), (128, 5, O.PROD), (200, 3, O.PROD), (200, 2, O.MSE),
             (128, 5, O.MSE), (128, 6, O.MSE), (128, 7, O.MSE), (128, 8, O.MSE), (200, 5, O.MSE), (200, 8, O.MSE),
             (2, 3, O.MSE), (2, 3, O.PROD), (3, 8, O.MSE)]


@pytest.mark.parametrize("d,bits,variant", DEQ_CASES)
def test_dequantize_oracle_codes(d, bits, variant):
    groups, n = 2, 700
    x = np.random.default_rng(d + bits).standard_normal((groups, n, d))
    cd = O.make_codec(d, bits, variant, 21, groups=groups)
    codec = tq.Codec(d, bits, variant, seed=21, groups=groups)
    keys = [_oracle_keys(cd, x[s], s) for s in range(groups)]
    got = codec.dequantize(_stored(cd, keys)).cpu().numpy()
    for s in range(groups):
        k = keys[s]
        if variant == O.MSE:
            ref = O.dequantize_mse(cd, k["idx"], k["norms"], s)
        else:
            ref = O.dequantize_prod(cd, k["idx"], k["signs"], k["norms"], k["rnorms"], s)
        check_rows(got[s], ref, f"dequant set {s}")


DQ_LAWS = ("gauss", "student3", "outlier", "uniform", "sparse")


def _law(name, rng, n, d):
    if name == "gauss":
        return rng.standard_normal((n, d))
    if name == "student3":
        return rng.standard_t(3, (n, d))
    if name == "outlier":  # four channels 30x the others
        return rng.standard_normal((n, d)) * np.where(np.arange(d) < 4, 30.0, 1.0)
    if name == "uniform":
        return rng.uniform(-1.0, 1.0, (n, d))
    return rng.standard_normal((n, d)) * (rng.random((n, d)) < 0.05)  # 95% zeros


@pytest.mark.parametrize("variant,bits", [(O.PROD, b) for b in (1, 2, 3, 4, 5)] + [(O.MSE, b) for b in (1, 2, 3, 4)])
def test_dequantize_margin_over_input_laws(variant, bits):
    """The d = 128 dequantize on oracle codes of five input laws, element by
    element against the oracle reconstruction in units of the row RMS.  The
    QJL term takes S^T as f16 hi + lo, so with at most 2 mse bits (two
    positive centroids, which the f16 decode-table scale makes nearly exact)
    every element is within 2e-5; with 3 and 4 mse bits the f16 centroid
    table leaves up to about 3.5e-4, inside the 1e-3 tolerance."""
    d, n = 128, 1500
    rng = np.random.default_rng(100 + 10 * bits + variant)
    cd = O.make_codec(d, bits, variant, 21)
    codec = tq.Codec(d, bits, variant, seed=21)
    limit = 2e-5 if cd.mse_bits <= 2 else REL_TOL
    for law in DQ_LAWS:
        k = _oracle_keys(cd, _law(law, rng, n, d), 0)
        got = codec.dequantize(_stored(cd, [k])).cpu().numpy()[0].astype(np.float64)
        if variant == O.MSE:
            ref = O.dequantize_mse(cd, k["idx"], k["norms"], 0)
        else:
            ref = O.dequantize_prod(cd, k["idx"], k["signs"], k["norms"], k["rnorms"], 0)
        rms = np.linalg.norm(ref, axis=1) / np.sqrt(d)
        live = rms > 0
        worst = float((np.max(np.abs(got - ref), axis=1)[live] / rms[live]).max())
        assert worst <= limit, f"{law}: worst element error {worst:.3g} of the row RMS"
        check_rows(got, ref, f"dequant {law}")


@pytest.mark.parametrize("variant,bits", [(O.MSE, 4), (O.PROD, 4)])
def test_dequantize_unaligned_output_matches(variant, bits):
    """An output that is not 16-byte aligned takes the generic kernel; both
    kernels reconstruct the same codes to the parity tolerance."""
    d, n = 128, 333
    x = np.random.default_rng(7).standard_normal((1, n, d))
    cd = O.make_codec(d, bits, variant, 3)
    codec = tq.Codec(d, bits, variant, seed=3)
    stored = _stored(cd, [_oracle_keys(cd, x[0], 0)])
    fast = codec.dequantize(stored).cpu().numpy()[0]
    buf = torch.empty(n * d + 1, dtype=torch.float32, device="cuda")
    view = buf[1:].view(1, n, d)  # 4-byte offset
    codec.dequantize(stored, out=view)
    slow = view.cpu().numpy()[0]
    check_rows(slow, fast.astype(np.float64), "generic vs fast dequantize")


LOGIT_CASES = [
    # d, bits, variant, n_sets, nq, n_keys
    (128, 4, O.PROD, 2, 4, 4096),
    (128, 3, O.PROD, 3, 4, 1000),
    (128, 2, O.PROD, 1, 12, 777),     # n_keys % 4 != 0 and nq > 8
    (128, 4, O.PROD, 2, 10, 1024),    # 8 heads in one launch, then 2 (16-byte logits stores)
    (128, 1, O.PROD, 2, 4, 512),
    (128, 4, O.MSE, 2, 4, 2048),
    (128, 3, O.MSE, 1, 1, 1200),
    (128, 5, O.PROD, 1, 3, 640),
    (200, 4, O.PROD, 2, 4, 600),
    (200, 2, O.MSE, 1, 5, 301),
    (128, 5, O.MSE, 2, 4, 700),
    (128, 6, O.MSE, 1, 9, 333),
    (128, 7, O.MSE, 1, 3, 500),
    (128, 8, O.MSE, 2, 4, 256),
    (200, 6, O.MSE, 1, 4, 300),
    (200, 8, O.MSE, 2, 2, 129),
    (2, 2, O.MSE, 1, 3, 100),
    (2, 4, O.PROD, 2, 2, 77),
]


@pytest.mark.parametrize("d,bits,variant,n_sets,nq,n_keys", LOGIT_CASES)
def test_logits_oracle_codes(d, bits, variant, n_sets, nq, n_keys):
    groups = min(n_sets, 2)
    rng = np.random.default_rng(d * bits + nq)
    x = rng.standard_normal((n_sets, n_keys, d))
    q = rng.standard_normal((n_sets, nq, d)).astype(np.float32)
    cd = O.make_codec(d, bits, variant, 31, groups=groups)
    codec = tq.Codec(d, bits, variant, seed=31, groups=groups)
    keys = [_oracle_keys(cd, x[s], s % groups) for s in range(n_sets)]
    got = codec.logits(_cuda(q), _stored(cd, keys)).cpu().numpy()
    for s in range(n_sets):
        ref = O.logits_plain(cd, q[s].astype(np.float64), keys[s], s % groups)
        check_rows(got[s], ref, f"logits set {s}")


def test_logits_decode_config_full_size_sampled():
    """16 batch x 8 KV heads x 131072 keys, 4 query heads per KV head, prod
    b=4, on a synthetic packed cache; sampled keys checked against the oracle."""
    sets, T, d = workloads.DEC_BATCH * workloads.DEC_KV_HEADS, workloads.DEC_TOKENS, workloads.DEC_DIM
    codec = tq.Codec(d, 4, tq.TQ_PROD, seed=0, groups=workloads.DEC_KV_HEADS)
    cd = O.make_codec(d, 4, O.PROD, 0, groups=workloads.DEC_KV_HEADS)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4)
    codes = torch.randint(0, 256, (sets, T, codec.code_row), dtype=torch.uint8, device="cuda", generator=gen)
    signs = torch.randint(0, 256, (sets, T, codec.sign_row), dtype=torch.uint8, device="cuda", generator=gen)
    norms = (10.0 + torch.randn((sets, T), device="cuda", generator=gen)).float()
    rnorms = torch.rand((sets, T), device="cuda", generator=gen) * 0.45 + 0.05
    q = workloads.decode_queries().reshape(sets, workloads.DEC_Q_PER_KV, d)
    out = codec.logits(_cuda(q), dict(codes=codes, signs=signs, norms=norms, rnorms=rnorms))
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    for s in rng.choice(sets, 12, replace=False):
        ks = np.sort(rng.choice(T, 300, replace=False))
        kt = torch.from_numpy(ks).cuda()
        keys = dict(idx=O.unpack(codes[s, kt].cpu().numpy(), 3, d),
                    signs=O.bits_to_signs(O.unpack(signs[s, kt].cpu().numpy(), 1, d)),
                    norms=norms[s, kt].cpu().numpy().astype(np.float64),
                    rnorms=rnorms[s, kt].cpu().numpy().astype(np.float64))
        ref = O.logits_fast(cd, q[s].astype(np.float64), keys, int(s) % 8)
        check_rows(out[s][:, kt].cpu().numpy(), ref, f"set {s}")


@pytest.mark.parametrize("n_sets,n_keys,variant,bits,nq", [
    (1, 1 << 25, O.PROD, 4, 4), (2, (1 << 25) + 64, O.PROD, 4, 10), (1, 1 << 25, O.MSE, 4, 4),
    (1, (1 << 25) + 64, O.MSE, 4, 4), (1, (1 << 26) + 100, O.MSE, 2, 6)])
def test_logits_past_the_fused_key_chunk(n_sets, n_keys, variant, bits, nq):
    """Sets of 2^25 keys (the most one launch of the fused logits kernel
    addresses; with mse b = 4 its 64-byte code rows make a set's codes exactly
    2^31 bytes) and longer ones, which run as chunks of 2^25 keys: two sets
    and two head groups (10 heads) at 2^25 + 64, and one set past 2^26 keys,
    where a launch takes 4 heads so that its output rows stay within 32-bit
    offsets.  Sampled keys (around each chunk boundary and the last 64 among
    them) of every set against the oracle."""
    codec = tq.Codec(128, bits, variant, seed=0)
    cd = O.make_codec(128, bits, variant, 0)
    mb = cd.mse_bits
    gen = torch.Generator(device="cuda")
    gen.manual_seed(15)
    keys = dict(codes=torch.randint(0, 256, (n_sets, n_keys, codec.code_row), dtype=torch.uint8, device="cuda",
                                    generator=gen),
                norms=10.0 + torch.randn((n_sets, n_keys), device="cuda", generator=gen))
    if variant == O.PROD:
        keys["signs"] = torch.randint(0, 256, (n_sets, n_keys, codec.sign_row), dtype=torch.uint8, device="cuda",
                                      generator=gen)
        keys["rnorms"] = torch.rand((n_sets, n_keys), device="cuda", generator=gen) * 0.45 + 0.05
    q = torch.randn((n_sets, nq, 128), device="cuda", generator=gen)
    out = codec.logits(q, keys)
    torch.cuda.synchronize()
    rng = np.random.default_rng(16)
    edges = [np.arange(max(c - 32, 0), min(c + 32, n_keys)) for c in range(1 << 25, n_keys, 1 << 25)]
    ks = np.unique(np.concatenate([rng.choice(n_keys, 300, replace=False), np.arange(n_keys - 64, n_keys), *edges]))
    kt = torch.from_numpy(ks).cuda()
    for s in range(n_sets):
        sk = dict(idx=O.unpack(keys["codes"][s, kt].cpu().numpy(), mb, 128),
                  norms=keys["norms"][s, kt].cpu().numpy().astype(np.float64))
        if variant == O.PROD:
            sk["signs"] = O.bits_to_signs(O.unpack(keys["signs"][s, kt].cpu().numpy(), 1, 128))
            sk["rnorms"] = keys["rnorms"][s, kt].cpu().numpy().astype(np.float64)
        ref = O.logits_fast(cd, q[s].cpu().numpy().astype(np.float64), sk, 0)
        check_rows(out[s][:, kt].cpu().numpy(), ref, f"n_keys {n_keys} set {s}")
    del keys, out


@pytest.mark.parametrize("bits", [4, 3])
def test_quantize_kv_config_full_size_sampled(bits):
    """The launch the bench times: K and V of one layer (16 sets = 2 tensors x
    8 KV heads x 32768 tokens x 128 bf16 with outlier channels) in one call,
    mse b = 4 and b = 3, set s on codec group s % 8; sampled vectors of every
    set, the V half included, checked against the oracle."""
    x = torch.cat([workloads.kv_tensor(2), workloads.kv_tensor(3)], 0).contiguous()
    codec = tq.Codec(128, bits, tq.TQ_MSE, seed=0, groups=8)
    cd = O.make_codec(128, bits, O.MSE, 0, groups=8)
    out = codec.quantize(x.cuda())
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    xf = x.float().numpy()
    gi, oi, oy = [], [], []
    for s in range(x.shape[0]):
        sel = np.sort(rng.choice(xf.shape[1], 384, replace=False))
        gidx = _gpu_idx(codec, out["codes"][s, torch.from_numpy(sel).cuda()], bits)
        idx, nu, y = O.quantize_mse(cd, xf[s, sel].astype(np.float64), s % 8)
        gi.append(gidx), oi.append(idx), oy.append(y)
        assert np.allclose(out["norms"][s].cpu().numpy()[sel], nu, rtol=1e-5)
    check_indices(np.concatenate(gi), np.concatenate(oi), np.concatenate(oy), cd.boundaries, f"kv b={bits}")


def test_quantize_kv_prod_full_size_sampled():
    """The KV key tensor (8 heads x 32768 tokens x 128 bf16) under
    TurboQuant_prod b=4 (3-bit mse + QJL), one codec group per head; sampled
    vectors checked against the oracle (indices, signs, both norms)."""
    k = workloads.kv_tensor(2)
    codec = tq.Codec(128, 4, tq.TQ_PROD, seed=0, groups=8)
    cd = O.make_codec(128, 4, O.PROD, 0, groups=8)
    out = codec.quantize(k.cuda())
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    xf = k.float().numpy()
    gi, oi, oy = [], [], []
    qjl = QJLCheck()
    for h in range(8):
        sel = np.sort(rng.choice(xf.shape[1], 256, replace=False))
        st = torch.from_numpy(sel).cuda()
        res = O.quantize_prod(cd, xf[h, sel].astype(np.float64), h)
        gidx = _gpu_idx(codec, out["codes"][h, st], 3)
        gi.append(gidx), oi.append(res["idx"]), oy.append(res["y"])
        qjl.add(cd, xf[h, sel], gidx, _gpu_idx(codec, out["signs"][h, st], 1), out["rnorms"][h].cpu().numpy()[sel], h)
        assert np.allclose(out["norms"][h].cpu().numpy()[sel], res["norms"], rtol=1e-5)
    check_indices(np.concatenate(gi), np.concatenate(oi), np.concatenate(oy), cd.boundaries, "kv prod b=4")
    qjl.check("kv prod b=4")


@pytest.mark.parametrize("variant", [O.MSE, O.PROD])
def test_dequantize_kv_config_full_size_sampled(variant):
    """K and V of the KV workload (16 sets x 32768 tokens x 128 bf16, the
    launch the bench times), b=4: the library's reconstruction of its own
    codes against the oracle's reconstruction of the same codes, on sampled
    rows of every set."""
    x = torch.cat([workloads.kv_tensor(2), workloads.kv_tensor(3)], 0).contiguous()
    codec = tq.Codec(128, 4, variant, seed=0, groups=8)
    cd = O.make_codec(128, 4, variant, 0, groups=8)
    stored = codec.quantize(x.cuda())
    rec = codec.dequantize(stored)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    mb = cd.mse_bits
    for s in range(x.shape[0]):
        sel = np.sort(rng.choice(x.shape[1], 128, replace=False))
        st = torch.from_numpy(sel).cuda()
        idx = O.unpack(stored["codes"][s, st].cpu().numpy(), mb, 128)
        nu = stored["norms"][s, st].cpu().numpy().astype(np.float64)
        if variant == O.MSE:
            ref = O.dequantize_mse(cd, idx, nu, s % 8)
        else:
            z = O.bits_to_signs(O.unpack(stored["signs"][s, st].cpu().numpy(), 1, 128))
            ga = stored["rnorms"][s, st].cpu().numpy().astype(np.float64)
            ref = O.dequantize_prod(cd, idx, z, nu, ga, s % 8)
        check_rows(rec[s, st].cpu().numpy(), ref, f"set {s}")


def test_calls_on_a_side_stream_match_the_default_stream():
    """The data calls enqueued on a side stream (default priority), right
    after their input is produced on that stream and with no host
    synchronisation in between, give the same bytes as on the default
    stream: the library launches on the stream it is given."""
    codec = tq.Codec(128, 4, tq.TQ_PROD, seed=3, groups=2)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(12)
    x_ref = torch.randn((2, 4096, 128), device="cuda", generator=gen).to(torch.bfloat16)
    q = torch.randn((2, 4, 128), device="cuda", generator=gen)
    ref = codec.quantize(x_ref)
    ref_dq = codec.dequantize(ref)
    ref_lg = codec.logits(q, ref)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        x = (x_ref.float() * 1.0).to(torch.bfloat16)  # produced on the side stream
        out = codec.quantize(x, stream=side)
        dq = codec.dequantize(out, stream=side)
        lg = codec.logits(q, out, stream=side)
    side.synchronize()
    for k in ("codes", "signs", "norms", "rnorms"):
        assert torch.equal(out[k], ref[k]), k
    assert torch.equal(dq, ref_dq)
    assert torch.equal(lg, ref_lg)


def test_graph_capture_replays_match_eager():
    """quantize and logits captured into one HIP graph (outputs allocated
    before the capture) and replayed four times, with eager work and
    synchronisations between the replays: every replay gives the eager bytes."""
    codec = tq.Codec(128, 4, tq.TQ_PROD, seed=5, groups=2)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(13)
    x = torch.randn((2, 4096, 128), device="cuda", generator=gen).to(torch.bfloat16)
    q = torch.randn((2, 4, 128), device="cuda", generator=gen)
    out = codec.empty_codes(2, 4096)
    lg = torch.empty((2, 4, 4096), device="cuda")
    codec.quantize(x, out=out)
    codec.logits(q, out, out=lg)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in out.items() if v is not None}
    ref_lg = lg.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            codec.quantize(x, out=out)
            codec.logits(q, out, out=lg)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        codec.quantize(x, out=out)
        codec.logits(q, out, out=lg)
    for r in range(4):
        for v in out.values():
            if v is not None:
                v.zero_()
        lg.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert torch.equal(out[k], v), f"replay {r}: {k}"
        assert torch.equal(lg, ref_lg), f"replay {r}: logits"


def test_graph_capture_covers_the_other_data_calls():
    """dequantize, the tiled TurboQuant_prod quantize (d = 200: it clears its
    residual-norm accumulator with a kernel), attention with a caller
    workspace, append, and the mixed-precision quantize and logits, captured
    into one HIP graph with every output allocated before the capture and
    replayed three times: every replay gives the eager bytes."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(14)
    kc = tq.Codec(128, 4, tq.TQ_PROD, seed=1, groups=2)
    vc = tq.Codec(128, 4, tq.TQ_MSE, seed=2, groups=2)
    tc = tq.Codec(200, 3, tq.TQ_PROD, seed=3)
    chans = np.stack([np.random.default_rng(g).permutation(128)[:64] for g in range(2)])
    mc = tq.MixedCodec(128, 2, tq.TQ_MSE, 4, chans, groups=2)
    xk = torch.randn((2, 2048, 128), device="cuda", generator=gen).to(torch.bfloat16)
    xv = torch.randn((2, 2048, 128), device="cuda", generator=gen).to(torch.bfloat16)
    xt = torch.randn((1, 3000, 200), device="cuda", generator=gen)
    q = torch.randn((2, 4, 128), device="cuda", generator=gen)
    xa = torch.randn((2, 128), device="cuda", generator=gen)
    rows = torch.tensor([5, 2048 + 7], dtype=torch.int64, device="cuda")
    keys, vals = kc.quantize(xk), vc.quantize(xv)
    flat = {k: (None if v is None else v.view(2 * 2048, *v.shape[2:]).clone()) for k, v in keys.items()}
    rec = torch.empty((2, 2048, 128), device="cuda")
    tout = tc.empty_codes(1, 3000)
    ws = torch.empty(max(kc.attention_workspace_bytes(vc, 4, 2, 2048), 1), dtype=torch.uint8, device="cuda")
    att = torch.empty((2, 4, 128), device="cuda")
    mout = mc.empty_codes(2, 2048)
    mws = mc.workspace(2, 2048, 4)
    mlg = torch.empty((2, 4, 2048), device="cuda")

    def calls():
        kc.dequantize(keys, out=rec)
        tc.quantize(xt, out=tout)
        kc.attention(q, keys, vc, vals, out=att, workspace=ws)
        kc.append(xa, rows, flat)
        mc.quantize(xk, out=mout, workspace=mws)
        mc.logits(q, mout, out=mlg, workspace=mws)

    cache = [v for v in flat.values() if v is not None]  # append writes only its rows
    outs = [rec, att, mlg] + [v for v in tout.values() if v is not None] + cache + \
        [v for p in mout for v in p.values() if v is not None]
    calls()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    for r in range(3):
        for o, e in zip(outs, ref):
            if any(o is c for c in cache):
                o.copy_(e)
                o[rows] = 0
            else:
                o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, ref)):
            assert torch.equal(o, e), f"replay {r}: output {i}"


# --------------------------------------------------------- statistics -----
@pytest.mark.parametrize("bits", [2, 4])
def test_gpu_mse_distortion_matches_codebook(bits):
    x = workloads.parity_vectors()
    codec = tq.Codec(128, bits, tq.TQ_MSE, seed=0)
    cd = O.make_codec(128, bits, O.MSE, 0)
    rec = codec.dequantize(codec.quantize(_cuda(x))).cpu().numpy()[0].astype(np.float64)
    nu = np.linalg.norm(x.astype(np.float64), axis=1)
    err = np.sum((rec / nu[:, None] - x / nu[:, None]) ** 2, axis=1)
    assert abs(err.mean() - cd.distortion) < 4 * err.std() / math.sqrt(err.size)


def _logits_all_queries(codec, q, keys):
    """Logits of every query of q ([nq, d], any nq) against one set of keys,
    in calls of at most 64 queries."""
    parts = [codec.logits(_cuda(q[i:i + 64])[None], keys)[0] for i in range(0, q.shape[0], 64)]
    return torch.cat(parts, 0).cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("bits", [2, 4])
def test_gpu_mse_inner_product_shrinkage(bits):
    """The parity workload (4096 vectors, all 256 queries): the least-squares
    slope of the GPU's <q, x_hat> (logits on its own codes) against the exact
    <q, x> is 1 - D_b, the centroid-condition invariant behind the 36% figure
    at one bit ([ttakun] rotation section)."""
    x = workloads.parity_vectors()
    q = workloads.parity_queries()
    codec = tq.Codec(128, bits, tq.TQ_MSE, seed=0)
    cd = O.make_codec(128, bits, O.MSE, 0)
    keys = codec.quantize(_cuda(x))
    lg = _logits_all_queries(codec, q, keys).ravel()
    exact = (q.astype(np.float64) @ x.astype(np.float64).T).ravel()
    slope = float(lg @ exact / (exact @ exact))
    assert slope == pytest.approx(1.0 - cd.distortion, rel=0.015)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_gpu_prod_inner_products_unbiased_over_vectors(bits):
    """The parity workload, all 256 queries: TurboQuant_prod logits on the
    GPU's own codes are unbiased estimates of <q, x> (per-query mean error
    over 4096 keys against its own spread, and the mean of those z-scores)."""
    x = workloads.parity_vectors()
    q = workloads.parity_queries()
    codec = tq.Codec(128, bits, tq.TQ_PROD, seed=0)
    keys = codec.quantize(_cuda(x))
    lg = _logits_all_queries(codec, q, keys)
    err = lg - q.astype(np.float64) @ x.astype(np.float64).T
    # per-query mean error over 4096 keys, compared with its own spread
    z = err.mean(axis=1) / (err.std(axis=1) / math.sqrt(x.shape[0]))
    assert np.abs(z).max() < 5.0 and abs(z.mean()) < 5.0 / math.sqrt(z.size) * 3
