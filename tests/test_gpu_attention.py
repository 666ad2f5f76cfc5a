"""GPU parity of decode attention over quantized keys and values: the HIP
library (through its C ABI) against the oracle's softmax(scale q k_hat^T) v_hat.

Keys and values are quantized by the oracle and handed to the library in the
stored layout, so both sides score the very same codes; the output rows are
compared with the reconstruction/logit bar (relative L2 error <= 1e-3 per
row, every element within 1e-3 of the row's RMS).
"""
import math

import numpy as np
import pytest
import torch

import kv_cache_compression_tq_amd as tq
import workloads
from oracle import tq_oracle as O
from parity import check_rows

pytestmark = pytest.mark.gpu


def _cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _oracle_codes(cd, x, group):
    """Oracle codes for x with float32-rounded norms (as stored)."""
    if cd.variant == O.MSE:
        idx, nu, _ = O.quantize_mse(cd, x, group)
        return dict(idx=idx, norms=nu.astype(np.float32).astype(np.float64))
    r = O.quantize_prod(cd, x, group)
    return dict(idx=r["idx"], signs=r["signs"], norms=r["norms"].astype(np.float32).astype(np.float64),
                rnorms=r["rnorms"].astype(np.float32).astype(np.float64))


def _stored(cd, per_set):
    out = {}
    if cd.mse_bits:
        out["codes"] = _cuda(np.stack([O.pack(k["idx"], cd.mse_bits) for k in per_set]))
    out["norms"] = _cuda(np.stack([k["norms"] for k in per_set]).astype(np.float32))
    if cd.variant == O.PROD:
        out["signs"] = _cuda(np.stack([O.pack(O.signs_to_bits(k["signs"]), 1) for k in per_set]))
        out["rnorms"] = _cuda(np.stack([k["rnorms"] for k in per_set]).astype(np.float32))
    return out


ATTN_CASES = [
    # d, (k variant, k bits), (v variant, v bits), n_sets, nq, n_keys, scale
    (128, (O.PROD, 4), (O.MSE, 4), 3, 4, 1000, None),
    (128, (O.PROD, 4), (O.MSE, 3), 2, 4, 4096 + 17, None),
    (128, (O.PROD, 3), (O.MSE, 2), 1, 1, 1, None),          # one key: the value itself
    (128, (O.PROD, 2), (O.MSE, 4), 1, 12, 777, 0.5),          # more than 8 heads
    (128, (O.MSE, 4), (O.MSE, 4), 2, 8, 640, None),
    (128, (O.PROD, 1), (O.MSE, 1), 1, 4, 300, None),
    (128, (O.PROD, 4), (O.PROD, 3), 2, 4, 513, None),         # prod values
    (128, (O.PROD, 5), (O.MSE, 4), 1, 3, 200, 0.0),           # scale 0: the mean value
    (200, (O.PROD, 2), (O.MSE, 3), 2, 4, 301, None),
    (96, (O.MSE, 3), (O.PROD, 2), 1, 2, 129, 0.25),
]


@pytest.mark.parametrize("d,kc,vc,n_sets,nq,n_keys,scale", ATTN_CASES)
def test_attention_oracle_codes(d, kc, vc, n_sets, nq, n_keys, scale):
    groups = min(n_sets, 2)
    rng = np.random.default_rng(d + 7 * kc[1] + vc[1] + nq)
    xk = rng.standard_normal((n_sets, n_keys, d))
    xv = rng.standard_normal((n_sets, n_keys, d))
    q = rng.standard_normal((n_sets, nq, d)).astype(np.float32)
    ck = O.make_codec(d, kc[1], kc[0], 41, groups=groups)
    cv = O.make_codec(d, vc[1], vc[0], 42, groups=groups)
    kcod = tq.Codec(d, kc[1], kc[0], seed=41, groups=groups)
    vcod = tq.Codec(d, vc[1], vc[0], seed=42, groups=groups)
    keys = [_oracle_codes(ck, xk[s], s % groups) for s in range(n_sets)]
    vals = [_oracle_codes(cv, xv[s], s % groups) for s in range(n_sets)]
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    got = kcod.attention(_cuda(q), _stored(ck, keys), vcod, _stored(cv, vals), scale=sc).cpu().numpy()
    for s in range(n_sets):
        ref = O.attention_plain(ck, cv, q[s].astype(np.float64), keys[s], vals[s], sc, s % groups)
        check_rows(got[s], ref, f"attention set {s}")


def test_attention_workspace_checks():
    d = 128
    kcod = tq.Codec(d, 4, tq.TQ_PROD, seed=1)
    vcod = tq.Codec(d, 4, tq.TQ_MSE, seed=2)
    need = kcod.attention_workspace_bytes(vcod, 4, 2, 1000)
    assert 0 < need < 2 * 4 * 1000 * 4  # the fused kernel's partials, not the unfused logits buffer
    x = torch.randn(2, 1000, d, device="cuda")
    keys, vals = kcod.quantize(x), vcod.quantize(x)
    q = torch.randn(2, 4, d, device="cuda")
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(tq.TQError):
        kcod.attention(q, keys, vcod, vals, workspace=small)
    other = tq.Codec(64, 4, tq.TQ_MSE, seed=2)
    with pytest.raises(tq.TQError):
        kcod.attention_workspace_bytes(other, 4, 2, 1000)


def test_attention_decode_config_full_size_sampled():
    """16 batch x 8 KV heads x 131072 keys (prod b=4) and values (mse b=4),
    4 query heads per KV head, on a synthetic packed cache; sampled sets
    checked against the oracle over all of their keys."""
    sets, T, d = workloads.DEC_BATCH * workloads.DEC_KV_HEADS, workloads.DEC_TOKENS, workloads.DEC_DIM
    kcod = tq.Codec(d, 4, tq.TQ_PROD, seed=0, groups=workloads.DEC_KV_HEADS)
    vcod = tq.Codec(d, 4, tq.TQ_MSE, seed=1, groups=workloads.DEC_KV_HEADS)
    ck = O.make_codec(d, 4, O.PROD, 0, groups=workloads.DEC_KV_HEADS)
    cv = O.make_codec(d, 4, O.MSE, 1, groups=workloads.DEC_KV_HEADS)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(6)
    keys = dict(codes=torch.randint(0, 256, (sets, T, kcod.code_row), dtype=torch.uint8, device="cuda", generator=gen),
                signs=torch.randint(0, 256, (sets, T, kcod.sign_row), dtype=torch.uint8, device="cuda", generator=gen),
                norms=(10.0 + torch.randn((sets, T), device="cuda", generator=gen)).float(),
                rnorms=torch.rand((sets, T), device="cuda", generator=gen) * 0.45 + 0.05)
    vals = dict(codes=torch.randint(0, 256, (sets, T, vcod.code_row), dtype=torch.uint8, device="cuda", generator=gen),
                norms=(10.0 + torch.randn((sets, T), device="cuda", generator=gen)).float())
    q = workloads.decode_queries().reshape(sets, workloads.DEC_Q_PER_KV, d)
    sc = 1.0 / math.sqrt(d)
    out = kcod.attention(_cuda(q), keys, vcod, vals, scale=sc)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    for s in rng.choice(sets, 3, replace=False):
        g = int(s) % workloads.DEC_KV_HEADS
        kd = dict(idx=O.unpack(keys["codes"][s].cpu().numpy(), 3, d),
                  signs=O.bits_to_signs(O.unpack(keys["signs"][s].cpu().numpy(), 1, d)),
                  norms=keys["norms"][s].cpu().numpy().astype(np.float64),
                  rnorms=keys["rnorms"][s].cpu().numpy().astype(np.float64))
        vd = dict(idx=O.unpack(vals["codes"][s].cpu().numpy(), 4, d),
                  norms=vals["norms"][s].cpu().numpy().astype(np.float64))
        ref = O.attention_plain(ck, cv, q[s].astype(np.float64), kd, vd, sc, g)
        check_rows(out[s].cpu().numpy(), ref, f"set {s}")
