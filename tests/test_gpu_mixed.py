"""GPU parity of outlier-channel mixed precision (two part codecs over a
channel split) against the oracle: quantize (indices, signs, norms per
part), dequantize and logits on the oracle's codes, and the KV workload at
2.5 and 3.5 bits per channel."""
import numpy as np
import pytest
import torch

import kv_cache_compression_tq_amd as tq
import workloads
from oracle import tq_oracle as O
from parity import QJLCheck, check_indices, check_rows

pytestmark = pytest.mark.gpu


def _cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _data(d, n_sets, n, n_out, groups, seed):
    rng = np.random.default_rng(seed)
    chans = np.stack([rng.permutation(d)[:n_out] for _ in range(groups)])
    x = rng.standard_normal((n_sets, n, d))
    for s in range(n_sets):
        x[s][:, chans[s % groups][:4]] *= 10.0  # outliers inside the outlier part
    return chans, x


def _check_part(codec, cd, got, ref, xpart, s, qjl, what):
    """Indices and norms of one part of set s; its QJL signs and residual
    norms (every vector, on the GPU's own indices) go to `qjl`."""
    gidx = None
    if cd.mse_bits:
        gidx = codec.unpack(got["codes"][s], cd.mse_bits).cpu().numpy()
        check_indices(gidx, ref["idx"], ref["y"], cd.boundaries, what)
    assert np.allclose(got["norms"][s].cpu().numpy(), ref["norms"], rtol=1e-5)
    if cd.variant == O.PROD:
        qjl.add(cd, xpart, gidx, codec.unpack(got["signs"][s], 1).cpu().numpy(), got["rnorms"][s].cpu().numpy(),
                s % cd.groups)


CASES = [(128, 64, 2, O.MSE), (128, 64, 3, O.MSE), (128, 64, 3, O.PROD), (128, 32, 2, O.PROD), (200, 40, 1, O.MSE)]


@pytest.mark.parametrize("d,n_out,bits,variant", CASES)
def test_mixed_quantize_matches_oracle(d, n_out, bits, variant):
    n_sets, n, groups = 3, 400, 2
    chans, x = _data(d, n_sets, n, n_out, groups, seed=d + n_out + bits)
    mc = tq.MixedCodec(d, bits, variant, 17, chans, groups=groups)
    mx = O.make_mixed(d, bits, variant, 17, chans, groups=groups)
    po, pr = mc.quantize(_cuda(x.astype(np.float32)))
    torch.cuda.synchronize()
    qo, qr = QJLCheck(), QJLCheck()
    for s in range(n_sets):
        xs = x[s].astype(np.float32).astype(np.float64)
        perm = mx.channels[s % groups]
        ro, rr = O.mixed_quantize(mx, xs, s % groups)
        _check_part(mc.outlier, mx.outlier, po, ro, xs[:, perm[:n_out]], s, qo, f"outlier part set {s}")
        _check_part(mc.regular, mx.regular, pr, rr, xs[:, perm[n_out:]], s, qr, f"regular part set {s}")
    if variant == O.PROD:
        qo.check("outlier part")
        qr.check("regular part")


def _stored(cd, parts_per_set):
    out = {}
    if cd.mse_bits:
        out["codes"] = _cuda(np.stack([O.pack(p["idx"], cd.mse_bits) for p in parts_per_set]))
    out["norms"] = _cuda(np.stack([p["norms"] for p in parts_per_set]).astype(np.float32))
    if cd.variant == O.PROD:
        out["signs"] = _cuda(np.stack([O.pack(O.signs_to_bits(p["signs"]), 1) for p in parts_per_set]))
        out["rnorms"] = _cuda(np.stack([p["rnorms"] for p in parts_per_set]).astype(np.float32))
    return out


def _f32_parts(p):
    q = dict(p)
    q["norms"] = p["norms"].astype(np.float32).astype(np.float64)
    if "rnorms" in p:
        q["rnorms"] = p["rnorms"].astype(np.float32).astype(np.float64)
    return q


@pytest.mark.parametrize("d,n_out,bits,variant", CASES)
def test_mixed_dequantize_and_logits_on_oracle_codes(d, n_out, bits, variant):
    n_sets, n, groups, nq = 2, 300, 2, 5
    chans, x = _data(d, n_sets, n, n_out, groups, seed=3 * d + bits)
    mc = tq.MixedCodec(d, bits, variant, 23, chans, groups=groups)
    mx = O.make_mixed(d, bits, variant, 23, chans, groups=groups)
    parts = [O.mixed_quantize(mx, x[s], s % groups) for s in range(n_sets)]
    parts = [(_f32_parts(po), _f32_parts(pr)) for po, pr in parts]
    stored = (_stored(mx.outlier, [p[0] for p in parts]), _stored(mx.regular, [p[1] for p in parts]))
    rec = mc.dequantize(stored).cpu().numpy()
    q = np.random.default_rng(1).standard_normal((n_sets, nq, d)).astype(np.float32)
    lg = mc.logits(_cuda(q), stored).cpu().numpy()
    for s in range(n_sets):
        check_rows(rec[s], O.mixed_dequantize(mx, parts[s], s % groups), f"dequantize set {s}")
        check_rows(lg[s], O.mixed_logits_plain(mx, q[s].astype(np.float64), parts[s], s % groups), f"logits set {s}")


@pytest.mark.parametrize("bits", [2, 3])
def test_mixed_kv_workload_sampled(bits):
    """8 KV heads x 32768 tokens x 128 bf16 with 4 outlier channels per head;
    per head the 64 channels of largest RMS form the outlier part
    (b + 0.5 bits per channel: 2.5 and 3.5)."""
    k = workloads.kv_tensor(2)
    xf = k.float().numpy()
    rms = np.sqrt((xf.astype(np.float64) ** 2).mean(axis=1))
    chans = np.argsort(-rms, axis=1)[:, :64]
    mc = tq.MixedCodec(128, bits, tq.TQ_MSE, 0, chans, groups=8)
    mx = O.make_mixed(128, bits, O.MSE, 0, chans, groups=8)
    po, pr = mc.quantize(k.cuda())
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    for h in range(8):
        sel = np.sort(rng.choice(xf.shape[1], 256, replace=False))
        ro, rr = O.mixed_quantize(mx, xf[h, sel].astype(np.float64), h)
        t = torch.from_numpy(sel).cuda()
        for codec, cd, got, ref in ((mc.outlier, mx.outlier, po, ro), (mc.regular, mx.regular, pr, rr)):
            gidx = codec.unpack(got["codes"][h, t], cd.mse_bits).cpu().numpy()
            check_indices(gidx, ref["idx"], ref["y"], cd.boundaries, f"head {h}")
            assert np.allclose(got["norms"][h, t].cpu().numpy(), ref["norms"], rtol=1e-5)


@pytest.mark.parametrize("bits", [1, 2, 3])
def test_mixed_fused_bf16_quantize(bits):
    """d = 128 with 64 outlier channels, TurboQuant_mse on bfloat16 input: the
    fused one-pass kernel (both rotations in one image, part norms from masked
    Gram products).  Indices and norms against the oracle, and every packed
    row byte for byte (padding included) against the oracle's packing of its
    indices; ragged n, two groups."""
    n_sets, n, groups = 3, 1001, 2
    chans, x = _data(128, n_sets, n, 64, groups, seed=40 + bits)
    xb = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
    xr = xb.float().numpy().astype(np.float64)
    mc = tq.MixedCodec(128, bits, tq.TQ_MSE, 29, chans, groups=groups)
    mx = O.make_mixed(128, bits, O.MSE, 29, chans, groups=groups)
    po, pr = mc.quantize(xb.cuda())
    torch.cuda.synchronize()
    for s in range(n_sets):
        ro, rr = O.mixed_quantize(mx, xr[s], s % groups)
        for codec, cd, got, ref, what in ((mc.outlier, mx.outlier, po, ro, "outlier"),
                                          (mc.regular, mx.regular, pr, rr, "regular")):
            gidx = codec.unpack(got["codes"][s], cd.mse_bits).cpu().numpy()
            check_indices(gidx, ref["idx"], ref["y"], cd.boundaries, f"{what} part set {s}")
            assert np.allclose(got["norms"][s].cpu().numpy(), ref["norms"], rtol=1e-5)
            # every row is the oracle's packing of its indices, padding included
            rows = got["codes"][s].cpu().numpy()
            assert np.array_equal(rows, O.pack(gidx, cd.mse_bits, rows.shape[1])), what


def test_mixed_fused_single_vector_and_zero_part():
    """One vector per set (a single partial stage) whose regular channels are
    all zero: the regular part's norm is 0 and its codes are those of y = 0."""
    chans = np.arange(64)[None, :]
    x = np.zeros((2, 1, 128), np.float32)
    x[:, 0, :64] = np.random.default_rng(5).standard_normal((2, 64))
    xb = torch.from_numpy(x).to(torch.bfloat16)
    mc = tq.MixedCodec(128, 2, tq.TQ_MSE, 3, chans, groups=1)
    mx = O.make_mixed(128, 2, O.MSE, 3, chans, groups=1)
    po, pr = mc.quantize(xb.cuda())
    torch.cuda.synchronize()
    for s in range(2):
        ro, rr = O.mixed_quantize(mx, xb[s].float().numpy().astype(np.float64), 0)
        assert pr["norms"][s].item() == 0.0
        assert np.array_equal(mc.regular.unpack(pr["codes"][s], 2).cpu().numpy(), rr["idx"])
        gidx = mc.outlier.unpack(po["codes"][s], 3).cpu().numpy()
        check_indices(gidx, ro["idx"], ro["y"], mx.outlier.boundaries, f"outlier set {s}")


@pytest.mark.parametrize("bits", [1, 2, 3])
def test_mixed_fused_logits(bits):
    """d = 128 with 64 outlier channels, TurboQuant_mse: the one-pass logits
    kernel over both parts' codes (9 heads: two head chunks; 1000 keys: full
    blocks and a ragged tail) against <q, x_hat> of the oracle's codes."""
    n_sets, n, groups, nq = 3, 1000, 2, 9
    chans, x = _data(128, n_sets, n, 64, groups, seed=60 + bits)
    mc = tq.MixedCodec(128, bits, tq.TQ_MSE, 31, chans, groups=groups)
    mx = O.make_mixed(128, bits, O.MSE, 31, chans, groups=groups)
    parts = [O.mixed_quantize(mx, x[s], s % groups) for s in range(n_sets)]
    parts = [(_f32_parts(po), _f32_parts(pr)) for po, pr in parts]
    stored = (_stored(mx.outlier, [p[0] for p in parts]), _stored(mx.regular, [p[1] for p in parts]))
    q = np.random.default_rng(bits).standard_normal((n_sets, nq, 128)).astype(np.float32)
    lg = mc.logits(_cuda(q), stored).cpu().numpy()
    for s in range(n_sets):
        check_rows(lg[s], O.mixed_logits_plain(mx, q[s].astype(np.float64), parts[s], s % groups), f"logits set {s}")


def test_mixed_decode_logits_full_size_sampled():
    """Decode logits on a 2.5-bit mixed key cache at the decode shape (16 batch
    x 8 KV heads x 131072 tokens, 4 query heads per KV head, the launch the
    bench times): a synthetic packed cache (random code bytes, norms about 10),
    sampled keys of 12 sets against the oracle's logits of the same codes."""
    sets, T, d, qh = workloads.DEC_BATCH * workloads.DEC_KV_HEADS, workloads.DEC_TOKENS, 128, workloads.DEC_Q_PER_KV
    rng = np.random.default_rng(7)
    chans = np.stack([rng.permutation(d)[:64] for _ in range(workloads.DEC_KV_HEADS)])
    mc = tq.MixedCodec(d, 2, tq.TQ_MSE, 0, chans, groups=workloads.DEC_KV_HEADS)
    mx = O.make_mixed(d, 2, O.MSE, 0, chans, groups=workloads.DEC_KV_HEADS)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(9)
    cache = mc.empty_codes(sets, T)
    for part in cache:
        part["codes"].copy_(torch.randint(0, 256, part["codes"].shape, dtype=torch.uint8, device="cuda", generator=gen))
        part["norms"].copy_(10.0 + torch.randn(part["norms"].shape, device="cuda", generator=gen))
    q = torch.randn((sets, qh, d), device="cuda", generator=gen)
    out = mc.logits(q, cache)
    torch.cuda.synchronize()
    for s in rng.choice(sets, 12, replace=False):
        kt = torch.from_numpy(np.sort(rng.choice(T, 300, replace=False))).cuda()
        parts = tuple(dict(idx=O.unpack(p["codes"][s, kt].cpu().numpy(), cd.mse_bits, 64),
                           norms=p["norms"][s, kt].cpu().numpy().astype(np.float64))
                      for cd, p in ((mx.outlier, cache[0]), (mx.regular, cache[1])))
        ref = O.mixed_logits_plain(mx, q[s].cpu().numpy().astype(np.float64), parts, int(s) % workloads.DEC_KV_HEADS)
        check_rows(out[s][:, kt].cpu().numpy(), ref, f"set {s}")


def test_mixed_fused_logits_past_the_key_chunk():
    """The one-pass mixed logits on two sets of 2^25 + 64 keys (two chunks of
    keys per set) and 10 heads (two head groups): sampled keys, those around
    the chunk boundary and the last 64 among them, against the oracle."""
    d, n_sets, n_keys, nq = 128, 2, (1 << 25) + 64, 10
    rng = np.random.default_rng(21)
    chans = np.stack([rng.permutation(d)[:64] for _ in range(2)])
    mc = tq.MixedCodec(d, 2, tq.TQ_MSE, 0, chans, groups=2)
    mx = O.make_mixed(d, 2, O.MSE, 0, chans, groups=2)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(22)
    cache = mc.empty_codes(n_sets, n_keys)
    for part in cache:
        part["codes"].copy_(torch.randint(0, 256, part["codes"].shape, dtype=torch.uint8, device="cuda", generator=gen))
        part["norms"].copy_(10.0 + torch.randn(part["norms"].shape, device="cuda", generator=gen))
    q = torch.randn((n_sets, nq, d), device="cuda", generator=gen)
    out = mc.logits(q, cache)
    torch.cuda.synchronize()
    ks = np.unique(np.concatenate([rng.choice(n_keys, 300, replace=False), np.arange(n_keys - 64, n_keys),
                                   np.arange((1 << 25) - 32, (1 << 25) + 32)]))
    kt = torch.from_numpy(ks).cuda()
    for s in range(n_sets):
        parts = tuple(dict(idx=O.unpack(p["codes"][s, kt].cpu().numpy(), cd.mse_bits, 64),
                           norms=p["norms"][s, kt].cpu().numpy().astype(np.float64))
                      for cd, p in ((mx.outlier, cache[0]), (mx.regular, cache[1])))
        ref = O.mixed_logits_plain(mx, q[s].cpu().numpy().astype(np.float64), parts, s % 2)
        check_rows(out[s][:, kt].cpu().numpy(), ref, f"set {s}")
    del cache, out


@pytest.mark.parametrize("n_out,bits,variant,nq", [(32, 2, O.PROD, 9), (4, 2, O.MSE, 1), (20, 3, O.MSE, 13)])
def test_mixed_composed_logits_part_buffers_do_not_overlap(n_out, bits, variant, nq):
    """The composed logits path keeps the two parts' gathered queries and the
    regular part's logits in one workspace.  Shapes where n_sets * nq * n_out
    floats is not a multiple of 256 bytes (so an overlap of the part buffers
    would corrupt the last query's regular coordinates): logits against the
    oracle for every query, with the workspace prefilled with NaN."""
    d, n_sets, n, groups = 128, 1, 257, 1
    chans, x = _data(d, n_sets, n, n_out, groups, seed=n_out + nq)
    mc = tq.MixedCodec(d, bits, variant, 41, chans, groups=groups)
    mx = O.make_mixed(d, bits, variant, 41, chans, groups=groups)
    parts = [(_f32_parts(po), _f32_parts(pr)) for po, pr in [O.mixed_quantize(mx, x[0], 0)]]
    stored = (_stored(mx.outlier, [parts[0][0]]), _stored(mx.regular, [parts[0][1]]))
    q = np.random.default_rng(nq).standard_normal((n_sets, nq, d)).astype(np.float32)
    ws = mc.workspace(n_sets, n, nq)
    ws.view(torch.uint8).fill_(0xFF)  # NaN bit patterns everywhere
    lg = mc.logits(_cuda(q), stored, workspace=ws).cpu().numpy()
    check_rows(lg[0], O.mixed_logits_plain(mx, q[0].astype(np.float64), parts[0], 0), "composed logits")


def test_mixed_calls_reject_bad_part_pointers_before_launching():
    """A NULL or misaligned array of either part fails with TQ_EINVAL before
    anything is enqueued: the outputs keep their contents."""
    import ctypes

    lib = tq.lib()
    d, n_sets, n, nq = 128, 1, 64, 4
    chans = np.arange(64)[None, :]
    for variant in (tq.TQ_MSE, tq.TQ_PROD):
        mc = tq.MixedCodec(d, 2, variant, 3, chans, groups=1)
        x = torch.randn((n_sets, n, d), device="cuda").to(torch.bfloat16)
        q = torch.randn((n_sets, nq, d), device="cuda")
        good = mc.quantize(x)
        torch.cuda.synchronize()
        ws = mc.workspace(n_sets, n, nq)
        out_lg = torch.full((n_sets, nq, n), 7.0, device="cuda")
        out_rec = torch.full((n_sets, n, d), 7.0, device="cuda")
        keys = ["codes", "norms"] + (["signs", "rnorms"] if variant == tq.TQ_PROD else [])
        for part in (0, 1):
            for key in keys:
                for bad in ("null", "misaligned"):
                    arrs = {k: tq._ptr_pair(good, k) for k in ("codes", "signs", "norms", "rnorms")}
                    base = good[part][key].data_ptr()
                    arrs[key][part] = None if bad == "null" else base + (4 if key in ("codes", "signs") else 2)
                    before = [t.clone() for p in good for t in p.values() if t is not None]
                    st_q = lib.tq_mixed_quantize(mc._h, ctypes.c_void_p(x.data_ptr()), tq.TQ_BF16, n_sets, n,
                                                 arrs["codes"], arrs["signs"], arrs["norms"], arrs["rnorms"],
                                                 ctypes.c_void_p(ws.data_ptr()), ws.numel(), None)
                    st_d = lib.tq_mixed_dequantize(mc._h, arrs["codes"], arrs["signs"], arrs["norms"], arrs["rnorms"],
                                                   n_sets, n, ctypes.c_void_p(out_rec.data_ptr()),
                                                   ctypes.c_void_p(ws.data_ptr()), ws.numel(), None)
                    st_l = lib.tq_mixed_logits(mc._h, ctypes.c_void_p(q.data_ptr()), nq, arrs["codes"], arrs["signs"],
                                               arrs["norms"], arrs["rnorms"], n_sets, n,
                                               ctypes.c_void_p(out_lg.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                                               ws.numel(), None)
                    torch.cuda.synchronize()
                    what = f"variant {variant} part {part} {key} {bad}"
                    assert (st_q, st_d, st_l) == (tq.TQ_EINVAL,) * 3, what
                    after = [t for p in good for t in p.values() if t is not None]
                    assert all(torch.equal(a, b) for a, b in zip(before, after)), what
                    assert torch.all(out_lg == 7.0) and torch.all(out_rec == 7.0), what
        mc.close()
