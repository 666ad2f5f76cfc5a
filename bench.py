"""Benchmark of the TurboQuant hot path on one MI355X.

Default workload (the metric's configuration): KV-cache compression of one
layer of a Llama-3.1-8B-shaped model -- K and V, each 8 KV heads x 32768 tokens
x head_dim 128 in bf16 with 4 outlier channels per head (x10), TurboQuant_mse
at b = 4 with one rotation per head.  One step = one tq_quantize call over both
tensors (524,288 vectors), inputs resident in HBM and rotated over enough
copies to defeat the 256 MB Infinity Cache.

The same JSON line also carries the decode-attention-logits phase: 16 batch x
8 KV heads x 131072 cached tokens stored as TurboQuant_prod b = 4 (3-bit mse +
1-bit QJL), 4 query heads per KV head, float32 logits -- timed the same way --
and the fused decode attention over that key cache plus a TurboQuant_mse b = 4
value cache of the same shape.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0


def _parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--skip-logits", action="store_true")
    p.add_argument("--skip-attention", action="store_true")
    p.add_argument("--skip-others", action="store_true",
                   help="skip the non-headline paths (prod quantize, dequantize, high-d, NN indexing)")
    p.add_argument("--skip-dense", action="store_true", help="skip the unquantized-key logits baseline")
    p.add_argument("--skip-ceilings", action="store_true", help="skip the in-tree stream and MFMA probes")
    p.add_argument("--kv-only", action="store_true",
                   help="of the other paths, run only the KV-shape ones (prod quantize, dequantize, mixed)")
    p.add_argument("--copy-probe", action="store_true",
                   help="also run one plain 1 GiB device-to-device copy (counter calibration)")
    return p.parse_args()


def counted_traffic(profile):
    """HBM bytes per launch from a committed counter summary under profiles/
    (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when the kernel
    sources have changed since those counters were taken."""
    import hashlib
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", profile)
    if not os.path.exists(path):
        return None
    fields = dict(line.split(": ", 1) for line in open(path).read().splitlines()
                  if line.startswith(("traffic_bytes_per_launch: ", "kernel_source_sha256_16: ")))
    h = hashlib.sha256()
    for f in ("fast128.hip", "device_common.h"):  # the sources that define the kernel's code
        with open(os.path.join(os.path.dirname(os.path.abspath(__file__)),
                               "kv_cache_compression_tq_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if fields.get("kernel_source_sha256_16") != h.hexdigest()[:16]:
        return None
    return float(fields["traffic_bytes_per_launch"])


def _events(torch, n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def time_launches(torch, fn, steps, warmup, copies):
    """Run fn(i) `warmup` then `steps` times back to back; return (wall ms per
    step from the host clock, mean ms per step from one pair of events
    recorded on the launch stream around the timed steps, median ms per step
    from a separate pass after the timed region with an event pair around
    each step)."""
    for i in range(warmup):
        fn(i % copies)
    torch.cuda.synchronize()
    e0, e1 = _events(torch, 2)
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        fn(i % copies)
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    mean = e0.elapsed_time(e1) / steps
    n = min(steps, 10)
    ev = _events(torch, 2 * n)
    for i in range(n):
        ev[2 * i].record()
        fn(i % copies)
        ev[2 * i + 1].record()
    torch.cuda.synchronize()
    per = [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(n)]
    return wall, mean, float(np.median(per))


def quantize_phase(torch, tq, workloads, steps, warmup):
    k = workloads.kv_tensor(2)
    v = workloads.kv_tensor(3)
    x = torch.cat([k, v], 0).contiguous()          # [16 sets][32768][128] bf16
    sets, n, d = x.shape
    copies = 4                                      # 4 x 128 MiB inputs > MALL
    xs = [x.cuda()] + [x.cuda() for _ in range(copies - 1)]
    codec = tq.Codec(d, 4, tq.TQ_MSE, seed=0, groups=workloads.KV_HEADS)
    outs = [codec.empty_codes(sets, n) for _ in range(copies)]

    def step(i):
        codec.quantize(xs[i], out=outs[i])

    wall, kern, kmed = time_launches(torch, step, steps, warmup, copies)
    # warm: the same input every step (128 MiB in + 34 MB out fit the 256 MB
    # Infinity Cache)
    _, kern_warm, _ = time_launches(torch, lambda i: codec.quantize(xs[0], out=outs[0]), steps, warmup, 1)
    vectors = sets * n
    bytes_per_vec = d * 2 + codec.code_row + 4      # bf16 in, packed codes, f32 norm
    algo_flops = 2 * d * d                          # y = Pi x
    # executed: two bf16 passes (Pi hi, Pi lo) plus the Gram product for the
    # norm (4 MFMAs of 16 x 16 x 32 per 16 vectors)
    exec_flops = 2 * 2 * d * d + 4 * 2 * 16 * 16 * 32 // 16
    achieved = vectors * bytes_per_vec / (kern * 1e-3) / 1e9
    return dict(vectors=vectors, wall_ms=wall, kernel_ms=kern, kernel_ms_median=kmed, kernel_ms_warm=kern_warm,
                bytes_per_vector=bytes_per_vec, achieved_gbs=achieved,
                achieved_gbs_warm=vectors * bytes_per_vec / (kern_warm * 1e-3) / 1e9,
                mfma_algo_tflops=vectors * algo_flops / (kern * 1e-3) / 1e12,
                mfma_exec_tflops=vectors * exec_flops / (kern * 1e-3) / 1e12, codec=codec, x=x)


def quantize_b3_phase(torch, tq, workloads, x, steps, warmup):
    sets, n, d = x.shape
    xs = [x.cuda() for _ in range(4)]
    codec = tq.Codec(d, 3, tq.TQ_MSE, seed=0, groups=workloads.KV_HEADS)
    outs = [codec.empty_codes(sets, n) for _ in range(4)]
    wall, kern, _ = time_launches(torch, lambda i: codec.quantize(xs[i], out=outs[i]), steps, warmup, 4)
    bpv = d * 2 + codec.code_row + 4
    return dict(kernel_ms=kern, vectors_per_s=sets * n / (kern * 1e-3),
                achieved_gbs=sets * n * bpv / (kern * 1e-3) / 1e9)


def logits_phase(torch, tq, workloads, steps, warmup):
    B, H, QH, T, d = (workloads.DEC_BATCH, workloads.DEC_KV_HEADS, workloads.DEC_Q_PER_KV,
                      workloads.DEC_TOKENS, workloads.DEC_DIM)
    sets = B * H
    codec = tq.Codec(d, 4, tq.TQ_PROD, seed=0, groups=H)
    cache = codec.empty_codes(sets, T)
    # build the cache: float32 N(0,1) keys drawn on the device, 8 sets at a time
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4)
    chunk = 8
    kbuf = torch.empty((chunk, T, d), dtype=torch.float32, device="cuda")
    t0 = time.perf_counter()
    for s0 in range(0, sets, chunk):
        kbuf.normal_(generator=gen)
        view = {k: (None if v is None else v[s0:s0 + chunk]) for k, v in cache.items()}
        # the chunk's sets map to groups s % H because chunk is a multiple of H
        codec.quantize(kbuf, out=view)
    torch.cuda.synchronize()
    build_s = time.perf_counter() - t0
    del kbuf
    q = torch.from_numpy(workloads.decode_queries().reshape(sets, QH, d)).cuda()
    out = torch.empty((sets, QH, T), dtype=torch.float32, device="cuda")
    wall, kern, kmed = time_launches(torch, lambda i: codec.logits(q, cache, out=out), steps, warmup, 1)
    keys = sets * T
    packed = keys * (codec.code_row + codec.sign_row + 8)
    written = sets * QH * T * 4
    del out
    return dict(keys=keys, wall_ms=wall, kernel_ms=kern, kernel_ms_median=kmed, cache_build_s=build_s,
                packed_bytes=packed, logits_bytes=written,
                packed_gbs=packed / (kern * 1e-3) / 1e9,
                total_gbs=(packed + written) / (kern * 1e-3) / 1e9, codec=codec, cache=cache, q=q)


def attention_phase(torch, tq, workloads, lp, steps, warmup):
    """Decode attention on the logits phase's key cache plus a value cache of
    the same shape (TurboQuant_mse b = 4 of float32 N(0,1) draws): one fused
    tq_attention call per step, softmax scale 1/sqrt(128)."""
    H, T, d = workloads.DEC_KV_HEADS, workloads.DEC_TOKENS, workloads.DEC_DIM
    kc, cache, q = lp["codec"], lp["cache"], lp["q"]
    sets, QH = q.shape[0], q.shape[1]
    vc = tq.Codec(d, 4, tq.TQ_MSE, seed=1, groups=H)
    vals = vc.empty_codes(sets, T)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(8)
    chunk = 8
    vbuf = torch.empty((chunk, T, d), dtype=torch.float32, device="cuda")
    for s0 in range(0, sets, chunk):
        vbuf.normal_(generator=gen)
        vc.quantize(vbuf, out={k: (None if v is None else v[s0:s0 + chunk]) for k, v in vals.items()})
    torch.cuda.synchronize()
    del vbuf
    ws = torch.empty(max(kc.attention_workspace_bytes(vc, QH, sets, T), 1), dtype=torch.uint8, device="cuda")
    out = torch.empty((sets, QH, d), dtype=torch.float32, device="cuda")
    scale = 1.0 / d ** 0.5
    wall, kern, kmed = time_launches(
        torch, lambda i: kc.attention(q, cache, vc, vals, scale=scale, out=out, workspace=ws), steps, warmup, 1)
    keys = sets * T
    packed = keys * (kc.code_row + kc.sign_row + 8 + vc.code_row + 4)
    # online append into the same caches: one new key and value per set, at the
    # last slot of each set (rows s * T + T - 1 of the flat [sets * T] cache)
    flat_k = {k: (None if v is None else v.view(sets * T, *v.shape[2:])) for k, v in cache.items()}
    flat_v = {k: (None if v is None else v.view(sets * T, *v.shape[2:])) for k, v in vals.items()}
    rows = torch.arange(sets, device="cuda", dtype=torch.int64) * T + (T - 1)
    xk = torch.randn((sets, d), generator=gen, device="cuda")
    xv = torch.randn((sets, d), generator=gen, device="cuda")

    def append_step(i):
        kc.append(xk, rows, flat_k)
        vc.append(xv, rows, flat_v)

    awall, akern, _ = time_launches(torch, append_step, steps, warmup, 1)
    return dict(keys=keys, wall_ms=wall, kernel_ms=kern, kernel_ms_median=kmed, packed_bytes=packed,
                packed_gbs=packed / (kern * 1e-3) / 1e9, workspace_bytes=ws.numel(), append_ms=akern,
                append_wall_ms=awall, sets=sets)


def hbm_probes(torch):
    """Plain torch kernels over 1 GiB streams, each after a 1 GiB fill so that
    no input is still held in the 256 MB Infinity Cache: a copy (torch.neg,
    one launch, the calibration of the byte counters; its duration is read from
    the kernel trace), a three-input one-output elementwise op (torch.addcmul:
    a quarter of the bytes written, close to the quantize and logits mixes) and
    a read-only reduction (torch.sum).  Returns GB/s of the last two (events
    around one launch each, after a small launch that loads the kernel)."""
    n = 1 << 28
    src = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    evict = torch.empty_like(src).fill_(2.0)
    torch.cuda.synchronize()
    torch.neg(src, out=dst)   # plain elementwise kernel (the only neg here): reads and writes 1 GiB
    torch.cuda.synchronize()
    small = torch.ones(4096, dtype=torch.float32, device="cuda")
    torch.addcmul(small, small, small)
    torch.sum(small)
    q = n // 4
    a, b, c, out = src[:q], src[q:2 * q], src[2 * q:3 * q], dst[:q]
    ev = _events(torch, 2)
    res = {}
    for name, fn, nbytes in (("addcmul_3r1w_gbs", lambda: torch.addcmul(a, b, c, out=out), 16 * q),
                             ("sum_read_gbs", lambda: torch.sum(src), 4 * n)):
        evict.fill_(2.0)
        torch.cuda.synchronize()
        ev[0].record()
        fn()
        ev[1].record()
        torch.cuda.synchronize()
        res[name] = nbytes / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e9
    del src, dst, evict, small
    return res


def _mean_launch_ms(torch, fn, reps=5, warm=1):
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    ev = _events(torch, 2)
    ev[0].record()
    for _ in range(reps):
        fn()
    ev[1].record()
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[1]) / reps


def other_paths_phase(torch, tq, workloads, x_kv, kv_only=False):
    """The rest of the hot path, timed once each (not the headline metric):
    TurboQuant_prod quantize and both dequantizes on the KV workload, the
    high-dimensional quantize (d = 1536, 1e5 vectors; d = 3072, 5e4) and the
    nearest-neighbour indexing (d = 200, 1e6 unit vectors).  Inputs are drawn
    on the device with the workloads' distributions.  kv_only: the KV-shape
    parts alone (prod quantize, dequantizes, mixed precision)."""
    res = {}
    sets, n, d = x_kv.shape
    xk = x_kv.cuda()
    for variant, name in ((tq.TQ_MSE, "mse"), (tq.TQ_PROD, "prod")):
        codec = tq.Codec(d, 4, variant, seed=0, groups=workloads.KV_HEADS)
        out = codec.empty_codes(sets, n)
        ms = _mean_launch_ms(torch, lambda: codec.quantize(xk, out=out))
        if variant == tq.TQ_PROD:
            res["kv_prod_b4_quantize_ms"] = ms
        rec = torch.empty((sets, n, d), dtype=torch.float32, device="cuda")
        ms = _mean_launch_ms(torch, lambda: codec.dequantize(out, out=rec))
        res[f"kv_{name}_b4_dequantize_ms"] = ms
        res[f"kv_{name}_b4_dequantize_gbs"] = (sets * n * (d * 4 + codec.code_row + codec.sign_row + 8)) / (ms * 1e-3) / 1e9
        del rec
    gen = torch.Generator(device="cuda")
    gen.manual_seed(9)
    for dd, nn in (() if kv_only else ((1536, 100_000), (3072, 50_000))):
        z = torch.randn((1, nn, dd), generator=gen, device="cuda")
        rho = torch.empty((1, nn, 1), device="cuda").log_normal_(0.0, 0.5, generator=gen)
        xh = z / z.norm(dim=2, keepdim=True) * rho
        del z
        for variant, name, bits in [(v, nm, b) for v, nm in ((tq.TQ_MSE, "mse"), (tq.TQ_PROD, "prod"))
                                    for b in (1, 2, 3, 4)]:
            codec = tq.Codec(dd, bits, variant, seed=0)
            out = codec.empty_codes(1, nn)
            ms = _mean_launch_ms(torch, lambda: codec.quantize(xh, out=out))
            # f32 input: 3 split-bf16 passes per GEMM.  mse: Pi x; prod: Pi x,
            # S x and M c, or S x alone when the mse stage has 0 bits (b = 1)
            mse_bits = bits if variant == tq.TQ_MSE else bits - 1
            gemm = 1 if variant == tq.TQ_MSE else (3 if mse_bits > 0 else 1)
            flops = 2.0 * nn * dd * dd * 3 * gemm
            # the method's own flops: Pi x, and for prod S r (one GEMM when
            # there is no mse stage)
            algo = 2.0 * nn * dd * dd * (1 if variant == tq.TQ_MSE else (2 if mse_bits > 0 else 1))
            res[f"d{dd}_{name}_b{bits}_quantize_ms"] = ms
            res[f"d{dd}_{name}_b{bits}_vectors_per_s"] = nn / (ms * 1e-3)
            res[f"d{dd}_{name}_b{bits}_mfma_frac_executed_bf16"] = flops / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS
            res[f"d{dd}_{name}_b{bits}_mfma_frac_algorithmic_bf16"] = algo / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS
        del xh
    # outlier-channel mixed precision on the KV workload: per head the 64
    # channels of largest RMS at b + 1 bits, the rest at b (2.5 and 3.5 bits)
    rms = xk.float().pow(2).mean(dim=1).sqrt()           # [16 sets][128]; groups from the key heads
    chans = torch.argsort(rms[:workloads.KV_HEADS], dim=1, descending=True)[:, :64].cpu().numpy()
    for bits in (2, 3):
        mc = tq.MixedCodec(d, bits, tq.TQ_MSE, 0, chans, groups=workloads.KV_HEADS)
        out = mc.empty_codes(sets, n)
        ws = mc.workspace(sets, n)
        ms = _mean_launch_ms(torch, lambda: mc.quantize(xk, out=out, workspace=ws))
        res[f"kv_mixed_{bits}.5bit_quantize_ms"] = ms
        res[f"kv_mixed_{bits}.5bit_vectors_per_s"] = sets * n / (ms * 1e-3)
        byts = sets * n * (d * 2 + mc.outlier.code_row + mc.regular.code_row + 8)
        res[f"kv_mixed_{bits}.5bit_gbs"] = byts / (ms * 1e-3) / 1e9
        del mc, out, ws
    # decode logits on a 2.5-bit mixed key cache (the decode shape: 16 x 8 KV
    # heads x 131072 tokens, 4 query heads per KV head), keys N(0,1) in bf16
    H, T, QH = workloads.DEC_KV_HEADS, workloads.DEC_TOKENS, workloads.DEC_Q_PER_KV
    dsets = workloads.DEC_BATCH * H
    mc = tq.MixedCodec(d, 2, tq.TQ_MSE, 0, chans, groups=H)
    cache = mc.empty_codes(dsets, T)
    kb = torch.empty((8, T, d), dtype=torch.bfloat16, device="cuda")
    ws = mc.workspace(8, T)
    for s0 in range(0, dsets, 8):
        kb.copy_(torch.randn((8, T, d), generator=gen, device="cuda"))
        mc.quantize(kb, out=tuple({k: (None if v is None else v[s0:s0 + 8]) for k, v in p.items()} for p in cache),
                    workspace=ws)
    del kb, ws
    qd = torch.randn((dsets, QH, d), generator=gen, device="cuda")
    lo = torch.empty((dsets, QH, T), device="cuda")
    wsl = mc.workspace(dsets, T, QH)
    ms = _mean_launch_ms(torch, lambda: mc.logits(qd, cache, out=lo, workspace=wsl))
    kbytes = dsets * T * (mc.outlier.code_row + mc.regular.code_row + 8)
    res["decode_mixed_2.5bit_logits_ms"] = ms
    res["decode_mixed_2.5bit_logits_packed_gbs"] = kbytes / (ms * 1e-3) / 1e9
    res["decode_mixed_2.5bit_logits_total_gbs"] = (kbytes + dsets * QH * T * 4) / (ms * 1e-3) / 1e9
    del mc, cache, qd, lo, wsl
    if kv_only:
        return res
    centres = torch.randn((workloads.NN_CENTRES, workloads.NN_D), generator=gen, device="cuda")
    centres /= centres.norm(dim=1, keepdim=True)
    m = torch.randint(0, workloads.NN_CENTRES, (workloads.NN_POINTS,), generator=gen, device="cuda")
    pts = centres[m] + workloads.NN_STD * torch.randn((workloads.NN_POINTS, workloads.NN_D), generator=gen,
                                                      device="cuda")
    pts = (pts / pts.norm(dim=1, keepdim=True)).unsqueeze(0).contiguous()
    qs = centres[torch.randint(0, workloads.NN_CENTRES, (workloads.NN_QUERIES,), generator=gen, device="cuda")]
    qs = qs + workloads.NN_STD * torch.randn((workloads.NN_QUERIES, workloads.NN_D), generator=gen, device="cuda")
    qs = (qs / qs.norm(dim=1, keepdim=True)).contiguous()
    # exact fp32 top-1 of every query over the unquantized points (queries in chunks)
    true1 = torch.empty(workloads.NN_QUERIES, dtype=torch.int64, device="cuda")
    for a in range(0, workloads.NN_QUERIES, 500):
        true1[a:a + 500] = torch.argmax(qs[a:a + 500] @ pts[0].T, dim=1)
    ks = (1, 2, 4, 8, 16, 32, 64)
    for bits in (2, 4):
        codec = tq.Codec(workloads.NN_D, bits, tq.TQ_PROD, seed=0)
        out = codec.empty_codes(1, workloads.NN_POINTS)
        res[f"nn_index_d200_prod_b{bits}_ms"] = _mean_launch_ms(torch, lambda: codec.quantize(pts, out=out))
        keys = {k: (None if v is None else v[0]) for k, v in out.items()}
        sc, ix = codec.topk(qs, keys, 64)
        ms = _mean_launch_ms(torch, lambda: codec.topk(qs, keys, 64), reps=3)
        res[f"nn_search_d200_prod_b{bits}_top64_ms"] = ms
        res[f"nn_search_d200_prod_b{bits}_pairs_per_s"] = workloads.NN_QUERIES * workloads.NN_POINTS / (ms * 1e-3)
        hit = ix.long() == true1[:, None]
        first = torch.where(hit.any(dim=1), hit.float().argmax(dim=1), torch.full_like(true1, 1 << 30))
        res[f"nn_recall_at_1_at_k_prod_b{bits}"] = {str(k): float((first < k).float().mean()) for k in ks}
        del out, keys, sc, ix
    del pts, qs, true1
    res.update(generic_paths(torch, tq, gen))
    return res


def generic_paths(torch, tq, gen):
    """Logits of one set of 2^25 + 64 keys (the fused kernel in two chunks of
    keys), then the dimension-generic kernels on shapes the fast kernels hand
    over to them: logits at d = 200 (NN index keys), a top-64 search at d =
    300 (score-then-select), and the quantize, dequantize and logits of mse
    b = 5 at d = 128 (more than 4 bits).  Random codes stand in for
    quantized keys where only the streaming rate matters."""
    res = {}
    nk = (1 << 25) + 64
    c = tq.Codec(128, 4, tq.TQ_PROD, seed=0)
    keys = dict(codes=torch.randint(0, 256, (nk, c.code_row), dtype=torch.uint8, device="cuda", generator=gen),
                signs=torch.randint(0, 256, (nk, c.sign_row), dtype=torch.uint8, device="cuda", generator=gen),
                norms=torch.rand(nk, device="cuda", generator=gen) + 0.5,
                rnorms=torch.rand(nk, device="cuda", generator=gen) * 0.2)
    q = torch.randn((1, 4, 128), device="cuda", generator=gen)
    lo = torch.empty((1, 4, nk), device="cuda")
    cache = {k: v.unsqueeze(0) for k, v in keys.items()}
    ms = _mean_launch_ms(torch, lambda: c.logits(q, cache, out=lo), reps=3)
    res["long_set_logits_2p25_keys_prod_b4_ms"] = ms
    res["long_set_logits_2p25_keys_prod_b4_packed_gbs"] = nk * 72 / (ms * 1e-3) / 1e9
    del keys, cache, lo
    # d = 200 keys, prod b = 4: the generic logits kernel (one set of 1e6 keys, 64 queries)
    c = tq.Codec(200, 4, tq.TQ_PROD, seed=0)
    x = torch.randn((1, 1_000_000, 200), device="cuda", generator=gen)
    kc = c.empty_codes(1, 1_000_000)
    c.quantize(x, out=kc)
    q = torch.randn((1, 64, 200), device="cuda", generator=gen)
    lo = torch.empty((1, 64, 1_000_000), device="cuda")
    ms = _mean_launch_ms(torch, lambda: c.logits(q, kc, out=lo), reps=3)
    res["generic_logits_d200_prod_b4_64q_ms"] = ms
    res["generic_logits_d200_prod_b4_64q_packed_gbs"] = 1_000_000 * (c.code_row + c.sign_row + 8) / (ms * 1e-3) / 1e9
    del x, kc, q, lo
    # top-64 search at d = 300, prod b = 3 (past the fused scan's d <= 256): score-then-select through the
    # generic logits kernel, 1000 queries x 10^5 keys
    c = tq.Codec(300, 3, tq.TQ_PROD, seed=0)
    x = torch.randn((1, 100_000, 300), device="cuda", generator=gen)
    kc = c.empty_codes(1, 100_000)
    c.quantize(x, out=kc)
    keys = {k: (None if v is None else v[0]) for k, v in kc.items()}
    q = torch.randn((1000, 300), device="cuda", generator=gen)
    ms = _mean_launch_ms(torch, lambda: c.topk(q, keys, 64), reps=3)
    res["generic_topk_d300_prod_b3_1000q_100k_top64_ms"] = ms
    res["generic_topk_d300_prod_b3_pairs_per_s"] = 1000 * 100_000 / (ms * 1e-3)
    del x, kc, keys, q
    # mse b = 5 at d = 128 (KV shape, 16 sets x 32768): generic quantize, dequantize, logits
    c = tq.Codec(128, 5, tq.TQ_MSE, seed=0, groups=8)
    x = torch.randn((16, 32768, 128), device="cuda", generator=gen).to(torch.bfloat16)
    kc = c.empty_codes(16, 32768)
    ms = _mean_launch_ms(torch, lambda: c.quantize(x, out=kc))
    res["generic_quant_kv_mse_b5_ms"] = ms
    res["generic_quant_kv_mse_b5_vectors_per_s"] = 16 * 32768 / (ms * 1e-3)
    rec = torch.empty((16, 32768, 128), device="cuda")
    ms = _mean_launch_ms(torch, lambda: c.dequantize(kc, out=rec))
    res["generic_dequant_kv_mse_b5_ms"] = ms
    q = torch.randn((16, 4, 128), device="cuda", generator=gen)
    lo = torch.empty((16, 4, 32768), device="cuda")
    ms = _mean_launch_ms(torch, lambda: c.logits(q, kc, out=lo))
    res["generic_logits_kv_mse_b5_ms"] = ms
    res["generic_logits_kv_mse_b5_packed_gbs"] = 16 * 32768 * (c.code_row + 4) / (ms * 1e-3) / 1e9
    return res


def ceilings_phase(torch, tq):
    """Memory-system and matrix-core ceilings from the library's own probe
    kernels: streams over 1 GiB of input (each after a 1 GiB fill of another
    buffer, so no input is still held in the 256 MB Infinity Cache) at the
    read/write mixes of the hot-path kernels, and a matrix-core loop with no
    memory traffic.  GB/s count bytes read plus bytes written.  The 1:8 mix
    (the d = 128 dequantize's) reads 128 MiB, cold, and writes 1 GiB."""
    grid = 2048                                   # 8 workgroups of 4 waves per CU
    n_in = 1 << 30
    src = torch.empty(n_in // 4, dtype=torch.int32, device="cuda").fill_(0x1234567)
    dst = torch.empty(n_in // 4, dtype=torch.int32, device="cuda")
    evict = torch.empty(n_in // 4, dtype=torch.int32, device="cuda")
    ev = _events(torch, 2)
    res = {}
    kinds = (("copy", 0, 1, 1), ("mix_4r1w", 1, 4, 1), ("mix_9r2w", 2, 9, 2), ("read_only", 3, 1, 0),
             ("mix_9r2w_logits_rows", 4, 9, 2), ("mix_1r8w", 5, 1, 8))
    for name, kind, r, w in kinds:
        tile_in = r * 64 * 16
        cap = n_in if w <= r else n_in * r // w      # the 1:8 mix reads 128 MiB and writes 1 GiB
        used = cap // tile_in * tile_in
        moved = used + used // r * w
        times = []
        for rep in range(4):
            evict.fill_(rep)
            torch.cuda.synchronize()
            ev[0].record()
            tq.probe_stream(kind, src[:used // 4], dst, grid)
            ev[1].record()
            torch.cuda.synchronize()
            if rep:                                # the first launch loads the kernel
                times.append(ev[0].elapsed_time(ev[1]))
        ms = float(np.median(times))
        res[f"{name}_gbs"] = moved / (ms * 1e-3) / 1e9
        res[f"{name}_ms"] = ms
    del src, dst, evict
    out = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
    iters = 20000
    for name, f16 in (("bf16", False), ("f16", True)):
        tq.probe_mfma(f16, 16, grid, out)          # load the kernel
        torch.cuda.synchronize()
        ev[0].record()
        tq.probe_mfma(f16, iters, grid, out)
        ev[1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1])
        flops = grid * 4 * iters * 8 * 2.0 * 16 * 16 * 32
        res[f"mfma_{name}_tflops"] = flops / (ms * 1e-3) / 1e12
    del out
    res["issue"] = issue_probe(torch, tq)
    return res


def issue_probe(torch, tq):
    """What a SIMD issues with one wave (as the d = 128 quantize runs) and with
    two: 48 independent float FMAs, 16 bf16 MFMAs, or both interleaved per
    iteration, one workgroup per CU.  Rates come from events around the launch
    (ns per instruction per SIMD); `ghz` is the waves' own clock reading
    (shader counter over the 100 MHz real-time counter, median over waves),
    and cycles = ns x ghz."""
    grid, iters = 256, 4096
    ev = _events(torch, 2)
    res = {}
    for wps in (1, 2):
        out = torch.zeros(2 * grid * 4 * wps, dtype=torch.int32, device="cuda")
        for mode, name, instrs in ((0, "valu48", 48), (1, "mfma16", 16), (2, "mfma16_valu48", 64)):
            tq.probe_issue(mode, wps, 16, grid, out)   # load the kernel
            torch.cuda.synchronize()
            ev[0].record()
            tq.probe_issue(mode, wps, iters, grid, out)
            ev[1].record()
            torch.cuda.synchronize()
            ms = ev[0].elapsed_time(ev[1])
            d = out.view(-1, 2).cpu().numpy().astype(np.uint32).astype(np.float64)
            ghz = float(np.median(d[:, 0] / (d[:, 1] * 10.0)))
            ns = ms * 1e6 / (iters * instrs * wps)              # per instruction per SIMD
            res[f"{name}_{wps}w"] = dict(ns_per_instr=round(ns, 3), ghz=round(ghz, 3),
                                         cycles_per_instr=round(ns * ghz, 2))
        del out
    res["note"] = ("per SIMD: valu48 = 48 independent float FMAs, mfma16 = 16 bf16 16x16x32 MFMAs, "
                   "mfma16_valu48 = both, one MFMA then three FMAs; 1w / 2w = waves per SIMD; event-timed")
    return res


def dense_logits_phase(torch, tq, workloads, steps, warmup, q):
    """The dense baseline at the decode shape: the same 16 x 8 x 131072 keys
    stored unquantized in float16 (the named comparison) and in float32 (the
    pages' 32-bit comparison), the same 32 query heads, float32 logits."""
    B, H, QH, T, d = (workloads.DEC_BATCH, workloads.DEC_KV_HEADS, workloads.DEC_Q_PER_KV,
                      workloads.DEC_TOKENS, workloads.DEC_DIM)
    sets = B * H
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4)
    out = torch.empty((sets, QH, T), dtype=torch.float32, device="cuda")
    res = {}
    for name, dtype in (("f16", torch.float16), ("f32", torch.float32)):
        keys = torch.empty((sets, T, d), dtype=dtype, device="cuda")
        for s0 in range(0, sets, 8):
            keys[s0:s0 + 8] = torch.randn((8, T, d), generator=gen, device="cuda").to(dtype)
        wall, kern, kmed = time_launches(torch, lambda i: tq.dense_logits(q, keys, out=out), steps, warmup, 1)
        kbytes = sets * T * d * keys.element_size()
        res[name] = dict(kernel_ms=kern, kernel_ms_median=kmed, wall_ms=wall, key_bytes=kbytes,
                         gbs=kbytes / (kern * 1e-3) / 1e9,
                         total_gbs=(kbytes + sets * QH * T * 4) / (kern * 1e-3) / 1e9)
        del keys
    del out
    return res


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return os.cpu_count() or 1


def _kv_quantize_rate(O, cd, xf, budget_s):
    """Oracle TurboQuant_mse b = 4 over the KV vectors in 8192-vector chunks
    (norm, rotate, boundary search, pack) for about budget_s."""
    done, t0, rows = 0, time.perf_counter(), 8192
    sets, n = xf.shape[0], xf.shape[1]
    while time.perf_counter() - t0 < budget_s and done < sets * n:
        s = (done // rows) % sets
        off = (done // (rows * sets)) * rows
        chunk = xf[s, off:off + rows].astype(np.float64)
        idx, nu, _ = O.quantize_mse(cd, chunk, s % cd.groups)
        O.pack(idx, 4)
        done += chunk.shape[0]
    return done, time.perf_counter() - t0


def _random_prod_keys(rng, n, d, mse_bits):
    return dict(idx=rng.integers(0, 1 << mse_bits, (n, d)), signs=np.where(rng.random((n, d)) < 0.5, -1, 1),
                norms=10.0 + rng.standard_normal(n), rnorms=0.05 + 0.45 * rng.random(n))


def cpu_baseline(workloads, x_bf16, budget_s=8.0):
    """The oracle (float64 NumPy, BLAS threads as the host gives them) timed on
    bounded samples of the workloads, beside the GPU figures of the same run.
    `value` is the headline leg (the KV quantize, vectors/s); the other legs
    time the oracle's fast logits form (rotated-domain inner products, equal to
    the plain form up to rounding) on the decode and nearest-neighbour shapes
    in 65,536-key chunks, and the d = 1536 quantize.  Inputs are seeded
    synthetic draws (random codes for the logits legs).  Totals for the full
    workloads are extrapolated linearly from the samples and labelled so."""
    from oracle import tq_oracle as O

    threads = _blas_threads()
    xf = x_bf16.float().numpy()
    cd = O.make_codec(128, 4, O.MSE, 0, groups=workloads.KV_HEADS)
    done, el = _kv_quantize_rate(O, cd, xf, budget_s)
    legs = {}
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            d1, e1 = _kv_quantize_rate(O, cd, xf, 3.0)
        legs["kv_quantize_single_thread_vectors_per_s"] = d1 / e1
    except Exception:
        pass
    rng = np.random.default_rng(11)
    # decode logits: prod b = 4 keys, 4 query heads per set, 65,536-key chunks
    kd = O.make_codec(128, 4, O.PROD, 0, groups=workloads.DEC_KV_HEADS)
    chunk, keys_done, t0 = 65536, 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        s = (keys_done // chunk) % (workloads.DEC_BATCH * workloads.DEC_KV_HEADS)
        keys = _random_prod_keys(rng, chunk, 128, 3)
        q = rng.standard_normal((workloads.DEC_Q_PER_KV, 128))
        O.logits_fast(kd, q, keys, s % kd.groups)
        keys_done += chunk
    el_l = time.perf_counter() - t0
    total_keys = workloads.DEC_BATCH * workloads.DEC_KV_HEADS * workloads.DEC_TOKENS
    legs["decode_logits"] = dict(keys_per_s=keys_done / el_l, packed_gbs=keys_done * 72 / el_l / 1e9,
                                 extrapolated_full_ms=total_keys / (keys_done / el_l) * 1e3,
                                 sample=f"{keys_done} keys (prod b=4, 4 heads) in {el_l:.1f} s")
    # high-dimensional quantize, d = 1536, mse b = 4
    hd = O.make_codec(1536, 4, O.MSE, 0)
    xh = workloads.highd_vectors(2000, 1536)
    t0 = time.perf_counter()
    idx, _, _ = O.quantize_mse(hd, xh.astype(np.float64))
    O.pack(idx, 4)
    el_h = time.perf_counter() - t0
    legs["highd_d1536_mse_b4"] = dict(vectors_per_s=2000 / el_h, extrapolated_1e5_s=1e5 / (2000 / el_h),
                                      sample="2000 of the 100000 vectors")
    # nearest-neighbour scoring: 100 queries x 1e6 prod b = 4 keys at d = 200
    nd = O.make_codec(workloads.NN_D, 4, O.PROD, 0)
    qn = rng.standard_normal((100, workloads.NN_D))
    t0 = time.perf_counter()
    for a in range(0, workloads.NN_POINTS, chunk):
        n = min(chunk, workloads.NN_POINTS - a)
        O.logits_fast(nd, qn, _random_prod_keys(rng, n, workloads.NN_D, 3))
    el_n = time.perf_counter() - t0
    pairs = 100 * workloads.NN_POINTS
    legs["nn_scoring_d200_prod_b4"] = dict(pairs_per_s=pairs / el_n,
                                           extrapolated_1e4_queries_s=el_n * workloads.NN_QUERIES / 100,
                                           sample="100 queries x 1e6 keys, extrapolated linearly to 1e4 queries")
    return dict(value=done / el, unit="vectors/s", cores=int(threads), host_cpu_count=os.cpu_count(),
                kind="oracle",
                sample=f"{done} of the {xf.shape[0] * xf.shape[1]} KV vectors (mse b=4: norm, rotate, "
                       f"boundary search, pack) in {el:.1f} s",
                legs=legs)


def main():
    args = _parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1 "
                                   "(the multi-GPU sharding is described in DESIGN.md, not built)"}))
        sys.exit(2)
    import torch

    import kv_cache_compression_tq_amd as tq
    import workloads

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    qp = quantize_phase(torch, tq, workloads, args.steps, args.warmup)
    q3 = quantize_b3_phase(torch, tq, workloads, qp["x"], args.steps, args.warmup)
    lp = None if args.skip_logits else logits_phase(torch, tq, workloads, args.steps, args.warmup)
    ap = None if (lp is None or args.skip_attention) else attention_phase(torch, tq, workloads, lp, args.steps,
                                                                          args.warmup)
    if lp is not None:
        qdec = lp["q"]
        del lp["cache"], lp["codec"], lp["q"]
        dense = None if args.skip_dense else dense_logits_phase(torch, tq, workloads, args.steps, args.warmup, qdec)
        del qdec
    else:
        dense = None
    other = None if args.skip_others else other_paths_phase(torch, tq, workloads, qp["x"], args.kv_only)
    ceil = None if args.skip_ceilings else ceilings_phase(torch, tq)
    cpu = None if args.no_cpu_baseline else cpu_baseline(workloads, qp["x"])
    probes = hbm_probes(torch) if args.copy_probe else None
    peak_meas = ceil["copy_gbs"] if ceil else None

    value = qp["vectors"] / (qp["wall_ms"] * 1e-3)
    line = {
        "metric": "quantized vectors/s and q·K̂ logit GB/s (d=128, b=4) vs MI355X HBM roofline",
        "value": value,
        "unit": "vectors/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": qp["wall_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "KV-cache quantize, K+V of one Llama-3.1-8B-shaped layer: 2 x 8 KV heads x "
                               "32768 tokens x 128, bf16, 4 outlier channels/head x10, TurboQuant_mse b=4, "
                               "one rotation per head",
                   "vectors_per_step": qp["vectors"], "d": 128, "bits": 4, "variant": "mse"},
        "roofline": {"bound": "hbm", "kernel": "k_quant128_mse<4>", "achieved": qp["achieved_gbs"],
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": qp["achieved_gbs"] / HBM_PEAK_GBS,
                     "traffic": counted_traffic("quant128_kv_mse_b4.md"),
                     "bytes_per_vector": qp["bytes_per_vector"],
                     "kernel_ms": qp["kernel_ms"],
                     "measured_peak": peak_meas,
                     "measured_peak_kind": "in-tree copy kernel, 1 GiB read + 1 GiB written, cold",
                     "frac_measured": qp["achieved_gbs"] / peak_meas if peak_meas else None,
                     "mix_ceiling": ceil["mix_4r1w_gbs"] if ceil else None,
                     "frac_of_mix_ceiling": qp["achieved_gbs"] / ceil["mix_4r1w_gbs"] if ceil else None,
                     "warm": {"kernel_ms": qp["kernel_ms_warm"], "achieved": qp["achieved_gbs_warm"],
                              "note": "one resident input, held in the 256 MB Infinity Cache"},
                     "mfma": {"dtype": "bf16", "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                              "measured_peak": ceil["mfma_bf16_tflops"] if ceil else None,
                              "algorithmic": qp["mfma_algo_tflops"],
                              "algorithmic_frac": qp["mfma_algo_tflops"] / BF16_MFMA_PEAK_TFLOPS,
                              "executed": qp["mfma_exec_tflops"],
                              "executed_frac": qp["mfma_exec_tflops"] / BF16_MFMA_PEAK_TFLOPS,
                              "note": "algorithmic = 2 d^2 flop per vector (y = Pi x); executed = the two split "
                                      "passes (Pi hi, Pi lo) plus the Gram product for the norm"}},
        "quantize_b3": {"kernel_ms": q3["kernel_ms"], "vectors_per_s": q3["vectors_per_s"],
                        "achieved_gbs": q3["achieved_gbs"], "frac": q3["achieved_gbs"] / HBM_PEAK_GBS},
    }
    if lp is not None:
        line["logits"] = {
            "metric": "q·K̂ logit GB/s on packed-code bytes",
            "value": lp["packed_gbs"], "unit": "GB/s", "ms_per_step": lp["wall_ms"],
            "config": {"workload": "decode attention logits: 16 batch x 8 KV heads x 131072 cached tokens, "
                                   "TurboQuant_prod b=4 (3-bit mse + 1-bit QJL), 32 query heads (4 per KV head), "
                                   "fp32 queries and logits", "keys": lp["keys"]},
            "roofline": {"bound": "hbm", "kernel": "k_logits128<3,prod>", "achieved": lp["packed_gbs"],
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": lp["packed_gbs"] / HBM_PEAK_GBS,
                         "traffic": counted_traffic("logits128_decode_prod_b4.md"),
                         "kernel_ms": lp["kernel_ms"],
                         "achieved_incl_logits_written": lp["total_gbs"],
                         "frac_incl_logits_written": lp["total_gbs"] / HBM_PEAK_GBS,
                         "measured_peak": peak_meas,
                         "frac_measured": lp["packed_gbs"] / peak_meas if peak_meas else None,
                         "mix_ceiling": ceil["mix_9r2w_logits_rows_gbs"] if ceil else None,
                         "mix_ceiling_kind": "in-tree stream, 72 B read + 16 B written per key, the kernel's "
                                             "4-byte four-row stores; GB/s on all bytes",
                         "frac_incl_logits_written_of_mix_ceiling":
                             lp["total_gbs"] / ceil["mix_9r2w_logits_rows_gbs"] if ceil else None},
            "cache_build_s": lp["cache_build_s"],
        }
        if dense is not None:
            line["logits"]["dense_baseline"] = {
                name: {"kernel": f"k_dense_logits128<{name}>", "kernel_ms": r["kernel_ms"],
                       "key_gbs": r["gbs"], "total_gbs": r["total_gbs"],
                       "frac_incl_logits_written": r["total_gbs"] / HBM_PEAK_GBS,
                       "quantized_speedup": r["kernel_ms"] / lp["kernel_ms"]}
                for name, r in dense.items()}
    if ap is not None:
        line["attention"] = {
            "metric": "softmax(q·K̂)·V̂ GB/s on packed K and V bytes",
            "value": ap["packed_gbs"], "unit": "GB/s", "ms_per_step": ap["wall_ms"],
            "config": {"workload": "decode attention: 16 batch x 8 KV heads x 131072 cached tokens, keys "
                                   "TurboQuant_prod b=4, values TurboQuant_mse b=4, 32 query heads (4 per KV "
                                   "head), fp32 queries and outputs, scale 1/sqrt(128)", "keys": ap["keys"]},
            "roofline": {"bound": "hbm", "kernel": "k_attn128<3,prod,4>", "achieved": ap["packed_gbs"],
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ap["packed_gbs"] / HBM_PEAK_GBS,
                         "traffic": counted_traffic("attn128_decode_prod4_mse4.md"),
                         "kernel_ms": ap["kernel_ms"], "bytes_per_key": ap["packed_bytes"] / ap["keys"]},
            "workspace_bytes": ap["workspace_bytes"],
        }
        line["append"] = {
            "metric": "online append latency: one new key (prod b=4) and value (mse b=4) per (batch, KV head) "
                      "written into the paged decode caches",
            "value": ap["append_ms"] * 1e3, "unit": "us per token step (K + V, 128 sets)",
            "higher_is_better": False, "wall_us_per_step": ap["append_wall_ms"] * 1e3,
            "vectors_per_s": 2 * ap["sets"] / (ap["append_ms"] * 1e-3),
        }
    if other is not None:
        if ceil is not None:   # the d = 128 dequantize against the stream with its 1:8 read/write mix
            for v in ("mse", "prod"):
                k = f"kv_{v}_b4_dequantize_gbs"
                if k in other:
                    other[f"kv_{v}_b4_dequantize_frac_of_mix_ceiling"] = other[k] / ceil["mix_1r8w_gbs"]
        line["other_paths"] = other
    if ceil is not None:
        line["ceilings"] = dict(ceil, note="in-tree probe kernels (probes.hip): 1 GiB streams (the 1:8 mix: 128 MiB read), cold, GB/s on "
                                           "bytes read + written; MFMA loops with no memory traffic")
    if probes is not None:
        line["hbm_probes"] = probes
    line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
