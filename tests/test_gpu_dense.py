"""GPU parity of the dense baseline (logits of unquantized float16 / float32
keys, the comparison the pages draw against 4-bit codes) against the plain
float64 dot product of the same values, and of the measurement probes'
arithmetic (what the stream kernels write)."""
import numpy as np
import pytest
import torch

import kv_cache_compression_tq_amd as tq
from parity import check_rows

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
@pytest.mark.parametrize("n_sets,nq,n_keys", [(3, 4, 1000), (2, 11, 4096), (1, 1, 63), (5, 8, 131)])
def test_dense_logits_match_the_plain_dot_product(dtype, n_sets, nq, n_keys):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(n_keys + nq)
    keys = torch.randn((n_sets, n_keys, 128), device="cuda", generator=gen).to(dtype)
    q = torch.randn((n_sets, nq, 128), device="cuda", generator=gen)
    out = tq.dense_logits(q, keys).cpu().numpy()
    k64 = keys.float().cpu().numpy().astype(np.float64)
    q64 = q.cpu().numpy().astype(np.float64)
    # float16 keys enter the MFMA exactly and the query's hi/lo f16 split
    # keeps 22 bits: 1e-5 of the row.  float32 keys and queries are both split
    # into bf16 hi/lo parts (about 2^-16 per product): 1e-4.
    tol = 1e-5 if dtype == torch.float16 else 1e-4
    for s in range(n_sets):
        check_rows(out[s], q64[s] @ k64[s].T, f"dense {dtype} set {s}", tol=tol)


def test_dense_logits_decode_shape_sampled():
    """The decode shape (128 sets x 4 heads x 131072 float16 keys): sampled
    keys of a few sets against the plain product."""
    sets, nq, T = 128, 4, 131072
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3)
    keys = torch.randn((sets, T, 128), device="cuda", generator=gen).to(torch.float16)
    q = torch.randn((sets, nq, 128), device="cuda", generator=gen)
    out = tq.dense_logits(q, keys)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    for s in rng.choice(sets, 6, replace=False):
        kt = torch.from_numpy(np.sort(rng.choice(T, 500, replace=False))).cuda()
        ref = q[s].cpu().numpy().astype(np.float64) @ keys[s, kt].float().cpu().numpy().astype(np.float64).T
        check_rows(out[s][:, kt].cpu().numpy(), ref, f"set {s}", tol=1e-5)


def test_stream_probes_write_the_xor_of_what_they_read():
    """Kinds 0-2 and 5 write, for every 64-unit tile, the XOR of the R words a lane
    read (plus the output word's index in its unit): checked on the host."""
    for kind, (r, w) in ((0, (1, 1)), (1, (4, 1)), (2, (9, 2)), (5, (1, 8))):
        tiles = 7
        src = torch.randint(0, 2 ** 31 - 1, (tiles * r * 64 * 4,), dtype=torch.int32, device="cuda")
        dst = torch.zeros((tiles * w * 64 * 4,), dtype=torch.int32, device="cuda")
        tq.probe_stream(kind, src, dst, grid=2)
        torch.cuda.synchronize()
        a = src.cpu().numpy().view(np.uint32).reshape(tiles, r, 64, 4)
        acc = np.bitwise_xor.reduce(a, axis=1)
        want = np.stack([acc + np.uint32(j) for j in range(w)], axis=1)
        assert np.array_equal(dst.cpu().numpy().view(np.uint32).reshape(tiles, w, 64, 4), want), kind


def test_issue_probe_reports_cycles_and_clock_per_wave():
    """Every wave of every mode writes its loop's shader cycles and real-time
    ticks; more iterations take proportionally more cycles, and the clock they
    imply lies within the chip's range."""
    grid = 8
    for wps in (1, 2):
        for mode in (0, 1, 2):
            res = []
            for iters in (256, 1024):
                out = torch.zeros(2 * grid * 4 * wps, dtype=torch.int32, device="cuda")
                tq.probe_issue(mode, wps, iters, grid, out)
                torch.cuda.synchronize()
                d = out.view(-1, 2).cpu().numpy().astype(np.uint32).astype(np.float64)
                assert np.all(d[:, 0] > 0) and np.all(d[:, 1] > 0), (mode, wps)
                ghz = d[:, 0] / (d[:, 1] * 10.0)
                assert np.all((ghz > 0.3) & (ghz < 4.0)), (mode, wps, ghz.min(), ghz.max())
                res.append(np.median(d[:, 0]))
            assert 2.5 < res[1] / res[0] < 5.5, (mode, wps, res)


def test_issue_probe_rejects_bad_arguments():
    out = torch.zeros(64, dtype=torch.int32, device="cuda")
    for args in ((3, 1, 16, 1), (0, 0, 16, 1), (0, 3, 16, 1), (0, 1, -1, 1), (0, 1, 16, 0), (0, 1, 16, 5000)):
        with pytest.raises(tq.TQError):
            tq.probe_issue(*args, out)
