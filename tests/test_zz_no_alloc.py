"""tq_attention_static, the attention entry point for callers that cannot
allocate device memory: through the C ABI, against tq_attention with a caller
workspace (the same kernels; the d = 128 kernel sums its blocks in a
run-dependent order, so the two agree to float32 rounding, checked at 1e-5 of
each row, a hundred times inside the parity bar), on two calls in a row (the
second smaller), with no device memory allocated by the call, and its
rejection of a shape whose workspace exceeds the fixed array."""
import ctypes

import numpy as np
import pytest
import torch

import kv_cache_compression_tq_amd as tq
from parity import check_rows

pytestmark = pytest.mark.gpu


def _cache(codec, n_sets, n_keys, gen):
    x = torch.randn((n_sets, n_keys, codec.d), device="cuda", generator=gen)
    return codec.quantize(x)


def _static_call(kc, vc, q, keys, vals, scale, out):
    n_sets, n_keys = keys["norms"].shape

    def p(t):
        return None if t is None else ctypes.c_void_p(t.data_ptr())

    return tq.lib().tq_attention_static(
        kc.handle, vc.handle, p(q), q.shape[1], p(keys.get("codes")), p(keys.get("signs")), p(keys["norms"]),
        p(keys.get("rnorms")), p(vals.get("codes")), p(vals.get("signs")), p(vals["norms"]), p(vals.get("rnorms")),
        n_sets, n_keys, ctypes.c_float(scale), p(out), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


# (d, key bits, key variant, value bits, value variant, [(n_sets, nq, n_keys) per call, the second smaller])
CASES = [
    (128, 4, tq.TQ_PROD, 4, tq.TQ_MSE, [(16, 4, 40000), (3, 2, 777)]),   # fused d = 128 kernels
    (96, 3, tq.TQ_PROD, 2, tq.TQ_PROD, [(4, 3, 9000), (2, 1, 130)]),     # any-d kernels
]


@pytest.mark.parametrize("d,kb,kv,vb,vv,calls", CASES)
def test_static_attention_matches_the_workspace_entry_point(d, kb, kv, vb, vv, calls):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(d + kb)
    kc = tq.Codec(d, kb, kv, seed=1, groups=2)
    vc = tq.Codec(d, vb, vv, seed=2, groups=2)
    scale = d ** -0.5
    for n_sets, nq, n_keys in calls:
        keys, vals = _cache(kc, n_sets, n_keys, gen), _cache(vc, n_sets, n_keys, gen)
        q = torch.randn((n_sets, nq, d), device="cuda", generator=gen)
        ref = kc.attention(q, keys, vc, vals, scale=scale)
        out = torch.full_like(ref, float("nan"))
        torch.cuda.synchronize()
        free_before = torch.cuda.mem_get_info()[0]
        st = _static_call(kc, vc, q, keys, vals, scale, out)
        torch.cuda.synchronize()
        free_after = torch.cuda.mem_get_info()[0]
        assert st == tq.TQ_OK, tq.lib().tq_last_error()
        check_rows(out.cpu().numpy(), ref.cpu().numpy(), f"{(n_sets, nq, n_keys)}: static workspace", tol=1e-5)
        assert free_after == free_before, "the call allocated device memory"
        # the binding's method reaches the same entry point
        again = kc.attention_static(q, keys, vc, vals, scale=scale)
        torch.cuda.synchronize()
        check_rows(again.cpu().numpy(), ref.cpu().numpy(), "binding method", tol=1e-5)


def test_static_attention_rejects_a_workspace_beyond_the_array():
    """The any-d kernels keep every logit in the workspace: 2 sets x 8 heads x
    300000 keys needs 19.2 MB > 16 MiB, so the call fails with TQ_EINVAL
    before enqueuing anything (the output keeps its contents)."""
    d, n_sets, nq, n_keys = 96, 2, 8, 300000
    kc = tq.Codec(d, 2, tq.TQ_MSE, seed=3)
    vc = tq.Codec(d, 2, tq.TQ_MSE, seed=4)
    need = kc.attention_workspace_bytes(vc, nq, n_sets, n_keys)
    assert need > (16 << 20)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    keys, vals = _cache(kc, n_sets, n_keys, gen), _cache(vc, n_sets, n_keys, gen)
    q = torch.randn((n_sets, nq, d), device="cuda", generator=gen)
    out = torch.full((n_sets, nq, d), 7.0, device="cuda")
    st = _static_call(kc, vc, q, keys, vals, 0.1, out)
    torch.cuda.synchronize()
    assert st == tq.TQ_EINVAL
    assert b"static workspace" in tq.lib().tq_last_error()
    assert torch.all(out == 7.0)
