"""Failure handling forced from the host (no kernel is made to fail): the
TQ_FAULT hooks drive the TQ_ENOMEM path of tq_init and the TQ_EHIP path of
every data call, and the library recovers once they are cleared."""
import os

import numpy as np
import pytest
import torch

import kv_cache_compression_tq_amd as tq

pytestmark = pytest.mark.gpu


@pytest.fixture
def fault():
    def set_(kind):
        os.environ["TQ_FAULT"] = kind

    yield set_
    os.environ.pop("TQ_FAULT", None)


def test_init_allocation_failure_returns_enomem_and_leaks_nothing(fault):
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    fault("alloc")
    for args in ((128, 4, tq.TQ_PROD, 1), (200, 3, tq.TQ_MSE, 2), (1536, 2, tq.TQ_PROD, 1)):
        with pytest.raises(tq.TQError) as e:
            tq.Codec(args[0], args[1], args[2], seed=0, groups=args[3])
        assert e.value.status == tq.TQ_ENOMEM
        assert "TQ_FAULT=alloc" in str(e.value)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0, "a failed init kept device memory"
    os.environ.pop("TQ_FAULT")
    c = tq.Codec(128, 4, tq.TQ_PROD, seed=0)
    assert c.code_row == 48


def test_launch_failure_returns_ehip_before_anything_is_enqueued(fault):
    d, n = 128, 256
    kc = tq.Codec(d, 4, tq.TQ_PROD, seed=1)
    vc = tq.Codec(d, 4, tq.TQ_MSE, seed=2)
    x = torch.randn((1, n, d), device="cuda")
    q = torch.randn((1, 4, d), device="cuda")
    keys, vals = kc.quantize(x), vc.quantize(x)
    torch.cuda.synchronize()
    out_codes = {k: (None if v is None else v.clone().fill_(0)) for k, v in keys.items()}
    lg = torch.full((1, 4, n), 7.0, device="cuda")
    rec = torch.full((1, n, d), 7.0, device="cuda")
    att = torch.full((1, 4, d), 7.0, device="cuda")
    fault("launch")
    calls = [
        lambda: kc.quantize(x, out=out_codes),
        lambda: kc.logits(q, keys, out=lg),
        lambda: kc.dequantize(keys, out=rec),
        lambda: kc.attention(q, keys, vc, vals, out=att),
        lambda: kc.attention_static(q, keys, vc, vals, out=att),
        lambda: kc.append(x[0, :1], torch.zeros(1, dtype=torch.int64, device="cuda"),
                          {k: (None if v is None else v[0]) for k, v in out_codes.items()}),
        lambda: kc.topk(q[0], {k: (None if v is None else v[0]) for k, v in keys.items()}, 4),
        lambda: tq.dense_logits(q, x.half(), out=lg),
    ]
    for i, call in enumerate(calls):
        with pytest.raises(tq.TQError) as e:
            call()
        assert e.value.status == tq.TQ_EHIP, i
        assert "TQ_FAULT=launch" in str(e.value), i
    torch.cuda.synchronize()
    assert all(v is None or not v.any() for v in out_codes.values())
    assert torch.all(lg == 7.0) and torch.all(rec == 7.0) and torch.all(att == 7.0)
    mc = tq.MixedCodec(d, 2, tq.TQ_MSE, 3, np.arange(64)[None, :])
    with pytest.raises(tq.TQError) as e:
        mc.quantize(x.to(torch.bfloat16))
    assert e.value.status == tq.TQ_EHIP
    os.environ.pop("TQ_FAULT")
    again = kc.quantize(x, out=out_codes)
    torch.cuda.synchronize()
    for k, v in keys.items():
        if v is not None:
            assert torch.equal(again[k], v), k
