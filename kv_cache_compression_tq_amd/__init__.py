"""Python binding of libtq.so, the TurboQuant hot path for AMD MI355X.

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch provides device memory and the current stream.  Importing this
package does not load the library; the first call does, and it raises if the
built library is missing (there is no fallback).
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["Codec", "MixedCodec", "lib", "library_path", "TQ_MSE", "TQ_PROD", "TQ_F32", "TQ_BF16", "TQ_F16",
           "TQError", "EXPORTED_SYMBOLS", "row_bytes", "dense_logits", "probe_stream", "probe_mfma",
           "probe_issue"]

TQ_MSE, TQ_PROD = 0, 1
TQ_F32, TQ_BF16, TQ_F16 = 0, 1, 2
TQ_OK, TQ_EINVAL, TQ_EUNSUPPORTED, TQ_ENOMEM, TQ_EHIP = 0, -1, -2, -3, -4

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int
_SIGS = {
    "tq_init": (_INT, [_INT, _INT, _INT, ctypes.c_uint64, ctypes.POINTER(_P)]),
    "tq_init_groups": (_INT, [_INT, _INT, _INT, ctypes.c_uint64, _INT, ctypes.POINTER(_P)]),
    "tq_destroy": (_INT, [_P]),
    "tq_layout": (_INT, [_P, ctypes.POINTER(_I64), ctypes.POINTER(_I64), ctypes.POINTER(_INT)]),
    "tq_quantize": (_INT, [_P, _P, _INT, _I64, _I64, _P, _P, _P, _P, _P]),
    "tq_dequantize": (_INT, [_P, _P, _P, _P, _P, _I64, _I64, _P, _P]),
    "tq_append": (_INT, [_P, _P, _INT, _I64, _P, _I64, _P, _P, _P, _P, _P]),
    "tq_logits": (_INT, [_P, _P, _I64, _P, _P, _P, _P, _I64, _I64, _P, _P]),
    "tq_attention": (_INT, [_P, _P, _P, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, ctypes.c_float, _P, _P,
                            ctypes.c_size_t, _P]),
    "tq_attention_workspace": (_INT, [_P, _P, _I64, _I64, _I64, ctypes.POINTER(ctypes.c_size_t)]),
    "tq_attention_static": (_INT, [_P, _P, _P, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, ctypes.c_float,
                                   _P, _P]),
    "tq_topk_workspace": (_INT, [_P, _I64, _I64, _INT, ctypes.POINTER(ctypes.c_size_t)]),
    "tq_topk": (_INT, [_P, _P, _I64, _P, _P, _P, _P, _I64, _INT, _P, _P, _P, ctypes.c_size_t, _P]),
    "tq_mixed_init": (_INT, [_INT, _INT, _INT, ctypes.c_uint64, _INT, _INT, _P, ctypes.POINTER(_P)]),
    "tq_mixed_destroy": (_INT, [_P]),
    "tq_mixed_parts": (_INT, [_P, ctypes.POINTER(_P), ctypes.POINTER(_P)]),
    "tq_mixed_workspace": (_INT, [_P, _I64, _I64, _I64, ctypes.POINTER(ctypes.c_size_t)]),
    "tq_mixed_quantize": (_INT, [_P, _P, _INT, _I64, _I64, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "tq_mixed_dequantize": (_INT, [_P, _P, _P, _P, _P, _I64, _I64, _P, _P, ctypes.c_size_t, _P]),
    "tq_mixed_logits": (_INT, [_P, _P, _I64, _P, _P, _P, _P, _I64, _I64, _P, _P, ctypes.c_size_t, _P]),
    "tq_dense_logits": (_INT, [_P, _I64, _P, _INT, _INT, _I64, _I64, _P, _P]),
    "tq_probe_stream": (_INT, [_INT, _P, _I64, _P, _I64, _INT, _P]),
    "tq_probe_mfma": (_INT, [_INT, _I64, _INT, _P, _P]),
    "tq_probe_issue": (_INT, [_INT, _INT, _I64, _INT, _P, _P]),
    "tq_strerror": (ctypes.c_char_p, [_INT]),
    "tq_last_error": (ctypes.c_char_p, []),
    "tq_get_tables": (_INT, [_P, _INT, _P, _P, _P, _P]),
    "tq_host_tables": (_INT, [_INT, _INT, _INT, ctypes.c_uint64, _INT, _P, _P, _P, _P]),
    "tq_pack": (_INT, [_P, _P, _INT, _I64, _P, _P]),
    "tq_unpack": (_INT, [_P, _P, _INT, _I64, _P, _P]),
}
EXPORTED_SYMBOLS = tuple(_SIGS)


class TQError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status}: {detail}")
        self.status = status


def library_path() -> str:
    return os.environ.get("TQ_LIBRARY", os.path.join(_HERE, "libtq.so"))


def lib() -> ctypes.CDLL:
    """Load libtq.so (once).  Raises FileNotFoundError when it is not built."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise FileNotFoundError(f"{path} is not built: run `python -m kv_cache_compression_tq_amd.build`")
        L = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def _check(status: int, where: str) -> None:
    if status != TQ_OK:
        detail = lib().tq_last_error().decode() or lib().tq_strerror(status).decode()
        raise TQError(status, where, detail)


def row_bytes(count: int, bits: int) -> int:
    return ((count * bits + 7) // 8 + 15) // 16 * 16


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class Codec:
    """A TurboQuant codec: d dimensions, b bits, variant TQ_MSE / TQ_PROD.

    Data methods take CUDA (HIP) torch tensors and enqueue on the current
    stream; outputs are allocated here with torch unless given.
    """

    def __init__(self, d: int, bits: int, variant: int = TQ_MSE, seed: int = 0, groups: int = 1, _borrowed=None):
        self.d, self.bits, self.variant, self.seed, self.groups = d, bits, variant, seed, groups
        if _borrowed is None:
            h = ctypes.c_void_p()
            _check(lib().tq_init_groups(d, bits, variant, seed, groups, ctypes.byref(h)), "tq_init_groups")
            self._owned = True
        else:  # a part codec owned by a MixedCodec
            h = _borrowed
            self._owned = False
        self._h = h
        cr, sr, mb = _I64(), _I64(), _INT()
        _check(lib().tq_layout(self._h, ctypes.byref(cr), ctypes.byref(sr), ctypes.byref(mb)), "tq_layout")
        self.code_row, self.sign_row, self.mse_bits = cr.value, sr.value, mb.value

    def close(self) -> None:
        if getattr(self, "_h", None):
            if getattr(self, "_owned", True):
                lib().tq_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def handle(self):
        return self._h

    # -- storage -----------------------------------------------------------
    def empty_codes(self, n_sets: int, n: int, device="cuda"):
        import torch

        codes = torch.zeros((n_sets, n, self.code_row), dtype=torch.uint8, device=device) if self.code_row else None
        norms = torch.empty((n_sets, n), dtype=torch.float32, device=device)
        signs = rnorms = None
        if self.variant == TQ_PROD:
            signs = torch.empty((n_sets, n, self.sign_row), dtype=torch.uint8, device=device)
            rnorms = torch.empty((n_sets, n), dtype=torch.float32, device=device)
        return dict(codes=codes, signs=signs, norms=norms, rnorms=rnorms)

    # -- hot path ----------------------------------------------------------
    def quantize(self, x, out=None, stream=None):
        """x: [n_sets, n, d] (or [n, d]) float32 or bfloat16 CUDA tensor."""
        import torch

        if x.dim() == 2:
            x = x.unsqueeze(0)
        if not x.is_contiguous():
            raise ValueError("x must be contiguous")
        dtype = {torch.float32: TQ_F32, torch.bfloat16: TQ_BF16}.get(x.dtype)
        if dtype is None:
            raise TypeError("x must be float32 or bfloat16")
        n_sets, n, d = x.shape
        if d != self.d:
            raise ValueError(f"last dimension {d} != codec d {self.d}")
        out = out or self.empty_codes(n_sets, n, x.device)
        _check(lib().tq_quantize(self._h, _ptr(x), dtype, n_sets, n, _ptr(out["codes"]), _ptr(out["signs"]),
                                 _ptr(out["norms"]), _ptr(out["rnorms"]), _stream(stream)), "tq_quantize")
        return out

    def append(self, x, rows, cache, stream=None):
        """Quantize x[n_sets, d] (float32 or bfloat16) and write set s's vector
        into row rows[s] (int64 CUDA tensor) of the cache dict (arrays shaped
        [cache_rows, ...] as empty_codes(1, cache_rows) returns, or any
        contiguous arrays with cache_rows rows)."""
        import torch

        if x.dim() != 2 or x.shape[1] != self.d or not x.is_contiguous():
            raise ValueError("x must be a contiguous [n_sets, d] tensor")
        dtype = {torch.float32: TQ_F32, torch.bfloat16: TQ_BF16}.get(x.dtype)
        if dtype is None:
            raise TypeError("x must be float32 or bfloat16")
        if rows.dtype != torch.int64 or rows.numel() != x.shape[0]:
            raise ValueError("rows must be an int64 tensor with one entry per set")
        cache_rows = cache["norms"].numel()
        _check(lib().tq_append(self._h, _ptr(x), dtype, x.shape[0], _ptr(rows), cache_rows, _ptr(cache.get("codes")),
                               _ptr(cache.get("signs")), _ptr(cache["norms"]), _ptr(cache.get("rnorms")),
                               _stream(stream)), "tq_append")
        return cache

    def dequantize(self, keys, out=None, stream=None):
        import torch

        norms = keys["norms"]
        n_sets, n = norms.shape
        if out is None:
            out = torch.empty((n_sets, n, self.d), dtype=torch.float32, device=norms.device)
        _check(lib().tq_dequantize(self._h, _ptr(keys.get("codes")), _ptr(keys.get("signs")), _ptr(norms),
                                   _ptr(keys.get("rnorms")), n_sets, n, _ptr(out), _stream(stream)),
               "tq_dequantize")
        return out

    def logits(self, q, keys, out=None, stream=None):
        """q: [n_sets, nq, d] float32; keys: dict from quantize.  Returns
        [n_sets, nq, n_keys] float32 raw inner products."""
        import torch

        if q.dim() == 2:
            q = q.unsqueeze(0)
        if q.dtype != torch.float32 or not q.is_contiguous():
            raise TypeError("q must be contiguous float32")
        norms = keys["norms"]
        n_sets, n_keys = norms.shape
        nq = q.shape[1]
        if q.shape[0] != n_sets or q.shape[2] != self.d:
            raise ValueError("q shape does not match the keys")
        if out is None:
            out = torch.empty((n_sets, nq, n_keys), dtype=torch.float32, device=norms.device)
        _check(lib().tq_logits(self._h, _ptr(q), nq, _ptr(keys.get("codes")), _ptr(keys.get("signs")), _ptr(norms),
                               _ptr(keys.get("rnorms")), n_sets, n_keys, _ptr(out), _stream(stream)), "tq_logits")
        return out

    def attention_workspace_bytes(self, values_codec: "Codec", nq: int, n_sets: int, n_keys: int) -> int:
        b = ctypes.c_size_t()
        _check(lib().tq_attention_workspace(self._h, values_codec.handle, nq, n_sets, n_keys, ctypes.byref(b)),
               "tq_attention_workspace")
        return b.value

    def attention(self, q, keys, values_codec: "Codec", values, scale=None, out=None, workspace=None, stream=None):
        """Decode attention: this codec holds the keys, `values_codec` the
        values.  q: [n_sets, nq, d] float32.  Returns [n_sets, nq, d] float32
        sum_t softmax_t(scale <q, k_hat_t>) v_hat_t (scale defaults to
        1/sqrt(d)).  `workspace` is a uint8 CUDA tensor (allocated here when
        not given)."""
        import math

        import torch

        if q.dim() == 2:
            q = q.unsqueeze(0)
        if q.dtype != torch.float32 or not q.is_contiguous():
            raise TypeError("q must be contiguous float32")
        n_sets, n_keys = keys["norms"].shape
        nq = q.shape[1]
        if q.shape[0] != n_sets or q.shape[2] != self.d or values["norms"].shape != keys["norms"].shape:
            raise ValueError("q, keys and values do not match")
        if scale is None:
            scale = 1.0 / math.sqrt(self.d)
        if out is None:
            out = torch.empty((n_sets, nq, self.d), dtype=torch.float32, device=q.device)
        need = self.attention_workspace_bytes(values_codec, nq, n_sets, n_keys)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        _check(lib().tq_attention(self._h, values_codec.handle, _ptr(q), nq, _ptr(keys.get("codes")),
                                  _ptr(keys.get("signs")), _ptr(keys["norms"]), _ptr(keys.get("rnorms")),
                                  _ptr(values.get("codes")), _ptr(values.get("signs")), _ptr(values["norms"]),
                                  _ptr(values.get("rnorms")), n_sets, n_keys, float(scale), _ptr(out),
                                  _ptr(workspace), workspace.numel(), _stream(stream)), "tq_attention")
        return out

    def attention_static(self, q, keys, values_codec: "Codec", values, scale=None, out=None, stream=None):
        """As attention, through tq_attention_static: the workspace is the
        library's fixed device array, so nothing is allocated when `out` is
        given (calls that overlap in time on one GPU race)."""
        import math

        import torch

        if q.dim() == 2:
            q = q.unsqueeze(0)
        if q.dtype != torch.float32 or not q.is_contiguous():
            raise TypeError("q must be contiguous float32")
        n_sets, n_keys = keys["norms"].shape
        nq = q.shape[1]
        if q.shape[0] != n_sets or q.shape[2] != self.d or values["norms"].shape != keys["norms"].shape:
            raise ValueError("q, keys and values do not match")
        if scale is None:
            scale = 1.0 / math.sqrt(self.d)
        if out is None:
            out = torch.empty((n_sets, nq, self.d), dtype=torch.float32, device=q.device)
        _check(lib().tq_attention_static(self._h, values_codec.handle, _ptr(q), nq, _ptr(keys.get("codes")),
                                         _ptr(keys.get("signs")), _ptr(keys["norms"]), _ptr(keys.get("rnorms")),
                                         _ptr(values.get("codes")), _ptr(values.get("signs")), _ptr(values["norms"]),
                                         _ptr(values.get("rnorms")), n_sets, n_keys, float(scale), _ptr(out),
                                         _stream(stream)), "tq_attention_static")
        return out

    def topk(self, q, keys, k: int, workspace=None, stream=None):
        """Top-k maximum inner product search: q [nq, d] float32 against one
        set of keys (the dict from quantize, set 0 or unbatched arrays).
        Returns (scores [nq, k] float32, indices [nq, k] int32), best first."""
        import torch

        if q.dim() != 2 or q.dtype != torch.float32 or not q.is_contiguous() or q.shape[1] != self.d:
            raise ValueError("q must be a contiguous [nq, d] float32 tensor")
        norms = keys["norms"].reshape(-1)
        n_keys, nq = norms.numel(), q.shape[0]
        b = ctypes.c_size_t()
        _check(lib().tq_topk_workspace(self._h, nq, n_keys, k, ctypes.byref(b)), "tq_topk_workspace")
        if workspace is None:
            workspace = torch.empty(max(b.value, 1), dtype=torch.uint8, device=q.device)
        scores = torch.empty((nq, k), dtype=torch.float32, device=q.device)
        idx = torch.empty((nq, k), dtype=torch.int32, device=q.device)
        _check(lib().tq_topk(self._h, _ptr(q), nq, _ptr(keys.get("codes")), _ptr(keys.get("signs")), _ptr(norms),
                             _ptr(keys.get("rnorms")), n_keys, k, _ptr(scores), _ptr(idx), _ptr(workspace),
                             workspace.numel(), _stream(stream)), "tq_topk")
        return scores, idx

    # -- test hooks ----------------------------------------------------------
    def tables(self, group: int = 0):
        import numpy as np

        d = self.d
        pi = np.empty((d, d), np.float32)
        s = np.empty((d, d), np.float32)
        L = 1 << self.mse_bits if self.mse_bits else 0
        c = np.empty(max(L, 1), np.float32)
        t = np.empty(max(L - 1, 1), np.float32)
        _check(lib().tq_get_tables(self._h, group, pi.ctypes.data, s.ctypes.data, c.ctypes.data, t.ctypes.data),
               "tq_get_tables")
        return dict(Pi=pi, S=s if self.variant == TQ_PROD else None, centroids=c[:L], boundaries=t[:max(L - 1, 0)])

    def pack(self, idx, bits: int, stream=None):
        import torch

        rows = idx.shape[0]
        out = torch.empty((rows, row_bytes(self.d, bits)), dtype=torch.uint8, device=idx.device)
        _check(lib().tq_pack(self._h, _ptr(idx), bits, rows, _ptr(out), _stream(stream)), "tq_pack")
        return out

    def unpack(self, packed, bits: int, stream=None):
        import torch

        rows = packed.shape[0]
        out = torch.empty((rows, self.d), dtype=torch.uint8, device=packed.device)
        _check(lib().tq_unpack(self._h, _ptr(packed), bits, rows, _ptr(out), _stream(stream)), "tq_unpack")
        return out


def _ptr_pair(parts, key):
    arr = (ctypes.c_void_p * 2)()
    for i, p in enumerate(parts):
        t = p.get(key)
        arr[i] = None if t is None else t.data_ptr()
    return arr


class MixedCodec:
    """Outlier-channel mixed precision: the channels out_channels[g] of group g
    are coded at bits + 1 by the `outlier` part codec (seed), the other
    channels at `bits` by the `regular` part codec (seed + 1).
    out_channels: [groups, n_out] integers."""

    def __init__(self, d: int, bits: int, variant: int, seed: int, out_channels, groups: int = 1):
        import numpy as np

        ch = np.ascontiguousarray(np.asarray(out_channels, dtype=np.int32).reshape(groups, -1))
        self.d, self.bits, self.variant, self.seed, self.groups = d, bits, variant, seed, groups
        self.n_out = ch.shape[1]
        h = ctypes.c_void_p()
        _check(lib().tq_mixed_init(d, bits, variant, seed, groups, self.n_out, ch.ctypes.data, ctypes.byref(h)),
               "tq_mixed_init")
        self._h = h
        ho, hr = ctypes.c_void_p(), ctypes.c_void_p()
        _check(lib().tq_mixed_parts(self._h, ctypes.byref(ho), ctypes.byref(hr)), "tq_mixed_parts")
        self.outlier = Codec(self.n_out, bits + 1, variant, seed, groups, _borrowed=ho)
        self.regular = Codec(d - self.n_out, bits, variant, seed + 1, groups, _borrowed=hr)

    def close(self) -> None:
        if getattr(self, "_h", None):
            self.outlier.close()
            self.regular.close()
            lib().tq_mixed_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace(self, n_sets: int, n: int, nq: int = 0, device="cuda"):
        import torch

        b = ctypes.c_size_t()
        _check(lib().tq_mixed_workspace(self._h, n_sets, n, nq, ctypes.byref(b)), "tq_mixed_workspace")
        return torch.empty(max(b.value, 1), dtype=torch.uint8, device=device)

    def empty_codes(self, n_sets: int, n: int, device="cuda"):
        return (self.outlier.empty_codes(n_sets, n, device), self.regular.empty_codes(n_sets, n, device))

    def quantize(self, x, out=None, workspace=None, stream=None):
        """x: [n_sets, n, d] float32 or bfloat16.  Returns (outlier, regular)
        dicts as Codec.quantize returns for each part."""
        import torch

        if x.dim() == 2:
            x = x.unsqueeze(0)
        dtype = {torch.float32: TQ_F32, torch.bfloat16: TQ_BF16}.get(x.dtype)
        if dtype is None or not x.is_contiguous() or x.shape[2] != self.d:
            raise ValueError("x must be a contiguous [n_sets, n, d] float32 / bfloat16 tensor")
        n_sets, n, _ = x.shape
        out = out or self.empty_codes(n_sets, n, x.device)
        ws = workspace if workspace is not None else self.workspace(n_sets, n, 0, x.device)
        _check(lib().tq_mixed_quantize(self._h, _ptr(x), dtype, n_sets, n, _ptr_pair(out, "codes"),
                                       _ptr_pair(out, "signs"), _ptr_pair(out, "norms"), _ptr_pair(out, "rnorms"),
                                       _ptr(ws), ws.numel(), _stream(stream)), "tq_mixed_quantize")
        return out

    def dequantize(self, parts, out=None, workspace=None, stream=None):
        import torch

        n_sets, n = parts[0]["norms"].shape
        if out is None:
            out = torch.empty((n_sets, n, self.d), dtype=torch.float32, device=parts[0]["norms"].device)
        ws = workspace if workspace is not None else self.workspace(n_sets, n, 0, out.device)
        _check(lib().tq_mixed_dequantize(self._h, _ptr_pair(parts, "codes"), _ptr_pair(parts, "signs"),
                                         _ptr_pair(parts, "norms"), _ptr_pair(parts, "rnorms"), n_sets, n, _ptr(out),
                                         _ptr(ws), ws.numel(), _stream(stream)), "tq_mixed_dequantize")
        return out

    def logits(self, q, parts, out=None, workspace=None, stream=None):
        import torch

        if q.dim() == 2:
            q = q.unsqueeze(0)
        if q.dtype != torch.float32 or not q.is_contiguous():
            raise TypeError("q must be contiguous float32")
        n_sets, n_keys = parts[0]["norms"].shape
        nq = q.shape[1]
        if out is None:
            out = torch.empty((n_sets, nq, n_keys), dtype=torch.float32, device=q.device)
        ws = workspace if workspace is not None else self.workspace(n_sets, n_keys, nq, q.device)
        _check(lib().tq_mixed_logits(self._h, _ptr(q), nq, _ptr_pair(parts, "codes"), _ptr_pair(parts, "signs"),
                                     _ptr_pair(parts, "norms"), _ptr_pair(parts, "rnorms"), n_sets, n_keys,
                                     _ptr(out), _ptr(ws), ws.numel(), _stream(stream)), "tq_mixed_logits")
        return out


def dense_logits(q, keys, out=None, stream=None):
    """Dense baseline: <q, k> over unquantized float16 / float32 keys.
    q: [n_sets, nq, d] float32, keys: [n_sets, n_keys, d]; returns
    [n_sets, nq, n_keys] float32 (tq_dense_logits)."""
    import torch

    dtype = {torch.float16: TQ_F16, torch.float32: TQ_F32}.get(keys.dtype)
    if dtype is None or not keys.is_contiguous() or q.dtype != torch.float32 or not q.is_contiguous():
        raise TypeError("keys must be contiguous float16/float32, q contiguous float32")
    n_sets, n_keys, d = keys.shape
    nq = q.shape[1]
    if out is None:
        out = torch.empty((n_sets, nq, n_keys), dtype=torch.float32, device=q.device)
    _check(lib().tq_dense_logits(_ptr(q), nq, _ptr(keys), dtype, d, n_sets, n_keys, _ptr(out), _stream(stream)),
           "tq_dense_logits")
    return out


def probe_stream(kind: int, src, dst, grid: int, stream=None):
    """One streaming probe kernel over the bytes of src (tq_probe_stream)."""
    _check(lib().tq_probe_stream(kind, _ptr(src), src.numel() * src.element_size(), _ptr(dst),
                                 dst.numel() * dst.element_size(), grid, _stream(stream)), "tq_probe_stream")


def probe_mfma(f16: bool, iters: int, grid: int, out, stream=None):
    """Back-to-back MFMAs with no memory traffic (tq_probe_mfma)."""
    _check(lib().tq_probe_mfma(int(f16), iters, grid, _ptr(out), _stream(stream)), "tq_probe_mfma")


def probe_issue(mode: int, waves_per_simd: int, iters: int, grid: int, out, stream=None):
    """Instruction-issue loops, per-wave cycles and real time (tq_probe_issue);
    out: int32 CUDA tensor of 2 * grid * 4 * waves_per_simd entries."""
    _check(lib().tq_probe_issue(mode, waves_per_simd, iters, grid, _ptr(out), _stream(stream)), "tq_probe_issue")


def host_tables(d: int, bits: int, variant: int, seed: int, group: int = 0):
    """The codec tables computed on the host only (no device needed)."""
    import numpy as np

    mse_bits = bits if variant == TQ_MSE else bits - 1
    L = 1 << mse_bits if mse_bits else 0
    pi = np.empty((d, d), np.float32)
    s = np.empty((d, d), np.float32)
    c = np.empty(max(L, 1), np.float32)
    t = np.empty(max(L - 1, 1), np.float32)
    _check(lib().tq_host_tables(d, bits, variant, seed, group, pi.ctypes.data, s.ctypes.data, c.ctypes.data,
                                t.ctypes.data), "tq_host_tables")
    return dict(Pi=pi, S=s if variant == TQ_PROD else None, centroids=c[:L], boundaries=t[:max(L - 1, 0)])
