"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle's
timing leg.

This module only draws inputs: it holds none of the quantizer's arithmetic
(no rotation, codebook, packing or scoring).  Shapes and value laws follow the
workloads the pages describe (KV caches of a Llama-3.1-8B-shaped layer, decode
attention logits with grouped query heads, an inner-product nearest-neighbour
index at d=200, high-dimensional vectors at d=1536/3072).  The pages measure on
LongBench / Needle-in-a-Haystack with trained weights and on GloVe-200; none of
those is available, so these generators stand in for them.
"""
from __future__ import annotations

import numpy as np

# --- small parity workload: d=128, n=4096 N(0,1), 256 N(0,1) queries -------
PARITY_D = 128
PARITY_N = 4096
PARITY_NQ = 256


def parity_vectors(n: int = PARITY_N, d: int = PARITY_D, seed: int = 0) -> np.ndarray:
    return np.random.default_rng(seed).standard_normal((n, d)).astype(np.float32)


def parity_queries(nq: int = PARITY_NQ, d: int = PARITY_D, seed: int = 1) -> np.ndarray:
    return np.random.default_rng(seed).standard_normal((nq, d)).astype(np.float32)


# --- KV cache of one layer: 8 KV heads x 32768 tokens x 128, bf16 ---------
KV_HEADS = 8
KV_TOKENS = 32768
KV_DIM = 128
KV_OUTLIER_CHANNELS = 4
KV_OUTLIER_SCALE = 10.0


def kv_tensor(seed: int, heads: int = KV_HEADS, tokens: int = KV_TOKENS, dim: int = KV_DIM):
    """[heads, tokens, dim] N(0,1) values with KV_OUTLIER_CHANNELS channels per
    head scaled by 10 (channel ids drawn per head from the same generator),
    rounded to bfloat16 (round-to-nearest-even).  Returns a torch bf16 CPU
    tensor.  seed 2 = keys, seed 3 = values."""
    import torch

    rng = np.random.default_rng(seed)
    x = rng.standard_normal((heads, tokens, dim), dtype=np.float32)
    for h in range(heads):
        ch = rng.choice(dim, size=KV_OUTLIER_CHANNELS, replace=False)
        x[h, :, ch] *= KV_OUTLIER_SCALE
    return torch.from_numpy(x).to(torch.bfloat16)


# --- decode logits: 16 batch x 8 KV heads x 131072 tokens, 32 query heads --
DEC_BATCH = 16
DEC_KV_HEADS = 8
DEC_Q_PER_KV = 4
DEC_TOKENS = 131072
DEC_DIM = 128


def decode_queries(seed: int = 5, batch: int = DEC_BATCH, q_heads: int = DEC_KV_HEADS * DEC_Q_PER_KV,
                   dim: int = DEC_DIM) -> np.ndarray:
    """[batch, 32, dim] float32 N(0,1); query head h reads KV head h // 4."""
    return np.random.default_rng(seed).standard_normal((batch, q_heads, dim), dtype=np.float32)


def decode_keys_device(seed: int, sets: int, tokens: int, dim: int, device, chunk_sets: int = 8):
    """[sets, tokens, dim] float32 N(0,1) drawn on the device with torch's
    generator, one chunk of sets at a time (the full config is 8.6 GB)."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = torch.empty((sets, tokens, dim), dtype=torch.float32, device=device)
    for s0 in range(0, sets, chunk_sets):
        s1 = min(sets, s0 + chunk_sets)
        out[s0:s1].normal_(generator=gen)
    return out


def random_packed_cache(seed: int, sets: int, tokens: int, code_row: int, sign_row: int,
                        code_bytes_used: int, sign_bytes_used: int):
    """A synthetic quantized cache: uniformly random code and sign bytes (padding
    bytes zero), norms ~ chi(d)-like positive values, residual norms in (0, 1).
    Used to exercise the scoring kernel independently of the quantizer."""
    rng = np.random.default_rng(seed)
    codes = np.zeros((sets, tokens, code_row), dtype=np.uint8)
    if code_bytes_used:
        codes[..., :code_bytes_used] = rng.integers(0, 256, (sets, tokens, code_bytes_used), dtype=np.uint8)
    signs = np.zeros((sets, tokens, max(sign_row, 0)), dtype=np.uint8)
    if sign_bytes_used:
        signs[..., :sign_bytes_used] = rng.integers(0, 256, (sets, tokens, sign_bytes_used), dtype=np.uint8)
    norms = (10.0 + rng.standard_normal((sets, tokens))).astype(np.float32)
    rnorms = rng.uniform(0.05, 0.5, (sets, tokens)).astype(np.float32)
    return codes, signs, norms, rnorms


# --- nearest-neighbour index: d=200, 1e6 points of a Gaussian mixture -------
NN_D = 200
NN_CENTRES = 1000
NN_POINTS = 1_000_000
NN_QUERIES = 10_000
NN_STD = 0.3


def nn_centres(seed: int = 6, k: int = NN_CENTRES, d: int = NN_D) -> np.ndarray:
    c = np.random.default_rng(seed).standard_normal((k, d))
    return (c / np.linalg.norm(c, axis=1, keepdims=True)).astype(np.float32)


def nn_points(n: int, seed: int, centres: np.ndarray, std: float = NN_STD) -> np.ndarray:
    """Unit-normalised points centre_m + std * N(0, I), m uniform.  seed 7 =
    database, seed 8 = queries."""
    rng = np.random.default_rng(seed)
    m = rng.integers(0, centres.shape[0], n)
    x = centres[m].astype(np.float64) + std * rng.standard_normal((n, centres.shape[1]))
    return (x / np.linalg.norm(x, axis=1, keepdims=True)).astype(np.float32)


# --- high-dimensional vectors: d=1536 (1e5) and d=3072 (5e4) ----------------
def highd_vectors(n: int, d: int, seed: int = 9) -> np.ndarray:
    """x = rho * Z / ||Z||, Z ~ N(0, I_d), rho ~ LogNormal(0, 0.5)."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((n, d), dtype=np.float32)
    rho = rng.lognormal(0.0, 0.5, n).astype(np.float32)
    return z / np.linalg.norm(z, axis=1, keepdims=True) * rho[:, None]
