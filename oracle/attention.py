"""Decode attention over the 4-bit KV cache.  TEST INFRASTRUCTURE ONLY (see
``oracle/__init__.py``).

Definition followed (QuaRot paper, attention paragraph and the attention
routines of its implementation appendix): during decoding the Decode routine
takes the current (rotated, FP16) query and the quantized cache that Init and
Append wrote, dequantizes keys and values, and computes ordinary softmax
attention of that one query over the cached positions -- the pages implement
it as a quantized variant of flash attention (online softmax), which changes
the evaluation order, not the result.  Queries and keys carry the same
head-wise rotation, so the scores equal those of the unrotated model (QuaRot
blog, "Quantizing the KV cache").

Here, for every batch b and query head hq, with kv head h = hq // (Hq / Hkv)
(grouped-query attention; the pages' models share heads this way in the 70B
shape) and positions j < L:

    k_j = dequant(K codes[b, h, j]),  v_j = dequant(V codes[b, h, j])
          (per group: code * scale + min, the asymmetric KV format)
    s_j = softmax_scale * (q[b, hq] . k_j)
    o   = sum_j softmax(s)_j * v_j

all in float64.  Parity of this function is pinned by ``tests/
test_oracle_attention.py`` against PyTorch's scaled_dot_product_attention on
the dequantized tensors, closed forms (equal keys -> the mean of the values,
one dominant key -> its value) and invariances (a shift of every score,
a common factor on the value scales).
"""
from __future__ import annotations

import numpy as np

from .kv import asym_dequant, unpack_uint4


def dequant_cache(cache_q: np.ndarray, cache_meta: np.ndarray, L: int, group: int) -> np.ndarray:
    """Packed cache [B, H, S_max, Dh/2] + meta [B, H, S_max, Dh/G, 2] -> float64 [B, H, L, Dh]."""
    codes = unpack_uint4(np.asarray(cache_q)[:, :, :L])
    meta = np.asarray(cache_meta, dtype=np.float16)[:, :, :L]
    return asym_dequant(codes, meta[..., 0], meta[..., 1], group)


def decode_attention(q: np.ndarray, k_cache_q, k_cache_meta, v_cache_q, v_cache_meta, L: int,
                     group: int, softmax_scale: float) -> np.ndarray:
    """q [B, Hq, Dh] -> attention output [B, Hq, Dh] (float64) over positions 0 .. L-1."""
    q = np.asarray(q, dtype=np.float64)
    b, hq, dh = q.shape
    k = dequant_cache(k_cache_q, k_cache_meta, L, group)     # [B, Hkv, L, Dh]
    v = dequant_cache(v_cache_q, v_cache_meta, L, group)
    hkv = k.shape[1]
    rep = hq // hkv
    kk = np.repeat(k, rep, axis=1)                           # [B, Hq, L, Dh]
    vv = np.repeat(v, rep, axis=1)
    s = softmax_scale * np.einsum("bhd,bhjd->bhj", q, kk)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=-1, keepdims=True)
    return np.einsum("bhj,bhjd->bhd", p, vv)
