"""Head-wise rotation of keys/queries and asymmetric 4-bit group quantization
of the KV cache.  TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Definitions followed:
* Keys and queries are rotated head-wise by the same Hadamard after the
  positional embedding, so scores q.k are unchanged (QuaRot paper, keys and
  queries paragraph: online head-wise Hadamard, post-RoPE caching; QuaRot
  blog, "Quantizing the KV cache": (qH).(kH) = q.k).  Values are not rotated
  online: their head-wise Hadamard is fused into W_v and W_out offline
  (QuaRot paper, attention paragraph).
* KV quantization is asymmetric, group size 128, clipping ratio 0.95 (QuaRot
  paper, implementation paragraph; KV bit-width study, Table 6).
* Init writes the prefill tokens into the cache, Append quantizes each new
  token and writes it at the next position (QuaRot paper, attention routines).

Reading taken for the asymmetric formula (the pages do not print it): per
group, min mn and max mx (both multiplied by the clipping ratio), fp16 scale
s = (mx - mn) / 15 and fp16 offset mn, codes q = clamp(round((y - mn) / s),
0, 15), dequantized as q * s + mn.  A constant group gets s = 0 and q = 0.
Cache layout: codes [B, H, S_max, Dh/2] (low nibble first), metadata
[B, H, S_max, Dh/G, 2] holding (scale, min) as fp16.

Other bit widths (QuaRot paper, KV bit-width study, Table 6: 2-, 3- and 4-bit
keys and values): b-bit codes use 2^b - 1 levels in place of 15, the same
formulas otherwise, and are kept in the 4-bit layout (the study measures
accuracy; the dequantization q * s + mn does not depend on b).
"""
from __future__ import annotations

import numpy as np

from .hadamard import rotate, rotate_unnormalised
from .quant import norm_constant

F32 = np.float32
F16 = np.float16


def pack_uint4(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes).astype(np.int64)
    assert c.min(initial=0) >= 0 and c.max(initial=0) <= 15
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_uint4(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed).astype(np.int64)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int64)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = (p >> 4) & 0xF
    return out.astype(np.uint8)


def asym_quant_math(y: np.ndarray, group: int, clip: float = 1.0, bits: int = 4):
    """float64 rows y [..., Dh] -> (uint8 codes [..., Dh], fp16 scale, fp16 min) per group."""
    levels = (1 << bits) - 1
    y = np.asarray(y, dtype=np.float64)
    dh = y.shape[-1]
    g = y.reshape(*y.shape[:-1], dh // group, group)
    mx = clip * g.max(axis=-1)
    mn = clip * g.min(axis=-1)
    s_h = ((mx - mn) / float(levels)).astype(F16)
    m_h = mn.astype(F16)
    s = s_h.astype(np.float64)[..., None]
    m = m_h.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        u = np.where(s > 0, (g - m) / np.where(s > 0, s, 1.0), 0.0)
    q = np.clip(np.rint(u), 0, levels).astype(np.uint8)
    return q.reshape(y.shape), s_h, m_h


def asym_quant_with_params(y: np.ndarray, group: int, s_h, m_h, bits: int = 4) -> np.ndarray:
    """Codes clamp(round_half_even((y - mn) / s), 0, 2^bits - 1) of float64 rows y [..., Dh]
    for given fp16 (s, mn) per group [..., Dh/G] (float64 arithmetic); s = 0 gives 0."""
    levels = (1 << bits) - 1
    y = np.asarray(y, dtype=np.float64)
    dh = y.shape[-1]
    g = y.reshape(*y.shape[:-1], dh // group, group)
    s = np.asarray(s_h, dtype=F16).astype(np.float64)[..., None]
    m = np.asarray(m_h, dtype=F16).astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        u = np.where(s > 0, (g - m) / np.where(s > 0, s, 1.0), 0.0)
    return np.clip(np.rint(u), 0, levels).astype(np.uint8).reshape(y.shape)


def asym_tie_distance(y: np.ndarray, group: int, s_h, m_h) -> np.ndarray:
    """| frac(|u|) - 0.5 | with u = (y - mn) / s per group (fp16 s, mn; u = 0 where s = 0):
    how far each pre-round value is from a .5 boundary."""
    y = np.asarray(y, dtype=np.float64)
    dh = y.shape[-1]
    g = y.reshape(*y.shape[:-1], dh // group, group)
    s = np.asarray(s_h, dtype=F16).astype(np.float64)[..., None]
    m = np.asarray(m_h, dtype=F16).astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        u = np.abs(np.where(s > 0, (g - m) / np.where(s > 0, s, 1.0), 0.0))
    return np.abs(u - np.floor(u) - 0.5).reshape(y.shape)


def asym_quant_recipe(z: np.ndarray, dh: int, rotated: bool, group: int, clip: float = 1.0,
                      bits: int = 4):
    """The fp32 step sequence of the kernel, from z = H (s * x) (or x if not rotated).

      y    = fp32(z * c), c = fp32(1/sqrt(Dh)) (y = z when not rotated)
      mx_c = fp32(clip * max y), mn_c = fp32(clip * min y)   per group
      s_h  = fp16_rne(fp32(mx_c - mn_c) / L), m_h = fp16_rne(mn_c)
      q    = 0 if s_h == 0 else clamp(round_half_even(fp32(y - m_h) * (1/s_h)), 0, L)
             (the last product rounded to an integer from its exact value)
    with L = 2^bits - 1 (15 for 4 bits).
    """
    levels = (1 << bits) - 1
    z32 = np.asarray(z, dtype=F32)
    c = norm_constant(dh, rotated)
    y = (z32 * c).astype(F32) if rotated else z32
    g = y.reshape(*y.shape[:-1], dh // group, group)
    clip32 = F32(clip)
    mx_c = (clip32 * g.max(axis=-1)).astype(F32)
    mn_c = (clip32 * g.min(axis=-1)).astype(F32)
    s_h = ((mx_c - mn_c).astype(F32) / F32(levels)).astype(F32).astype(F16)
    m_h = mn_c.astype(F16)
    s32 = s_h.astype(F32)
    with np.errstate(divide="ignore"):
        inv = np.where(s32 > 0, F32(1.0) / np.where(s32 > 0, s32, F32(1.0)), F32(0.0)).astype(F32)
    diff = (g - m_h.astype(F32)[..., None]).astype(F32)
    prod = diff.astype(np.float64) * inv.astype(np.float64)[..., None]
    q = np.clip(np.rint(prod), 0, levels).astype(np.uint8)
    return q.reshape(y.shape), s_h, m_h


def asym_dequant(codes, s_h, m_h, group: int) -> np.ndarray:
    q = np.asarray(codes, dtype=np.float64)
    dh = q.shape[-1]
    g = q.reshape(*q.shape[:-1], dh // group, group)
    s = np.asarray(s_h, dtype=F16).astype(np.float64)[..., None]
    m = np.asarray(m_h, dtype=F16).astype(np.float64)[..., None]
    return (g * s + m).reshape(q.shape)


def kv_rotate_quant_cache(kv: np.ndarray, signs, rotated: bool, group: int, clip: float,
                          cache_q: np.ndarray, cache_meta: np.ndarray, start_pos: int,
                          mode: str = "math", bits: int = 4):
    """Quantize kv [B, S_new, H, Dh] and write it into the cache at start_pos.. (in place).

    mode "math": float64 rotation and quantization; mode "recipe": the fp32
    step sequence applied to the exact float64 rotation (bit-exact reference
    when the rotation is exact in fp32).  Returns the float64 rotated values.
    """
    kv = np.asarray(kv, dtype=np.float64)
    b, s_new, h, dh = kv.shape
    if rotated:
        y = rotate(kv, signs)
        z = rotate_unnormalised(kv, signs)
    else:
        y = kv
        z = kv
    if mode == "math":
        q, s_h, m_h = asym_quant_math(y, group, clip, bits)
    else:
        q, s_h, m_h = asym_quant_recipe(z, dh, rotated, group, clip, bits)
    packed = pack_uint4(q)                          # [B, S_new, H, Dh/2]
    cache_q[:, :, start_pos:start_pos + s_new, :] = np.transpose(packed, (0, 2, 1, 3))
    meta = np.stack([s_h, m_h], axis=-1)            # [B, S_new, H, Dh/G, 2]
    cache_meta[:, :, start_pos:start_pos + s_new] = np.transpose(meta, (0, 2, 1, 3, 4))
    return y


def gqa_scores(q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """Raw scores S[b, hq, i, j] = q[b, i, hq] . k[b, j, hq // (Hq / Hkv)] (float64)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    hq, hkv = q.shape[2], k.shape[2]
    rep = hq // hkv
    kk = np.repeat(k, rep, axis=2)                  # [B, Sk, Hq, Dh]
    return np.einsum("bihd,bjhd->bhij", q, kk)
