"""Shared comparison rules for the GPU parity tests (not a test module).

The rules, derived from the arithmetic (fp32 accumulation vs the oracle's fp64):
  R1  rotated values: per row max|z_gpu - z64| / max|z64| <= 1e-3.
  R2  scales: equal to the oracle's fp16 scale or one fp16 ulp apart.
  R3  codes: with u = y64 / s_gpu (the scale the GPU stored, so that an R2
      one-ulp row does not cascade into its codes), q_gpu == clamp(RNE(u)),
      except that |diff| == 1 is allowed where u lies within 1e-3 of a .5
      boundary.  Asymmetric (KV): u = (y64 - min_gpu) / s_gpu, same window.
  R4  on inputs whose transform is exact in fp32 (grid inputs), codes and
      scales are bit-identical to the oracle's fp32 recipe.
"""
from __future__ import annotations

import numpy as np

from oracle import kv as okv
from oracle import quant as oq

R1_TOL = 1e-3
TIE_TOL = 1e-3


def f16_ulp_diff(a, b):
    """Distance in fp16 ulps between two fp16 arrays of the same sign."""
    ia = np.asarray(a, dtype=np.float16).view(np.int16).astype(np.int64)
    ib = np.asarray(b, dtype=np.float16).view(np.int16).astype(np.int64)
    return np.abs(ia - ib)


def check_rotation(z_gpu, z64, tol=R1_TOL):
    z_gpu = np.asarray(z_gpu, dtype=np.float64)
    denom = np.maximum(np.abs(z64).max(axis=-1), 1e-30)
    rel = np.abs(z_gpu - z64).max(axis=-1) / denom
    assert rel.max() <= tol, f"R1: max row error {rel.max():.3e} > {tol}"
    return float(rel.max())


def check_codes_given_scale(q_gpu, s_gpu, y64, bits=4):
    """R3 on unpacked codes: the oracle's codes from the GPU's stored scale
    (float64 division), a +-1 difference allowed only within TIE_TOL of a .5
    boundary.  s_gpu has one scale per row of y64 (its last axis)."""
    q_ref = oq.sym_quant_with_scale(y64, s_gpu, bits)
    diff = np.asarray(q_gpu).astype(np.int64) - q_ref.astype(np.int64)
    assert np.abs(diff).max(initial=0) <= 1, "R3: code off by more than 1"
    bad = (diff != 0) & (oq.tie_distance(y64, s_gpu) >= TIE_TOL)
    assert not bad.any(), f"R3: {int(bad.sum())} codes differ away from a .5 boundary"
    return int((diff != 0).sum())


def check_scales(s_gpu, y64, clip, bits=4):
    """R2: fp16 scales equal to the float64 oracle's or one ulp apart."""
    s_ref = oq.sym_scale_math(y64, clip, bits)
    ulps = f16_ulp_diff(s_gpu, s_ref)
    assert ulps.max(initial=0) <= 1, f"R2: scale off by {ulps.max()} ulp"
    return int((ulps > 0).sum())


def check_sym_codes(q_gpu_packed, s_gpu, y64, clip):
    """R2 + R3 of packed INT4 codes against the float64 math-mode oracle."""
    ulp_rows = check_scales(s_gpu, y64, clip)
    flips = check_codes_given_scale(oq.unpack_int4(q_gpu_packed), s_gpu, y64)
    return dict(scale_ulp_rows=ulp_rows, code_flips=flips)


def check_sym_exact(q_gpu_packed, s_gpu, z_exact, d, rotated, clip):
    """R4: bit-exact against the fp32 recipe on an exactly representable z."""
    q_ref, s_ref = oq.sym_quant_recipe(z_exact.astype(np.float32), d, rotated, clip)
    assert np.array_equal(np.asarray(s_gpu).view(np.uint16), s_ref.view(np.uint16)), "R4: scales"
    assert np.array_equal(np.asarray(q_gpu_packed), oq.pack_int4(q_ref)), "R4: packed codes"


def check_asym(codes_gpu, s_gpu, m_gpu, y64, group, clip, bits=4):
    """KV analogue of R2 + R3 (codes unpacked, [..., Dh]); 2^bits - 1 levels.
    Codes are compared with the oracle's codes for the GPU's stored (scale, min)."""
    _, s_ref, m_ref = okv.asym_quant_math(y64, group, clip, bits)
    us = f16_ulp_diff(s_gpu, s_ref)
    um = f16_ulp_diff(m_gpu, m_ref)
    assert us.max() <= 1 and um.max() <= 1, f"KV scale/min ulps {us.max()}/{um.max()}"
    q_ref = okv.asym_quant_with_params(y64, group, s_gpu, m_gpu, bits)
    diff = codes_gpu.astype(np.int64) - q_ref.astype(np.int64)
    assert np.abs(diff).max(initial=0) <= 1, "KV: code off by more than 1"
    tie = okv.asym_tie_distance(y64, group, s_gpu, m_gpu)
    bad = (diff != 0) & (tie >= TIE_TOL)
    assert not bad.any(), f"KV: {int(bad.sum())} codes differ away from a .5 boundary"


def decode_bound(q, k_q, k_meta, v_q, v_meta, L, group, softmax_scale, ref):
    """Per-element error bound of the Decode routine's output against the
    float64 oracle, derived from the kernel's arithmetic (first order):

      weights  each p_j s_j enters the value product rounded to fp16:
               |err| <= 2^-11 p_j s_j + 2^-25 (the subnormal spacing), times
               the code c_j <= 15, over sum_j p_j >= 1 (the largest weight is 1):
               2^-11 o_sc + 15 L 2^-25, with o_sc = sum p s c / sum p, the
               oracle's output over values with their minima set to 0;
      scores   codes times fp16 query operands are exact; the fp32 sums over
               the 128 dims (and of the query) lose at most 128 2^-24 of the sum
               of magnitudes A_j = s_j sum|q||c_j| + |min_j| sum|q|, and a few
               roundings of the scale, the fma, the max subtraction and exp2 add
               up to 0.2 2^-17 more: relative error of p_j
               eps <= 1.2 2^-17 scale A_max + 2^-21, which moves the normalised
               output by at most 2 eps max|v|;
      sums     fp32 accumulation of the output rows and of sum p over at most
               L + 64 terms: 2 (L + 64) 2^-24 max|v|;
      output   one rounding to fp16: 2^-11 |ref| + 2^-25.
    q [B, Hq, Dh]; caches as the oracle takes them; ref the oracle's output."""
    from oracle import attention as oatt
    q = np.asarray(q, dtype=np.float64)
    B, Hq, Dh = q.shape
    Hkv = k_q.shape[1]
    rep = Hq // Hkv
    v_meta0 = np.array(v_meta, dtype=np.float16, copy=True)
    v_meta0[..., 1] = 0
    o_sc = oatt.decode_attention(q, k_q, k_meta, v_q, v_meta0, L, group, softmax_scale)
    vdeq = oatt.dequant_cache(v_q, v_meta, L, group)                        # [B, Hkv, L, Dh]
    vmax = np.repeat(np.abs(vdeq).max(axis=(2, 3)), rep, axis=1)[..., None]  # [B, Hq, 1]
    codes = okv.unpack_uint4(np.asarray(k_q)[:, :, :L]).astype(np.float64)  # [B, Hkv, L, Dh]
    km = np.asarray(k_meta, dtype=np.float16)[:, :, :L].astype(np.float64)
    ks = km[..., 0, 0] if km.ndim == 5 else km[..., 0]                    # one group per head
    kmin = km[..., 0, 1] if km.ndim == 5 else km[..., 1]
    aq = np.abs(q)
    qc = np.einsum("bgrd,bgjd->bgrj", aq.reshape(B, Hkv, rep, Dh), codes)  # sum |q| c
    A = ks[:, :, None, :] * qc + np.abs(kmin)[:, :, None, :] * aq.sum(-1).reshape(B, Hkv, rep)[..., None]
    amax = A.max(axis=-1).reshape(B, Hq)[..., None]
    eps = 1.2 * 2.0 ** -17 * softmax_scale * amax + 2.0 ** -21
    return (2.0 ** -11 * o_sc + 15 * L * 2.0 ** -25 + 2 * eps * vmax
            + 2 * (L + 64) * 2.0 ** -24 * vmax + 2.0 ** -11 * np.abs(ref) + 2.0 ** -25)
