"""Shared comparison rules for the GPU parity tests (not a test module).

The rules, derived from the arithmetic (fp32 accumulation vs the oracle's fp64):
  R1  rotated values: per row max|z_gpu - z64| / max|z64| <= 1e-3.
  R2  scales: equal to the oracle's fp16 scale or one fp16 ulp apart.
  R3  codes: equal, except |diff| == 1 where the oracle's pre-round value u lies
      within 1e-3 of a .5 boundary.  On a row whose stored scale is one ulp off
      the window widens by the shift that ulp causes, |u| |s_gpu - s| / s with
      |u| <= 7.5 (asymmetric: (15 |ds| + |dmin|) / s).
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


def check_sym_codes(q_gpu_packed, s_gpu, y64, clip):
    """R2 + R3 against the float64 math-mode oracle."""
    q_ref, s_ref = oq.sym_quant_math(y64, clip)
    ulps = f16_ulp_diff(s_gpu, s_ref)
    assert ulps.max() <= 1, f"R2: scale off by {ulps.max()} ulp"
    q_gpu = oq.unpack_int4(q_gpu_packed).astype(np.int64)
    diff = q_gpu - q_ref.astype(np.int64)
    assert np.abs(diff).max(initial=0) <= 1, "R3: code off by more than 1"
    tie = oq.tie_distance(y64, s_ref)
    s_r = s_ref.astype(np.float64)
    shift = np.where(s_r > 0, 7.5 * np.abs(np.asarray(s_gpu, np.float64) - s_r) / np.where(s_r > 0, s_r, 1), 0)
    win = TIE_TOL + shift[..., None]
    bad = (diff != 0) & (tie >= win)
    assert not bad.any(), f"R3: {int(bad.sum())} codes differ away from a .5 boundary"
    return dict(scale_ulp_rows=int((ulps > 0).sum()), code_flips=int((diff != 0).sum()))


def check_sym_exact(q_gpu_packed, s_gpu, z_exact, d, rotated, clip):
    """R4: bit-exact against the fp32 recipe on an exactly representable z."""
    q_ref, s_ref = oq.sym_quant_recipe(z_exact.astype(np.float32), d, rotated, clip)
    assert np.array_equal(np.asarray(s_gpu).view(np.uint16), s_ref.view(np.uint16)), "R4: scales"
    assert np.array_equal(np.asarray(q_gpu_packed), oq.pack_int4(q_ref)), "R4: packed codes"


def check_asym(codes_gpu, s_gpu, m_gpu, y64, group, clip, bits=4):
    """KV analogue of R2 + R3 (codes unpacked, [..., Dh]); 2^bits - 1 levels."""
    levels = (1 << bits) - 1
    q_ref, s_ref, m_ref = okv.asym_quant_math(y64, group, clip, bits)
    us = f16_ulp_diff(s_gpu, s_ref)
    um = f16_ulp_diff(m_gpu, m_ref)
    assert us.max() <= 1 and um.max() <= 1, f"KV scale/min ulps {us.max()}/{um.max()}"
    diff = codes_gpu.astype(np.int64) - q_ref.astype(np.int64)
    assert np.abs(diff).max(initial=0) <= 1
    tie = okv.asym_tie_distance(y64, group, s_ref, m_ref)
    s_r = s_ref.astype(np.float64)
    ds = np.abs(np.asarray(s_gpu, np.float64) - s_r)
    dm = np.abs(np.asarray(m_gpu, np.float64) - m_ref.astype(np.float64))
    shift = np.where(s_r > 0, (levels * ds + dm) / np.where(s_r > 0, s_r, 1), 0)
    win = TIE_TOL + np.repeat(shift, group, axis=-1).reshape(diff.shape)
    bad = (diff != 0) & (tie >= win)
    assert not bad.any(), f"KV: {int(bad.sum())} codes differ away from a .5 boundary"
