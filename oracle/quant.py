"""Per-token symmetric INT4 round-to-nearest quantization and nibble packing.
TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Definition (QuaRot paper, activation-quantization paragraph; QuaRot blog,
"The outlier problem, stated precisely"): the scale of a row is its largest
absolute value divided by 7 (2^(b-1) - 1 for b = 4), the row is divided by the
scale and rounded to the nearest integer.  The implementation paragraph adds a
constant clipping ratio (0.9 for these inputs), so s = clip * max|y| / 7, and
INT4's range clamps the codes to [-8, 7].

Other bit widths (QuaRot paper, results with 6- and 8-bit round-to-nearest
weights and activations, Table 9): b-bit symmetric codes use
s = clip * max|y| / (2^(b-1) - 1) and clamp to [-2^(b-1), 2^(b-1) - 1]; b = 4 is
the INT4 case above.  Codes of b > 4 bits are stored one per byte (int8).

Readings taken where the pages are silent:
* ties round half to even (IEEE default, and what PyTorch's round does);
* the stored scale is fp16 and the division uses that stored value, so codes
  times the stored scale is exactly the dequantization the GEMM applies;
* a row whose scale is 0 (all zeros, or an fp16 underflow) gets codes 0;
* packing: byte j holds code 2j in its low nibble and code 2j+1 in its high
  nibble, two's complement.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
F16 = np.float16


# ---------------------------------------------------------------------------
# Packing
# ---------------------------------------------------------------------------

def pack_int4(codes: np.ndarray) -> np.ndarray:
    """int codes in [-8, 7], last axis even -> uint8 with 2 codes per byte."""
    c = np.asarray(codes).astype(np.int64)
    assert c.shape[-1] % 2 == 0
    assert c.min(initial=0) >= -8 and c.max(initial=0) <= 7
    lo = c[..., 0::2] & 0xF
    hi = c[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """uint8 bytes -> int8 codes (low nibble first), sign-extended."""
    p = np.asarray(packed).astype(np.int64)
    lo = p & 0xF
    hi = (p >> 4) & 0xF
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    out = np.where(out >= 8, out - 16, out)
    return out.astype(np.int8)


# ---------------------------------------------------------------------------
# Math mode (float64)
# ---------------------------------------------------------------------------

def code_range(bits: int) -> tuple[int, int, int]:
    """(qmax, lo, hi) of b-bit symmetric codes: qmax = 2^(b-1) - 1, range [-2^(b-1), qmax]."""
    assert 2 <= bits <= 8
    qmax = (1 << (bits - 1)) - 1
    return qmax, -(1 << (bits - 1)), qmax


def sym_scale_math(y: np.ndarray, clip: float = 1.0, bits: int = 4) -> np.ndarray:
    """fp16 per-row scale: fp16(clip * max|y| / qmax) computed in float64 (qmax = 7 for INT4)."""
    y = np.asarray(y, dtype=np.float64)
    amax = np.abs(y).max(axis=-1)
    return (clip * amax / float(code_range(bits)[0])).astype(F16)


def sym_quant_with_scale(y: np.ndarray, scale_f16: np.ndarray, bits: int = 4) -> np.ndarray:
    """Codes clamp(round_half_even(y / s), lo, hi) for given fp16 scales (float64 division);
    [-8, 7] for INT4."""
    _, lo, hi = code_range(bits)
    y = np.asarray(y, dtype=np.float64)
    s = np.asarray(scale_f16, dtype=F16).astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        u = np.where(s > 0, y / np.where(s > 0, s, 1.0), 0.0)
    return np.clip(np.rint(u), lo, hi).astype(np.int8)


def sym_quant_math(y: np.ndarray, clip: float = 1.0, bits: int = 4) -> tuple[np.ndarray, np.ndarray]:
    """(int8 codes, fp16 scales) of the float64 rows y."""
    s = sym_scale_math(y, clip, bits)
    return sym_quant_with_scale(y, s, bits), s


def tie_distance(y: np.ndarray, scale_f16: np.ndarray) -> np.ndarray:
    """| frac(|y/s|) - 0.5 |: how far each pre-round value is from a .5 boundary."""
    y = np.asarray(y, dtype=np.float64)
    s = np.asarray(scale_f16, dtype=F16).astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        u = np.abs(np.where(s > 0, y / np.where(s > 0, s, 1.0), 0.0))
    return np.abs(u - np.floor(u) - 0.5)


# ---------------------------------------------------------------------------
# Recipe mode (the fp32 step sequence the kernels implement)
# ---------------------------------------------------------------------------

def norm_constant(d: int, rotated: bool) -> np.float32:
    """c = fp32 rounding of the float64 value 1/sqrt(d) (1 when not rotated)."""
    if not rotated:
        return F32(1.0)
    return F32(1.0 / np.sqrt(np.float64(d)))


def sym_quant_recipe(z: np.ndarray, d: int, rotated: bool, clip: float = 1.0, bits: int = 4
                     ) -> tuple[np.ndarray, np.ndarray]:
    """Codes and fp16 scales from the fp32 transform output z = H (s * x).

    Steps, per row (every arithmetic step rounds to fp32 unless stated):
      c   = fp32(1/sqrt(d))            (1 when not rotated)
      a   = max|z| * c                 (max commutes with the monotone rounding)
      s_h = fp16_rne((clip * a) / 7)
      m   = c * (1 / s_h)              (m = 0 when s_h == 0)
      q   = clamp(round_half_even(z * m), -8, 7), the product z * m rounded
            to an integer directly from its exact value.
    """
    z32 = np.asarray(z, dtype=F32)
    c = np.full(z32.shape[:-1], norm_constant(d, rotated), dtype=F32)
    return sym_quant_recipe_rows(z32, c, clip, bits)


def sym_quant_recipe_rows(z: np.ndarray, c: np.ndarray, clip: float = 1.0, bits: int = 4
                          ) -> tuple[np.ndarray, np.ndarray]:
    """The recipe of sym_quant_recipe() with one fp32 constant c per row: the
    quantizer input is y = z * c, with z the exact fp32 row (the transform
    output, or the input itself) and c its normalisation.  For b bits the 7
    becomes qmax = 2^(b-1) - 1 and the clamp [-2^(b-1), qmax]."""
    qmax, lo, hi = code_range(bits)
    z32 = np.asarray(z, dtype=F32)
    c = np.asarray(c, dtype=F32)
    clip32 = F32(clip)
    az = np.abs(z32).max(axis=-1)
    a = (az * c).astype(F32)
    s = ((clip32 * a).astype(F32) / F32(qmax)).astype(F32)
    s_h = s.astype(F16)
    s_h32 = s_h.astype(F32)
    with np.errstate(divide="ignore"):
        inv = np.where(s_h32 > 0, F32(1.0) / np.where(s_h32 > 0, s_h32, F32(1.0)), F32(0.0)).astype(F32)
    m = (c * inv).astype(F32)
    # z and m are fp32, so their float64 product is exact; rint rounds it
    # half-to-even straight to an integer (the kernel does the same with one
    # fused multiply-add against 1.5 * 2^23).
    prod = z32.astype(np.float64) * m.astype(np.float64)[..., None]
    q = np.clip(np.rint(prod), lo, hi).astype(np.int8)
    return q, s_h


# ---------------------------------------------------------------------------
# Group-wise scales (QuaRot paper: group-wise quantization with different
# group sizes, one of its studied variants): the row is cut into groups of G
# consecutive elements along K and each group gets its own scale.
# ---------------------------------------------------------------------------

def sym_quant_groups_math(y: np.ndarray, group: int, clip: float = 1.0, bits: int = 4):
    """(codes [..., d], fp16 scales [..., d/G]) with one symmetric scale per group."""
    y = np.asarray(y, dtype=np.float64)
    d = y.shape[-1]
    assert d % group == 0
    g = y.reshape(*y.shape[:-1], d // group, group)
    q, s = sym_quant_math(g, clip, bits)
    return q.reshape(y.shape), s


def sym_quant_groups_recipe(z: np.ndarray, c: np.ndarray, group: int, clip: float = 1.0,
                            bits: int = 4):
    """The fp32 recipe per group: sym_quant_recipe_rows() on every group of G
    elements of each row, with the row's constant c."""
    z32 = np.asarray(z, dtype=F32)
    d = z32.shape[-1]
    g = z32.reshape(*z32.shape[:-1], d // group, group)
    cg = np.broadcast_to(np.asarray(c, dtype=F32)[..., None], g.shape[:-1])
    q, s = sym_quant_recipe_rows(g, cg, clip, bits)
    return q.reshape(z32.shape), s


def dequant(codes: np.ndarray, scale_f16: np.ndarray) -> np.ndarray:
    """float64 codes * scale."""
    return np.asarray(codes, dtype=np.float64) * np.asarray(scale_f16, dtype=F16).astype(np.float64)[..., None]

