"""The two remaining online steps of QuaRot's quantized transformer block, in
float64 (math mode) and as the fp32 recipe the kernels follow.
TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

* RMSNorm without its scale, feeding the per-token INT4 quantizer of the
  QKV, gate and up inputs.  QuaRot paper, section on the method (the scale
  diag(alpha) of RMSNorm is absorbed into the next weights, so the block only
  divides each row by its RMS) and the activation-quantization paragraph
  (RMSNorm without scaling stays in FP32, then the per-token quantizer).
  Definition: y = x / sqrt(mean(x^2) + eps).  The pages write the normalised
  row as x / ||x||; the usual RMS form differs from that by the constant
  sqrt(d) (and eps), which the per-token quantizer cannot see: codes depend
  on y / max|y| only, and the scale carries the constant.  eps is an argument
  (the pages give none).

* Hadamard heads, the block before the O projection: Z <- Z (H_{n_h} (x) I),
  where Z is the attention output, n_h the number of heads and the identity
  has the head dimension.  QuaRot paper, the attention-block paragraph on
  (H_{n_h} (x) I)(I (x) H_{d_h}) = H, and the description of Figure 6.  The
  pages use a plain (not randomized) Walsh-Hadamard transform here; with the
  1/sqrt(n_h) normalisation it is orthogonal.  Element index i = h d_h + j
  (numpy ``kron``), so H_{n_h} mixes the heads at a fixed position j.
"""
from __future__ import annotations

import numpy as np

from .hadamard import fwht
from .quant import F16, F32, sym_quant_math, sym_quant_recipe_rows


# ---------------------------------------------------------------------------
# RMSNorm (no scale) + per-token INT4
# ---------------------------------------------------------------------------

def rms_multiplier(x: np.ndarray, eps: float) -> np.ndarray:
    """r = 1 / sqrt(mean(x^2) + eps) per row, float64."""
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / np.sqrt(np.mean(x * x, axis=-1) + float(eps))


def rmsnorm(x: np.ndarray, eps: float) -> np.ndarray:
    """y = x * r (RMSNorm without the learned scale), float64."""
    x = np.asarray(x, dtype=np.float64)
    return x * rms_multiplier(x, eps)[..., None]


def rmsnorm_quant_math(x: np.ndarray, eps: float, clip: float = 1.0, bits: int = 4):
    """Float64 reference of the fused op: (codes, fp16 scales, y64)."""
    y = rmsnorm(x, eps)
    q, s = sym_quant_math(y, clip, bits)
    return q, s, y


def rmsnorm_quant_recipe(x_f16: np.ndarray, r_f32: np.ndarray, clip: float = 1.0, bits: int = 4):
    """Codes and fp16 scales the kernel derives from x and its fp32 multiplier r.

    The quantizer input is y = x * r with x exact (fp16 -> fp32) and r one fp32
    per row, so it is the rotate+quantize recipe with the per-row constant c
    replaced by r: a = max|x| * r, s_h = fp16((clip * a) / 7),
    m = r * (1 / s_h), q = clamp(rne(x * m), -8, 7).  How r itself is rounded
    (the order of the fp32 sum of squares) is left to the kernel and checked
    against rms_multiplier() within its error bound.
    """
    x32 = np.asarray(x_f16, dtype=F16).astype(F32)
    return sym_quant_recipe_rows(x32, np.asarray(r_f32, dtype=F32), clip, bits)


# ---------------------------------------------------------------------------
# Hadamard heads + per-token INT4
# ---------------------------------------------------------------------------

def hadamard_heads_unnormalised(x: np.ndarray, n_heads: int) -> np.ndarray:
    """z = (H_{n_h} (x) I_{d_h}) x along the last axis, float64, no 1/sqrt(n_h)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert d % n_heads == 0
    dh = d // n_heads
    heads = x.reshape(x.shape[:-1] + (n_heads, dh))
    # move the head index last, transform it, move it back
    z = fwht(np.swapaxes(heads, -1, -2))
    return np.swapaxes(z, -1, -2).reshape(x.shape)


def hadamard_heads(x: np.ndarray, n_heads: int) -> np.ndarray:
    """y = (H_{n_h} (x) I) x / sqrt(n_h) (orthogonal), float64."""
    return hadamard_heads_unnormalised(x, n_heads) / np.sqrt(np.float64(n_heads))


def hadamard_heads_quant_math(x: np.ndarray, n_heads: int, clip: float = 1.0, bits: int = 4):
    """Float64 reference of the fused op: (codes, fp16 scales, y64)."""
    y = hadamard_heads(x, n_heads)
    q, s = sym_quant_math(y, clip, bits)
    return q, s, y


def hadamard_heads_quant_recipe(z: np.ndarray, n_heads: int, clip: float = 1.0, bits: int = 4):
    """Codes and fp16 scales from the fp32 transform output z (no 1/sqrt(n_h)),
    with c = fp32(1/sqrt(n_h)) per row, as in the rotate+quantize recipe."""
    z32 = np.asarray(z, dtype=F32)
    c = np.full(z32.shape[:-1], F32(1.0 / np.sqrt(np.float64(n_heads))), dtype=F32)
    return sym_quant_recipe_rows(z32, c, clip, bits)
