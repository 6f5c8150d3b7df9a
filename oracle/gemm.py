"""W4A4 GEMM: exact INT4 x INT4 -> INT32 product and the scale epilogue.
TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Definition (QuaRot paper, activation-quantization paragraph; performance
paragraph: INT4 GEMM with an INT32 accumulator): acc[t, n] = sum_k
A_q[t, k] W_q[n, k] exactly, then the output is acc times the token (row)
scale times the channel (column) scale.

Group-wise scales (one of the paper's studied variants): the accumulator of
each group of G consecutive k is scaled by that group's token and channel
scales and the groups are summed in fp32.

Reading taken: the pages cast the INT32 result to FP16 before scaling; that
overflows once |acc| > 65504 (|acc| can reach 64 K), so the epilogue works in
fp32 as Y = fp16_rne(fp32(fp32(acc) * a_s[t]) * w_s[n]).
"""
from __future__ import annotations

import numpy as np

from .quant import unpack_int4

F32 = np.float32
F16 = np.float16


def int_matmul_exact(a_codes: np.ndarray, w_codes: np.ndarray) -> np.ndarray:
    """acc = A W^T for int codes of at most 8 bits, exact, as int64.

    float64 BLAS is exact here: every product and partial sum is an integer of
    magnitude <= 2^14 K < 2^53, so no rounding happens in any summation order.
    """
    a = np.asarray(a_codes, dtype=np.float64)
    w = np.asarray(w_codes, dtype=np.float64)
    assert a.shape[-1] == w.shape[-1]
    assert np.abs(a).max(initial=0) <= 128 and np.abs(w).max(initial=0) <= 128
    assert a.shape[-1] * (1 << 14) < 2 ** 53
    return (a @ w.T).astype(np.int64)


int4_matmul_exact = int_matmul_exact


def int4_matmul_bruteforce(a_codes: np.ndarray, w_codes: np.ndarray) -> np.ndarray:
    """Triple loop in Python integers (tiny shapes only)."""
    a = np.asarray(a_codes).astype(int).tolist()
    w = np.asarray(w_codes).astype(int).tolist()
    return np.array([[sum(x * y for x, y in zip(ar, wr)) for wr in w] for ar in a], dtype=np.int64)


def w4a4_acc(a_packed: np.ndarray, w_packed: np.ndarray) -> np.ndarray:
    """Exact int64 accumulators from packed operands [T, K/2] and [N, K/2]."""
    return int4_matmul_exact(unpack_int4(a_packed), unpack_int4(w_packed))


def epilogue_recipe(acc: np.ndarray, a_scale: np.ndarray, w_scale: np.ndarray) -> np.ndarray:
    """fp16 Y = fp16_rne(fp32(fp32(acc) * a_s[t]) * w_s[n]).

    fp32(acc) is exact for INT4 codes (|acc| <= 64 K < 2^24); 8-bit codes can
    pass 2^24, and the conversion then rounds to nearest even."""
    acc32 = np.asarray(acc).astype(F32)
    a_s = np.asarray(a_scale, dtype=F16).astype(F32)[:, None]
    w_s = np.asarray(w_scale, dtype=F16).astype(F32)[None, :]
    with np.errstate(over="ignore"):
        y = ((acc32 * a_s).astype(F32) * w_s).astype(F32)
        return y.astype(F16)


def epilogue_math(acc: np.ndarray, a_scale: np.ndarray, w_scale: np.ndarray) -> np.ndarray:
    """float64 acc * a_s[t] * w_s[n]."""
    a_s = np.asarray(a_scale, dtype=F16).astype(np.float64)[:, None]
    w_s = np.asarray(w_scale, dtype=F16).astype(np.float64)[None, :]
    return np.asarray(acc, dtype=np.float64) * a_s * w_s


def w8a8_gemm(a_codes, a_scale, w_codes, w_scale) -> tuple[np.ndarray, np.ndarray]:
    """(fp16 Y, int64 acc) of the linear layer on b-bit codes stored one per
    byte (int8 [T, K] and [N, K]; QuaRot paper, 6- and 8-bit RTN results)."""
    acc = int_matmul_exact(a_codes, w_codes)
    return epilogue_recipe(acc, a_scale, w_scale), acc


def w4a4_gemm(a_packed, a_scale, w_packed, w_scale) -> tuple[np.ndarray, np.ndarray]:
    """(fp16 Y, int64 acc) of the W4A4 linear layer."""
    acc = w4a4_acc(a_packed, w_packed)
    return epilogue_recipe(acc, a_scale, w_scale), acc


def w4a4_gemm_groups_math(a_packed, a_scales, w_packed, w_scales, group: int) -> np.ndarray:
    """float64 Y = sum over groups g of acc_g * a_s[t, g] * w_s[n, g], acc_g the
    exact product of the codes of group g (group-wise scales on both operands)."""
    a = unpack_int4(a_packed).astype(np.float64)
    w = unpack_int4(w_packed).astype(np.float64)
    K = a.shape[-1]
    y = np.zeros((a.shape[0], w.shape[0]))
    for gi in range(K // group):
        sl = slice(gi * group, (gi + 1) * group)
        acc = a[:, sl] @ w[:, sl].T
        y += acc * np.asarray(a_scales, F16)[:, gi].astype(np.float64)[:, None] \
            * np.asarray(w_scales, F16)[:, gi].astype(np.float64)[None, :]
    return y


def w4a4_gemm_groups_recipe(a_packed, a_scales, w_packed, w_scales, group: int):
    """(fp16 Y, int64 per-group accumulators [G, T, N]) in the fp32 step order of
    the kernel: for g = 0, 1, ... in turn,
        p = fp32(fp32(fp32(acc_g) * a_s[t, g]) * w_s[n, g]);  f = fp32(f + p),
    starting from f = 0, then Y = fp16(f)."""
    a = unpack_int4(a_packed)
    w = unpack_int4(w_packed)
    K = a.shape[-1]
    f = np.zeros((a.shape[0], w.shape[0]), dtype=F32)
    accs = []
    for gi in range(K // group):
        sl = slice(gi * group, (gi + 1) * group)
        acc = int_matmul_exact(a[:, sl], w[:, sl])
        accs.append(acc)
        a_s = np.asarray(a_scales, F16)[:, gi].astype(F32)[:, None]
        w_s = np.asarray(w_scales, F16)[:, gi].astype(F32)[None, :]
        with np.errstate(over="ignore"):
            p = ((acc.astype(F32) * a_s).astype(F32) * w_s).astype(F32)
            f = (f + p).astype(F32)
    with np.errstate(over="ignore"):
        return f.astype(F16), np.stack(accs)
