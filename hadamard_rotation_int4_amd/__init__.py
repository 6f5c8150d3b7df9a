"""Python binding of libquarot_hip.so (QuaRot online Hadamard + INT4 hot path on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/qr.h``.  PyTorch supplies device
memory and the current stream.  If the shared library is missing the import
still succeeds, but the first call raises, naming the build command; nothing
falls back to a CPU or PyTorch implementation.

Functions (same names as the C entry points without the ``qr_`` prefix):
  hadamard_quant(x, signs, clip_ratio, rotate=True, z_dbg=False, fp16_transform=False)
      -> (q_u8, scale_f16[, z])
  hadamard(x, signs, out_dtype=torch.float32, out=None) -> y
  w4a4_gemm(a_q, a_scale, w_q, w_scale, acc_dbg=False) -> y_f16[, acc_i32]
  kv_rotate_quant(kv, signs, group, clip_ratio, cache_q, cache_meta, start_pos,
                  rotate=True, z_dbg=False) -> None[, z]
  rmsnorm_quant(x, eps, clip_ratio, r_dbg=False) -> (q_u8, scale_f16[, r])
  hadamard_heads_quant(x, n_heads, clip_ratio, z_dbg=False) -> (q_u8, scale_f16[, z])
  hadamard_quant_i8 / rmsnorm_quant_i8 / hadamard_heads_quant_i8(..., bits=8)
      -> (q_i8, scale_f16[, dbg]): b-bit codes one per byte (2 <= bits <= 8)
  w8a8_gemm(a_q, a_scale, w_q, w_scale, acc_dbg=False) -> y_f16[, acc_i32]
  hadamard_quant_groups(x, signs, clip_ratio, group) -> (q_u8, scale_f16 [T, d/group][, z])
  w4a4_gemm_groups(a_q, a_scale [T, K/group], w_q, w_scale [N, K/group], group) -> y_f16
  kv_decode_attention(q, k_q, k_meta, v_q, v_meta, L, group, scale, out=None, workspace=None)
  kv_decode_attention_noalloc(q, k_q, k_meta, v_q, v_meta, L, group, scale, out=None)
      -> out_f16: the same Decode routine with the library's static scratch
  hadamard_factor(d) -> (n, m);  abi_version();  status_str(code)
"""
from __future__ import annotations

import ctypes
import math
import os
from pathlib import Path

LIB_PATH = Path(__file__).resolve().parent / "lib" / "libquarot_hip.so"

QR_ROT_NONE = 0
QR_ROT_HADAMARD = 1
QR_ROT_HADAMARD_F16 = 2

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m hadamard_rotation_int4_amd.build`"
            " (there is no CPU or PyTorch fallback)")
    lib = ctypes.CDLL(str(LIB_PATH))
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    lib.qr_abi_version.restype = ctypes.c_int
    lib.qr_abi_version.argtypes = []
    lib.qr_status_str.restype = ctypes.c_char_p
    lib.qr_status_str.argtypes = [ctypes.c_int]
    lib.qr_hadamard_factor.restype = ctypes.c_int
    lib.qr_hadamard_factor.argtypes = [i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.qr_hadamard_quant.restype = ctypes.c_int
    lib.qr_hadamard_quant.argtypes = [vp, i64, i32, i64, ctypes.c_int, vp, f32, vp, vp, vp, vp]
    lib.qr_hadamard.restype = ctypes.c_int
    lib.qr_hadamard.argtypes = [vp, i64, i32, i64, vp, vp, i32, vp]
    lib.qr_w4a4_gemm.restype = ctypes.c_int
    lib.qr_w4a4_gemm.argtypes = [vp, vp, i64, vp, vp, i64, i64, vp, vp, vp]
    lib.qr_kv_rotate_quant.restype = ctypes.c_int
    lib.qr_kv_rotate_quant.argtypes = [vp, i32, i32, i32, i32, i64, ctypes.c_int, vp, i32, f32,
                                       vp, vp, i32, i32, vp, vp]
    lib.qr_rmsnorm_quant.restype = ctypes.c_int
    lib.qr_rmsnorm_quant.argtypes = [vp, i64, i32, i64, f32, f32, vp, vp, vp, vp]
    lib.qr_hadamard_heads_quant.restype = ctypes.c_int
    lib.qr_hadamard_heads_quant.argtypes = [vp, i64, i32, i32, i64, f32, vp, vp, vp, vp]
    lib.qr_hadamard_quant_i8.restype = ctypes.c_int
    lib.qr_hadamard_quant_i8.argtypes = [vp, i64, i32, i64, ctypes.c_int, vp, f32, i32, vp, vp, vp,
                                         vp]
    lib.qr_rmsnorm_quant_i8.restype = ctypes.c_int
    lib.qr_rmsnorm_quant_i8.argtypes = [vp, i64, i32, i64, f32, f32, i32, vp, vp, vp, vp]
    lib.qr_hadamard_heads_quant_i8.restype = ctypes.c_int
    lib.qr_hadamard_heads_quant_i8.argtypes = [vp, i64, i32, i32, i64, f32, i32, vp, vp, vp, vp]
    lib.qr_hadamard_quant_groups.restype = ctypes.c_int
    lib.qr_hadamard_quant_groups.argtypes = [vp, i64, i32, i64, ctypes.c_int, vp, f32, i32, vp, vp,
                                             vp, vp]
    lib.qr_w4a4_gemm_groups.restype = ctypes.c_int
    lib.qr_w4a4_gemm_groups.argtypes = [vp, vp, i64, vp, vp, i64, i64, i32, vp, vp]
    lib.qr_w8a8_gemm.restype = ctypes.c_int
    lib.qr_w8a8_gemm.argtypes = [vp, vp, i64, vp, vp, i64, i64, vp, vp, vp]
    lib.qr_kv_rotate_quant_bits.restype = ctypes.c_int
    lib.qr_kv_rotate_quant_bits.argtypes = [vp, i32, i32, i32, i32, i64, ctypes.c_int, vp, i32, f32,
                                            i32, vp, vp, i32, i32, vp, vp]
    lib.qr_kv_decode_workspace_bytes.restype = i64
    lib.qr_kv_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.qr_kv_decode_attention.restype = ctypes.c_int
    lib.qr_kv_decode_attention.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, i32, i32, i32,
                                           f32, vp, vp, i64, vp]
    lib.qr_kv_decode_attention_noalloc.restype = ctypes.c_int
    lib.qr_kv_decode_attention_noalloc.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, i32,
                                                   i32, i32, f32, vp, vp]
    lib.qr_calibrate_mfma_i8.restype = ctypes.c_int
    lib.qr_calibrate_mfma_i8.argtypes = [vp, i32, i32, vp, vp, vp]
    lib.qr_calibrate_stream.restype = ctypes.c_int
    lib.qr_calibrate_stream.argtypes = [vp, i64, vp, i32, vp]
    _lib = lib
    return lib


def lib_loaded_path() -> str:
    _load()
    return str(LIB_PATH)


def abi_version() -> int:
    return int(_load().qr_abi_version())


def status_str(code: int) -> str:
    return _load().qr_status_str(int(code)).decode()


def _check(code: int, what: str) -> None:
    if code != 0:
        raise RuntimeError(f"{what}: {status_str(code)}")


def hadamard_factor(d: int) -> tuple[int, int]:
    n, m = ctypes.c_int32(), ctypes.c_int32()
    _check(_load().qr_hadamard_factor(int(d), ctypes.byref(n), ctypes.byref(m)),
           f"qr_hadamard_factor({d})")
    return n.value, m.value


# ---------------------------------------------------------------------------
# torch marshalling
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, dtype, name, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


def _signs(signs, d, device):
    torch = _torch()
    if signs is None:
        return None
    _need(signs, torch.int8, "signs", 1)
    if signs.numel() != d or not signs.is_contiguous():
        raise ValueError(f"signs must be a contiguous int8 vector of length {d}")
    if signs.device != device:
        raise ValueError("signs must be on the same device as x")
    return signs


def hadamard_quant(x, signs=None, clip_ratio: float = 1.0, rotate: bool = True,
                   z_dbg: bool = False, out=None, stream=None, fp16_transform: bool = False):
    """Rotate (optionally) and quantize the rows of x [T, d] (fp16, row stride % 8 == 0).

    Returns (q uint8 [T, d/2], scale fp16 [T]) and, with z_dbg, z fp32 [T, d].
    ``out`` may pass preallocated (q, scale) tensors.  ``fp16_transform`` selects
    QR_ROT_HADAMARD_F16 (the transform's additions in fp16; d = 28672 and 11008).
    """
    torch = _torch()
    _need(x, torch.float16, "x", 2)
    if x.numel() and x.stride(1) != 1:
        raise ValueError("x rows must be contiguous (stride(1) == 1)")
    T, d = x.shape
    s = _signs(signs, d, x.device) if rotate else None
    if out is None:
        q = torch.empty((T, d // 2), dtype=torch.uint8, device=x.device)
        sc = torch.empty((T,), dtype=torch.float16, device=x.device)
    else:
        q, sc = out
        _need(q, torch.uint8, "q")
        _need(sc, torch.float16, "scale")
        if q.numel() != T * (d // 2) or not q.is_contiguous() or sc.numel() != T:
            raise ValueError("out tensors have the wrong size or layout")
    z = torch.empty((T, d), dtype=torch.float32, device=x.device) if z_dbg else None
    code = _load().qr_hadamard_quant(_ptr(x), T, d, x.stride(0) if T > 0 else d,
                                     (QR_ROT_HADAMARD_F16 if fp16_transform else QR_ROT_HADAMARD)
                                     if rotate else QR_ROT_NONE, _ptr(s),
                                     float(clip_ratio), _ptr(q), _ptr(sc), _ptr(z), _stream(stream))
    _check(code, "qr_hadamard_quant")
    return (q, sc, z) if z_dbg else (q, sc)


def _quant_out(out, T, d, device, i8=False):
    """(codes, scales) outputs: packed uint8 [T, d/2], or int8 [T, d] one code per byte."""
    torch = _torch()
    qdt, qw = (torch.int8, d) if i8 else (torch.uint8, d // 2)
    if out is None:
        return (torch.empty((T, qw), dtype=qdt, device=device),
                torch.empty((T,), dtype=torch.float16, device=device))
    q, sc = out
    _need(q, qdt, "q")
    _need(sc, torch.float16, "scale")
    if q.numel() != T * qw or not q.is_contiguous() or sc.numel() != T:
        raise ValueError("out tensors have the wrong size or layout")
    return q, sc


def _rows(x):
    torch = _torch()
    _need(x, torch.float16, "x", 2)
    if x.numel() and x.stride(1) != 1:
        raise ValueError("x rows must be contiguous (stride(1) == 1)")
    return x.shape


def rmsnorm_quant(x, eps: float = 1e-5, clip_ratio: float = 1.0, r_dbg: bool = False,
                  out=None, stream=None):
    """RMSNorm without scale (fp32) + per-token INT4 of the rows of x [T, d] (fp16).

    Returns (q uint8 [T, d/2], scale fp16 [T]) and, with r_dbg, the fp32
    multiplier r = 1/sqrt(mean(x^2) + eps) per row."""
    torch = _torch()
    _need(x, torch.float16, "x", 2)
    if x.numel() and x.stride(1) != 1:
        raise ValueError("x rows must be contiguous (stride(1) == 1)")
    T, d = x.shape
    q, sc = _quant_out(out, T, d, x.device)
    r = torch.empty((T,), dtype=torch.float32, device=x.device) if r_dbg else None
    code = _load().qr_rmsnorm_quant(_ptr(x), T, d, x.stride(0) if T > 0 else d, float(eps),
                                    float(clip_ratio), _ptr(q), _ptr(sc), _ptr(r), _stream(stream))
    _check(code, "qr_rmsnorm_quant")
    return (q, sc, r) if r_dbg else (q, sc)


def hadamard_heads_quant(x, n_heads: int, clip_ratio: float = 1.0, z_dbg: bool = False,
                         out=None, stream=None):
    """Hadamard heads (H_nh (x) I) / sqrt(nh) + per-token INT4 of the rows of x [T, nh*dh].

    Returns (q uint8 [T, d/2], scale fp16 [T]) and, with z_dbg, z fp32 [T, d]
    (the transform before 1/sqrt(nh))."""
    torch = _torch()
    _need(x, torch.float16, "x", 2)
    if x.numel() and x.stride(1) != 1:
        raise ValueError("x rows must be contiguous (stride(1) == 1)")
    T, d = x.shape
    if n_heads <= 0 or d % n_heads:
        raise ValueError(f"row width {d} is not a multiple of n_heads={n_heads}")
    q, sc = _quant_out(out, T, d, x.device)
    z = torch.empty((T, d), dtype=torch.float32, device=x.device) if z_dbg else None
    code = _load().qr_hadamard_heads_quant(_ptr(x), T, int(n_heads), d // int(n_heads),
                                           x.stride(0) if T > 0 else d, float(clip_ratio),
                                           _ptr(q), _ptr(sc), _ptr(z), _stream(stream))
    _check(code, "qr_hadamard_heads_quant")
    return (q, sc, z) if z_dbg else (q, sc)


def hadamard_quant_i8(x, signs=None, clip_ratio: float = 1.0, bits: int = 8,
                      rotate: bool = True, z_dbg: bool = False, out=None, stream=None):
    """As hadamard_quant with b-bit codes one per byte: (q int8 [T, d], scale[, z])."""
    torch = _torch()
    T, d = _rows(x)
    s = _signs(signs, d, x.device) if rotate else None
    q, sc = _quant_out(out, T, d, x.device, i8=True)
    z = torch.empty((T, d), dtype=torch.float32, device=x.device) if z_dbg else None
    code = _load().qr_hadamard_quant_i8(_ptr(x), T, d, x.stride(0) if T > 0 else d,
                                        QR_ROT_HADAMARD if rotate else QR_ROT_NONE, _ptr(s),
                                        float(clip_ratio), int(bits), _ptr(q), _ptr(sc), _ptr(z),
                                        _stream(stream))
    _check(code, "qr_hadamard_quant_i8")
    return (q, sc, z) if z_dbg else (q, sc)


def hadamard_quant_groups(x, signs=None, clip_ratio: float = 1.0, group: int = 128,
                          rotate: bool = True, z_dbg: bool = False, out=None, stream=None):
    """As hadamard_quant with one scale per group of `group` elements:
    (q uint8 [T, d/2], scale fp16 [T, d/group][, z])."""
    torch = _torch()
    T, d = _rows(x)
    s = _signs(signs, d, x.device) if rotate else None
    if out is None:
        q = torch.empty((T, d // 2), dtype=torch.uint8, device=x.device)
        sc = torch.empty((T, max(d // max(group, 1), 1)), dtype=torch.float16, device=x.device)
    else:
        q, sc = out
        _need(q, torch.uint8, "q")
        _need(sc, torch.float16, "scale")
        if q.numel() != T * (d // 2) or not q.is_contiguous() or not sc.is_contiguous() or \
                sc.numel() != T * (d // max(group, 1)):
            raise ValueError("out tensors have the wrong size or layout")
    z = torch.empty((T, d), dtype=torch.float32, device=x.device) if z_dbg else None
    code = _load().qr_hadamard_quant_groups(_ptr(x), T, d, x.stride(0) if T > 0 else d,
                                            QR_ROT_HADAMARD if rotate else QR_ROT_NONE, _ptr(s),
                                            float(clip_ratio), int(group), _ptr(q), _ptr(sc),
                                            _ptr(z), _stream(stream))
    _check(code, "qr_hadamard_quant_groups")
    return (q, sc, z) if z_dbg else (q, sc)


def rmsnorm_quant_i8(x, eps: float = 1e-5, clip_ratio: float = 1.0, bits: int = 8,
                     r_dbg: bool = False, out=None, stream=None):
    """As rmsnorm_quant with b-bit codes one per byte: (q int8 [T, d], scale[, r])."""
    torch = _torch()
    T, d = _rows(x)
    q, sc = _quant_out(out, T, d, x.device, i8=True)
    r = torch.empty((T,), dtype=torch.float32, device=x.device) if r_dbg else None
    code = _load().qr_rmsnorm_quant_i8(_ptr(x), T, d, x.stride(0) if T > 0 else d, float(eps),
                                       float(clip_ratio), int(bits), _ptr(q), _ptr(sc), _ptr(r),
                                       _stream(stream))
    _check(code, "qr_rmsnorm_quant_i8")
    return (q, sc, r) if r_dbg else (q, sc)


def hadamard_heads_quant_i8(x, n_heads: int, clip_ratio: float = 1.0, bits: int = 8,
                            z_dbg: bool = False, out=None, stream=None):
    """As hadamard_heads_quant with b-bit codes one per byte: (q int8 [T, d], scale[, z])."""
    torch = _torch()
    T, d = _rows(x)
    if n_heads <= 0 or d % n_heads:
        raise ValueError(f"row width {d} is not a multiple of n_heads={n_heads}")
    q, sc = _quant_out(out, T, d, x.device, i8=True)
    z = torch.empty((T, d), dtype=torch.float32, device=x.device) if z_dbg else None
    code = _load().qr_hadamard_heads_quant_i8(_ptr(x), T, int(n_heads), d // int(n_heads),
                                              x.stride(0) if T > 0 else d, float(clip_ratio),
                                              int(bits), _ptr(q), _ptr(sc), _ptr(z),
                                              _stream(stream))
    _check(code, "qr_hadamard_heads_quant_i8")
    return (q, sc, z) if z_dbg else (q, sc)


def hadamard(x, signs=None, out_dtype=None, stream=None, out=None):
    """y = H_d diag(s) x / sqrt(d) row-wise; x fp16 [T, d]; y fp32 (default) or fp16.

    ``out``: optional preallocated contiguous [T, d] tensor of ``out_dtype``."""
    torch = _torch()
    out_dtype = (out.dtype if out is not None else torch.float32) if out_dtype is None else out_dtype
    _need(x, torch.float16, "x", 2)
    if x.numel() and x.stride(1) != 1:
        raise ValueError("x rows must be contiguous (stride(1) == 1)")
    if out_dtype not in (torch.float32, torch.float16):
        raise ValueError("out_dtype must be float32 or float16")
    T, d = x.shape
    s = _signs(signs, d, x.device)
    if out is not None:
        _need(out, out_dtype, "out", 2)
        if tuple(out.shape) != (T, d) or not out.is_contiguous():
            raise ValueError("out must be a contiguous [T, d] tensor")
        y = out
    else:
        y = torch.empty((T, d), dtype=out_dtype, device=x.device)
    code = _load().qr_hadamard(_ptr(x), T, d, x.stride(0) if T > 0 else d, _ptr(s), _ptr(y),
                               1 if out_dtype == torch.float32 else 0, _stream(stream))
    _check(code, "qr_hadamard")
    return y


def w4a4_gemm(a_q, a_scale, w_q, w_scale, acc_dbg: bool = False, out=None, stream=None):
    """Y fp16 [T, N] = dequant(A_q W_q^T); a_q uint8 [T, K/2], w_q uint8 [N, K/2]."""
    return _gemm(a_q, a_scale, w_q, w_scale, acc_dbg, out, stream, False)


def w8a8_gemm(a_q, a_scale, w_q, w_scale, acc_dbg: bool = False, out=None, stream=None):
    """Y fp16 [T, N] = dequant(A_q W_q^T); a_q int8 [T, K], w_q int8 [N, K] (codes one per byte)."""
    return _gemm(a_q, a_scale, w_q, w_scale, acc_dbg, out, stream, True)


def w4a4_gemm_groups(a_q, a_scale, w_q, w_scale, group: int, out=None, stream=None):
    """Y fp16 [T, N] with group-wise scales: a_q uint8 [T, K/2], a_scale fp16 [T, K/group],
    w_q uint8 [N, K/2], w_scale fp16 [N, K/group]."""
    torch = _torch()
    _need(a_q, torch.uint8, "a_q", 2)
    _need(w_q, torch.uint8, "w_q", 2)
    _need(a_scale, torch.float16, "a_scale", 2)
    _need(w_scale, torch.float16, "w_scale", 2)
    for name, t in (("a_q", a_q), ("w_q", w_q), ("a_scale", a_scale), ("w_scale", w_scale)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    T, kh = a_q.shape
    N, kh2 = w_q.shape
    K = 2 * kh
    if kh != kh2 or group <= 0 or K % group or tuple(a_scale.shape) != (T, K // group) or \
            tuple(w_scale.shape) != (N, K // group):
        raise ValueError("inconsistent GEMM operand shapes")
    y = torch.empty((T, N), dtype=torch.float16, device=a_q.device) if out is None else out
    if out is not None:
        _need(y, torch.float16, "out", 2)
        if tuple(y.shape) != (T, N) or not y.is_contiguous():
            raise ValueError("out must be a contiguous fp16 [T, N] tensor")
    code = _load().qr_w4a4_gemm_groups(_ptr(a_q), _ptr(a_scale), T, _ptr(w_q), _ptr(w_scale), N,
                                       K, int(group), _ptr(y), _stream(stream))
    _check(code, "qr_w4a4_gemm_groups")
    return y


def _gemm(a_q, a_scale, w_q, w_scale, acc_dbg, out, stream, i8):
    torch = _torch()
    cdt = torch.int8 if i8 else torch.uint8
    _need(a_q, cdt, "a_q", 2)
    _need(w_q, cdt, "w_q", 2)
    _need(a_scale, torch.float16, "a_scale", 1)
    _need(w_scale, torch.float16, "w_scale", 1)
    for name, t in (("a_q", a_q), ("w_q", w_q), ("a_scale", a_scale), ("w_scale", w_scale)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    T, kh = a_q.shape
    N, kh2 = w_q.shape
    if kh != kh2 or a_scale.numel() != T or w_scale.numel() != N:
        raise ValueError("inconsistent GEMM operand shapes")
    K = kh if i8 else 2 * kh
    y = torch.empty((T, N), dtype=torch.float16, device=a_q.device) if out is None else out
    if out is not None:
        _need(y, torch.float16, "out", 2)
        if tuple(y.shape) != (T, N) or not y.is_contiguous():
            raise ValueError("out must be a contiguous fp16 [T, N] tensor")
    acc = torch.empty((T, N), dtype=torch.int32, device=a_q.device) if acc_dbg else None
    fn = _load().qr_w8a8_gemm if i8 else _load().qr_w4a4_gemm
    code = fn(_ptr(a_q), _ptr(a_scale), T, _ptr(w_q), _ptr(w_scale), N, K, _ptr(y), _ptr(acc),
              _stream(stream))
    _check(code, "qr_w8a8_gemm" if i8 else "qr_w4a4_gemm")
    return (y, acc) if acc_dbg else y


def kv_rotate_quant(kv, signs, group: int, clip_ratio: float, cache_q, cache_meta,
                    start_pos: int, rotate: bool = True, z_dbg: bool = False, stream=None,
                    bits: int = 4):
    """Quantize kv fp16 [B, S_new, H, Dh] (last dim contiguous, heads packed) into the cache.

    cache_q uint8 [B, H, S_max, Dh/2]; cache_meta fp16 [B, H, S_max, Dh/group, 2].
    bits in {2, 3, 4}: codes with 2^bits - 1 levels, in the same 4-bit layout.
    Returns z fp32 [B, S_new, H, Dh] when z_dbg.
    """
    torch = _torch()
    _need(kv, torch.float16, "kv", 4)
    _need(cache_q, torch.uint8, "cache_q", 4)
    _need(cache_meta, torch.float16, "cache_meta", 5)
    B, S_new, H, Dh = kv.shape
    if kv.stride(3) != 1 or kv.stride(2) != Dh or (S_new > 1 and kv.stride(0) != S_new * kv.stride(1)):
        raise ValueError("kv must be [B, S_new, H, Dh] with heads packed and one token stride")
    if not cache_q.is_contiguous() or not cache_meta.is_contiguous():
        raise ValueError("cache tensors must be contiguous")
    S_max = cache_q.shape[2]
    if tuple(cache_q.shape) != (B, H, S_max, Dh // 2) or \
            tuple(cache_meta.shape) != (B, H, S_max, Dh // group, 2):
        raise ValueError("cache tensors have the wrong shape")
    ld = kv.stride(1) if S_new > 1 else (kv.stride(0) if B > 1 else H * Dh)
    s = _signs(signs, Dh, kv.device) if rotate else None
    z = torch.empty((B, S_new, H, Dh), dtype=torch.float32, device=kv.device) if z_dbg else None
    rot = QR_ROT_HADAMARD if rotate else QR_ROT_NONE
    if bits == 4:
        code = _load().qr_kv_rotate_quant(_ptr(kv), B, S_new, H, Dh, ld, rot, _ptr(s), int(group),
                                          float(clip_ratio), _ptr(cache_q), _ptr(cache_meta),
                                          S_max, int(start_pos), _ptr(z), _stream(stream))
    else:
        code = _load().qr_kv_rotate_quant_bits(_ptr(kv), B, S_new, H, Dh, ld, rot, _ptr(s),
                                               int(group), float(clip_ratio), int(bits),
                                               _ptr(cache_q), _ptr(cache_meta), S_max,
                                               int(start_pos), _ptr(z), _stream(stream))
    _check(code, "qr_kv_rotate_quant" if bits == 4 else "qr_kv_rotate_quant_bits")
    return z


def kv_decode_workspace_bytes(B: int, Hq: int, Hkv: int, Dh: int, L: int) -> int:
    return int(_load().qr_kv_decode_workspace_bytes(B, Hq, Hkv, Dh, L))


def _decode_args(q, k_cache_q, k_cache_meta, v_cache_q, v_cache_meta, group, softmax_scale, out):
    torch = _torch()
    _need(q, torch.float16, "q", 3)
    for t, nm in ((k_cache_q, "k_cache_q"), (v_cache_q, "v_cache_q")):
        _need(t, torch.uint8, nm, 4)
    for t, nm in ((k_cache_meta, "k_cache_meta"), (v_cache_meta, "v_cache_meta")):
        _need(t, torch.float16, nm, 5)
    B, Hq, Dh = q.shape
    _, Hkv, S_max, _ = k_cache_q.shape
    for t in (q, k_cache_q, v_cache_q, k_cache_meta, v_cache_meta):
        if not t.is_contiguous():
            raise ValueError("q and the cache tensors must be contiguous")
    if tuple(k_cache_q.shape) != (B, Hkv, S_max, Dh // 2) or tuple(v_cache_q.shape) != tuple(k_cache_q.shape) \
            or tuple(k_cache_meta.shape) != (B, Hkv, S_max, Dh // group, 2) \
            or tuple(v_cache_meta.shape) != tuple(k_cache_meta.shape):
        raise ValueError("cache tensors have the wrong shape")
    scale = float(softmax_scale) if softmax_scale is not None else 1.0 / math.sqrt(Dh)
    o = out if out is not None else torch.empty((B, Hq, Dh), dtype=torch.float16, device=q.device)
    if out is not None:
        _need(o, torch.float16, "out", 3)
        if tuple(o.shape) != (B, Hq, Dh) or not o.is_contiguous():
            raise ValueError("out must be a contiguous fp16 [B, Hq, Dh] tensor")
    return B, Hq, Hkv, Dh, S_max, scale, o


def kv_decode_attention(q, k_cache_q, k_cache_meta, v_cache_q, v_cache_meta, L: int,
                        group: int = 128, softmax_scale: float | None = None, out=None,
                        workspace=None, stream=None):
    """Decode attention of q fp16 [B, Hq, Dh] over positions 0 .. L-1 of the 4-bit cache.

    Caches as qr_kv_rotate_quant writes them: codes uint8 [B, Hkv, S_max, Dh/2],
    meta fp16 [B, Hkv, S_max, Dh/group, 2].  Returns fp16 [B, Hq, Dh].
    """
    torch = _torch()
    B, Hq, Hkv, Dh, S_max, scale, o = _decode_args(q, k_cache_q, k_cache_meta, v_cache_q,
                                                   v_cache_meta, group, softmax_scale, out)
    nbytes = kv_decode_workspace_bytes(B, Hq, Hkv, Dh, int(L)) if B > 0 else 0
    if workspace is None:
        workspace = torch.empty((max(nbytes, 4),), dtype=torch.uint8, device=q.device)
    code = _load().qr_kv_decode_attention(_ptr(q), B, Hq, Hkv, Dh, _ptr(k_cache_q),
                                          _ptr(k_cache_meta), _ptr(v_cache_q), _ptr(v_cache_meta),
                                          S_max, int(L), int(group), scale, _ptr(o),
                                          _ptr(workspace), workspace.numel() * workspace.element_size(),
                                          _stream(stream))
    _check(code, "qr_kv_decode_attention")
    return o


def kv_decode_attention_noalloc(q, k_cache_q, k_cache_meta, v_cache_q, v_cache_meta, L: int,
                                group: int = 128, softmax_scale: float | None = None, out=None,
                                stream=None):
    """kv_decode_attention through the allocation-free entry point (the library's
    static per-GPU scratch instead of a workspace).  Pass ``out`` to allocate
    nothing on this side either."""
    B, Hq, Hkv, Dh, S_max, scale, o = _decode_args(q, k_cache_q, k_cache_meta, v_cache_q,
                                                   v_cache_meta, group, softmax_scale, out)
    code = _load().qr_kv_decode_attention_noalloc(_ptr(q), B, Hq, Hkv, Dh, _ptr(k_cache_q),
                                                  _ptr(k_cache_meta), _ptr(v_cache_q),
                                                  _ptr(v_cache_meta), S_max, int(L), int(group),
                                                  scale, _ptr(o), _stream(stream))
    _check(code, "qr_kv_decode_attention_noalloc")
    return o


def calibrate_mfma_i8(fragments, grid: int, iters: int, clocks: bool = False, stream=None):
    """Register-only loop of the GEMM's int8 MFMA (measurement support, not part
    of the method): ``fragments`` is int8 [64, 16] on the GPU.  Returns the
    int32 [grid * 256] per-thread checksums and, with ``clocks``, the uint64
    [grid, 4] counters (shader clock start/end, 100 MHz counter start/end)."""
    torch = _torch()
    _need(fragments, torch.int8, "fragments", 2)
    if tuple(fragments.shape) != (64, 16) or not fragments.is_contiguous():
        raise ValueError("fragments must be a contiguous int8 [64, 16] tensor")
    dev = fragments.device
    chk = torch.empty((int(grid) * 256,), dtype=torch.int32, device=dev)
    clk = torch.empty((int(grid), 4), dtype=torch.uint64, device=dev) if clocks else None
    code = _load().qr_calibrate_mfma_i8(_ptr(fragments), int(grid), int(iters), _ptr(chk),
                                        _ptr(clk), _stream(stream))
    _check(code, "qr_calibrate_mfma_i8")
    return (chk, clk) if clocks else chk


def calibrate_stream(src, grid: int, out=None, stream=None):
    """Plain stream with the rotate+quant traffic mix (measurement support, not
    part of the method): ``src`` is a contiguous GPU tensor whose byte size is a
    multiple of 16; returns uint32 [bytes / 16], the XOR of each 16-byte chunk's
    four dwords."""
    torch = _torch()
    if not isinstance(src, torch.Tensor) or not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous GPU tensor")
    nbytes = src.numel() * src.element_size()
    if nbytes % 16:
        raise ValueError("src must hold a whole number of 16-byte chunks")
    n16 = nbytes // 16
    if out is None:
        out = torch.empty((n16,), dtype=torch.uint32, device=src.device)
    elif out.dtype != torch.uint32 or out.numel() != n16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous uint32 tensor of bytes / 16 elements")
    code = _load().qr_calibrate_stream(_ptr(src), n16, _ptr(out), int(grid), _stream(stream))
    _check(code, "qr_calibrate_stream")
    return out
