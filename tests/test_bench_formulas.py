"""CPU pins of the algorithmic-byte formulas behind bench.py's roofline figures: each
equals the summed sizes of the tensors the entry point reads and writes, in the
layouts include/qr.h documents (every input read once, every output written once)."""
import numpy as np
import pytest

import bench


def nbytes(*shapes_dtypes):
    return sum(int(np.prod(s)) * np.dtype(t).itemsize for s, t in shapes_dtypes)


@pytest.mark.parametrize("T,d", [(1, 4096), (37, 8192), (65536, 28672), (2048, 11008)])
def test_rotate_quant_bytes(T, d):
    # x fp16 [T, d] in; codes uint8 [T, d/2] and scales fp16 [T] out
    assert bench.hq_bytes(T, d) == nbytes(((T, d), np.float16), ((T, d // 2), np.uint8),
                                          ((T,), np.float16))
    # b-bit codes one per byte
    assert bench.i8_bytes(T, d) == nbytes(((T, d), np.float16), ((T, d), np.int8), ((T,), np.float16))


@pytest.mark.parametrize("T,N,K", [(65536, 28672, 8192), (1, 4096, 4096), (300, 260, 192)])
def test_gemm_bytes_and_ops(T, N, K):
    # A codes [T, K/2], W codes [N, K/2], fp16 scales [T] and [N] in; fp16 Y [T, N] out
    assert bench.gemm_bytes(T, N, K) == nbytes(((T, K // 2), np.uint8), ((N, K // 2), np.uint8),
                                               ((T,), np.float16), ((N,), np.float16),
                                               ((T, N), np.float16))
    assert bench.gemm8_bytes(T, N, K) == nbytes(((T, K), np.int8), ((N, K), np.int8),
                                                ((T,), np.float16), ((N,), np.float16),
                                                ((T, N), np.float16))
    assert bench.gemm_ops(T, N, K) == 2 * T * N * K      # one multiply and one add per MAC


@pytest.mark.parametrize("rows,dh,group", [(32 * 2048 * 8, 128, 128), (96, 64, 32)])
def test_kv_bytes(rows, dh, group):
    # fp16 [rows, dh] in; codes uint8 [rows, dh/2] and fp16 (scale, min) [rows, dh/group, 2] out
    assert bench.kv_bytes(rows, dh, group) == nbytes(((rows, dh), np.float16),
                                                     ((rows, dh // 2), np.uint8),
                                                     ((rows, dh // group, 2), np.float16))
    assert bench.rot_bytes(rows, dh) == nbytes(((rows, dh), np.float16), ((rows, dh), np.float16))


@pytest.mark.parametrize("b,hkv,hq,L,dh,group", [(32, 8, 64, 2098, 128, 128), (1, 2, 16, 300, 128, 128)])
def test_decode_bytes(b, hkv, hq, L, dh, group):
    # K and V caches over L positions (codes + (scale, min)) and the fp16 query in; fp16 output out
    cache = nbytes(((b, hkv, L, dh // 2), np.uint8), ((b, hkv, L, dh // group, 2), np.float16))
    assert bench.decode_bytes(b, hkv, hq, L, dh, group) == 2 * cache + nbytes(
        ((b, hq, dh), np.float16), ((b, hq, dh), np.float16))


def test_calibrated_mfma_ceiling_matches_its_source():
    # the committed register-loop calibration was taken on the current calibration
    # kernel source, and lies between the datasheet peak's power-limited share and it
    tops = bench.calibrated_mfma_tops()
    assert tops is not None
    assert 3000.0 < tops < bench.INT8_PEAK_TOPS


def test_calibrated_stream_ceiling_matches_its_source():
    gbs = bench.calibrated_stream_gbs()
    assert gbs is not None
    assert 4000.0 < gbs < bench.HBM_PEAK_GBS
