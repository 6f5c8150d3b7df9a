"""GPU parity of the b-bit variants (codes one per byte; 6- and 8-bit RTN of the
QuaRot paper's Table 9) against the oracle, through the C ABI:
qr_hadamard_quant_i8, qr_rmsnorm_quant_i8, qr_hadamard_heads_quant_i8 and
qr_w8a8_gemm.

Rules: the INT4 ones (tests/parity.py) with the b-bit code range -- R1 on the
transform, R2/R3 end to end against float64, bit-exact codes and scales against
the oracle's fp32 recipe on the GPU's own transform output (or RMS multiplier),
and bit-exact int32 accumulators and fp16 outputs of the GEMM.
"""
import numpy as np
import pytest

import workloads as wl
from oracle import block as ob
from oracle import gemm as og
from oracle import hadamard as oh
from oracle import quant as oq

from parity import check_codes_given_scale, check_rotation, check_scales

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
qr = pytest.importorskip("hadamard_rotation_int4_amd")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def check_codes_bits(q_gpu, s_gpu, y64, clip, bits):
    """R2 + R3 for b-bit codes against float64."""
    check_scales(s_gpu, y64, clip, bits)
    check_codes_given_scale(q_gpu, s_gpu, y64, bits)


# ---------------------------------------------------------------------------
# rotate + quantize, b-bit
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [8, 6])
@pytest.mark.parametrize("d", [128, 1024, 4096, 8192, 56, 3584, 28672, 344, 11008])
def test_hadamard_quant_i8_gaussian(d, bits):
    T = 13
    x = wl.activations(41, 0, T, d, n_outliers=min(4, d // 8))
    s = wl.signs(41, d)
    q, sc, z = (host(t) for t in qr.hadamard_quant_i8(dev(x), dev(s), 1.0, bits, z_dbg=True))
    z64 = oh.rotate_unnormalised(x.astype(np.float64), s)
    check_rotation(z, z64)
    check_codes_bits(q, sc, z64 / np.sqrt(d), 1.0, bits)
    q_rec, s_rec = oq.sym_quant_recipe(z, d, True, 1.0, bits)
    assert np.array_equal(sc.view(np.uint16), s_rec.view(np.uint16))
    assert np.array_equal(q, q_rec)


@pytest.mark.parametrize("d", [1024, 3584, 11008, 28672])
def test_hadamard_quant_i8_row_stride(d):
    # rows 16 elements into a wider buffer (row stride d + 64) on every kernel
    # family of the b-bit quantizer
    T, bits = 9, 8
    big = wl.activations(42, 0, T, d + 64, n_outliers=4)
    s = wl.signs(42, d)
    q, sc, z = (host(t) for t in qr.hadamard_quant_i8(dev(big)[:, 16:16 + d], dev(s), 1.0, bits,
                                                      z_dbg=True))
    x = big[:, 16:16 + d]
    z64 = oh.rotate_unnormalised(x.astype(np.float64), s)
    check_rotation(z, z64)
    check_codes_bits(q, sc, z64 / np.sqrt(d), 1.0, bits)
    q_rec, s_rec = oq.sym_quant_recipe(z, d, True, 1.0, bits)
    assert np.array_equal(sc.view(np.uint16), s_rec.view(np.uint16))
    assert np.array_equal(q, q_rec)


@pytest.mark.parametrize("bits", [8, 6, 4])
def test_hadamard_quant_i8_clip_and_no_rotation(bits):
    d = 4096
    x = wl.grid_activations(42, 0, 9, d)
    q, sc, z = (host(t) for t in qr.hadamard_quant_i8(dev(x), None, 0.5, bits, rotate=False,
                                                       z_dbg=True))
    assert np.array_equal(z, x.astype(np.float32))
    q_rec, s_rec = oq.sym_quant_recipe(x.astype(np.float32), d, False, 0.5, bits)
    assert np.array_equal(sc.view(np.uint16), s_rec.view(np.uint16)) and np.array_equal(q, q_rec)
    _, lo, hi = oq.code_range(bits)
    assert q.min() == lo and q.max() == hi


@pytest.mark.parametrize("d", [4096, 28672, 11008])
def test_i8_with_four_bits_matches_the_int4_kernels(d):
    # grid inputs: both transforms are exact, so the 4-bit codes one per byte
    # must be the nibbles the INT4 kernel packs
    x = wl.grid_activations(43, 0, 11, d)
    s = wl.signs(43, d)
    q8, s8 = qr.hadamard_quant_i8(dev(x), dev(s), 1.0, 4)
    q4, s4 = qr.hadamard_quant(dev(x), dev(s), 1.0)
    assert np.array_equal(host(s8).view(np.uint16), host(s4).view(np.uint16))
    assert np.array_equal(host(q8), oq.unpack_int4(host(q4)))


@pytest.mark.parametrize("bits", [8, 6])
@pytest.mark.parametrize("d", [28672, 11008, 8192])
def test_hadamard_quant_i8_edge_rows(d, bits):
    # zero row, constant row, a row whose scale is an fp16 subnormal (clamped
    # path), a single spike, a Gaussian row; bit-exact against the recipe
    s = wl.signs(44, d)
    x = np.zeros((5, d), dtype=np.float16)
    x[1] = 1.0
    x[2] = (wl.grid_activations(44, 0, 1, d)[0].astype(np.float64) * 2.0 ** -20).astype(np.float16)
    x[3, d // 3] = 3.0
    x[4] = wl.activations(44, 1, 1, d)[0]
    q, sc, z = (host(t) for t in qr.hadamard_quant_i8(dev(x), dev(s), 1.0, bits, z_dbg=True))
    z64 = oh.rotate_unnormalised(x.astype(np.float64), s)
    assert np.array_equal(z[:4].astype(np.float64), z64[:4])
    q_rec, s_rec = oq.sym_quant_recipe(z, d, True, 1.0, bits)
    assert np.array_equal(sc.view(np.uint16), s_rec.view(np.uint16)) and np.array_equal(q, q_rec)
    assert sc[0] == 0 and not q[0].any()


# ---------------------------------------------------------------------------
# RMSNorm and Hadamard heads, b-bit
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [8, 6])
@pytest.mark.parametrize("d", [72, 4096, 8192])
def test_rmsnorm_quant_i8(d, bits):
    x = wl.activations(44, 0, 21, d, n_outliers=min(5, d // 8))
    q, sc, r = (host(t) for t in qr.rmsnorm_quant_i8(dev(x), 1e-5, 1.0, bits, r_dbg=True))
    r64 = ob.rms_multiplier(x, 1e-5)
    assert (np.abs(r.astype(np.float64) - r64) / r64).max() <= 2e-5
    check_codes_bits(q, sc, x.astype(np.float64) * r64[:, None], 1.0, bits)
    q_rec, s_rec = ob.rmsnorm_quant_recipe(x, r, 1.0, bits)
    assert np.array_equal(sc.view(np.uint16), s_rec.view(np.uint16)) and np.array_equal(q, q_rec)


@pytest.mark.parametrize("bits", [8, 6])
@pytest.mark.parametrize("nh,dh", [(64, 128), (32, 128), (8, 64), (16, 512)])
def test_heads_quant_i8(nh, dh, bits):
    x = wl.activations(45, nh, 19, nh * dh)
    q, sc, z = (host(t) for t in qr.hadamard_heads_quant_i8(dev(x), nh, 1.0, bits, z_dbg=True))
    z64 = ob.hadamard_heads_unnormalised(x, nh)
    check_rotation(z, z64)
    check_codes_bits(q, sc, z64 / np.sqrt(nh), 1.0, bits)
    q_rec, s_rec = ob.hadamard_heads_quant_recipe(z, nh, 1.0, bits)
    assert np.array_equal(sc.view(np.uint16), s_rec.view(np.uint16)) and np.array_equal(q, q_rec)


# ---------------------------------------------------------------------------
# W8A8 GEMM
# ---------------------------------------------------------------------------

def int8_codes(seed, rows, k, lo=-128, hi=127):
    return np.random.default_rng(seed).integers(lo, hi + 1, size=(rows, k)).astype(np.int8)


@pytest.mark.parametrize("T,N,K", [(37, 100, 4096), (300, 520, 1040), (1, 64, 256), (64, 256, 8192),
                                   (513, 260, 4112), (256, 256, 128), (700, 900, 16)])
def test_w8a8_gemm_bit_exact(T, N, K):
    a = int8_codes(T * 7 + 1, T, K)
    w = int8_codes(N * 11 + 2, N, K)
    asc = wl.positive_scales(46, 0, T, 1e-4, 1e-2)
    wsc = wl.positive_scales(46, 1, N, 1e-4, 1e-2)
    y, acc = qr.w8a8_gemm(dev(a), dev(asc), dev(w), dev(wsc), acc_dbg=True)
    y_ref, acc_ref = og.w8a8_gemm(a, asc, w, wsc)
    assert np.array_equal(host(acc).astype(np.int64), acc_ref)
    assert np.array_equal(host(y).view(np.uint16), y_ref.view(np.uint16))


def test_w8a8_gemm_extreme_codes_past_2_24():
    # |acc| up to 2^14 K: fp32(acc) rounds to nearest even in the epilogue
    T, N, K = 64, 192, 8192
    a = int8_codes(47, T, K, -128, -100)
    w = int8_codes(48, N, K, -128, -90)
    asc = np.full(T, 2.0 ** -12, np.float16)
    wsc = wl.positive_scales(49, 0, N, 1e-4, 1e-3)
    y, acc = qr.w8a8_gemm(dev(a), dev(asc), dev(w), dev(wsc), acc_dbg=True)
    y_ref, acc_ref = og.w8a8_gemm(a, asc, w, wsc)
    assert acc_ref.min() > 2 ** 24
    assert np.array_equal(host(acc).astype(np.int64), acc_ref)
    assert np.array_equal(host(y).view(np.uint16), y_ref.view(np.uint16))


@pytest.mark.parametrize("bits", [8, 6])
def test_w8a8_linear_end_to_end(bits):
    # X, W rotated by the same randomized Hadamard and quantized to b bits; the
    # GEMM's accumulators are exact on the GPU's codes, and the output is close
    # to the unquantized product (more so at 8 bits than at 6)
    T, N, K = 64, 512, 4096
    x = wl.activations(50, 0, T, K, n_outliers=4, lo=50, hi=50)
    w = wl.weights(50, 1, N, K)
    s = wl.signs(50, K)
    qa, sa = qr.hadamard_quant_i8(dev(x), dev(s), 1.0, bits)
    qw, sw = qr.hadamard_quant_i8(dev(w), dev(s), 1.0, bits)
    y, acc = qr.w8a8_gemm(qa, sa, qw, sw, acc_dbg=True)
    acc_ref = og.int_matmul_exact(host(qa), host(qw))
    assert np.array_equal(host(acc).astype(np.int64), acc_ref)
    y_ref = og.epilogue_recipe(acc_ref, host(sa), host(sw))
    assert np.array_equal(host(y).view(np.uint16), y_ref.view(np.uint16))
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    err = np.linalg.norm(host(y).astype(np.float64) - exact) / np.linalg.norm(exact)
    # rounding noise of both operands: step max|row| / qmax with max|row| about
    # 4.5 standard deviations after the rotation, uniform error step / sqrt(12);
    # twice that as the bound
    qmax = oq.code_range(bits)[0]
    assert err < 2 * np.sqrt(2) * 4.5 / qmax / np.sqrt(12), err


@pytest.mark.parametrize("T,N,K", [(65536, 8192, 8192), (2048, 11008, 4096)])
def test_w8a8_gemm_full_size_sampled(T, N, K):
    g = torch.Generator(device="cuda")
    g.manual_seed(T + N + K)
    a = torch.randint(-128, 128, (T, K), generator=g, device="cuda", dtype=torch.int8)
    w = torch.randint(-128, 128, (N, K), generator=g, device="cuda", dtype=torch.int8)
    asc = torch.rand((T,), generator=g, device="cuda").mul(1e-3).add(1e-4).half()
    wsc = torch.rand((N,), generator=g, device="cuda").mul(1e-3).add(1e-4).half()
    y = qr.w8a8_gemm(a, asc, w, wsc)
    rows = np.unique(np.r_[np.random.default_rng(51).choice(T, 48, replace=False), 0, T - 1])
    cols = np.unique(np.r_[np.random.default_rng(52).choice(N, 512, replace=False), 0, N - 1])
    ri, ci = torch.as_tensor(rows, device="cuda"), torch.as_tensor(cols, device="cuda")
    y_ref, _ = og.w8a8_gemm(host(a[ri]), host(asc[ri]), host(w[ci]), host(wsc[ci]))
    assert np.array_equal(host(y[ri][:, ci]).view(np.uint16), y_ref.view(np.uint16))
