"""Pins for the oracle's symmetric INT4 quantizer, packing and GEMM."""
import json
import os

import numpy as np
import pytest

import workloads as wl
from oracle import gemm, hadamard as had, quant
from oracle import quant as oq

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_pack_order_hand_built():
    # byte j: code 2j in the low nibble, code 2j+1 in the high nibble, two's complement
    codes = np.array([[1, -1, 7, -8, 0, 3]])
    assert quant.pack_int4(codes).tolist() == [[0xF1, 0x87, 0x30]]
    assert quant.unpack_int4(np.array([[0xF1, 0x87, 0x30]], dtype=np.uint8)).tolist() == codes.tolist()


def test_pack_roundtrip_all_pairs():
    a, b = np.meshgrid(np.arange(-8, 8), np.arange(-8, 8))
    codes = np.stack([a.ravel(), b.ravel()], axis=1)
    packed = quant.pack_int4(codes)
    assert sorted(packed.ravel().tolist()) == list(range(256))
    assert np.array_equal(quant.unpack_int4(packed), codes)


def test_scale_one_gives_plain_rounding():
    # max|y| = 7 -> s = 1 exactly, so codes are round-half-even(y)
    y = np.array([[7.0, 2.5, -2.5, 3.5, -0.5, 0.5, 1.5, 0.0, -6.49, 4.51]])
    q, s = quant.sym_quant_math(y)
    assert s.tolist() == [1.0]
    assert q.tolist() == [[7, 2, -2, 4, 0, 0, 2, 0, -6, 5]]
    q2, s2 = quant.sym_quant_recipe(y.astype(np.float32), 10, rotated=False)
    assert q2.tolist() == q.tolist() and s2.tolist() == [1.0]


def test_blog_bucket_example():
    g = json.load(open(os.path.join(GOLDEN, "blog_quant_bucket_example.json")))
    a, b = g["values_same_bucket"]
    y = np.array([[g["row_max"], a, b, -1.0]])
    q, s = quant.sym_quant_math(y)
    assert float(s[0]) == pytest.approx(g["expected_scale"], rel=1e-3)  # fp16 scale
    assert q[0, 0] == g["expected_code_of_max"]
    assert q[0, 1] == q[0, 2]


def test_clip_drives_plus_eight_to_seven():
    # clip 0.9: s = 0.9 for max 7, 7/0.9 = 7.78 rounds to 8 -> clamped to 7; -7.78 -> -8 is kept
    y = np.array([[7.0, -7.0, 0.9, -0.40]])
    q, s = quant.sym_quant_math(y, clip=0.9)
    assert float(s[0]) == pytest.approx(0.9, rel=1e-3)
    assert q.tolist() == [[7, -8, 1, 0]]
    q2, _ = quant.sym_quant_recipe(y.astype(np.float32), 4, rotated=False, clip=0.9)
    assert q2.tolist() == q.tolist()


def test_zero_row():
    y = np.zeros((2, 16))
    y[1, 3] = 1.0
    q, s = quant.sym_quant_math(y)
    assert s[0] == 0 and not q[0].any()
    q2, s2 = quant.sym_quant_recipe(y.astype(np.float32), 16, rotated=True)
    assert s2[0] == 0 and not q2[0].any()


def test_recipe_agrees_with_math_away_from_ties():
    d = 4096
    x = wl.activations(1, 0, 64, d, n_outliers=4, lo=50, hi=50)
    s = wl.signs(1, d)
    y64 = had.rotate(x.astype(np.float64), s)
    z32 = had.rotate_unnormalised(x.astype(np.float64), s).astype(np.float32)
    qm, sm = quant.sym_quant_math(y64)
    qr, sr = quant.sym_quant_recipe(z32, d, rotated=True)
    # scales: equal or one fp16 ulp apart
    ulp = np.abs(sm.astype(np.float32).view(np.int32) - sr.astype(np.float32).view(np.int32))
    assert (sm == sr).mean() > 0.9
    assert np.all(np.abs(sm.view(np.int16).astype(int) - sr.view(np.int16).astype(int)) <= 1), ulp
    diff = qm.astype(int) - qr.astype(int)
    assert np.abs(diff).max() <= 1
    near = quant.tie_distance(y64, sm) < 4e-3
    assert not np.any((diff != 0) & ~near)


def test_rotation_removes_outliers_and_improves_sqnr():
    # Qualitative pin (QuaRot paper Fig. 1; QuaRot blog outlier demo): after the
    # rotation the per-token INT4 quantization error drops sharply.
    d = 4096
    x = wl.activations(1, 0, 32, d, n_outliers=4, lo=50, hi=50).astype(np.float64)
    s = wl.signs(1, d)

    def sqnr(y):
        q, sc = quant.sym_quant_math(y)
        err = quant.dequant(q, sc) - y
        return 10 * np.log10((y ** 2).sum() / (err ** 2).sum())

    plain, rotated = sqnr(x), sqnr(had.rotate(x, s))
    assert rotated > plain + 10.0


# ----------------------------- GEMM ----------------------------------------

def test_gemm_exact_vs_bruteforce():
    rng = np.random.default_rng(3)
    a = rng.integers(-8, 8, size=(5, 64))
    w = rng.integers(-8, 8, size=(7, 64))
    assert np.array_equal(gemm.int4_matmul_exact(a, w), gemm.int4_matmul_bruteforce(a, w))
    # from packed bytes, through the unpack path
    ap, wp = quant.pack_int4(a), quant.pack_int4(w)
    assert np.array_equal(gemm.w4a4_acc(ap, wp), gemm.int4_matmul_bruteforce(a, w))


def test_gemm_extreme_magnitude():
    k = 28672
    a = np.full((2, k), -8)
    w = np.full((3, k), -8)
    w[1] = 7
    acc = gemm.int4_matmul_exact(a, w)
    assert acc[0, 0] == 64 * k and acc[0, 1] == -56 * k


def test_epilogue_values():
    acc = np.array([[1000, -3, 0], [1835008, 7, 65536 * 16]])
    a_s = np.array([0.5, 0.25], dtype=np.float16)
    w_s = np.array([0.25, 2.0, 1.0], dtype=np.float16)
    y = gemm.epilogue_recipe(acc, a_s, w_s)
    assert y[0].tolist() == [125.0, -3.0, 0.0]
    assert y[1, 1] == np.float16(3.5)
    assert np.isinf(y[1, 2])  # 262144 overflows fp16 -> +inf
    np.testing.assert_allclose(gemm.epilogue_math(acc, a_s, w_s)[0], [125.0, -3.0, 0.0])


def test_tiny_w4a4_linear_tracks_fp_product():
    # End-to-end on the tiny workload shape (scaled down in N): rotate both X and W
    # with the same R, quantize, multiply: the result tracks X W^T.
    d, n = 4096, 64
    x = wl.activations(1, 0, 32, d, n_outliers=4, lo=50, hi=50).astype(np.float64)
    w = wl.weights(1, 1, n, d).astype(np.float64)
    s = wl.signs(1, d)
    qa, sa = quant.sym_quant_math(had.rotate(x, s))
    qw, sw = quant.sym_quant_math(had.rotate(w, s))
    y, acc = gemm.w4a4_gemm(quant.pack_int4(qa), sa, quant.pack_int4(qw), sw)
    ref = x @ w.T
    rel = np.linalg.norm(y.astype(np.float64) - ref) / np.linalg.norm(ref)
    # Uniform INT4 noise with step max/7 on a Gaussian row whose max is ~4 sigma
    # has relative rms ~ 4 / (7 sqrt(12)) = 0.165 per operand, ~0.23 for two.
    assert rel < 0.3
    # without the rotation the same quantization is far worse
    qa0, sa0 = quant.sym_quant_math(x)
    qw0, sw0 = quant.sym_quant_math(w)
    y0, _ = gemm.w4a4_gemm(quant.pack_int4(qa0), sa0, quant.pack_int4(qw0), sw0)
    rel0 = np.linalg.norm(y0.astype(np.float64) - ref) / np.linalg.norm(ref)
    assert rel0 > 2 * rel


# ---------------------------------------------------------------------------
# b-bit codes (6- and 8-bit round-to-nearest, QuaRot paper Table 9)
# ---------------------------------------------------------------------------

def test_bbit_code_ranges():
    assert oq.code_range(4) == (7, -8, 7)
    assert oq.code_range(6) == (31, -32, 31)
    assert oq.code_range(8) == (127, -128, 127)
    assert oq.code_range(2) == (1, -2, 1)


def test_bbit_unit_scale_rows_round_half_even():
    # max|y| = qmax gives scale exactly 1, so the codes are rne(y)
    q, s = oq.sym_quant_math(np.array([[127.0, -63.5, 0.5, 1.5, -2.5, 100.49]]), 1.0, 8)
    assert s[0] == 1.0 and q.tolist() == [[127, -64, 0, 2, -2, 100]]
    q, s = oq.sym_quant_math(np.array([[31.0, -31.0, 15.5, -2.5, 0.0, 30.5]]), 1.0, 6)
    assert s[0] == 1.0 and q.tolist() == [[31, -31, 16, -2, 0, 30]]
    q, s = oq.sym_quant_math(np.array([[1.0, -1.0, 0.5, -0.5]]), 1.0, 2)
    assert s[0] == 1.0 and q.tolist() == [[1, -1, 0, 0]]


def test_bbit_clip_reaches_the_asymmetric_minimum():
    # clip 1/2: |y| / s ~ 2 qmax, clamped to [-2^(b-1), qmax]
    for bits in (6, 8):
        qmax, lo, hi = oq.code_range(bits)
        q, s = oq.sym_quant_math(np.array([[100.0, -100.0, 0.0, 1.0]]), 0.5, bits)
        assert s[0] == np.float16(0.5 * 100.0 / qmax)
        assert q[0, 0] == hi and q[0, 1] == lo and q[0, 2] == 0


def test_bbit_four_bits_is_the_int4_quantizer():
    y = np.random.default_rng(31).standard_normal((8, 256)) * 3
    for clip in (1.0, 0.9):
        q4, s4 = oq.sym_quant_math(y, clip)
        qb, sb = oq.sym_quant_math(y, clip, 4)
        assert np.array_equal(q4, qb) and np.array_equal(s4, sb)


@pytest.mark.parametrize("bits", [6, 8])
def test_bbit_recipe_agrees_with_math(bits):
    rng = np.random.default_rng(40 + bits)
    z = (rng.integers(-2000, 2000, size=(16, 512)) / 8.0).astype(np.float32)  # exact fp32 rows
    q_rec, s_rec = oq.sym_quant_recipe(z, 512, True, 1.0, bits)
    q64, s64 = oq.sym_quant_math(z.astype(np.float64) / np.sqrt(512), 1.0, bits)
    assert np.abs(s_rec.view(np.int16).astype(int) - s64.view(np.int16).astype(int)).max() <= 1
    diff = q_rec.astype(int) - q64.astype(int)
    assert np.abs(diff).max() <= 1
    qmax = oq.code_range(bits)[0]
    # the 8-bit codes' relative resolution is 1/127: the reconstruction error is
    # at most half a step of the scale
    recon = q_rec.astype(np.float64) * s_rec.astype(np.float64)[:, None]
    y = z.astype(np.float64) / np.sqrt(512)
    assert (np.abs(recon - y) <= 0.5 * s_rec.astype(np.float64)[:, None] * (1 + 1e-2)).all()
    assert np.abs(q_rec).max() <= qmax


def test_int8_gemm_bruteforce_and_epilogue_rounding():
    rng = np.random.default_rng(50)
    a = rng.integers(-128, 128, size=(5, 96)).astype(np.int8)
    w = rng.integers(-128, 128, size=(7, 96)).astype(np.int8)
    assert np.array_equal(gemm.int_matmul_exact(a, w), gemm.int4_matmul_bruteforce(a, w))
    # extreme codes: -128 * -128 summed over K stays exact in int64
    big = np.full((1, 4096), -128, np.int8)
    assert gemm.int_matmul_exact(big, big)[0, 0] == 128 * 128 * 4096
    # accumulators past 2^24 (8-bit codes) still give the nearest fp16 of acc * a_s * w_s
    acc = np.array([[2 ** 24 + 1, 2 ** 24 + 3, 2 ** 25 + 2, -(2 ** 24) - 1]])
    y = gemm.epilogue_recipe(acc, np.full(1, 2.0 ** -10, np.float16), np.full(4, 2.0 ** -10, np.float16))
    assert y.astype(np.float64).tolist() == [[16.0, 16.0, 32.0, -16.0]]
    yq, accq = gemm.w8a8_gemm(a, np.ones(5, np.float16), w, np.ones(7, np.float16))
    assert np.array_equal(accq, gemm.int4_matmul_bruteforce(a, w))


# ---------------------------------------------------------------------------
# Group-wise scales
# ---------------------------------------------------------------------------

def test_groups_with_one_group_is_per_token():
    y = np.random.default_rng(70).standard_normal((6, 256)) * 3
    qg, sg = oq.sym_quant_groups_math(y, 256)
    q, s = oq.sym_quant_math(y)
    assert np.array_equal(qg, q) and np.array_equal(sg[:, 0], s)
    z = (np.random.default_rng(71).integers(-500, 500, size=(6, 256)) / 4.0).astype(np.float32)
    c = np.full(6, np.float32(1 / 16), np.float32)
    qg, sg = oq.sym_quant_groups_recipe(z, c, 256)
    q, s = oq.sym_quant_recipe(z, 256, True)
    assert np.array_equal(qg, q) and np.array_equal(sg[:, 0], s)


def test_groups_scale_each_group_on_its_own():
    # group 0 holds an outlier, group 1 small values: group 1's codes keep their
    # resolution, which a per-token scale would crush to zero
    y = np.zeros((1, 256))
    y[0, :128] = np.linspace(-1, 1, 128)
    y[0, 5] = 70.0
    y[0, 128:] = np.linspace(-0.1, 0.1, 128)
    q, s = oq.sym_quant_groups_math(y, 128)
    assert s[0, 0] == np.float16(10.0) and s[0, 1] == np.float16(0.1 / 7)
    assert np.abs(q[0, 128:]).max() == 7
    qt, _ = oq.sym_quant_math(y)
    assert np.abs(qt[0, 128:]).max() == 0


@pytest.mark.parametrize("group", [64, 128, 256])
def test_groups_gemm_recipe_and_math(group):
    rng = np.random.default_rng(72 + group)
    T, N, K = 5, 7, 512
    a = quant.pack_int4(rng.integers(-8, 8, size=(T, K)))
    w = quant.pack_int4(rng.integers(-8, 8, size=(N, K)))
    asc = rng.uniform(1e-3, 1e-1, size=(T, K // group)).astype(np.float16)
    wsc = rng.uniform(1e-3, 1e-1, size=(N, K // group)).astype(np.float16)
    y, accs = gemm.w4a4_gemm_groups_recipe(a, asc, w, wsc, group)
    # the per-group accumulators sum to the full product
    assert np.array_equal(accs.sum(axis=0), gemm.w4a4_acc(a, w))
    ua, uw = quant.unpack_int4(a), quant.unpack_int4(w)
    g0 = gemm.int4_matmul_bruteforce(ua[:, :group], uw[:, :group])
    assert np.array_equal(accs[0], g0)
    y64 = gemm.w4a4_gemm_groups_math(a, asc, w, wsc, group)
    assert np.allclose(y.astype(np.float64), y64, rtol=2e-3, atol=1e-6)
    # one group over all of K is the per-token epilogue
    y1, _ = gemm.w4a4_gemm_groups_recipe(a, asc[:, :1], w, wsc[:, :1], K)
    assert np.array_equal(y1.view(np.uint16), gemm.epilogue_recipe(
        gemm.w4a4_acc(a, w), asc[:, 0], wsc[:, 0]).view(np.uint16))


# ------------------------- tie distance (R3's window) -------------------------
# Hand values of u = y / s: 2.5 and -2.5 sit on a .5 boundary (distance 0),
# integers are as far from one as possible (0.5), -3.4996 is 4e-4 away.  The
# scale is used as the fp16 value that is stored, so 0.1 acts as
# 0.0999755859375 and y = 0.25 lands 6.1e-4 past 2.5, not on it.

def test_tie_distance_hand_values():
    y = np.array([[1.25, -1.25, 1.0, 3.5, -1.7498, 0.375, 0.0]])
    got = quant.tie_distance(y, np.array([0.5], dtype=np.float16))
    want = [0.0, 0.0, 0.5, 0.5, 4e-4, 0.25, 0.5]
    assert np.allclose(got, [want], rtol=0, atol=1e-12)


def test_tie_distance_uses_the_fp16_scale_of_each_row():
    y = np.array([[0.25, 0.25], [0.25, 0.75]])
    s = np.array([0.1, 0.5], dtype=np.float64)  # row 0's scale is not an fp16 number
    got = quant.tie_distance(y, s)
    u0 = 0.25 / 0.0999755859375                  # = 2.50061..., the stored fp16 scale
    assert np.allclose(got[0], abs(u0 - 2.5), rtol=0, atol=1e-12) and abs(u0 - 2.5) > 6e-4
    assert np.allclose(got[1], [0.0, 0.0], atol=0)  # 0.5 and 1.5


def test_tie_distance_zero_scale_row_is_never_a_tie():
    got = quant.tie_distance(np.array([[0.0, 3.0]]), np.array([0.0], dtype=np.float16))
    assert got.tolist() == [[0.5, 0.5]]


def test_quant_with_scale_hand_values():
    # s = 0.5: u = (2.5, -2.5, 3.5, 7.6, -9, 0.26) -> RNE (2, -2, 4, 8 -> 7, -9 -> -8, 0)
    y = np.array([[1.25, -1.25, 1.75, 3.8, -4.5, 0.13]])
    q = quant.sym_quant_with_scale(y, np.array([0.5], dtype=np.float16))
    assert q.tolist() == [[2, -2, 4, 7, -8, 0]]
    assert quant.sym_quant_with_scale(y, np.array([0.0], dtype=np.float16)).tolist() == [[0] * 6]
