"""GPU parity: qr_hadamard_quant and qr_hadamard against the oracle (through the C ABI)."""
import numpy as np
import pytest

import workloads as wl
from oracle import hadamard as oh
from oracle import quant as oq

from parity import check_rotation, check_sym_codes, check_sym_exact

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
qr = pytest.importorskip("hadamard_rotation_int4_amd")

WIDTHS = [8, 16, 64, 128, 256, 512, 1024, 2048, 4096, 8192, 56, 224, 3584, 28672, 344, 11008]


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def run(x, signs, clip=1.0, rotate=True):
    xs = dev(x)
    s = dev(signs) if signs is not None else None
    q, sc, z = qr.hadamard_quant(xs, s, clip, rotate=rotate, z_dbg=True)
    return host(q), host(sc), host(z)


@pytest.mark.parametrize("d", WIDTHS)
def test_gaussian_with_outliers(d):
    T = 37  # several waves/blocks plus a ragged tail
    x = wl.activations(1, 0, T, d, n_outliers=min(4, d // 8), lo=50, hi=50)
    s = wl.signs(1, d)
    q, sc, z = run(x, s)
    z64 = oh.rotate_unnormalised(x.astype(np.float64), s)
    check_rotation(z, z64)
    check_sym_codes(q, sc, z64 / np.sqrt(d), 1.0)


# Row counts just past one full pass of each kernel's grid: 2048 rows for the
# d = 2^n kernel (512 workgroups x 4 wavefronts), 512 rows for d = 28672 and 11008
# (512 workgroups, a row each); the first workgroup then carries one more row,
# through its prefetch / double-buffer path.  Every row is checked.
@pytest.mark.parametrize("d,T", [(8192, 2049), (4096, 2049), (28672, 513), (11008, 513),
                                 (28672, 1025)])
def test_one_row_past_a_full_grid_pass(d, T):
    x = wl.activations(7, 1, T, d, n_outliers=5, lo=20, hi=100)
    s = wl.signs(7, d)
    q, sc, z = run(x, s)
    z64 = oh.rotate_unnormalised(x.astype(np.float64), s)
    check_rotation(z, z64)
    check_sym_codes(q, sc, z64 / np.sqrt(d), 1.0)


@pytest.mark.parametrize("d", [128, 512, 4096, 8192, 28672, 11008])
def test_grid_inputs_bit_exact(d):
    T = 21
    x = wl.grid_activations(1, d, T, d)
    s = wl.signs(2, d)
    q, sc, z = run(x, s)
    z_exact = oh.rotate_unnormalised(x.astype(np.float64), s)
    assert np.array_equal(z.astype(np.float64), z_exact), "transform must be exact on grid inputs"
    check_sym_exact(q, sc, z_exact, d, True, 1.0)


@pytest.mark.parametrize("d", [128, 4096, 8192, 28672, 11008])
@pytest.mark.parametrize("clip", [0.9, 0.5])
def test_clip_ratio(d, clip):
    T = 9
    x = wl.grid_activations(3, d, T, d)
    s = wl.signs(3, d)
    q, sc, z = run(x, s, clip=clip)
    z_exact = oh.rotate_unnormalised(x.astype(np.float64), s)
    check_sym_exact(q, sc, z_exact, d, True, clip)
    codes = oq.unpack_int4(q)
    assert codes.min() >= -8 and codes.max() <= 7
    if clip <= 0.5:
        assert (codes == 7).any() and (codes == -8).any()


@pytest.mark.parametrize("d", [4096, 28672])
def test_plain_hadamard_signs_none(d):
    x = wl.activations(4, 0, 5, d)
    q, sc, z = run(x, None)
    z64 = oh.rotate_unnormalised(x.astype(np.float64), None)
    check_rotation(z, z64)
    check_sym_codes(q, sc, z64 / np.sqrt(d), 1.0)


@pytest.mark.parametrize("d", [4096, 4000, 11008])
def test_quant_only(d):
    x = wl.grid_activations(5, d, 11, d)
    q, sc, z = run(x, None, rotate=False)
    assert np.array_equal(z, x.astype(np.float32))
    check_sym_exact(q, sc, x.astype(np.float64), d, False, 1.0)


@pytest.mark.parametrize("d", [128, 512, 4096, 344, 3584, 11008, 28672])
def test_row_stride_and_views(d):
    # every kernel family (d/8 lanes per row, one wavefront per row, LDS-staged,
    # H_172 and H_4 (x) H_28 on the matrix cores) on rows 16 elements into a
    # wider buffer, with a row stride of d + 64
    T = 10
    big = wl.activations(6, 0, T, d + 64)
    view = dev(big)[:, 16:16 + d]
    s = wl.signs(6, d)
    q, sc, z = qr.hadamard_quant(view, dev(s), 1.0, z_dbg=True)
    z64 = oh.rotate_unnormalised(big[:, 16:16 + d].astype(np.float64), s)
    check_rotation(host(z), z64)
    check_sym_codes(host(q), host(sc), z64 / np.sqrt(d), 1.0)


@pytest.mark.parametrize("d", [128, 8192, 28672, 11008])
def test_edge_rows(d):
    # zero row, constant row, a row scaled into fp16 subnormal scales, a huge row
    # (s * x constant, so all its energy lands in few outputs and the scale
    # overflows fp16 to +inf -> codes 0), a single spike
    s = wl.signs(7, d)
    x = np.zeros((6, d), dtype=np.float16)
    x[1] = 1.0
    x[2] = (wl.grid_activations(7, d, 1, d)[0].astype(np.float64) * 2.0 ** -20).astype(np.float16)
    x[3] = (60000.0 * s).astype(np.float16)
    x[4, d // 3] = 3.0
    x[5] = wl.activations(7, 1, 1, d)[0]
    q, sc, z = run(x, s)
    z64 = oh.rotate_unnormalised(x.astype(np.float64), s)
    # rows 0..4 are exact in fp32; the recipe decides their codes and scales bit for bit
    assert np.array_equal(z[:3].astype(np.float64), z64[:3])
    check_sym_exact(q[:5], sc[:5], z64[:5], d, True, 1.0)
    assert sc[0] == 0 and not q[0].any()
    assert np.isinf(sc[3]) and not q[3].any()
    codes = oq.unpack_int4(q)
    assert codes.min() >= -8 and codes.max() <= 7


def test_empty_and_single_row():
    x = dev(np.zeros((0, 4096), dtype=np.float16))
    q, sc = qr.hadamard_quant(x)
    assert q.shape == (0, 2048) and sc.shape == (0,)
    x1 = wl.activations(8, 0, 1, 8192)
    s = wl.signs(8, 8192)
    q, sc, z = run(x1, s)
    check_rotation(z, oh.rotate_unnormalised(x1.astype(np.float64), s))


@pytest.mark.parametrize("d", [128, 1024, 8192, 28672, 11008])
@pytest.mark.parametrize("f32", [True, False])
def test_rotate_only(d, f32):
    x = wl.activations(9, 0, 13, d)
    s = wl.signs(9, d)
    y = host(qr.hadamard(dev(x), dev(s), out_dtype=torch.float32 if f32 else torch.float16))
    y64 = oh.rotate(x.astype(np.float64), s)
    check_rotation(y, y64, tol=1e-3)
    if not f32:
        # fp16 output: one rounding of the fp32 value
        assert np.abs(y.astype(np.float64) - y64).max() <= 2 ** -10 * np.abs(y64).max() + 1e-6


def test_determinism():
    d = 8192
    x = wl.activations(10, 0, 64, d)
    s = wl.signs(10, d)
    a = run(x, s)
    b = run(x, s)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


# ---- QR_ROT_HADAMARD_F16 (the transform's additions in fp16, d = 28672, 11008) ----
# Bound from the arithmetic (include/qr.h): R fp16 roundings, each relative
# 2^-11 of a vector that the remaining scaled-orthogonal stages carry to ||z||,
# plus the fp16 subnormal term (absolute 2^-25 before the factor 2^e, grown by
# sqrt(2) per remaining stage); the quantization of the returned values is the
# fp32 recipe, bit for bit.
F16_WIDTHS = {28672: (9, 7), 11008: (7, 8)}   # d -> (roundings R, scaling exponent e)


def f16_bound(z64, d):
    R, e = F16_WIDTHS[d]
    S = sum(2.0 ** (j / 2) for j in range(R))
    return R * 2.0 ** -11 * np.linalg.norm(z64, axis=-1) + 2.0 ** (e - 25) * S * np.sqrt(d)


def run_f16(x, s, clip=1.0):
    q, sc, z = qr.hadamard_quant(dev(x), dev(s) if s is not None else None, clip, z_dbg=True,
                                 fp16_transform=True)
    return host(q), host(sc), host(z)


@pytest.mark.parametrize("d", sorted(F16_WIDTHS))
@pytest.mark.parametrize("clip", [1.0, 0.9])
def test_fp16_transform_bound_and_recipe(d, clip):
    T = 37
    x = wl.activations(11, 0, T, d, n_outliers=4, lo=50, hi=50)
    s = wl.signs(11, d)
    q, sc, z = run_f16(x, s, clip)
    # the quantizer input is 2^e times fp16 values
    f = 2.0 ** F16_WIDTHS[d][1]
    assert np.array_equal((z / f).astype(np.float16).astype(np.float32) * f, z)
    z64 = oh.rotate_unnormalised(x.astype(np.float64), s)
    err = np.linalg.norm(z.astype(np.float64) - z64, axis=-1)
    bound = f16_bound(z64, d)
    assert (err <= bound).all(), f"max err/bound {(err / bound).max():.3f}"
    check_sym_exact(q, sc, z.astype(np.float64), d, True, clip)
    # the codes agree with the fp32 transform's except near rounding ties
    q32, sc32, z32 = run(x, s, clip)
    assert (oq.unpack_int4(q).astype(np.int64) != oq.unpack_int4(q32)).mean() < 0.05


@pytest.mark.parametrize("d", sorted(F16_WIDTHS))
def test_fp16_transform_edge_rows(d):
    x = np.zeros((5, d), dtype=np.float16)
    x[1] = 1.0                                   # constant row
    x[2, d // 3] = 3.0                           # one spike
    x[3] = wl.activations(12, 1, 1, d)[0]
    x[4] = (wl.activations(12, 2, 1, d)[0].astype(np.float64) * 2.0 ** -12).astype(np.float16)
    q, sc, z = run_f16(x, None)
    z64 = oh.rotate_unnormalised(x.astype(np.float64), None)
    err = np.linalg.norm(z.astype(np.float64) - z64, axis=-1)
    assert (err <= f16_bound(z64, d)).all()
    check_sym_exact(q, sc, z.astype(np.float64), d, True, 1.0)
    assert sc[0] == 0 and not q[0].any()


def test_fp16_transform_other_widths_unsupported():
    x = dev(wl.activations(13, 0, 2, 4096))
    with pytest.raises(RuntimeError):
        qr.hadamard_quant(x, None, 1.0, fp16_transform=True)
