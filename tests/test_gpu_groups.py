"""GPU parity of the group-wise variant (one scale per group of consecutive k;
QuaRot paper, group-wise quantization study) against the oracle, through the
C ABI: qr_hadamard_quant_groups, and qr_w4a4_gemm_groups when present.

Rules: R1 on the transform; per group, scales equal or one fp16 ulp apart and
codes equal or +-1 within 1e-3 of a .5 boundary against float64; bit-exact
codes and scales against the oracle's fp32 recipe on the GPU's own z; the
GEMM bit-exact against the oracle's fp32 recipe.
"""
import numpy as np
import pytest

import workloads as wl
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


def check_group_codes(q_packed, s_gpu, y64, group, clip):
    T, d = y64.shape
    yg = y64.reshape(T, d // group, group)
    check_scales(s_gpu, yg, clip)
    check_codes_given_scale(oq.unpack_int4(q_packed).reshape(T, d // group, group), s_gpu, yg)


@pytest.mark.parametrize("d,group", [(d, gr) for d in (512, 4096, 8192, 11008, 28672)
                                      for gr in (64, 128, 256) if d % gr == 0])
def test_quant_groups(d, group):
    T = 11
    x = wl.activations(80, 0, T, d, n_outliers=min(5, d // 8))
    s = wl.signs(80, d)
    q, sc, z = (host(t) for t in qr.hadamard_quant_groups(dev(x), dev(s), 1.0, group, z_dbg=True))
    assert sc.shape == (T, d // group)
    z64 = oh.rotate_unnormalised(x.astype(np.float64), s)
    check_rotation(z, z64)
    check_group_codes(q, sc, z64 / np.sqrt(d), group, 1.0)
    c = np.full(T, oq.norm_constant(d, True), np.float32)
    q_rec, s_rec = oq.sym_quant_groups_recipe(z, c, group)
    assert np.array_equal(sc.view(np.uint16), s_rec.view(np.uint16))
    assert np.array_equal(q, oq.pack_int4(q_rec))


@pytest.mark.parametrize("d", [4096, 11008])
def test_quant_groups_row_stride(d):
    # rows 16 elements into a wider buffer (row stride d + 64)
    T, group = 7, 128
    big = wl.activations(81, 0, T, d + 64, n_outliers=5)
    s = wl.signs(81, d)
    q, sc, z = (host(t) for t in qr.hadamard_quant_groups(dev(big)[:, 16:16 + d], dev(s), 1.0,
                                                          group, z_dbg=True))
    z64 = oh.rotate_unnormalised(big[:, 16:16 + d].astype(np.float64), s)
    check_rotation(z, z64)
    check_group_codes(q, sc, z64 / np.sqrt(d), group, 1.0)
    c = np.full(T, oq.norm_constant(d, True), np.float32)
    q_rec, s_rec = oq.sym_quant_groups_recipe(z, c, group)
    assert np.array_equal(sc.view(np.uint16), s_rec.view(np.uint16))
    assert np.array_equal(q, oq.pack_int4(q_rec))


@pytest.mark.parametrize("clip", [1.0, 0.5])
def test_quant_groups_no_rotation_edge_rows(clip):
    d, group = 4096, 128
    x = wl.grid_activations(81, 0, 6, d)
    x[0] = 0.0                                          # zero row: every scale 0
    x[1, :group] = 0.0                                  # one zero group
    x[2, 5] = 60000.0                                   # one huge group
    x[3] = (x[3].astype(np.float64) * 2.0 ** -20).astype(np.float16)  # subnormal scales
    q, sc, z = (host(t) for t in qr.hadamard_quant_groups(dev(x), None, clip, group, rotate=False,
                                                          z_dbg=True))
    assert np.array_equal(z, x.astype(np.float32))
    q_rec, s_rec = oq.sym_quant_groups_recipe(x.astype(np.float32), np.ones(6, np.float32), group,
                                              clip)
    assert np.array_equal(sc.view(np.uint16), s_rec.view(np.uint16))
    assert np.array_equal(q, oq.pack_int4(q_rec))
    assert not sc[0].any() and sc[1, 0] == 0


def test_quant_groups_one_group_is_the_per_token_quantizer():
    # group = d on an exact input: the same codes and scales as qr_hadamard_quant
    d = 512
    x = wl.grid_activations(82, 0, 9, d)
    s = wl.signs(82, d)
    qg, sg = qr.hadamard_quant_groups(dev(x), dev(s), 1.0, 512)
    q, sc = qr.hadamard_quant(dev(x), dev(s), 1.0)
    assert np.array_equal(host(qg), host(q))
    assert np.array_equal(host(sg)[:, 0].view(np.uint16), host(sc).view(np.uint16))


def scales(seed, rows, groups, lo=1e-3, hi=1e-1):
    g = np.random.default_rng(seed)
    return np.exp(g.uniform(np.log(lo), np.log(hi), size=(rows, groups))).astype(np.float16)


@pytest.mark.parametrize("T,N,K,group", [
    (T, N, K, gr)
    for T, N, K in ((37, 100, 4096), (300, 260, 2048), (129, 513, 1536), (1, 64, 512),
                    (256, 256, 11008), (70, 90, 4160))
    for gr in (64, 128, 256, 512) if K % gr == 0])  # a group size divides K
def test_gemm_groups_bit_exact(T, N, K, group):
    a = wl.packed_codes(83, T, T, K)
    w = wl.packed_codes(83, 1000 + N, N, K)
    asc, wsc = scales(T + group, T, K // group), scales(N + group, N, K // group)
    y = host(qr.w4a4_gemm_groups(dev(a), dev(asc), dev(w), dev(wsc), group))
    y_ref, _ = og.w4a4_gemm_groups_recipe(a, asc, w, wsc, group)
    assert np.array_equal(y.view(np.uint16), y_ref.view(np.uint16))


def test_linear_groups_end_to_end():
    # rotated X and W quantized group-wise, then the grouped GEMM: bit-exact on
    # the GPU's codes, and closer to X W^T than per-token / per-channel scales
    T, N, K, group = 64, 512, 4096, 128
    x = wl.activations(84, 0, T, K, n_outliers=4, lo=50, hi=50)
    w = wl.weights(84, 1, N, K)
    s = dev(wl.signs(84, K))
    qa, sa = qr.hadamard_quant_groups(dev(x), s, 1.0, group)
    qw, sw = qr.hadamard_quant_groups(dev(w), s, 1.0, group)
    y = host(qr.w4a4_gemm_groups(qa, sa, qw, sw, group)).astype(np.float64)
    y_ref, _ = og.w4a4_gemm_groups_recipe(host(qa), host(sa), host(qw), host(sw), group)
    assert np.array_equal(y.astype(np.float16).view(np.uint16), y_ref.view(np.uint16))
    qa1, sa1 = qr.hadamard_quant(dev(x), s, 1.0)
    qw1, sw1 = qr.hadamard_quant(dev(w), s, 1.0)
    y1 = host(qr.w4a4_gemm(qa1, sa1, qw1, sw1)).astype(np.float64)
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    err_g = np.linalg.norm(y - exact) / np.linalg.norm(exact)
    err_t = np.linalg.norm(y1 - exact) / np.linalg.norm(exact)
    assert err_g < err_t, (err_g, err_t)
