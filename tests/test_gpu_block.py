"""GPU parity: qr_rmsnorm_quant and qr_hadamard_heads_quant against the oracle
(through the C ABI), at small ragged sizes, edge rows, and the full Llama-2
shapes in the launch configurations bench.py times (sampled rows at T = 65536).

Rules (tests/parity.py):
  * RMSNorm: the GPU's fp32 multiplier r against the float64 r within 2e-5
    relative (the fp32 sum of <= 16384 exact squares, accumulated in a lane's
    registers and then across 64 lanes, is within (d / 64 + 6) 2^-24 of the
    exact sum relative, and the division, addition, square root and reciprocal
    add four roundings); codes and scales end to end against y64 = x r64 (R2,
    R3); and bit-exact against the oracle's fp32 recipe on the GPU's own r (R4).
  * Hadamard heads: z against the float64 transform (R1), codes and scales end
    to end (R2, R3), bit-exact recipe on the GPU's own z (R4), and exact z on
    grid inputs.
"""
import numpy as np
import pytest

import workloads as wl
from oracle import block as ob
from oracle import quant as oq

from parity import check_rotation, check_sym_codes

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
qr = pytest.importorskip("hadamard_rotation_int4_amd")

R_TOL = 2e-5


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


# ---------------------------------------------------------------------------
# RMSNorm (no scale) + INT4
# ---------------------------------------------------------------------------

def check_rms(x, q, sc, r, eps, clip):
    r64 = ob.rms_multiplier(x, eps)
    rel = np.abs(r.astype(np.float64) - r64) / np.maximum(r64, 1e-300)
    assert rel.max() <= R_TOL, f"r: relative error {rel.max():.3e}"
    check_sym_codes(q, sc, x.astype(np.float64) * r64[:, None], clip)
    q_rec, s_rec = ob.rmsnorm_quant_recipe(x, r, clip)
    assert np.array_equal(sc.view(np.uint16), s_rec.view(np.uint16)), "R4: scales"
    assert np.array_equal(q, oq.pack_int4(q_rec)), "R4: packed codes"


@pytest.mark.parametrize("d", [8, 72, 512, 1000, 4096, 4104, 8192, 11008, 16384])
def test_rmsnorm_quant_gaussian_with_outliers(d):
    T = 37
    x = wl.activations(21, 0, T, d, n_outliers=min(5, d // 8))
    q, sc, r = qr.rmsnorm_quant(dev(x), 1e-5, 1.0, r_dbg=True)
    check_rms(x, host(q), host(sc), host(r), 1e-5, 1.0)


@pytest.mark.parametrize("clip", [0.9, 0.5])
@pytest.mark.parametrize("eps", [0.0, 1e-5])
def test_rmsnorm_quant_clip_and_eps(clip, eps):
    x = wl.activations(22, 0, 19, 4096)
    q, sc, r = qr.rmsnorm_quant(dev(x), eps, clip, r_dbg=True)
    check_rms(x, host(q), host(sc), host(r), eps, clip)
    codes = oq.unpack_int4(host(q))
    assert codes.min() >= -8 and codes.max() <= 7
    if clip <= 0.5:
        assert (codes == 7).any() and (codes == -8).any()


def test_rmsnorm_quant_edge_rows():
    d = 8192
    x = np.zeros((6, d), dtype=np.float16)
    x[1] = 1.0                                      # constant row: r = 1/sqrt(1 + eps)
    x[2, 17] = 3.0                                  # single spike
    x[3] = (wl.activations(23, 0, 1, d)[0].astype(np.float64) * 2.0 ** -20).astype(np.float16)
    x[4] = (wl.activations(23, 1, 1, d, n_outliers=0)[0].astype(np.float64) * 1000).astype(np.float16)
    x[5] = wl.activations(23, 2, 1, d)[0]
    for eps in (1e-5, 0.0):
        q, sc, r = (host(t) for t in qr.rmsnorm_quant(dev(x), eps, 1.0, r_dbg=True))
        q_rec, s_rec = ob.rmsnorm_quant_recipe(x, r, 1.0)
        assert np.array_equal(sc.view(np.uint16), s_rec.view(np.uint16))
        assert np.array_equal(q, oq.pack_int4(q_rec))
        assert sc[0] == 0 and not q[0].any()
        if eps == 0.0:
            assert r[0] == 0.0                      # 0 / 0 row: r defined as 0
            check_rms(x[1:], q[1:], sc[1:], r[1:], eps, 1.0)
        else:
            check_rms(x, q, sc, r, eps, 1.0)


def test_rmsnorm_quant_row_stride_and_empty():
    d, T = 4096, 10
    big = wl.activations(24, 0, T, d + 64)
    q, sc, r = qr.rmsnorm_quant(dev(big)[:, 32:32 + d], 1e-5, 1.0, r_dbg=True)
    check_rms(big[:, 32:32 + d], host(q), host(sc), host(r), 1e-5, 1.0)
    q, sc = qr.rmsnorm_quant(dev(np.zeros((0, d), np.float16)))
    assert q.shape == (0, d // 2) and sc.shape == (0,)


# ---------------------------------------------------------------------------
# Hadamard heads + INT4
# ---------------------------------------------------------------------------

def check_heads(x, nh, q, sc, z, clip):
    z64 = ob.hadamard_heads_unnormalised(x, nh)
    check_rotation(z, z64)
    check_sym_codes(q, sc, z64 / np.sqrt(nh), clip)
    q_rec, s_rec = ob.hadamard_heads_quant_recipe(z, nh, clip)
    assert np.array_equal(sc.view(np.uint16), s_rec.view(np.uint16)), "R4: scales"
    assert np.array_equal(q, oq.pack_int4(q_rec)), "R4: packed codes"


HEAD_SHAPES = [(64, 128), (32, 128), (16, 128), (8, 64), (2, 32), (64, 8), (32, 256), (16, 512),
               (4, 256)]


@pytest.mark.parametrize("nh,dh", HEAD_SHAPES)
def test_heads_quant_gaussian_with_outliers(nh, dh):
    T = 37
    x = wl.activations(25, nh, T, nh * dh, n_outliers=5)
    q, sc, z = qr.hadamard_heads_quant(dev(x), nh, 1.0, z_dbg=True)
    check_heads(x, nh, host(q), host(sc), host(z), 1.0)


@pytest.mark.parametrize("nh,dh", [(64, 128), (32, 128), (8, 64)])
def test_heads_quant_grid_inputs_exact(nh, dh):
    x = wl.grid_activations(26, nh, 21, nh * dh)
    q, sc, z = (host(t) for t in qr.hadamard_heads_quant(dev(x), nh, 1.0, z_dbg=True))
    z_exact = ob.hadamard_heads_unnormalised(x, nh)
    assert np.array_equal(z.astype(np.float64), z_exact)
    q_rec, s_rec = ob.hadamard_heads_quant_recipe(z_exact, nh, 1.0)
    assert np.array_equal(sc.view(np.uint16), s_rec.view(np.uint16))
    assert np.array_equal(q, oq.pack_int4(q_rec))


@pytest.mark.parametrize("clip", [0.9, 0.5])
def test_heads_quant_clip(clip):
    x = wl.activations(27, 0, 13, 4096)
    q, sc, z = qr.hadamard_heads_quant(dev(x), 32, clip, z_dbg=True)
    check_heads(x, 32, host(q), host(sc), host(z), clip)


def test_heads_quant_edge_rows_stride_and_empty():
    nh, dh = 64, 128
    d = nh * dh
    x = np.zeros((5, d + 64), dtype=np.float16)
    x[1, :d] = 1.0                                 # all energy lands in head 0
    x[2, 5] = -2.0                                 # one spike spreads to every head
    x[3, :d] = (wl.grid_activations(28, 0, 1, d)[0].astype(np.float64) * 2.0 ** -20).astype(np.float16)
    x[4, :d] = wl.activations(28, 1, 1, d)[0]
    x[:, d:] = 7.0                                 # past the row: must be ignored
    q, sc, z = (host(t) for t in qr.hadamard_heads_quant(dev(x)[:, :d], nh, 1.0, z_dbg=True))
    check_heads(x[:, :d], nh, q, sc, z, 1.0)
    assert sc[0] == 0 and not q[0].any()
    q, sc = qr.hadamard_heads_quant(dev(np.zeros((0, d), np.float16)), nh)
    assert q.shape == (0, d // 2) and sc.shape == (0,)


# ---------------------------------------------------------------------------
# Full Llama-2 sizes (the bench's block workloads)
# ---------------------------------------------------------------------------

def sample_rows(T, seed, x_abs_max):
    g = np.random.default_rng(seed)
    rows = set(g.choice(T, size=min(T, 256), replace=False).tolist())
    rows |= {0, T - 1}
    rows |= set(np.argsort(x_abs_max)[-4:].tolist())
    return np.array(sorted(rows))


@pytest.mark.parametrize("T,d", [(65536, 8192), (2048, 4096)])
def test_rmsnorm_quant_full_size(T, d):
    x = wl.activations_torch(torch, "cuda", 31, d, T, d)
    q, sc, r = qr.rmsnorm_quant(x, 1e-5, 1.0, r_dbg=True)
    amax = host(x.abs().amax(dim=1).float())
    rows = sample_rows(T, 31, amax)
    idx = torch.as_tensor(rows, device="cuda")
    check_rms(host(x[idx]), host(q[idx]), host(sc[idx]), host(r[idx]), 1e-5, 1.0)


@pytest.mark.parametrize("T,nh,dh", [(65536, 64, 128), (2048, 32, 128)])
def test_heads_quant_full_size(T, nh, dh):
    d = nh * dh
    x = wl.activations_torch(torch, "cuda", 32, d, T, d)
    q, sc = qr.hadamard_heads_quant(x, nh, 1.0)
    _, _, z = qr.hadamard_heads_quant(x[:1], nh, 1.0, z_dbg=True)  # warm a z_dbg launch too
    amax = host(x.abs().amax(dim=1).float())
    rows = sample_rows(T, 32, amax)
    idx = torch.as_tensor(rows, device="cuda")
    xs = host(x[idx])
    z64 = ob.hadamard_heads_unnormalised(xs, nh)
    check_sym_codes(host(q[idx]), host(sc[idx]), z64 / np.sqrt(nh), 1.0)
    # the same rows through the z_dbg launch: R1 and the bit-exact recipe
    qz, scz, zz = qr.hadamard_heads_quant(x[idx].contiguous(), nh, 1.0, z_dbg=True)
    assert np.array_equal(host(qz), host(q[idx])) and np.array_equal(host(scz), host(sc[idx]))
    check_heads(xs, nh, host(qz), host(scz), host(zz), 1.0)
