"""Pins of oracle/block.py (RMSNorm-without-scale + INT4, Hadamard heads + INT4)
against facts fixed outside the oracle: a library routine, closed forms, the
pages' Kronecker identity, brute-force dense matrices and invariances."""
import numpy as np
import pytest

from oracle import block as ob
from oracle import hadamard as oh
from oracle import quant as oq


# ---------------------------------------------------------------------------
# RMSNorm without scale
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("eps", [0.0, 1e-5, 1e-2])
def test_rmsnorm_matches_torch_rms_norm(eps):
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(3).standard_normal((9, 96)) * 3.0
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (96,), eps=eps).numpy()
    np.testing.assert_allclose(ob.rmsnorm(x, eps), ref, rtol=1e-13, atol=0)


def test_rmsnorm_closed_forms():
    # constant row c: y = c / sqrt(c^2 + eps)
    c, eps = 2.5, 0.25
    y = ob.rmsnorm(np.full((1, 16), c), eps)
    np.testing.assert_allclose(y, c / np.sqrt(c * c + eps), rtol=1e-15)
    # [3, 4] with eps = 0: mean square 12.5
    y = ob.rmsnorm(np.array([[3.0, 4.0]]), 0.0)
    np.testing.assert_allclose(y, [[3 / np.sqrt(12.5), 4 / np.sqrt(12.5)]], rtol=1e-15)


def test_rmsnorm_is_the_pages_unit_norm_times_sqrt_d():
    # the pages normalise a row as x / ||x||; with eps = 0 the RMS form is that times sqrt(d)
    x = np.random.default_rng(4).standard_normal((5, 128))
    y = ob.rmsnorm(x, 0.0)
    np.testing.assert_allclose(y, np.sqrt(128) * x / np.linalg.norm(x, axis=-1, keepdims=True),
                               rtol=1e-13)
    # and is invariant to rescaling the row
    np.testing.assert_allclose(ob.rmsnorm(7.25 * x, 0.0), y, rtol=1e-13)


def test_rmsnorm_commutes_with_rotation():
    # the property the method relies on: RMSNorm(x Q) = RMSNorm(x) Q for orthogonal Q
    x = np.random.default_rng(5).standard_normal((6, 64))
    s = np.where(np.random.default_rng(6).random(64) < 0.5, -1, 1)
    lhs = ob.rmsnorm(oh.rotate(x, s), 1e-5)
    rhs = oh.rotate(ob.rmsnorm(x, 1e-5), s)
    np.testing.assert_allclose(lhs, rhs, atol=1e-12)


def test_rmsnorm_quant_hand_examples():
    # mean square 4 -> r = 1/2 exactly; y = [1, -1, 1, -1]; scale fp16(1/7); codes +-7
    x = np.array([[2.0, -2.0, 2.0, -2.0]], dtype=np.float16)
    q, s, y = ob.rmsnorm_quant_math(x, 0.0)
    assert s[0] == np.float16(1.0 / 7.0)
    assert q.tolist() == [[7, -7, 7, -7]]
    qr_, sr = ob.rmsnorm_quant_recipe(x, np.array([0.5], dtype=np.float32))
    assert sr[0] == s[0] and np.array_equal(qr_, q)
    # one spike: [4, 0, 0, 0] -> r = 1/2, y = [2, 0, 0, 0], codes [7, 0, 0, 0]
    x = np.array([[4.0, 0.0, 0.0, 0.0]], dtype=np.float16)
    q, s, _ = ob.rmsnorm_quant_math(x, 0.0)
    assert s[0] == np.float16(2.0 / 7.0) and q.tolist() == [[7, 0, 0, 0]]


def test_rmsnorm_quant_zero_row():
    x = np.zeros((2, 32), dtype=np.float16)
    q, s = ob.rmsnorm_quant_recipe(x, ob.rms_multiplier(x, 1e-5).astype(np.float32))
    assert np.all(q == 0) and np.all(s == 0)


def test_rmsnorm_quant_recipe_agrees_with_math():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((64, 4096)) * np.where(rng.random(4096) < 0.002, 40, 1)).astype(np.float16)
    eps = 1e-5
    r32 = ob.rms_multiplier(x, eps).astype(np.float32)
    q_rec, s_rec = ob.rmsnorm_quant_recipe(x, r32)
    q64, s64, y64 = ob.rmsnorm_quant_math(x, eps)
    assert np.abs(s_rec.view(np.int16).astype(int) - s64.view(np.int16).astype(int)).max() <= 1
    diff = q_rec.astype(int) - q64.astype(int)
    assert np.abs(diff).max() <= 1
    tie = oq.tie_distance(y64, s64)
    assert not ((diff != 0) & (tie > 1e-3)).any()


def test_rmsnorm_quant_recipe_catches_a_missing_rms():
    # a recipe that forgot r (r = 1) gives the same codes (the quantizer is
    # scale-invariant) but scales off by the RMS: the scale check must see it
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((4, 256)) * 5).astype(np.float16)
    r32 = ob.rms_multiplier(x, 1e-5).astype(np.float32)
    _, s_ok = ob.rmsnorm_quant_recipe(x, r32)
    _, s_bad = ob.rmsnorm_quant_recipe(x, np.ones(4, np.float32))
    _, s64, _ = ob.rmsnorm_quant_math(x, 1e-5)
    assert np.array_equal(s_ok, s64)
    assert not np.array_equal(s_bad, s64)


# ---------------------------------------------------------------------------
# Hadamard heads
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("nh,dh", [(2, 4), (4, 8), (8, 16), (32, 8), (16, 16)])
def test_heads_equals_dense_kronecker(nh, dh):
    n = int(np.log2(nh))
    dense = np.kron(oh.sylvester(n), np.eye(dh, dtype=np.int64))
    x = np.random.default_rng(nh * 100 + dh).integers(-50, 50, size=(3, nh * dh))
    z = ob.hadamard_heads_unnormalised(x, nh)
    assert np.array_equal(z, (x @ dense.T).astype(np.float64))


@pytest.mark.parametrize("nh,dh", [(4, 8), (32, 8), (8, 32)])
def test_heads_completes_the_full_hadamard(nh, dh):
    # the pages' identity (H_{n_h} (x) I)(I (x) H_{d_h}) = H_{n_h d_h}: the heads
    # block applied after a head-wise H_{d_h} gives the full Sylvester transform
    nd = nh * dh
    x = np.random.default_rng(nd).integers(-9, 9, size=(2, nd)).astype(np.float64)
    per_head = (x.reshape(2, nh, dh) @ oh.sylvester(int(np.log2(dh))).T).reshape(2, nd)
    full = x @ oh.sylvester(int(np.log2(nd))).T
    assert np.array_equal(ob.hadamard_heads_unnormalised(per_head, nh), full)


def test_heads_orthogonal_and_involution():
    x = np.random.default_rng(11).standard_normal((7, 64 * 128))
    y = ob.hadamard_heads(x, 64)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)
    # H/sqrt(n) is symmetric and orthogonal, so applying it twice is the identity
    np.testing.assert_allclose(ob.hadamard_heads(y, 64), x, atol=1e-12)


def test_heads_single_head_spreads_evenly():
    # only head 0 non-zero: column 0 of H is all ones, so every head gets x_0 / sqrt(n_h)
    nh, dh = 32, 128
    x = np.zeros((1, nh * dh))
    x[0, :dh] = np.arange(1, dh + 1)
    y = ob.hadamard_heads(x, nh).reshape(nh, dh)
    np.testing.assert_allclose(y, np.tile(np.arange(1, dh + 1) / np.sqrt(nh), (nh, 1)), rtol=1e-15)


def test_heads_quant_recipe_agrees_with_math():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((32, 4096)).astype(np.float16)
    z = ob.hadamard_heads_unnormalised(x, 32)   # exact in fp32 (sums of 32 fp16)
    q_rec, s_rec = ob.hadamard_heads_quant_recipe(z, 32)
    q64, s64, y64 = ob.hadamard_heads_quant_math(x, 32)
    assert np.array_equal(s_rec, s64)
    diff = q_rec.astype(int) - q64.astype(int)
    tie = oq.tie_distance(y64, s64)
    assert not ((diff != 0) & (tie > 1e-3)).any()


def test_block_quantizers_take_the_bit_width():
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((4, 256)) * 4).astype(np.float16)
    q8, s8, y = ob.rmsnorm_quant_math(x, 1e-5, 1.0, 8)
    assert np.array_equal(s8, oq.sym_scale_math(y, 1.0, 8))
    assert np.abs(q8).max() == 127
    qh, sh, yh = ob.hadamard_heads_quant_math(x, 4, 1.0, 6)
    assert np.abs(qh).max() == 31 and np.array_equal(sh, oq.sym_scale_math(yh, 1.0, 6))
