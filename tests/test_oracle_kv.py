"""Pins for the oracle's KV rotation and asymmetric group quantization."""
import numpy as np
import pytest

import workloads as wl
from oracle import hadamard as had, kv


def test_constant_group():
    y = np.full((1, 128), 0.37)
    q, s, m = kv.asym_quant_math(y, 128)
    assert s.ravel().tolist() == [0.0] and not q.any()
    np.testing.assert_allclose(kv.asym_dequant(q, s, m, 128), np.float16(0.37))
    q2, s2, m2 = kv.asym_quant_recipe(y.astype(np.float32), 128, rotated=False, group=128)
    assert s2.ravel().tolist() == [0.0] and not q2.any() and m2.tolist() == m.tolist()


def test_ramp_group_codes():
    # y = mn + k * s with s, mn exact in fp16 -> codes are k exactly
    k = np.tile(np.arange(16), 8)
    y = (-1.5 + 0.25 * k).astype(np.float64)[None, :]
    q, s, m = kv.asym_quant_math(y, 128)
    assert float(s[0, 0]) == 0.25 and float(m[0, 0]) == -1.5
    assert np.array_equal(q[0], k)
    q2, _, _ = kv.asym_quant_recipe(y.astype(np.float32), 128, rotated=False, group=128)
    assert np.array_equal(q2[0], k)


def test_clip_clamps_both_ends():
    y = np.linspace(-1.0, 1.0, 128)[None, :]
    q, s, m = kv.asym_quant_math(y, 128, clip=0.5)
    assert q[0, 0] == 0 and q[0, -1] == 15
    assert float(m[0, 0]) == -0.5


def test_group_split():
    y = np.concatenate([np.zeros(64), np.arange(64.0)])[None, :]
    q, s, m = kv.asym_quant_math(y, 64)
    assert s.shape == (1, 2) and s[0, 0] == 0 and float(m[0, 1]) == 0.0
    assert q[0, -1] == 15


def test_pack_uint4():
    assert kv.pack_uint4(np.array([[1, 15, 0, 8]])).tolist() == [[0xF1, 0x80]]
    assert kv.unpack_uint4(np.array([[0xF1, 0x80]], dtype=np.uint8)).tolist() == [[1, 15, 0, 8]]


def test_score_invariance_under_headwise_rotation():
    # (qR)(kR)^T = q k^T when queries and keys share the head-wise rotation
    # (QuaRot blog "Quantizing the KV cache"; QuaRot paper keys/queries paragraph)
    b, s, hq, hkv, dh = 2, 5, 8, 2, 128
    q = wl.kv_tensor(5, 10, b, s, hq, dh).astype(np.float64)
    k = wl.kv_tensor(5, 11, b, s, hkv, dh).astype(np.float64)
    sg = wl.signs(5, dh)
    ref = kv.gqa_scores(q, k)
    got = kv.gqa_scores(had.rotate(q, sg), had.rotate(k, sg))
    rel = np.abs(got - ref).max() / np.abs(ref).max()
    assert rel < 1e-12


def test_gqa_mapping():
    q = np.zeros((1, 1, 4, 2))
    k = np.zeros((1, 1, 2, 2))
    q[0, 0, :, 0] = [1, 2, 3, 4]
    k[0, 0, :, 0] = [10, 100]
    s = kv.gqa_scores(q, k)[0, :, 0, 0]
    assert s.tolist() == [10, 20, 300, 400]  # q-heads 0,1 -> kv 0; 2,3 -> kv 1


def test_cache_append_positions():
    b, h, dh, smax = 2, 3, 128, 10
    cache_q = np.full((b, h, smax, dh // 2), 0xAA, dtype=np.uint8)
    meta = np.full((b, h, smax, 1, 2), -7.0, dtype=np.float16)
    x = wl.kv_tensor(5, 20, b, 4, h, dh)
    sg = wl.signs(5, dh)
    kv.kv_rotate_quant_cache(x, sg, True, 128, 0.95, cache_q, meta, start_pos=3)
    assert np.all(cache_q[:, :, :3] == 0xAA) and np.all(cache_q[:, :, 7:] == 0xAA)
    assert np.all(meta[:, :, :3] == -7.0) and np.all(meta[:, :, 7:] == -7.0)
    q, s, m = kv.asym_quant_math(had.rotate(x.astype(np.float64), sg), 128, 0.95)
    assert np.array_equal(cache_q[1, 2, 3 + 1], kv.pack_uint4(q[1, 1, 2]))
    assert meta[0, 1, 5, 0, 0] == s[0, 2, 1, 0] and meta[0, 1, 5, 0, 1] == m[0, 2, 1, 0]


@pytest.mark.parametrize("rotated", [True, False])
def test_recipe_agrees_with_math_away_from_ties(rotated):
    x = wl.kv_tensor(5, 1, 4, 16, 8, 128).astype(np.float64)
    sg = wl.signs(5, 128)
    y = had.rotate(x, sg) if rotated else x
    z = had.rotate_unnormalised(x, sg) if rotated else x
    qm, sm, mm = kv.asym_quant_math(y, 128, 0.95)
    qr, sr, mr = kv.asym_quant_recipe(z.astype(np.float32), 128, rotated, 128, 0.95)
    d_s = np.abs(sm.view(np.int16).astype(int) - sr.view(np.int16).astype(int))
    d_m = np.abs(mm.view(np.int16).astype(int) - mr.view(np.int16).astype(int))
    assert d_s.max() <= 1 and d_m.max() <= 1
    diff = qm.astype(int) - qr.astype(int)
    assert np.abs(diff).max() <= 1
    near = kv.asym_tie_distance(y, 128, sm, mm) < 5e-3
    assert not np.any((diff != 0) & ~near)


# ---------------------------------------------------------------------------
# 2- and 3-bit KV (QuaRot paper, KV bit-width study, Table 6)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [2, 3])
def test_bbit_ramp_group_codes(bits):
    # y = mn + k s with s, mn exact in fp16 and k = 0 .. 2^b - 1: codes are k
    levels = (1 << bits) - 1
    k = np.tile(np.arange(levels + 1), 128 // (levels + 1))
    y = (-1.5 + 0.25 * k).astype(np.float64)[None, :]
    q, s, m = kv.asym_quant_math(y, 128, bits=bits)
    assert float(s[0, 0]) == 0.25 and float(m[0, 0]) == -1.5 and np.array_equal(q[0], k)
    q2, s2, m2 = kv.asym_quant_recipe(y.astype(np.float32), 128, rotated=False, group=128, bits=bits)
    assert np.array_equal(q2[0], k) and s2[0, 0] == s[0, 0]


@pytest.mark.parametrize("bits", [2, 3])
def test_bbit_range_and_error(bits):
    levels = (1 << bits) - 1
    y = np.random.default_rng(60 + bits).standard_normal((16, 128))
    q, s, m = kv.asym_quant_math(y, 128, bits=bits)
    assert q.min() == 0 and q.max() == levels
    # reconstruction error within half a step (plus the fp16 rounding of scale and min)
    err = np.abs(kv.asym_dequant(q, s, m, 128) - y)
    step = s.astype(np.float64)[..., 0][:, None]
    assert (err <= 0.5 * step * (1 + 1e-2) + 1e-3 * np.abs(y).max()).all()
    # four bits reproduce the INT4 functions
    q4, s4, m4 = kv.asym_quant_math(y, 128)
    q4b, s4b, m4b = kv.asym_quant_math(y, 128, bits=4)
    assert np.array_equal(q4, q4b) and np.array_equal(s4, s4b) and np.array_equal(m4, m4b)


# ------------------- asymmetric tie distance and given (s, mn) -------------------
# s = 0.25 and mn = fp16(-0.9) = -0.89990234375, so mn / s is not an integer: a
# helper that forgot to subtract mn, added it, or took another group's (s, mn)
# would move these values.  Group 0's u = (y - mn) / s = 2.5, 2, 0, 14.5;
# group 1 (s = 0.5, mn = 1) has u = 0.25, 3.5, 15.75 (clamped to 15), -1 (to 0).

def _two_groups():
    m0 = float(np.float16(-0.9))
    y0 = m0 + 0.25 * np.array([2.5, 2.0, 0.0, 14.5])
    y1 = 1.0 + 0.5 * np.array([0.25, 3.5, 15.75, -1.0])
    s = np.array([[0.25, 0.5]], dtype=np.float16)
    m = np.array([[m0, 1.0]], dtype=np.float16)
    return np.concatenate([y0, y1])[None, :], s, m


def test_asym_tie_distance_hand_values():
    y, s, m = _two_groups()
    got = kv.asym_tie_distance(y, 4, s, m)
    assert np.allclose(got, [[0.0, 0.5, 0.5, 0.0, 0.25, 0.0, 0.25, 0.5]], rtol=0, atol=1e-12)


def test_asym_quant_with_params_hand_values():
    y, s, m = _two_groups()
    q = kv.asym_quant_with_params(y, 4, s, m)
    assert q.tolist() == [[2, 2, 0, 14, 0, 4, 15, 0]]
    q3 = kv.asym_quant_with_params(y, 4, s, m, bits=3)  # 7 levels: 14 -> 7, 15 -> 7
    assert q3.tolist() == [[2, 2, 0, 7, 0, 4, 7, 0]]
    z = kv.asym_quant_with_params(y, 4, np.zeros_like(s), m)
    assert not z.any()
