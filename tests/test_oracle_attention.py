"""Pins for the oracle's decode attention over the 4-bit KV cache.

Independent references: PyTorch's scaled_dot_product_attention (float64, CPU)
on the dequantized cache, closed forms and invariances.
"""
import numpy as np
import pytest

from oracle import attention as att
from oracle import kv

torch = pytest.importorskip("torch")


def random_cache(rng, b, h, s_max, dh, group):
    codes = rng.integers(0, 16, size=(b, h, s_max, dh))
    meta = np.stack([rng.uniform(0.01, 0.2, size=(b, h, s_max, dh // group)),
                     rng.uniform(-1.5, 0.0, size=(b, h, s_max, dh // group))], axis=-1)
    return kv.pack_uint4(codes), meta.astype(np.float16)


@pytest.mark.parametrize("b,hq,hkv,dh,group,L,s_max", [
    (2, 4, 2, 64, 64, 37, 40),
    (1, 8, 1, 128, 128, 300, 300),
    (3, 6, 6, 32, 16, 5, 9),
])
def test_matches_torch_sdpa(b, hq, hkv, dh, group, L, s_max):
    rng = np.random.default_rng(b * 100 + hq)
    kq, km = random_cache(rng, b, hkv, s_max, dh, group)
    vq, vm = random_cache(rng, b, hkv, s_max, dh, group)
    q = rng.normal(size=(b, hq, dh)).astype(np.float16)
    scale = 1.0 / np.sqrt(dh)
    got = att.decode_attention(q, kq, km, vq, vm, L, group, scale)
    # independent: dequantize, repeat kv heads (grouped-query convention), SDPA
    k = torch.from_numpy(att.dequant_cache(kq, km, L, group)).repeat_interleave(hq // hkv, dim=1)
    v = torch.from_numpy(att.dequant_cache(vq, vm, L, group)).repeat_interleave(hq // hkv, dim=1)
    qt = torch.from_numpy(q.astype(np.float64))[:, :, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, k, v, scale=scale)[:, :, 0, :]
    np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-12)


def test_dequant_layout():
    # code 2j sits in the low nibble of byte j; value = code * scale + min per group
    codes = np.arange(16, dtype=np.int64)[None, None, None, :]
    meta = np.array([[[[[0.5, -2.0], [0.25, 1.0]]]]], dtype=np.float16)  # two groups of 8
    out = att.dequant_cache(kv.pack_uint4(codes), meta, 1, 8)[0, 0, 0]
    expect = np.concatenate([np.arange(8) * 0.5 - 2.0, np.arange(8, 16) * 0.25 + 1.0])
    np.testing.assert_array_equal(out, expect)


def test_equal_keys_give_mean_of_values():
    rng = np.random.default_rng(1)
    b, h, L, dh = 1, 1, 50, 32
    kcodes = np.tile(rng.integers(0, 16, size=(1, 1, 1, dh)), (1, 1, L, 1))
    km = np.tile(np.array([0.1, -0.7], dtype=np.float16), (b, h, L, 1, 1))
    vq, vm = random_cache(rng, b, h, L, dh, dh)
    q = rng.normal(size=(b, h, dh)).astype(np.float16)
    got = att.decode_attention(q, kv.pack_uint4(kcodes), km, vq, vm, L, dh, 0.3)
    mean = att.dequant_cache(vq, vm, L, dh).mean(axis=2)
    np.testing.assert_allclose(got, mean, rtol=0, atol=1e-12)


def test_dominant_key_returns_its_value():
    rng = np.random.default_rng(2)
    b, h, L, dh = 1, 1, 20, 16
    kcodes = np.zeros((b, h, L, dh), dtype=np.int64)
    kcodes[0, 0, 7] = 15                                    # key 7 aligned with q = +1
    km = np.tile(np.array([1.0, 0.0], dtype=np.float16), (b, h, L, 1, 1))
    vq, vm = random_cache(rng, b, h, L, dh, dh)
    q = np.ones((b, h, dh), dtype=np.float16)
    got = att.decode_attention(q, kv.pack_uint4(kcodes), km, vq, vm, L, dh, 1.0)
    # scores: 240 for key 7, 0 elsewhere -> weight of the rest is 19 e^-240
    np.testing.assert_allclose(got[0, 0], att.dequant_cache(vq, vm, L, dh)[0, 0, 7], rtol=0,
                               atol=1e-90)


def test_invariant_to_key_min_shift_and_linear_in_value_scale():
    rng = np.random.default_rng(3)
    b, hq, hkv, L, dh = 2, 4, 2, 33, 64
    kq, km = random_cache(rng, b, hkv, L, dh, dh)
    km[..., 1] = (np.round(km[..., 1].astype(np.float64) * 64) / 64).astype(np.float16)
    vq, vm = random_cache(rng, b, hkv, L, dh, dh)
    q = rng.normal(size=(b, hq, dh)).astype(np.float16)
    base = att.decode_attention(q, kq, km, vq, vm, L, dh, 0.2)
    # one group per key: shifting every key min by the same delta adds
    # delta * sum(q) to every score of a head, which softmax ignores
    km2 = km.copy()
    km2[..., 1] = (km[..., 1].astype(np.float64) + 0.5).astype(np.float16)
    assert np.array_equal(km2[..., 1].astype(np.float64), km[..., 1].astype(np.float64) + 0.5)
    np.testing.assert_allclose(att.decode_attention(q, kq, km2, vq, vm, L, dh, 0.2), base,
                               rtol=1e-12, atol=1e-12)
    # doubling every value scale and min doubles the output
    vm2 = (vm.astype(np.float64) * 2).astype(np.float16)
    np.testing.assert_allclose(att.decode_attention(q, kq, km, vq, vm2, L, dh, 0.2), 2 * base,
                               rtol=1e-12, atol=1e-12)


def test_positions_past_length_are_ignored():
    rng = np.random.default_rng(4)
    kq, km = random_cache(rng, 1, 1, 40, 32, 32)
    vq, vm = random_cache(rng, 1, 1, 40, 32, 32)
    q = rng.normal(size=(1, 1, 32)).astype(np.float16)
    a = att.decode_attention(q, kq, km, vq, vm, 25, 32, 0.5)
    kq2, vq2 = kq.copy(), vq.copy()
    kq2[:, :, 25:] = 0xFF
    vq2[:, :, 25:] = 0x77
    np.testing.assert_array_equal(att.decode_attention(q, kq2, km, vq2, vm, 25, 32, 0.5), a)
