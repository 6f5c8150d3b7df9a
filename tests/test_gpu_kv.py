"""GPU parity: qr_kv_rotate_quant (Init + Append into the packed cache) and the
score invariance of rotated queries/keys."""
import numpy as np
import pytest

import workloads as wl
from oracle import hadamard as oh
from oracle import kv as okv

from parity import check_asym, check_rotation

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
qr = pytest.importorskip("hadamard_rotation_int4_amd")

SENT_Q = 0xA5
SENT_M = np.float16(-3.5)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def fresh_cache(B, H, S_max, Dh, group):
    cq = torch.full((B, H, S_max, Dh // 2), SENT_Q, dtype=torch.uint8, device="cuda")
    cm = torch.full((B, H, S_max, Dh // group, 2), float(SENT_M), dtype=torch.float16, device="cuda")
    return cq, cm


@pytest.mark.parametrize("rot", [True, False])
@pytest.mark.parametrize("Dh,group", [(128, 128), (128, 32), (64, 64), (256, 128), (32, 8)])
def test_init_append_grid_bit_exact(rot, Dh, group):
    B, H, S0, steps, clip = 3, 4, 19, 5, 0.95
    S_max = S0 + steps + 2
    x = wl.grid_activations(5, Dh + group, B * (S0 + steps) * H, Dh).reshape(B, S0 + steps, H, Dh)
    s = wl.signs(5, Dh)
    cq, cm = fresh_cache(B, H, S_max, Dh, group)
    ref_q = np.full((B, H, S_max, Dh // 2), SENT_Q, dtype=np.uint8)
    ref_m = np.full((B, H, S_max, Dh // group, 2), SENT_M, dtype=np.float16)
    qr.kv_rotate_quant(dev(x[:, :S0]), dev(s), group, clip, cq, cm, 0, rotate=rot)
    okv.kv_rotate_quant_cache(x[:, :S0], s, rot, group, clip, ref_q, ref_m, 0, mode="recipe")
    for i in range(steps):
        qr.kv_rotate_quant(dev(x[:, S0 + i:S0 + i + 1]), dev(s), group, clip, cq, cm, S0 + i, rotate=rot)
        okv.kv_rotate_quant_cache(x[:, S0 + i:S0 + i + 1], s, rot, group, clip, ref_q, ref_m, S0 + i,
                                  mode="recipe")
    assert np.array_equal(host(cq), ref_q)
    assert np.array_equal(host(cm).view(np.uint16), ref_m.view(np.uint16))


@pytest.mark.parametrize("rot", [True, False])
def test_gaussian_outliers_tolerance(rot):
    B, H, S, Dh, group, clip = 4, 8, 33, 128, 128, 0.95
    x = wl.kv_tensor(5, 0, B, S, H, Dh)
    s = wl.signs(5, Dh)
    cq, cm = fresh_cache(B, H, S, Dh, group)
    z = qr.kv_rotate_quant(dev(x), dev(s), group, clip, cq, cm, 0, rotate=rot, z_dbg=True)
    x64 = x.astype(np.float64)
    z64 = oh.rotate_unnormalised(x64, s) if rot else x64
    check_rotation(host(z).reshape(-1, Dh), z64.reshape(-1, Dh))
    y64 = z64 / np.sqrt(Dh) if rot else x64
    codes = okv.unpack_uint4(np.transpose(host(cq), (0, 2, 1, 3)))     # [B, S, H, Dh]
    meta = np.transpose(host(cm), (0, 2, 1, 3, 4))                   # [B, S, H, G, 2]
    check_asym(codes, meta[..., 0], meta[..., 1], y64, group, clip)


def test_scores_invariant_under_rotation():
    # 70B-shaped GQA (8 query heads per KV head), scaled down in batch and length
    B, S, Hq, Hkv, Dh = 2, 40, 16, 2, 128
    q = wl.kv_tensor(5, 10, B, S, Hq, Dh)
    k = wl.kv_tensor(5, 11, B, S, Hkv, Dh)
    s = wl.signs(5, Dh)
    qrot = host(qr.hadamard(dev(q.reshape(-1, Dh)), dev(s))).reshape(B, S, Hq, Dh)
    cq, cm = fresh_cache(B, Hkv, S, Dh, 128)
    z = host(qr.kv_rotate_quant(dev(k), dev(s), 128, 0.95, cq, cm, 0, z_dbg=True))
    krot = z.astype(np.float64) / np.sqrt(Dh)
    ref = okv.gqa_scores(q.astype(np.float64), k.astype(np.float64))
    got = okv.gqa_scores(qrot.astype(np.float64), krot)
    rel = np.abs(got - ref).max(axis=-1) / np.abs(ref).max(axis=-1)
    assert rel.max() <= 1e-3


def test_untouched_positions_and_noop():
    B, H, Dh = 2, 3, 128
    cq, cm = fresh_cache(B, H, 8, Dh, 128)
    x = wl.kv_tensor(5, 3, B, 2, H, Dh)
    qr.kv_rotate_quant(dev(x), dev(wl.signs(5, Dh)), 128, 1.0, cq, cm, 5)
    hq, hm = host(cq), host(cm)
    assert np.all(hq[:, :, :5] == SENT_Q) and np.all(hq[:, :, 7:] == SENT_Q)
    assert np.all(hm[:, :, :5] == SENT_M) and np.all(hm[:, :, 7:] == SENT_M)
    assert not np.all(hq[:, :, 5:7] == SENT_Q)
    qr.kv_rotate_quant(dev(x[:, :0]), None, 128, 1.0, cq, cm, 8)   # S_new = 0 at the end: no-op
    assert np.array_equal(host(cq), hq)


@pytest.mark.parametrize("signed", [True, False])
def test_strided_tokens_and_plain_hadamard(signed):
    # tokens padded to H * Dh + 64 elements (a slice of a wider projection
    # output); signs NULL is the plain Hadamard (all +1).  Grid inputs: the
    # cache is bit-exact against the oracle's recipe.
    B, S, H, Dh, G, clip = 2, 21, 3, 128, 128, 0.95
    ld = H * Dh + 64
    x = wl.grid_activations(5, 77, B * S, ld).reshape(B, S, ld)
    s = wl.signs(5, Dh) if signed else None
    xt = dev(x)[:, :, :H * Dh].reshape(B, S, H, Dh)     # token stride ld, heads packed
    assert xt.stride(1) == ld
    cq, cm = fresh_cache(B, H, S + 3, Dh, G)
    qr.kv_rotate_quant(xt, dev(s) if signed else None, G, clip, cq, cm, 2)
    ref_q = np.full((B, H, S + 3, Dh // 2), SENT_Q, dtype=np.uint8)
    ref_m = np.full((B, H, S + 3, 1, 2), SENT_M, dtype=np.float16)
    okv.kv_rotate_quant_cache(x[:, :, :H * Dh].reshape(B, S, H, Dh), s, True, G, clip, ref_q, ref_m,
                              2, mode="recipe")
    assert np.array_equal(host(cq), ref_q)
    assert np.array_equal(host(cm).view(np.uint16), ref_m.view(np.uint16))


@pytest.mark.parametrize("rot", [True, False])
def test_cache_only_dword_aligned(rot):
    # cache_q needs only 4-byte alignment: a view 4 bytes into a buffer (the Dh = 128
    # kernel writes each row's 64 bytes as 16-byte pieces at that address); Init and
    # one Append on grid inputs are bit-exact against the oracle's recipe, and the
    # bytes around the view stay untouched.
    B, S, H, Dh, G, clip = 2, 21, 3, 128, 128, 0.95
    S_max = S + 4
    x = wl.grid_activations(5, 91, B * (S + 1) * H, Dh).reshape(B, S + 1, H, Dh)
    s = wl.signs(5, Dh)
    n = B * H * S_max * (Dh // 2)
    buf = torch.full((n + 16,), SENT_Q, dtype=torch.uint8, device="cuda")
    cq = buf[4:4 + n].view(B, H, S_max, Dh // 2)
    assert cq.data_ptr() % 16 == 4
    cm = torch.full((B, H, S_max, 1, 2), float(SENT_M), dtype=torch.float16, device="cuda")
    ref_q = np.full((B, H, S_max, Dh // 2), SENT_Q, dtype=np.uint8)
    ref_m = np.full((B, H, S_max, 1, 2), SENT_M, dtype=np.float16)
    qr.kv_rotate_quant(dev(x[:, :S]), dev(s), G, clip, cq, cm, 1, rotate=rot)
    okv.kv_rotate_quant_cache(x[:, :S], s, rot, G, clip, ref_q, ref_m, 1, mode="recipe")
    qr.kv_rotate_quant(dev(x[:, S:]), dev(s), G, clip, cq, cm, S + 1, rotate=rot)
    okv.kv_rotate_quant_cache(x[:, S:], s, rot, G, clip, ref_q, ref_m, S + 1, mode="recipe")
    assert np.array_equal(host(cq), ref_q)
    assert np.array_equal(host(cm).view(np.uint16), ref_m.view(np.uint16))
    hb = host(buf)
    assert np.all(hb[:4] == SENT_Q) and np.all(hb[4 + n:] == SENT_Q)
