"""GPU parity: 2- and 3-bit K/V (QuaRot paper, KV bit-width study, Table 6)
through qr_kv_rotate_quant_bits, and the Decode routine over such caches."""
import numpy as np
import pytest

import workloads as wl
from oracle import attention as oatt
from oracle import hadamard as oh
from oracle import kv as okv

from parity import check_asym, check_rotation, decode_bound

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
qr = pytest.importorskip("hadamard_rotation_int4_amd")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("rot", [True, False])
@pytest.mark.parametrize("Dh,group", [(128, 128), (128, 32), (64, 64)])
def test_init_append_grid_bit_exact(bits, rot, Dh, group):
    B, H, S0, steps, clip = 2, 4, 13, 3, 0.95
    S_max = S0 + steps
    x = wl.grid_activations(6, Dh + bits, B * S_max * H, Dh).reshape(B, S_max, H, Dh)
    s = wl.signs(6, Dh)
    cq = torch.zeros((B, H, S_max, Dh // 2), dtype=torch.uint8, device="cuda")
    cm = torch.zeros((B, H, S_max, Dh // group, 2), dtype=torch.float16, device="cuda")
    ref_q = np.zeros((B, H, S_max, Dh // 2), np.uint8)
    ref_m = np.zeros((B, H, S_max, Dh // group, 2), np.float16)
    qr.kv_rotate_quant(dev(x[:, :S0]), dev(s), group, clip, cq, cm, 0, rotate=rot, bits=bits)
    okv.kv_rotate_quant_cache(x[:, :S0], s, rot, group, clip, ref_q, ref_m, 0, mode="recipe",
                              bits=bits)
    for i in range(steps):
        qr.kv_rotate_quant(dev(x[:, S0 + i:S0 + i + 1]), dev(s), group, clip, cq, cm, S0 + i,
                           rotate=rot, bits=bits)
        okv.kv_rotate_quant_cache(x[:, S0 + i:S0 + i + 1], s, rot, group, clip, ref_q, ref_m,
                                  S0 + i, mode="recipe", bits=bits)
    assert np.array_equal(host(cq), ref_q)
    assert np.array_equal(host(cm).view(np.uint16), ref_m.view(np.uint16))
    assert okv.unpack_uint4(host(cq)).max() <= (1 << bits) - 1


@pytest.mark.parametrize("bits", [2, 3])
def test_gaussian_outliers_tolerance(bits):
    B, H, S, Dh, group, clip = 4, 8, 33, 128, 128, 0.95
    x = wl.kv_tensor(6, 1, B, S, H, Dh)
    s = wl.signs(6, Dh)
    cq = torch.zeros((B, H, S, Dh // 2), dtype=torch.uint8, device="cuda")
    cm = torch.zeros((B, H, S, Dh // group, 2), dtype=torch.float16, device="cuda")
    z = qr.kv_rotate_quant(dev(x), dev(s), group, clip, cq, cm, 0, z_dbg=True, bits=bits)
    z64 = oh.rotate_unnormalised(x.astype(np.float64), s)
    check_rotation(host(z).reshape(-1, Dh), z64.reshape(-1, Dh))
    codes = okv.unpack_uint4(np.transpose(host(cq), (0, 2, 1, 3)))
    meta = np.transpose(host(cm), (0, 2, 1, 3, 4))
    check_asym(codes, meta[..., 0], meta[..., 1], z64 / np.sqrt(Dh), group, clip, bits)


@pytest.mark.parametrize("kbits,vbits", [(3, 3), (4, 3), (4, 2)])
def test_decode_over_low_bit_cache(kbits, vbits):
    # the Decode routine reads code * scale + min whatever the width; compare
    # with the oracle's attention over the same dequantized cache
    B, Hkv, Hq, Dh, G, L = 2, 2, 8, 128, 128, 300
    k = wl.kv_tensor(6, 2, B, L, Hkv, Dh)
    v = wl.kv_tensor(6, 3, B, L, Hkv, Dh)
    s = wl.signs(6, Dh)
    caches = []
    for t, bits, rot in ((k, kbits, True), (v, vbits, False)):
        cq = torch.zeros((B, Hkv, L, Dh // 2), dtype=torch.uint8, device="cuda")
        cm = torch.zeros((B, Hkv, L, Dh // G, 2), dtype=torch.float16, device="cuda")
        qr.kv_rotate_quant(dev(t), dev(s) if rot else None, G, 0.95, cq, cm, 0, rotate=rot,
                           bits=bits)
        caches += [cq, cm]
    q = wl.queries(6, 4, B, Hq, Dh)
    qrot = qr.hadamard(dev(q.reshape(-1, Dh)), dev(s), torch.float16).view(B, Hq, Dh)
    scale = 1.0 / np.sqrt(Dh)
    ws = torch.empty((qr.kv_decode_workspace_bytes(B, Hq, Hkv, Dh, L),), dtype=torch.uint8,
                     device="cuda")
    out = qr.kv_decode_attention(qrot, *caches, L, G, scale, workspace=ws)
    ref = oatt.decode_attention(host(qrot), *(host(c) for c in caches), L, G, scale)
    err = np.abs(host(out).astype(np.float64) - ref)
    bound = decode_bound(host(qrot), *(host(c) for c in caches), L, G, scale, ref)
    assert (err <= bound).all(), float((err / bound).max())
