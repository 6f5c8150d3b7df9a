"""GPU parity: qr_kv_decode_attention (the Decode routine over the 4-bit cache)
against the float64 oracle.

Tolerance: the per-element bound parity.decode_bound derives from the
kernel's arithmetic -- the fp16 rounding of each weight p_j s_j (relative
2^-11, plus the fp16 subnormal spacing), the fp32 score sums over exact code
products (relative 2^-17 of the sum of magnitudes, which moves each weight and
so the output by at most twice that times max|v|), the fp32 sums over the
positions, and the final rounding to fp16 (2^-11 |ref|).

Cases: one position, ragged lengths around the 256-position chunk, grouped-
query ratios 1, 8 and 16, a sharp softmax, many splits, the Llama-2-70B decode
shape (batch 32, 64 query / 8 KV heads, 2048 + 50 positions) on sampled
sequences, and the cache written by qr_kv_rotate_quant (Init + Appends) read
back by the Decode routine.
"""
import numpy as np
import pytest

import workloads as wl
from oracle import attention as oatt
from oracle import hadamard as oh
from oracle import kv as okv
from parity import decode_bound

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
qr = pytest.importorskip("hadamard_rotation_int4_amd")

WID = 9  # workload id of the seeded decode inputs


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def check(got, ref, q, k_q, k_meta, v_q, v_meta, L, group, scale):
    err = np.abs(got.astype(np.float64) - ref)
    bound = decode_bound(q, k_q, k_meta, v_q, v_meta, L, group, scale, ref)
    worst = float((err / bound).max())
    print(f"decode L={L}: max error / bound = {worst:.3f}, max error {err.max():.3e}")
    assert worst <= 1.0, f"max error / bound = {worst:.3f}"
    return worst


@pytest.mark.parametrize("B,Hq,Hkv,S_max,L,qstd", [
    (2, 16, 2, 600, 1, 1.0),
    (2, 16, 2, 600, 17, 1.0),
    (2, 16, 2, 600, 256, 1.0),
    (2, 16, 2, 600, 257, 1.0),
    (2, 16, 2, 600, 600, 1.0),
    (3, 4, 4, 300, 300, 1.0),       # one query head per KV head
    (1, 16, 1, 1030, 1029, 1.0),    # 16 query heads per KV head
    (2, 16, 2, 700, 650, 8.0),      # sharp softmax
    (1, 8, 1, 5000, 4999, 1.0),     # 20 chunks, one split each
])
def test_decode_random_cache(B, Hq, Hkv, S_max, L, qstd):
    Dh = group = 128
    tid = B * 1000 + L
    kq, km = wl.kv_cache_random(WID, tid, B, Hkv, S_max, Dh, group)
    vq, vm = wl.kv_cache_random(WID, tid + 1, B, Hkv, S_max, Dh, group)
    q = wl.queries(WID, tid, B, Hq, Dh, qstd)
    scale = 1.0 / np.sqrt(Dh)
    got = host(qr.kv_decode_attention(dev(q), dev(kq), dev(km), dev(vq), dev(vm), L, group, scale))
    ref = oatt.decode_attention(q, kq, km, vq, vm, L, group, scale)
    check(got, ref, q, kq, km, vq, vm, L, group, scale)


def test_decode_workspace_and_out_reuse():
    B, Hq, Hkv, S_max, Dh = 2, 16, 2, 900, 128
    kq, km = wl.kv_cache_random(WID, 50, B, Hkv, S_max, Dh, Dh)
    vq, vm = wl.kv_cache_random(WID, 51, B, Hkv, S_max, Dh, Dh)
    q = wl.queries(WID, 50, B, Hq, Dh)
    args = [dev(a) for a in (q, kq, km, vq, vm)]
    nbytes = qr.kv_decode_workspace_bytes(B, Hq, Hkv, Dh, S_max)
    ws = torch.full((nbytes,), 0x7F, dtype=torch.uint8, device="cuda")   # stale contents
    out = torch.empty((B, Hq, Dh), dtype=torch.float16, device="cuda")
    for L in (900, 300, 37):    # a longer call leaves records a shorter one must not read
        qr.kv_decode_attention(*args, L, 128, 0.1, out=out, workspace=ws)
        ref = oatt.decode_attention(q, kq, km, vq, vm, L, 128, 0.1)
        check(host(out), ref, q, kq, km, vq, vm, L, 128, 0.1)


@pytest.mark.parametrize("L", [2049, 2098])
def test_decode_70b_shape_sampled(L):
    kvw = wl.WORKLOADS["70b_kv"].kv
    B, Hq, Hkv, Dh, G = kvw["batch"], kvw["q_heads"], kvw["kv_heads"], kvw["head_dim"], kvw["group"]
    S_max = kvw["prefill"] + kvw["decode"]
    cuda = torch.device("cuda")
    kq, km = wl.kv_cache_random_torch(torch, cuda, WID, 70, B, Hkv, S_max, Dh, G)
    vq, vm = wl.kv_cache_random_torch(torch, cuda, WID, 71, B, Hkv, S_max, Dh, G)
    q = dev(wl.queries(WID, 70, B, Hq, Dh))
    scale = 1.0 / np.sqrt(Dh)
    got = host(qr.kv_decode_attention(q, kq, km, vq, vm, L, G, scale))
    bs = np.array([0, 13, 22, B - 1])
    bi = torch.as_tensor(bs, device=cuda)
    sub = [host(t.index_select(0, bi)) for t in (q, kq, km, vq, vm)]
    ref = oatt.decode_attention(*sub, L, G, scale)
    check(got[bs], ref, *sub, L, G, scale)


def test_decode_reads_the_cache_that_init_and_append_write():
    """K and V of exact-in-fp32 grid values go through qr_kv_rotate_quant (Init of
    300 positions, then 5 Appends), bit-exactly like the oracle's recipe; the
    Decode routine then reads the GPU cache and the oracle its own."""
    B, Hkv, Hq, Dh, G, P, steps, clip = 2, 2, 16, 128, 128, 300, 5, 0.95
    S_max = P + steps
    s = wl.signs(WID, Dh)
    kx = wl.grid_activations(WID, 1, B * S_max * Hkv, Dh).reshape(B, S_max, Hkv, Dh)
    vx = wl.grid_activations(WID, 2, B * S_max * Hkv, Dh).reshape(B, S_max, Hkv, Dh)
    caches = {}
    for name, x, rot in (("k", kx, True), ("v", vx, False)):
        cq = torch.zeros((B, Hkv, S_max, Dh // 2), dtype=torch.uint8, device="cuda")
        cm = torch.zeros((B, Hkv, S_max, Dh // G, 2), dtype=torch.float16, device="cuda")
        rq = np.zeros((B, Hkv, S_max, Dh // 2), dtype=np.uint8)
        rm = np.zeros((B, Hkv, S_max, Dh // G, 2), dtype=np.float16)
        qr.kv_rotate_quant(dev(x[:, :P]), dev(s), G, clip, cq, cm, 0, rotate=rot)
        okv.kv_rotate_quant_cache(x[:, :P], s, rot, G, clip, rq, rm, 0, mode="recipe")
        for i in range(steps):
            qr.kv_rotate_quant(dev(x[:, P + i:P + i + 1]), dev(s), G, clip, cq, cm, P + i, rotate=rot)
            okv.kv_rotate_quant_cache(x[:, P + i:P + i + 1], s, rot, G, clip, rq, rm, P + i,
                                      mode="recipe")
        assert np.array_equal(host(cq), rq)
        assert np.array_equal(host(cm).view(np.uint16), rm.view(np.uint16))
        caches[name] = (cq, cm, rq, rm)
    # the query carries the keys' head-wise rotation (computed by the oracle, fp16)
    q = oh.rotate(wl.queries(WID, 3, B, Hq, Dh).astype(np.float64), s).astype(np.float16)
    scale = 1.0 / np.sqrt(Dh)
    for L in (P, S_max):
        got = host(qr.kv_decode_attention(dev(q), caches["k"][0], caches["k"][1], caches["v"][0],
                                          caches["v"][1], L, G, scale))
        ref = oatt.decode_attention(q, caches["k"][2], caches["k"][3], caches["v"][2],
                                    caches["v"][3], L, G, scale)
        check(got, ref, q, caches["k"][2], caches["k"][3], caches["v"][2], caches["v"][3], L, G,
              scale)
