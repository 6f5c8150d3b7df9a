"""The allocation-free Decode entry point (qr_kv_decode_attention_noalloc,
called through the C ABI) against the entry point with a caller workspace:
bit-identical outputs on two calls in a row, the second one smaller, both
with the positions split over several workgroups so that the static scratch
holds the split records; then a shape that needs no scratch at all."""
import ctypes

import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
qr = pytest.importorskip("hadamard_rotation_int4_amd")


def vp(t):
    return ctypes.c_void_p(t.data_ptr())


def call_noalloc(q, kq, km, vq, vm, L, scale, out):
    B, Hq, Dh = q.shape
    Hkv, S_max = kq.shape[1], kq.shape[2]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return qr._load().qr_kv_decode_attention_noalloc(vp(q), B, Hq, Hkv, Dh, vp(kq), vp(km),
                                                     vp(vq), vp(vm), S_max, L, 128, scale,
                                                     vp(out), stream)


def call_workspace(q, kq, km, vq, vm, L, scale, out):
    B, Hq, Dh = q.shape
    Hkv, S_max = kq.shape[1], kq.shape[2]
    n = qr.kv_decode_workspace_bytes(B, Hq, Hkv, Dh, L)
    ws = torch.empty((max(n, 4),), dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return qr._load().qr_kv_decode_attention(vp(q), B, Hq, Hkv, Dh, vp(kq), vp(km), vp(vq),
                                             vp(vm), S_max, L, 128, scale, vp(out), vp(ws), n,
                                             stream)


def inputs(tid, B, Hq, Hkv, S_max):
    kq, km = wl.kv_cache_random(94, tid, B, Hkv, S_max, 128, 128)
    vq, vm = wl.kv_cache_random(94, tid + 1, B, Hkv, S_max, 128, 128)
    q = wl.queries(94, tid, B, Hq, 128)
    return [torch.from_numpy(a).cuda() for a in (q, kq, km, vq, vm)]


# (B, Hq, Hkv, S_max, L, splits > 1): the second call is smaller than the first
CASES = [(2, 16, 2, 3000, 3000), (1, 8, 1, 800, 700), (32, 64, 8, 300, 300)]


def test_noalloc_matches_workspace_entry_point():
    scale = 1.0 / np.sqrt(128)
    for i, (B, Hq, Hkv, S_max, L) in enumerate(CASES):
        print(f"noalloc case B={B} Hq={Hq} Hkv={Hkv} L={L}", flush=True)
        args = inputs(10 * i, B, Hq, Hkv, S_max)
        got = torch.full((B, Hq, 128), 7.0, dtype=torch.float16, device="cuda")
        ref = torch.empty((B, Hq, 128), dtype=torch.float16, device="cuda")
        assert call_noalloc(*args, L, scale, got) == 0
        assert call_workspace(*args, L, scale, ref) == 0
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"case {i}"


def test_noalloc_rejects_a_call_beyond_its_scratch():
    # 255 sequences of one KV head with 16 query heads split over 2 x 256-position
    # chunks: 4.2 MB of records, more than the 4 MiB static buffer; nothing runs.
    assert qr.kv_decode_workspace_bytes(255, 16, 1, 128, 512) > 4 << 20
    code = qr._load().qr_kv_decode_attention_noalloc(None, 255, 16, 1, 128, None, None, None, None,
                                                     512, 512, 128, 0.088, None, None)
    assert code == 7, qr.status_str(code)
