"""Guard bands: every output of the hot path is written into the middle of a
larger buffer filled with a poison byte, on ragged shapes (T and N not
multiples of any tile, K with a tail past the K step, row widths whose last
chunk is partial), and the bytes around it must come back untouched.  An
out-of-bounds store would otherwise land in a neighbouring allocation without
any error.  The outputs themselves are compared with a plain call's."""
import ctypes

import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
qr = pytest.importorskip("hadamard_rotation_int4_amd")

GUARD = 4096          # bytes on each side
POISON = 0xA5


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


class Guarded:
    """A device view of `nbytes` bytes between two poisoned guard bands."""

    def __init__(self, nbytes, dtype, shape):
        self.n = nbytes
        self.buf = torch.full((nbytes + 2 * GUARD,), POISON, dtype=torch.uint8, device="cuda")
        self.view = self.buf[GUARD:GUARD + nbytes].view(dtype).view(shape)

    def check(self):
        torch.cuda.synchronize()
        b = self.buf.cpu().numpy()
        lo, hi = b[:GUARD], b[GUARD + self.n:]
        assert (lo == POISON).all(), f"write below the output at {np.flatnonzero(lo != POISON)[-1] - GUARD}"
        assert (hi == POISON).all(), f"write past the output at +{np.flatnonzero(hi != POISON)[0]}"


def guarded_like(shape, dtype):
    nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    return Guarded(nbytes, dtype, shape)


@pytest.mark.parametrize("d", [344, 4096, 8192, 11008, 28672])
@pytest.mark.parametrize("T", [1, 37])
def test_hadamard_quant(T, d):
    x = dev(wl.activations(90, 0, T, d, n_outliers=4))
    s = dev(wl.signs(90, d))
    q_ref, sc_ref = qr.hadamard_quant(x, s)
    q, sc = guarded_like((T, d // 2), torch.uint8), guarded_like((T,), torch.float16)
    qr.hadamard_quant(x, s, out=(q.view, sc.view))
    q.check(), sc.check()
    assert torch.equal(q.view, q_ref) and torch.equal(sc.view, sc_ref)
    q8, sc8 = guarded_like((T, d), torch.int8), guarded_like((T,), torch.float16)
    qr.hadamard_quant_i8(x, s, 1.0, 8, out=(q8.view, sc8.view))
    q8.check(), sc8.check()


@pytest.mark.parametrize("T,d", [(37, 8192), (5, 4096)])
def test_block_quantizers(T, d):
    x = dev(wl.activations(91, 0, T, d, n_outliers=4))
    for fn, args in ((qr.rmsnorm_quant, (1e-5, 1.0)), (qr.hadamard_heads_quant, (64, 1.0))):
        q, sc = guarded_like((T, d // 2), torch.uint8), guarded_like((T,), torch.float16)
        fn(x, *args, out=(q.view, sc.view))
        q.check(), sc.check()
        q_ref, sc_ref = fn(x, *args)
        assert torch.equal(q.view, q_ref) and torch.equal(sc.view, sc_ref)


# tiled (128 x 128 and 256 x 256) and weight-streaming shapes with ragged T, N and K tails
GEMM_SHAPES = [(300, 260, 192), (4000, 4000, 320), (3000, 4100, 4160), (17, 100, 4160),
               (64, 33, 64), (1, 4100, 11008), (65, 129, 448)]


@pytest.mark.parametrize("T,N,K", GEMM_SHAPES)
@pytest.mark.parametrize("bits", [4, 8])
def test_gemm_outputs(T, N, K, bits):
    if bits == 4:
        a, w = dev(wl.packed_codes(92, 0, T, K)), dev(wl.packed_codes(92, 1, N, K))
        fn = qr._load().qr_w4a4_gemm
    else:
        a = dev(wl.packed_codes(92, 2, T, 2 * K).view(np.int8))
        w = dev(wl.packed_codes(92, 3, N, 2 * K).view(np.int8))
        fn = qr._load().qr_w8a8_gemm
    asc, wsc = dev(wl.positive_scales(92, 0, T)), dev(wl.positive_scales(92, 1, N))
    y, acc = guarded_like((T, N), torch.float16), guarded_like((T, N), torch.int32)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    code = fn(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(asc.data_ptr()), T,
              ctypes.c_void_p(w.data_ptr()), ctypes.c_void_p(wsc.data_ptr()), N, K,
              ctypes.c_void_p(y.view.data_ptr()), ctypes.c_void_p(acc.view.data_ptr()), stream)
    assert code == 0, qr.status_str(code)
    y.check(), acc.check()
    gemm = qr.w4a4_gemm if bits == 4 else qr.w8a8_gemm
    y_ref, acc_ref = gemm(a, asc, w, wsc, acc_dbg=True)
    assert torch.equal(acc.view, acc_ref) and torch.equal(y.view.view(torch.int16), y_ref.view(torch.int16))


@pytest.mark.parametrize("B,Hq,Hkv,L", [(2, 16, 2, 601), (32, 64, 8, 300), (1, 8, 1, 3000)])
def test_decode_output_and_workspace(B, Hq, Hkv, L):
    Dh = G = 128
    kq, km = wl.kv_cache_random(93, 0, B, Hkv, L, Dh, G)
    vq, vm = wl.kv_cache_random(93, 1, B, Hkv, L, Dh, G)
    args = [dev(t) for t in (wl.queries(93, 0, B, Hq, Dh), kq, km, vq, vm)]
    nws = qr.kv_decode_workspace_bytes(B, Hq, Hkv, Dh, L)
    ws = Guarded(max(nws, 4), torch.uint8, (max(nws, 4),))
    out = guarded_like((B, Hq, Dh), torch.float16)
    qr.kv_decode_attention(*args, L, G, 0.088, out=out.view, workspace=ws.view)
    out.check(), ws.check()
    ref = qr.kv_decode_attention(*args, L, G, 0.088)
    assert torch.equal(out.view, ref)
