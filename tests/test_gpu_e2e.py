"""End-to-end parity on the tiny W4A4 linear: rotate + quantize X and W on the
GPU, run the W4A4 GEMM, compare with the oracle's own chain."""
import numpy as np
import pytest

import workloads as wl
from oracle import gemm as og
from oracle import hadamard as oh
from oracle import quant as oq

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
qr = pytest.importorskip("hadamard_rotation_int4_amd")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.mark.parametrize("d,N", [(4096, 4096), (11008, 512), (28672, 256)])
def test_linear_chain(d, N):
    W = wl.WORKLOADS["tiny"]
    T = 32
    x = wl.activations(W.wid, 0, T, d, n_outliers=4, lo=50, hi=50)
    w = wl.weights(W.wid, 1, N, d)
    s = wl.signs(W.wid, d)
    xs, ws, ss = dev(x), dev(w), dev(s)
    qa, sa = qr.hadamard_quant(xs, ss)
    qw, sw = qr.hadamard_quant(ws, ss)          # weight prep: per output channel, T := N
    y = host(qr.w4a4_gemm(qa, sa, qw, sw))
    qa, sa, qw, sw = host(qa), host(sa), host(qw), host(sw)
    # the oracle's own chain, float64 rotation + math-mode quantization
    qa_r, sa_r = oq.sym_quant_math(oh.rotate(x.astype(np.float64), s))
    qw_r, sw_r = oq.sym_quant_math(oh.rotate(w.astype(np.float64), s))
    y_ref = og.epilogue_recipe(og.int4_matmul_exact(qa_r, qw_r), sa_r, sw_r).astype(np.float64)
    fa = (oq.unpack_int4(qa) != qa_r).sum(axis=1) + 8 * (sa != sa_r)
    fw = (oq.unpack_int4(qw) != qw_r).sum(axis=1) + 8 * (sw != sw_r)
    # each flipped code moves acc by at most 8; a 1-ulp scale moves Y by <= 2^-10 relative
    bound = (2.0 ** -9 * np.abs(y_ref)
             + 8.5 * (fa[:, None] + fw[None, :]) * sa_r.astype(np.float64)[:, None] * sw_r.astype(np.float64)[None, :]
             + 1e-7)
    err = np.abs(y.astype(np.float64) - y_ref)
    assert np.all(err <= bound)
    assert (fa == 0).mean() > 0.5
    # and the chain tracks the unquantized product (INT4 noise on both operands)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    rel = np.linalg.norm(y.astype(np.float64) - ref) / np.linalg.norm(ref)
    assert rel < 0.3


def sqnr_db(y, ref):
    return 10 * np.log10(np.sum(ref ** 2) / np.sum((y - ref) ** 2))


def test_rotation_improves_sqnr():
    # the point of the method: with outlier channels, the W4A4 product of the
    # rotated operands tracks X W^T far better than quantizing them as they are
    W = wl.WORKLOADS["tiny"]
    T, N, d = 32, 1024, 4096
    x = wl.activations(W.wid, 0, T, d, n_outliers=4, lo=50, hi=50)
    w = wl.weights(W.wid, 1, N, d)
    s = dev(wl.signs(W.wid, d))
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    ys = {}
    for rot in (True, False):
        qa, sa = qr.hadamard_quant(dev(x), s, rotate=rot)
        qw, sw = qr.hadamard_quant(dev(w), s, rotate=rot)
        ys[rot] = host(qr.w4a4_gemm(qa, sa, qw, sw)).astype(np.float64)
    rotated, plain = sqnr_db(ys[True], ref), sqnr_db(ys[False], ref)
    assert rotated > plain + 6.0, (rotated, plain)
    assert rotated > 10.0, rotated
