"""GPU parity: qr_w4a4_gemm against the oracle's exact integer GEMM and fp32 epilogue."""
import numpy as np
import pytest

import workloads as wl
from oracle import gemm as og
from oracle import quant as oq

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
qr = pytest.importorskip("hadamard_rotation_int4_amd")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def run(ap, asc, wp, wsc):
    y, acc = qr.w4a4_gemm(dev(ap), dev(asc), dev(wp), dev(wsc), acc_dbg=True)
    return host(y), host(acc)


SHAPES = [(1, 1, 64), (7, 100, 128), (300, 260, 192), (33, 17, 4096), (256, 256, 256),
          (513, 300, 1024), (64, 640, 11008), (257, 513, 320), (2, 4096, 128)]

# Shapes that steer the entry point to each of its kernels.  T >= 65 runs the
# tiled kernel, with 256 x 256 tiles (one workgroup per compute unit) or
# 128 x 128 tiles (two per compute unit), whichever the launcher estimates
# faster: 256 x 256 wins only when its grid fills the 256 compute units in
# clearly fewer rounds.  The small shapes of SHAPES all take 128 x 128;
#   (4096, 4096, 512)  -> 256 x 256 tiles (256 tiles fill the machine once);
#   (2048, 4096, 512)  -> 128 x 128 tiles;
#   (1 | 8 | 32 | 64, ...) -> weight-streaming kernel with 1, 1, 2, 4 row blocks,
#   at the Llama-2-7B decode widths, including K = 11008 (K % 128 == 0) and
#   K = 4160 (a final half block of 64).
# The 256 x 256 tiles with ragged edges and a K tail are covered by
# test_256_tiles_ragged_edges_and_k_tail below.
KERNEL_SHAPES = [(4096, 4096, 512), (2048, 4096, 512), (640, 384, 256), (1, 12288, 4096),
                 (8, 4096, 4096), (32, 11008, 4096), (64, 4096, 11008), (17, 100, 4160),
                 (64, 33, 64)]


def picks_256_tiles(T, N):
    """The launcher's tile choice for T >= 65 (rounds of 256 tiles of 256 x 256
    at throughput 1, against rounds of 512 tiles of 128 x 128 at 0.46 each)."""
    r44 = -(-(-(-T // 256) * -(-N // 256)) // 256)
    r22 = -(-(-(-T // 128) * -(-N // 128)) // 512)
    return r22 * 128 * 128 / 0.46 > r44 * 256 * 256


# 256 x 256 tiles whose last tile row and column are partial, with K tails of
# 64 and 192 past the 256-element K step (and one without a tail); N = 3999 is
# odd, so output rows are not 4-byte aligned and every store is per element.
# K = 64, 192 and 256 are single K steps (the copies of the first step are the
# only ones; 64 and 192 also clear the chunks past K in it).
RAGGED_256 = [(4000, 4000, 320), (3000, 4100, 4160), (3900, 3850, 448), (4000, 4000, 512),
              (4000, 3999, 320), (4000, 4000, 64), (3900, 4000, 192), (4000, 4000, 256)]


def _edge_sample(n, seed):
    rest = np.random.default_rng(seed).choice(n, 40, replace=False)
    return np.unique(np.r_[0, 1, 255, 256, n - 257, n - 256, n - 2, n - 1, rest])


@pytest.mark.parametrize("T,N,K", RAGGED_256)
@pytest.mark.parametrize("bits", [4, 8])
def test_256_tiles_ragged_edges_and_k_tail(T, N, K, bits):
    assert picks_256_tiles(T, N)
    if bits == 4:
        a = wl.packed_codes(3, 0, T, K)
        w = wl.packed_codes(3, 1, N, K)
    else:
        a = wl.packed_codes(3, 2, T, 2 * K).view(np.int8)
        w = wl.packed_codes(3, 3, N, 2 * K).view(np.int8)
    asc = wl.positive_scales(3, 0, T)
    wsc = wl.positive_scales(3, 1, N)
    gemm = qr.w4a4_gemm if bits == 4 else qr.w8a8_gemm
    y_plain = host(gemm(dev(a), dev(asc), dev(w), dev(wsc)))      # the kernel without acc_dbg
    y, acc = (host(t) for t in gemm(dev(a), dev(asc), dev(w), dev(wsc), acc_dbg=True))
    rows, cols = _edge_sample(T, T + K), _edge_sample(N, N + K)
    if bits == 4:
        acc_ref = og.w4a4_acc(a[rows], w[cols])
    else:
        acc_ref = og.int_matmul_exact(a[rows], w[cols])
    assert np.array_equal(acc[np.ix_(rows, cols)].astype(np.int64), acc_ref)
    y_ref = og.epilogue_recipe(acc_ref, asc[rows], wsc[cols])
    assert np.array_equal(y[np.ix_(rows, cols)].view(np.uint16), y_ref.view(np.uint16))
    assert np.array_equal(y_plain.view(np.uint16), y.view(np.uint16))


@pytest.mark.parametrize("T,N,K", SHAPES + KERNEL_SHAPES)
def test_random_codes_bit_exact(T, N, K):
    ap = wl.packed_codes(1, 0, T, K)
    wp = wl.packed_codes(1, 1, N, K)
    asc = wl.positive_scales(1, 0, T)
    wsc = wl.positive_scales(1, 1, N)
    y, acc = run(ap, asc, wp, wsc)
    acc_ref = og.w4a4_acc(ap, wp)
    assert np.array_equal(acc.astype(np.int64), acc_ref)
    y_ref = og.epilogue_recipe(acc_ref, asc, wsc)
    assert np.array_equal(y.view(np.uint16), y_ref.view(np.uint16))


def test_extreme_magnitude():
    T, N, K = 40, 70, 28672
    ap = np.full((T, K // 2), 0x88, dtype=np.uint8)   # every code -8
    wp = np.full((N, K // 2), 0x88, dtype=np.uint8)
    wp[1::2] = 0x77                                   # every code +7
    asc = np.full(T, 2.0 ** -10, dtype=np.float16)
    wsc = np.full(N, 2.0 ** -10, dtype=np.float16)
    y, acc = run(ap, asc, wp, wsc)
    assert acc[0, 0] == 64 * K and acc[0, 1] == -56 * K
    assert np.array_equal(y.view(np.uint16), og.epilogue_recipe(og.w4a4_acc(ap, wp), asc, wsc).view(np.uint16))


@pytest.mark.parametrize("T,N", [(40, 70), (300, 260), (4000, 4000)])
@pytest.mark.parametrize("bits", [4, 8])
def test_largest_k(T, N, bits):
    """K = 131008, the largest the entry points take (|256 acc| < 2^31 for INT4,
    |acc| < 2^31 for codes down to -128), on each kernel (weight streaming for
    INT4, 128 x 128 and 256 x 256 tiles): row 0 of A at the most negative code
    against W rows at the most negative and the most positive code gives the
    largest magnitudes; the other rows are random.  Sampled rows and columns
    against the exact integer product and the epilogue recipe."""
    K = 131008
    print(f"gemm largest K: bits={bits} T={T} N={N} K={K}", flush=True)
    if bits == 4:
        ap = wl.packed_codes(4, 0, T, K)
        wp = wl.packed_codes(4, 1, N, K)
        lo, hi, fill_lo, fill_hi = -8, 7, 0x88, 0x77
    else:
        ap = wl.packed_codes(4, 2, T, 2 * K).view(np.int8)
        wp = wl.packed_codes(4, 3, N, 2 * K).view(np.int8)
        lo, hi, fill_lo, fill_hi = -128, 127, -128, 127
    ap[0] = fill_lo
    wp[0] = fill_lo
    wp[1] = fill_hi
    asc = wl.positive_scales(4, 0, T, 1e-6, 1e-4)
    wsc = wl.positive_scales(4, 1, N, 1e-6, 1e-4)
    gemm = qr.w4a4_gemm if bits == 4 else qr.w8a8_gemm
    y, acc = (host(t) for t in gemm(dev(ap), dev(asc), dev(wp), dev(wsc), acc_dbg=True))
    assert acc[0, 0] == lo * lo * K and acc[0, 1] == lo * hi * K
    rows = np.unique(np.r_[0, 1, T - 1, np.random.default_rng(T).choice(T, min(T, 24), replace=False)])
    cols = np.unique(np.r_[0, 1, N - 1, np.random.default_rng(N).choice(N, min(N, 24), replace=False)])
    if bits == 4:
        acc_ref = og.w4a4_acc(ap[rows], wp[cols])
    else:
        acc_ref = og.int_matmul_exact(ap[rows], wp[cols])
    assert np.array_equal(acc[np.ix_(rows, cols)].astype(np.int64), acc_ref)
    y_ref = og.epilogue_recipe(acc_ref, asc[rows], wsc[cols])
    assert np.array_equal(y[np.ix_(rows, cols)].view(np.uint16), y_ref.view(np.uint16))


def test_epilogue_overflow_and_zero_scales():
    T, N, K = 9, 33, 256
    ap = wl.packed_codes(2, 0, T, K)
    wp = wl.packed_codes(2, 1, N, K)
    asc = wl.positive_scales(2, 0, T, 1.0, 1000.0)
    asc[3] = 0.0
    wsc = wl.positive_scales(2, 1, N, 1.0, 1000.0)
    y, acc = run(ap, asc, wp, wsc)
    y_ref = og.epilogue_recipe(og.w4a4_acc(ap, wp), asc, wsc)
    assert np.isinf(y_ref).any()
    assert np.array_equal(y.view(np.uint16), y_ref.view(np.uint16))


def test_output_without_debug_matches():
    T, N, K = 100, 300, 4096
    ap = wl.packed_codes(3, 0, T, K)
    wp = wl.packed_codes(3, 1, N, K)
    asc = wl.positive_scales(3, 0, T)
    wsc = wl.positive_scales(3, 1, N)
    y = host(qr.w4a4_gemm(dev(ap), dev(asc), dev(wp), dev(wsc)))
    y_ref = og.epilogue_recipe(og.w4a4_acc(ap, wp), asc, wsc)
    assert np.array_equal(y.view(np.uint16), y_ref.view(np.uint16))


@pytest.mark.parametrize("T,N,K", [(300, 260, 448), (4000, 4000, 320)])
def test_output_only_dword_aligned(T, N, K):
    # y_f16 needs only 4-byte alignment: an output 4 bytes into a buffer (the
    # epilogue writes 16-byte row pieces at that alignment), for the 128 x 128 and
    # the 256 x 256 tiles; bit-exact against the oracle's epilogue on sampled rows
    # and columns, and the bytes around the view untouched.
    ap = wl.packed_codes(3, 4, T, K)
    wp = wl.packed_codes(3, 5, N, K)
    asc = wl.positive_scales(3, 4, T)
    wsc = wl.positive_scales(3, 5, N)
    buf = torch.full((T * N + 8,), -2.0, dtype=torch.float16, device="cuda")
    y = buf[2:2 + T * N].view(T, N)
    assert y.data_ptr() % 16 == 4
    qr.w4a4_gemm(dev(ap), dev(asc), dev(wp), dev(wsc), out=y)
    rows, cols = _edge_sample(T, 7), _edge_sample(N, 8)
    y_ref = og.epilogue_recipe(og.w4a4_acc(ap[rows], wp[cols]), asc[rows], wsc[cols])
    assert np.array_equal(host(y)[np.ix_(rows, cols)].view(np.uint16), y_ref.view(np.uint16))
    hb = host(buf)
    assert np.all(hb[:2] == -2.0) and np.all(hb[2 + T * N:] == -2.0)


def test_empty():
    z = dev(np.zeros((0, 32), dtype=np.uint8))
    w = dev(np.zeros((5, 32), dtype=np.uint8))
    y = qr.w4a4_gemm(z, dev(np.zeros(0, np.float16)), w, dev(np.ones(5, np.float16)))
    assert tuple(y.shape) == (0, 5)
