"""The calibration kernels behind the practical ceilings the rooflines quote:
qr_calibrate_mfma_i8 (the GEMM's int8 MFMA in a register-only loop): every
wavefront's checksums add up to the exact integer sum include/qr.h states, and
the clock counters advance; qr_calibrate_stream (the rotate+quant traffic mix):
every output dword is the XOR fold of its 16-byte input chunk."""
import numpy as np
import pytest
import torch

import hadamard_rotation_int4_amd as qr

pytestmark = pytest.mark.gpu


def gemm_like_fragments(seed):
    """16 q with q uniform in -8..7: the int8 values the W4A4 GEMM feeds its
    matrix cores after unpacking INT4 codes."""
    rng = np.random.default_rng(seed)
    return (16 * rng.integers(-8, 8, size=(64, 16))).astype(np.int8)


def wave_sum(frag, iters):
    """iters * sum_j sum_{h, e} (sum_{l in half h} A_l[e]) (sum_{l in half h} B_{j,l}[e])
    modulo 2^32, B_{j,l} = row (l + 7 + 16 j) mod 64, as a brute-force sum over
    the 32 x 32 x 32 products of each chain."""
    f = frag.astype(np.int64)
    total = 0
    for j in range(4):
        b = f[(np.arange(64) + 7 + 16 * j) % 64]
        A = np.concatenate([f[:32], f[32:]], axis=1)      # [m, k]: lanes m and m + 32
        B = np.concatenate([b[:32], b[32:]], axis=1)      # [n, k]
        total += int((A @ B.T).sum())
    return (iters * total) % 2**32


@pytest.mark.parametrize("grid,iters,seed", [(8, 1000, 0), (300, 37, 1), (1, 1, 2)])
def test_checksums_exact(grid, iters, seed):
    print(f"calibrate grid={grid} iters={iters} seed={seed}", flush=True)
    frag = gemm_like_fragments(seed)
    chk, clk = qr.calibrate_mfma_i8(torch.from_numpy(frag).cuda(), grid, iters, clocks=True)
    torch.cuda.synchronize()
    per_wave = chk.cpu().numpy().astype(np.int64).reshape(grid * 4, 64).sum(1) % 2**32
    assert (per_wave == wave_sum(frag, iters)).all()
    c = clk.view(torch.int64).cpu().numpy()
    assert (c[:, 1] > c[:, 0]).all() and (c[:, 3] >= c[:, 2]).all()


def test_without_clocks():
    frag = gemm_like_fragments(3)
    chk = qr.calibrate_mfma_i8(torch.from_numpy(frag).cuda(), 4, 10)
    torch.cuda.synchronize()
    per_wave = chk.cpu().numpy().astype(np.int64).reshape(16, 64).sum(1) % 2**32
    assert (per_wave == wave_sum(frag, 10)).all()


@pytest.mark.parametrize("n16,grid", [(1, 1), (511, 1), (513, 1), (100003, 7), (1 << 20, 2048)])
def test_stream_xor_fold(n16, grid):
    print(f"calibrate stream n16={n16} grid={grid}", flush=True)
    src = np.random.default_rng(n16).integers(0, 2**32, size=(n16, 4), dtype=np.uint32)
    out = qr.calibrate_stream(torch.from_numpy(src).cuda(), grid)
    torch.cuda.synchronize()
    ref = src[:, 0] ^ src[:, 1] ^ src[:, 2] ^ src[:, 3]
    assert np.array_equal(out.cpu().numpy(), ref)
