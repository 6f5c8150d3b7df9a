"""GPU parity at the full sizes of the Llama-2 workloads, in the launch
configurations that bench.py times.

Inputs are seeded and synthetic (workloads.py).  Large tensors are drawn on the
device by torch's seeded generator; the checks copy sampled rows (or the whole
output, where it is small) back to the host and hand the oracle the same
*inputs* -- never a value the HIP path produced.

* 7B prefill (T = 2048): rotate + quantize at d = 4096 and d = 11008 = 64 * 172,
  every row (rules R1-R3 of tests/parity.py); the five W4A4 GEMMs on seeded
  codes, bit-exact accumulators and outputs on sampled rows.
* 7B decode (T in {1, 8, 32, 64}): the same rotations, every row, and the five
  GEMMs through the weight-streaming kernel, bit-exact everywhere.
* 70B prefill (T = 65536): rotate + quantize at d = 8192 and d = 28672 =
  1024 * 28 on sampled rows (seeded, plus the first, the last and the rows with
  the largest |x|); the five GEMMs on sampled rows x sampled columns, bit-exact.
* 70B KV cache (batch 32, 2048 prompt tokens + 50 decode steps, 8 KV heads of
  128): Init then 50 Appends into one cache, the whole cache checked (R8), and
  the invariance of the attention scores under the head-wise rotation of
  queries and keys (R7) on the 50 decode queries and 64 prompt positions.
"""
import numpy as np
import pytest

import workloads as wl
from oracle import gemm as og
from oracle import hadamard as oh
from oracle import kv as okv

from parity import check_asym, check_rotation, check_sym_codes

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
qr = pytest.importorskip("hadamard_rotation_int4_amd")

W7 = wl.WORKLOADS["7b_prefill"]
W7D = wl.WORKLOADS["7b_decode"]
W70 = wl.WORKLOADS["70b_prefill"]
W70KV = wl.WORKLOADS["70b_kv"]


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def rotated_checked(x, s, z):
    """The float64 oracle's z = H (s * x), after checking the GPU's z against it (R1)."""
    z64 = oh.rotate_unnormalised(x.astype(np.float64), s)
    check_rotation(z, z64)
    return z64


def codes_gpu(seed, rows, cols_half):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randint(0, 256, (rows, cols_half), generator=g, device="cuda", dtype=torch.uint8)


def scales_gpu(seed, n, lo=1e-3, hi=1e-1):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    u = torch.rand((n,), generator=g, device="cuda", dtype=torch.float64)
    return torch.exp(np.log(lo) + u * (np.log(hi) - np.log(lo))).to(torch.float16)


# ---------------------------------------------------------------------------
# 7B prefill and decode: rotation + quantization, every row
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T", [2048, 1, 8, 32, 64])
@pytest.mark.parametrize("d", [4096, 11008])
def test_7b_rotate_quant_all_rows(T, d):
    wid = W7.wid if T == 2048 else W7D.wid
    x = wl.activations(wid, 10 + d, T, d, W7.n_outliers, W7.outlier_lo, W7.outlier_hi)
    s = wl.signs(wid, d)
    q, sc, z = qr.hadamard_quant(dev(x), dev(s), 1.0, z_dbg=True)
    z64 = rotated_checked(x, s, host(z))
    check_sym_codes(host(q), host(sc), z64 / np.sqrt(d), 1.0)


# ---------------------------------------------------------------------------
# 7B GEMMs on seeded codes: prefill (sampled rows) and decode (all rows)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T", [2048, 1, 8, 32, 64])
@pytest.mark.parametrize("lin", [l.name for l in W7.linears])
def test_7b_gemm_bit_exact(T, lin):
    L = {l.name: l for l in W7.linears}[lin]
    seed = 1000 * T + len(lin)
    a = codes_gpu(seed, T, L.k // 2)
    w = codes_gpu(seed + 1, L.n, L.k // 2)
    asc, wsc = scales_gpu(seed + 2, T), scales_gpu(seed + 3, L.n)
    y, acc = qr.w4a4_gemm(a, asc, w, wsc, acc_dbg=True)
    rows = np.arange(T) if T <= 64 else np.unique(np.concatenate(
        [[0, T - 1], np.random.default_rng(seed).choice(T, 126, replace=False)]))
    ri = torch.as_tensor(rows, device="cuda")
    ah = host(a.index_select(0, ri))
    acc_ref = og.w4a4_acc(ah, host(w))
    assert np.array_equal(host(acc.index_select(0, ri)).astype(np.int64), acc_ref)
    y_ref = og.epilogue_recipe(acc_ref, host(asc)[rows], host(wsc))
    assert np.array_equal(host(y.index_select(0, ri)).view(np.uint16), y_ref.view(np.uint16))


# ---------------------------------------------------------------------------
# 70B prefill, T = 65536: the bench's launches, sampled rows / columns
# ---------------------------------------------------------------------------

def sample_rows(T, x, seed):
    rng = np.random.default_rng(seed)
    big = torch.topk(x.abs().amax(dim=1).float(), 8).indices.cpu().numpy()
    return np.unique(np.concatenate([[0, T - 1], big, rng.choice(T, 512, replace=False)]))


@pytest.mark.parametrize("d", [8192, 28672])
def test_70b_rotate_quant_sampled_rows(d):
    T = W70.tokens[0]
    x = wl.activations_torch(torch, torch.device("cuda"), W70.wid, 10 + d, T, d, W70.n_outliers,
                             W70.outlier_lo, W70.outlier_hi)
    s = wl.signs(W70.wid, d)
    q, sc = qr.hadamard_quant(x, dev(s), 1.0)
    rows = sample_rows(T, x, d)
    ri = torch.as_tensor(rows, device="cuda")
    xs = host(x.index_select(0, ri))
    z64 = oh.rotate_unnormalised(xs.astype(np.float64), s)
    stats = check_sym_codes(host(q.index_select(0, ri)), host(sc)[rows], z64 / np.sqrt(d), 1.0)
    assert stats["code_flips"] <= 1e-4 * xs.size


@pytest.mark.parametrize("lin", [l.name for l in W70.linears])
def test_70b_gemm_sampled_bit_exact(lin):
    L = {l.name: l for l in W70.linears}[lin]
    T = W70.tokens[0]
    seed = 7000 + len(lin)
    a = codes_gpu(seed, T, L.k // 2)
    w = codes_gpu(seed + 1, L.n, L.k // 2)
    asc, wsc = scales_gpu(seed + 2, T), scales_gpu(seed + 3, L.n)
    y = qr.w4a4_gemm(a, asc, w, wsc)
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 62, replace=False)]))
    cols = np.unique(np.concatenate([[0, L.n - 1], rng.choice(L.n, 510, replace=False)]))
    ri, ci = torch.as_tensor(rows, device="cuda"), torch.as_tensor(cols, device="cuda")
    acc_ref = og.w4a4_acc(host(a.index_select(0, ri)), host(w.index_select(0, ci)))
    y_ref = og.epilogue_recipe(acc_ref, host(asc)[rows], host(wsc)[cols])
    got = host(y.index_select(0, ri).index_select(1, ci))
    assert np.array_equal(got.view(np.uint16), y_ref.view(np.uint16))


# ---------------------------------------------------------------------------
# 70B KV cache: Init + 50 Appends, whole cache; score invariance
# ---------------------------------------------------------------------------

def test_70b_kv_cache_init_append():
    kv = W70KV.kv
    B, P, Dn, H, Dh, G = kv["batch"], kv["prefill"], kv["decode"], kv["kv_heads"], kv["head_dim"], kv["group"]
    S = P + Dn
    cuda = torch.device("cuda")
    s = wl.signs(W70KV.wid, Dh)
    sd = dev(s)
    for tid, rot in ((0, True), (1, False)):           # K rotated, V not
        x = wl.kv_tensor_torch(torch, cuda, W70KV.wid, tid, B, S, H, Dh, kv["outlier"])
        cq = torch.zeros((B, H, S, Dh // 2), dtype=torch.uint8, device=cuda)
        cm = torch.zeros((B, H, S, Dh // G, 2), dtype=torch.float16, device=cuda)
        qr.kv_rotate_quant(x[:, :P].contiguous(), sd, G, 0.95, cq, cm, 0, rotate=rot)     # Init
        for i in range(Dn):                                                                   # Append
            qr.kv_rotate_quant(x[:, P + i:P + i + 1], sd, G, 0.95, cq, cm, P + i, rotate=rot)
        x64 = host(x).astype(np.float64)
        y64 = oh.rotate(x64, s) if rot else x64
        codes = okv.unpack_uint4(np.transpose(host(cq), (0, 2, 1, 3)))      # [B, S, H, Dh]
        meta = np.transpose(host(cm), (0, 2, 1, 3, 4))                      # [B, S, H, G, 2]
        check_asym(codes, meta[..., 0], meta[..., 1], y64, G, 0.95)


def test_70b_scores_invariant_under_rotation():
    kv = W70KV.kv
    B, P, Dn, H, Hq, Dh = kv["batch"], kv["prefill"], kv["decode"], kv["kv_heads"], kv["q_heads"], kv["head_dim"]
    S = P + Dn
    cuda = torch.device("cuda")
    s = wl.signs(W70KV.wid, Dh)
    k = wl.kv_tensor_torch(torch, cuda, W70KV.wid, 0, B, S, H, Dh, kv["outlier"])
    q = wl.kv_tensor_torch(torch, cuda, W70KV.wid, 2, B, S, Hq, Dh, 1.0)
    rng = np.random.default_rng(5)
    qpos = np.concatenate([np.sort(rng.choice(P, 64, replace=False)), np.arange(P, S)])
    for b in np.sort(rng.choice(B, 2, replace=False)):
        kb = k[b].reshape(-1, Dh)
        qb = q[b].index_select(0, torch.as_tensor(qpos, device=cuda)).reshape(-1, Dh)
        krot = host(qr.hadamard(kb, dev(s), torch.float32)).reshape(1, S, H, Dh).astype(np.float64)
        qrot = host(qr.hadamard(qb, dev(s), torch.float32)).reshape(1, len(qpos), Hq, Dh).astype(np.float64)
        k64 = host(kb).reshape(1, S, H, Dh).astype(np.float64)
        q64 = host(qb).reshape(1, len(qpos), Hq, Dh).astype(np.float64)
        ref = okv.gqa_scores(q64, k64)
        got = okv.gqa_scores(qrot, krot)
        rel = np.abs(got - ref).max(axis=-1) / np.abs(ref).max(axis=-1)
        assert rel.max() <= 1e-3
