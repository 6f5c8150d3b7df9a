"""Seeded synthetic inputs for the five Llama-2-shaped workloads.

This module is shared by the tests, the bench and the oracle checks.  It draws
random numbers and arranges them into the shapes of the workloads; it holds
none of the method's arithmetic (no rotation, no quantization, no GEMM).

Recipe (stated once, used everywhere):
* numpy ``Generator(PCG64(SeedSequence([workload_id, tensor_id])))``, values
  drawn in float64 and rounded to fp16 (round half to even).
* Activations: N(0, 1) with a few planted outlier channels, the same columns
  for every token (transformer outlier channels are systematic across tokens,
  QuaRot blog "The outlier problem, stated precisely"; Fig. 1 of the QuaRot
  paper shows them at the FFN input).  Outlier columns are drawn without
  replacement and scaled by a factor drawn uniformly from [lo, hi].
* Weights: N(0, 0.02^2), i.e. standard deviation 0.02.
* Signs: uniform +-1 (int8).
* KV: N(0, 1) with one seeded x30 outlier dimension per head.
For large tensors the same recipe runs on the GPU through ``torch`` with a
seeded Philox generator (``*_torch`` functions); those streams differ from
numpy's, and the full-size checks copy sampled rows of the device tensor back
to the host instead of regenerating them.

Stream ids: tensor_id 0 = X, 1.. = each weight, 100 + d = signs of width d,
200 = outlier picks, 300.. = KV tensors, 400.. = codes/scales for GEMM-only
checks.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

F16 = np.float16


def rng(workload_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([workload_id, tensor_id])))


# ---------------------------------------------------------------------------
# Workload table (shapes from the five Llama-2 configurations)
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Linear:
    name: str
    n: int          # output channels
    k: int          # reduction width (= rotation width d of its input)
    input: str      # which activation feeds it


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    tokens: tuple[int, ...]
    hidden: int
    linears: tuple[Linear, ...] = field(default_factory=tuple)
    n_outliers: int = 5
    outlier_lo: float = 20.0
    outlier_hi: float = 100.0
    kv: dict | None = None


def _llama_block(hidden: int, qkv_n: int, ffn: int) -> tuple[Linear, ...]:
    return (
        Linear("qkv", qkv_n, hidden, "attn_in"),
        Linear("o", hidden, hidden, "o_in"),
        Linear("gate", ffn, hidden, "ffn_in"),
        Linear("up", ffn, hidden, "ffn_in"),
        Linear("down", hidden, ffn, "down_in"),
    )


WORKLOADS: dict[str, Workload] = {
    # Tiny W4A4 linear: X fp16 [32, 4096], 4 outlier channels x50, W [4096, 4096].
    "tiny": Workload(1, "tiny W4A4 linear", (32,), 4096,
                     (Linear("linear", 4096, 4096, "x"),), n_outliers=4,
                     outlier_lo=50.0, outlier_hi=50.0),
    # Llama-2-7B one-block prefill, T = 2048.
    "7b_prefill": Workload(2, "Llama-2-7B one-block prefill", (2048,), 4096,
                           _llama_block(4096, 12288, 11008)),
    # Llama-2-7B decode shapes, T in {1, 8, 32, 64}.
    "7b_decode": Workload(3, "Llama-2-7B decode", (1, 8, 32, 64), 4096,
                          _llama_block(4096, 12288, 11008)),
    # Llama-2-70B one-block prefill, batch 32 x seq 2048.
    "70b_prefill": Workload(4, "Llama-2-70B one-block prefill", (65536,), 8192,
                            _llama_block(8192, 10240, 28672)),
    # Llama-2-70B KV path: batch 32, context 2048 + 50 decode steps.
    "70b_kv": Workload(5, "Llama-2-70B KV cache", (32 * 2048,), 8192, (),
                       kv=dict(batch=32, prefill=2048, decode=50, kv_heads=8,
                               q_heads=64, head_dim=128, group=128, outlier=30.0)),
}


# ---------------------------------------------------------------------------
# numpy generators
# ---------------------------------------------------------------------------

def outlier_columns(workload_id: int, d: int, count: int, lo: float, hi: float, tag: int = 0):
    g = rng(workload_id, 200 + tag)
    cols = g.choice(d, size=count, replace=False)
    scale = g.uniform(lo, hi, size=count)
    return cols, scale


def activations(workload_id: int, tensor_id: int, t: int, d: int, n_outliers: int = 5,
                lo: float = 20.0, hi: float = 100.0) -> np.ndarray:
    """fp16 [t, d], N(0,1) with planted outlier columns."""
    g = rng(workload_id, tensor_id)
    x = g.standard_normal((t, d))
    if n_outliers:
        cols, scale = outlier_columns(workload_id, d, n_outliers, lo, hi, tag=tensor_id)
        x[:, cols] *= scale[None, :]
    return x.astype(F16)


def weights(workload_id: int, tensor_id: int, n: int, k: int, std: float = 0.02) -> np.ndarray:
    g = rng(workload_id, tensor_id)
    return (g.standard_normal((n, k)) * std).astype(F16)


def signs(workload_id: int, d: int) -> np.ndarray:
    g = rng(workload_id, 100 + d)
    return np.where(g.integers(0, 2, size=d) == 0, 1, -1).astype(np.int8)


def kv_tensor(workload_id: int, tensor_id: int, b: int, s: int, h: int, dh: int,
              outlier: float = 30.0) -> np.ndarray:
    """fp16 [b, s, h, dh], N(0,1) with one seeded outlier dimension per head."""
    g = rng(workload_id, 300 + tensor_id)
    x = g.standard_normal((b, s, h, dh))
    dims = g.integers(0, dh, size=h)
    x[:, :, np.arange(h), dims] *= outlier
    return x.astype(F16)


def grid_activations(workload_id: int, tensor_id: int, t: int, d: int, bits: int = 6,
                     frac_bits: int = 2) -> np.ndarray:
    """fp16 values k / 2^frac_bits with |k| < 2^bits.

    Any +-1 combination of d such values is a multiple of 2^-frac_bits below
    d * 2^(bits - frac_bits) in magnitude, so for d * 2^bits <= 2^24 every
    partial sum of a Hadamard transform is exact in fp32, whatever the
    summation order.
    """
    g = rng(workload_id, 500 + tensor_id)
    k = g.integers(-(1 << bits) + 1, 1 << bits, size=(t, d))
    return (k.astype(np.float64) / (1 << frac_bits)).astype(F16)


def packed_codes(workload_id: int, tensor_id: int, rows: int, k: int) -> np.ndarray:
    """Uniformly random bytes [rows, k/2]: two uniformly random int4 codes each."""
    g = rng(workload_id, 400 + tensor_id)
    return g.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)


def positive_scales(workload_id: int, tensor_id: int, n: int, lo: float = 1e-3,
                    hi: float = 1e-1) -> np.ndarray:
    g = rng(workload_id, 450 + tensor_id)
    return np.exp(g.uniform(np.log(lo), np.log(hi), size=n)).astype(F16)


def kv_cache_random(workload_id: int, tensor_id: int, b: int, h: int, s_max: int, dh: int,
                    group: int, scale_lo: float = 0.01, scale_hi: float = 0.2,
                    min_lo: float = -1.5, min_hi: float = 0.0):
    """A filled 4-bit cache: uniformly random packed codes uint8 [b, h, s_max, dh/2] and
    fp16 (scale, min) pairs [b, h, s_max, dh/group, 2] drawn uniformly in the given ranges."""
    g = rng(workload_id, 600 + tensor_id)
    codes = g.integers(0, 256, size=(b, h, s_max, dh // 2), dtype=np.uint8)
    meta = np.stack([g.uniform(scale_lo, scale_hi, size=(b, h, s_max, dh // group)),
                     g.uniform(min_lo, min_hi, size=(b, h, s_max, dh // group))], axis=-1)
    return codes, meta.astype(F16)


def queries(workload_id: int, tensor_id: int, b: int, h: int, dh: int, std: float = 1.0):
    """fp16 [b, h, dh] ~ N(0, std^2): one decoding query per sequence."""
    g = rng(workload_id, 700 + tensor_id)
    return (g.standard_normal((b, h, dh)) * std).astype(F16)


# ---------------------------------------------------------------------------
# torch generators (large tensors, generated on the device)
# ---------------------------------------------------------------------------

def _torch_gen(torch, device, workload_id: int, tensor_id: int):
    g = torch.Generator(device=device)
    g.manual_seed(int(workload_id) * 1_000_003 + int(tensor_id))
    return g


def activations_torch(torch, device, workload_id: int, tensor_id: int, t: int, d: int,
                      n_outliers: int = 5, lo: float = 20.0, hi: float = 100.0):
    g = _torch_gen(torch, device, workload_id, tensor_id)
    x = torch.randn((t, d), generator=g, device=device, dtype=torch.float32)
    if n_outliers:
        cols, scale = outlier_columns(workload_id, d, n_outliers, lo, hi, tag=tensor_id)
        x[:, torch.as_tensor(cols, device=device)] *= torch.as_tensor(scale, device=device,
                                                                      dtype=torch.float32)
    return x.to(torch.float16)


def weights_torch(torch, device, workload_id: int, tensor_id: int, n: int, k: int,
                  std: float = 0.02):
    g = _torch_gen(torch, device, workload_id, tensor_id)
    return (torch.randn((n, k), generator=g, device=device, dtype=torch.float32) * std).to(
        torch.float16)


def kv_tensor_torch(torch, device, workload_id: int, tensor_id: int, b: int, s: int, h: int,
                    dh: int, outlier: float = 30.0):
    g = _torch_gen(torch, device, workload_id, 300 + tensor_id)
    x = torch.randn((b, s, h, dh), generator=g, device=device, dtype=torch.float32)
    dims = rng(workload_id, 300 + tensor_id).integers(0, dh, size=h)
    x[:, :, torch.arange(h, device=device), torch.as_tensor(dims, device=device)] *= outlier
    return x.to(torch.float16)


def kv_cache_random_torch(torch, device, workload_id: int, tensor_id: int, b: int, h: int,
                          s_max: int, dh: int, group: int, scale_lo: float = 0.01,
                          scale_hi: float = 0.2, min_lo: float = -1.5, min_hi: float = 0.0):
    g = _torch_gen(torch, device, workload_id, 600 + tensor_id)
    codes = torch.randint(0, 256, (b, h, s_max, dh // 2), generator=g, device=device,
                          dtype=torch.uint8)
    u = torch.rand((b, h, s_max, dh // group, 2), generator=g, device=device, dtype=torch.float32)
    lo = torch.tensor([scale_lo, min_lo], device=device)
    hi = torch.tensor([scale_hi, min_hi], device=device)
    return codes, (lo + u * (hi - lo)).to(torch.float16)
