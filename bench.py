"""Benchmark of the QuaRot online-rotation + INT4 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload 70b_prefill|7b_prefill|7b_decode|70b_kv|70b_block|7b_block|
                                70b_block_w8a8|7b_block_w8a8]
                    [--no-cpu-baseline] [--copy-calibration] [--mfma-calibration]
                    [--stream-calibration] [--fp16-hadamard]

One step is one pass of the whole hot path over one batch of synthetic input
(inputs resident in HBM; weights prepared offline and not timed):

* prefill (default: Llama-2-70B block, T = 65536 = batch 32 x seq 2048):
  fused Hadamard rotation + per-token INT4 quantization of the four GEMM inputs
  (attention input, attention output, FFN input -- shared by gate and up -- and
  the down-projection input, d = K of its GEMM); the five W4A4 GEMMs (QKV, O,
  gate, up, down) with the scale epilogue; head-wise Hadamard + asymmetric
  4-bit group-128 quantization of K and V into the cache (Init of the prompt);
  the head-wise rotation of Q.  With --fp16-hadamard the down-projection
  rotation (d = 28672, or 11008 for 7b_prefill) runs the fp16 variant of the
  transform (QR_ROT_HADAMARD_F16) instead of the default fp32 one.
* 70b_block / 7b_block: the same block with the model's own online path
  (QuaRot paper, Figures 3 and 6): RMSNorm without scale + INT4 in front of
  QKV and of gate/up, the Hadamard-heads transform + INT4 in front of O, the
  full online Hadamard + INT4 only in front of down.  The same five GEMMs in
  fp16 (torch.matmul) are timed separately as context: the pages' speedups
  are against an FP16 block.  The _w8a8 forms run the same online path with
  8-bit codes one per byte and the W8A8 GEMM (the pages' 8-bit RTN setting).
* 7b_decode: the same four rotations and five GEMMs at T = 1, 8, 32 and 64.
* 70b_kv: K/V Init of a 32 x 2048-token prompt (8 KV heads of 128), the
  rotation of its queries (64 heads), then 50 decode steps of Append K, V,
  rotate one query token and the Decode attention of that query over the
  4-bit cache (2049 .. 2098 positions).

Prints one JSON line.  ``value`` is the step's GEMM int-ops per second (TOPS)
for the prefill workloads and its algorithmic HBM bytes per second (GB/s) for
the memory-bound ones.  ``roofline`` covers the step's dominant kernel;
``roofline_hadamard_quant`` covers the fused rotation + quantization against
the HBM roofline.  Each launch is bracketed by HIP events on the stream it runs
on.  ``traffic`` is read from the committed rocprofv3 counter summary of that
kernel and workload (profiles/traffic_*.txt) when the kernel source still
matches the hash recorded there, else null.  ``cpu_baseline`` is the oracle
timed on the host on a bounded sample.

--copy-calibration runs only a plain device copy of 1 GiB (ten times), the
reference kernel that scales the FETCH_SIZE / WRITE_SIZE counters, and
prints its rate: the practical HBM ceiling of a read + write stream.

--mfma-calibration runs only the library's register-only loop of the GEMM's
int8 MFMA (qr_calibrate_mfma_i8: no memory traffic, 8 wavefronts per SIMD)
and prints the int-op rate it sustains, the shader clock it ran at and the
fraction of the int8 peak at that clock: the practical ceiling of the matrix
cores under the chip's power limit.

--stream-calibration runs only the library's plain stream with the rotate+quant
traffic mix (qr_calibrate_stream: 1 GiB read, 256 MiB written, non-temporal)
and prints its rate: the practical HBM ceiling of that mix.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA (5.0 POP/s)
METRIC = "fused Hadamard+INT4-quant HBM GB/s; W4A4 GEMM TOPS at Llama-2 shapes"
CSRC = ROOT / "hadamard_rotation_int4_amd" / "csrc"
# Workloads whose working set fits in the 256 MB Infinity Cache (MALL).
SMALL_WORKING_SET = ("7b_prefill", "7b_decode", "70b_kv", "7b_block", "7b_block_w8a8")
COLD_REPS = 5
KERNEL_SOURCE = {"w4a4_gemm": "w4a4_gemm.hip", "hadamard_quant": "hadamard_quant.hip",
                 "kv_rotate_quant": "kv_quant.hip", "hadamard": "hadamard_quant.hip",
                 "kv_decode_attention": "kv_decode.hip", "rmsnorm_quant": "block_quant.hip",
                 "hadamard_heads_quant": "block_quant.hip", "w8a8_gemm": "w4a4_gemm.hip",
                 "hadamard_quant_i8": "hadamard_quant.hip", "rmsnorm_quant_i8": "block_quant.hip",
                 "hadamard_heads_quant_i8": "block_quant.hip",
                 "hadamard_quant_groups": "hadamard_quant.hip", "w4a4_gemm_groups": "w4a4_gemm.hip"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="70b_prefill",
                    choices=["70b_prefill", "7b_prefill", "7b_decode", "70b_kv", "70b_block",
                             "7b_block", "70b_block_w8a8", "7b_block_w8a8"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=2048)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--mfma-calibration", action="store_true")
    ap.add_argument("--stream-calibration", action="store_true")
    ap.add_argument("--group", type=int, default=0,
                    help="prefill workloads: group-wise scales of this group size on both GEMM "
                         "operands (group-wise quantizer and grouped GEMM)")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the fp16 / hipBLASLt int8 context timings of the block workloads")
    ap.add_argument("--fp16-hadamard", action="store_true",
                    help="down-projection rotation with the fp16 transform")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the compact results of the other four configurations that the "
                         "default (70B prefill) run adds")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# Algorithmic work per launch (each input read once, each output written once)
# ---------------------------------------------------------------------------

def hq_bytes(T, d):
    """Fused rotate + quant: read fp16 x, write packed codes and the fp16 scale
    (signs and H_m tables are cache resident)."""
    return T * (2 * d + d // 2 + 2)


def gemm_ops(T, N, K):
    return 2 * T * N * K


def gemm_bytes(T, N, K):
    """A codes + W codes + both scale vectors + the fp16 output."""
    return T * K // 2 + N * K // 2 + 2 * T + 2 * N + 2 * T * N


def kv_bytes(rows, dh, group):
    """Per (token, head) row: fp16 in, packed codes + fp16 (scale, min) per group out."""
    return rows * (2 * dh + dh // 2 + 4 * (dh // group))


def rot_bytes(rows, dh):
    """Rotation only, fp16 in and out."""
    return rows * 4 * dh


def decode_bytes(b, hkv, hq, L, dh, group):
    """Decode routine: the K and V caches of L positions (packed codes + fp16 (scale, min)
    per group) read once, the fp16 queries in and the fp16 outputs out."""
    return 2 * b * hkv * L * (dh // 2 + 4 * (dh // group)) + 2 * 2 * b * hq * dh


# ---------------------------------------------------------------------------
# Workload construction: a list of launches (kernel, label, bytes, ops, fn)
# ---------------------------------------------------------------------------

def i8_bytes(T, d):
    """b-bit quantizer: read fp16 x, write one byte per code and the fp16 scale."""
    return T * (2 * d + d + 2)


def gemm8_bytes(T, N, K):
    return T * K + N * K + 2 * T + 2 * N + 2 * T * N


def make_block(torch, qr, wl, W, T, dev, with_kv, f16_down=False, quarot=False, bits=4,
               group=0):
    lin = {l.name: l for l in W.linears}
    H, ffn, wid = W.hidden, lin["down"].k, W.wid
    inputs = {}
    for i, name in enumerate(("attn_in", "o_in", "ffn_in", "down_in")):
        d = ffn if name == "down_in" else H
        inputs[name] = wl.activations_torch(torch, dev, wid, 10 + i, T, d, W.n_outliers,
                                            W.outlier_lo, W.outlier_hi)
    signs = {d: torch.from_numpy(wl.signs(wid, d)).to(dev) for d in (H, ffn)}
    # weights: random init, rotated by the same R_K and quantized per output
    # channel with the library's own kernel (offline preparation, not timed)
    i8 = bits != 4
    wq = {}
    for i, (name, l) in enumerate(lin.items()):
        w = wl.weights_torch(torch, dev, wid, 1 + i, l.n, l.k)
        wq[name] = (qr.hadamard_quant_i8(w, signs[l.k], 1.0, bits) if i8
                    else qr.hadamard_quant_groups(w, signs[l.k], 1.0, group) if group
                    else qr.hadamard_quant(w, signs[l.k], 1.0))
        del w
    qbuf = {n: (torch.empty((T, x.shape[1]) if i8 else (T, x.shape[1] // 2),
                            dtype=torch.int8 if i8 else torch.uint8, device=dev),
                torch.empty((T, x.shape[1] // group) if group else (T,), dtype=torch.float16,
                            device=dev)) for n, x in inputs.items()}
    ybuf = {n: torch.empty((T, l.n), dtype=torch.float16, device=dev) for n, l in lin.items()}
    L = []
    tag = f"T{T}:" if not with_kv else ""
    for name, x in inputs.items():
        if group:
            L.append(("hadamard_quant_groups", tag + name, T * (2 * x.shape[1] + x.shape[1] // 2
                                                              + 2 * (x.shape[1] // group)), 0,
                      (lambda x=x, name=name: qr.hadamard_quant_groups(
                          x, signs[x.shape[1]], 1.0, group, out=qbuf[name])), qbuf[name]))
            continue
        if i8:
            # b-bit codes one per byte: the model's online path with the _i8 quantizers
            if name in ("attn_in", "ffn_in"):
                fn = (lambda x=x, name=name: qr.rmsnorm_quant_i8(x, 1e-5, 1.0, bits, out=qbuf[name]))
                kname = "rmsnorm_quant_i8"
            elif name == "o_in":
                fn = (lambda x=x, name=name: qr.hadamard_heads_quant_i8(x, H // 128, 1.0, bits,
                                                                        out=qbuf[name]))
                kname = "hadamard_heads_quant_i8"
            else:
                fn = (lambda x=x, name=name: qr.hadamard_quant_i8(x, signs[x.shape[1]], 1.0, bits,
                                                                  out=qbuf[name]))
                kname = "hadamard_quant_i8"
            L.append((kname, tag + name, i8_bytes(T, x.shape[1]), 0, fn, qbuf[name]))
            continue
        if quarot and name in ("attn_in", "ffn_in"):
            # the residual rotation is fused into the weights; RMSNorm (no scale) + INT4 online
            L.append(("rmsnorm_quant", tag + name, hq_bytes(T, x.shape[1]), 0,
                      (lambda x=x, name=name: qr.rmsnorm_quant(x, 1e-5, 1.0, out=qbuf[name])),
                      qbuf[name]))
            continue
        if quarot and name == "o_in":
            # (I (x) H_dh) is fused into W_v / W_out; Hadamard heads + INT4 online
            L.append(("hadamard_heads_quant", tag + name, hq_bytes(T, x.shape[1]), 0,
                      (lambda x=x, name=name: qr.hadamard_heads_quant(x, H // 128, 1.0,
                                                                      out=qbuf[name])),
                      qbuf[name]))
            continue
        f16 = f16_down and name == "down_in" and x.shape[1] in (28672, 11008)
        L.append(("hadamard_quant", tag + name + (":fp16" if f16 else ""), hq_bytes(T, x.shape[1]), 0,
                  (lambda x=x, name=name, f16=f16: qr.hadamard_quant(
                      x, signs[x.shape[1]], 1.0, out=qbuf[name], fp16_transform=f16)), qbuf[name]))
    for name, l in lin.items():
        if group:
            L.append(("w4a4_gemm_groups", tag + name,
                      gemm_bytes(T, l.n, l.k) + 2 * (T + l.n) * (l.k // group - 1),
                      gemm_ops(T, l.n, l.k),
                      (lambda name=name, l=l: qr.w4a4_gemm_groups(*qbuf[l.input], *wq[name], group,
                                                                   out=ybuf[name])), (ybuf[name],)))
            continue
        if i8:
            L.append(("w8a8_gemm", tag + name, gemm8_bytes(T, l.n, l.k), gemm_ops(T, l.n, l.k),
                      (lambda name=name, l=l: qr.w8a8_gemm(*qbuf[l.input], *wq[name],
                                                            out=ybuf[name])), (ybuf[name],)))
            continue
        L.append(("w4a4_gemm", tag + name, gemm_bytes(T, l.n, l.k), gemm_ops(T, l.n, l.k),
                  (lambda name=name, l=l: qr.w4a4_gemm(*qbuf[l.input], *wq[name],
                                                        out=ybuf[name])), (ybuf[name],)))
    desc = None
    if with_kv:
        # KV: 70B-shaped heads (8 KV heads, 64 query heads, head_dim 128) over the same tokens
        Hkv, Hq, Dh, G = 8, H // 128, 128, 128
        B = 32 if T % 32 == 0 else 1
        S = T // B
        k_in = wl.kv_tensor_torch(torch, dev, 5, 0, B, S, Hkv, Dh)
        v_in = wl.kv_tensor_torch(torch, dev, 5, 1, B, S, Hkv, Dh)
        q_in = wl.activations_torch(torch, dev, 5, 2, T * Hq, Dh, 0)
        kv_signs = torch.from_numpy(wl.signs(5, Dh)).to(dev)
        cache = {n: (torch.empty((B, Hkv, S, Dh // 2), dtype=torch.uint8, device=dev),
                     torch.empty((B, Hkv, S, Dh // G, 2), dtype=torch.float16, device=dev))
                 for n in ("k", "v")}
        qout = torch.empty((T * Hq, Dh), dtype=torch.float16, device=dev)
        L.append(("kv_rotate_quant", "k", kv_bytes(T * Hkv, Dh, G), 0,
                  lambda: qr.kv_rotate_quant(k_in, kv_signs, G, 0.95, *cache["k"], 0), cache["k"]))
        L.append(("kv_rotate_quant", "v", kv_bytes(T * Hkv, Dh, G), 0,
                  lambda: qr.kv_rotate_quant(v_in, None, G, 0.95, *cache["v"], 0, rotate=False),
                  cache["v"]))
        L.append(("hadamard", "q", rot_bytes(T * Hq, Dh), 0,
                  lambda: qr.hadamard(q_in, kv_signs, torch.float16, out=qout), (qout,)))
        desc = (f"K/V init into a 4-bit cache ({B}x{S}x{Hkv}x{Dh}, group {G}), "
                f"Q rotation ({Hq} heads)")
    return L, lin, desc


def fp16_linears(torch, wl, W, T, dev):
    """The block's five linear layers in fp16 (torch.matmul): the FP16 baseline
    the pages' block speedups are measured against (context, not the path)."""
    lin = {l.name: l for l in W.linears}
    xs = {}
    for i, name in enumerate(("attn_in", "o_in", "ffn_in", "down_in")):
        d = lin["down"].k if name == "down_in" else W.hidden
        xs[name] = wl.activations_torch(torch, dev, W.wid, 10 + i, T, d, W.n_outliers,
                                        W.outlier_lo, W.outlier_hi)
    L = []
    for i, (name, l) in enumerate(lin.items()):
        w = wl.weights_torch(torch, dev, W.wid, 1 + i, l.n, l.k)
        y = torch.empty((T, l.n), dtype=torch.float16, device=dev)
        L.append(("fp16_gemm", name, gemm_bytes(T, l.n, l.k), gemm_ops(T, l.n, l.k),
                  (lambda x=xs[l.input], w=w, y=y: torch.matmul(x, w.t(), out=y)), (y,)))
    return L


def make_kv_decode(torch, qr, wl, W, dev):
    kv = W.kv
    B, P, Dn, H, Hq, Dh, G = (kv["batch"], kv["prefill"], kv["decode"], kv["kv_heads"],
                              kv["q_heads"], kv["head_dim"], kv["group"])
    S = P + Dn
    k = wl.kv_tensor_torch(torch, dev, W.wid, 0, B, S, H, Dh, kv["outlier"])
    v = wl.kv_tensor_torch(torch, dev, W.wid, 1, B, S, H, Dh, kv["outlier"])
    q = wl.kv_tensor_torch(torch, dev, W.wid, 2, B, S, Hq, Dh, 1.0)
    kp, vp = k[:, :P].contiguous(), v[:, :P].contiguous()
    qp = q[:, :P].reshape(-1, Dh)
    s = torch.from_numpy(wl.signs(W.wid, Dh)).to(dev)
    cache = {n: (torch.empty((B, H, S, Dh // 2), dtype=torch.uint8, device=dev),
                 torch.empty((B, H, S, Dh // G, 2), dtype=torch.float16, device=dev))
             for n in ("k", "v")}
    qo_p = torch.empty((B * P * Hq, Dh), dtype=torch.float16, device=dev)
    L = [("kv_rotate_quant", "k:init", kv_bytes(B * P * H, Dh, G), 0,
          lambda: qr.kv_rotate_quant(kp, s, G, 0.95, *cache["k"], 0), cache["k"]),
         ("kv_rotate_quant", "v:init", kv_bytes(B * P * H, Dh, G), 0,
          lambda: qr.kv_rotate_quant(vp, None, G, 0.95, *cache["v"], 0, rotate=False), cache["v"]),
         ("hadamard", "q:prompt", rot_bytes(B * P * Hq, Dh), 0,
          lambda: qr.hadamard(qp, s, torch.float16, out=qo_p), (qo_p,))]
    qo_d = [torch.empty((B * Hq, Dh), dtype=torch.float16, device=dev) for _ in range(Dn)]
    att_o = [torch.empty((B, Hq, Dh), dtype=torch.float16, device=dev) for _ in range(Dn)]
    ws = torch.empty((qr.kv_decode_workspace_bytes(B, Hq, H, Dh, S),), dtype=torch.uint8, device=dev)
    scale = 1.0 / Dh ** 0.5
    for i in range(Dn):
        qd = q[:, P + i].reshape(-1, Dh)
        L.append(("kv_rotate_quant", f"k:append{i}", kv_bytes(B * H, Dh, G), 0,
                  lambda i=i: qr.kv_rotate_quant(k[:, P + i:P + i + 1], s, G, 0.95, *cache["k"], P + i),
                  cache["k"]))
        L.append(("kv_rotate_quant", f"v:append{i}", kv_bytes(B * H, Dh, G), 0,
                  lambda i=i: qr.kv_rotate_quant(v[:, P + i:P + i + 1], None, G, 0.95, *cache["v"],
                                                 P + i, rotate=False), cache["v"]))
        L.append(("hadamard", f"q:decode{i}", rot_bytes(B * Hq, Dh), 0,
                  lambda qd=qd, i=i: qr.hadamard(qd, s, torch.float16, out=qo_d[i]), (qo_d[i],)))
        L.append(("kv_decode_attention", f"decode{i}", decode_bytes(B, H, Hq, P + i + 1, Dh, G), 0,
                  lambda i=i: qr.kv_decode_attention(qo_d[i].view(B, Hq, Dh), *cache["k"], *cache["v"],
                                                     P + i + 1, G, scale, out=att_o[i], workspace=ws),
                  (att_o[i],)))
    desc = (f"Llama-2-70B KV path: batch {B}, {P}-token prompt + {Dn} decode steps, {H} KV heads "
            f"and {Hq} query heads of {Dh}; K/V Init + Append into the 4-bit cache (group {G}, "
            f"clip 0.95), head-wise rotation of K and Q, Decode attention of each step's query "
            f"over the cache ({P + 1}..{S} positions)")
    return L, desc


# ---------------------------------------------------------------------------
# Timing
# ---------------------------------------------------------------------------

def _median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def run_timed(torch, launches, steps, warmup):
    """Eager launches; HIP events around every launch and every step.  Returns
    (mean ms per step over the timed region, per-launch median ms over the steps,
    wall seconds, per-step ms)."""
    for _ in range(warmup):
        for l in launches:
            l[4]()
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in launches] for _ in range(steps)]
    tb = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    tb[0].record()
    for k in range(steps):
        for i, l in enumerate(launches):
            ev[k][i][0].record()
            l[4]()
            ev[k][i][1].record()
        tb[k + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per = [_median([ev[k][i][0].elapsed_time(ev[k][i][1]) for k in range(steps)])
           for i in range(len(launches))]
    step_ms = [tb[k].elapsed_time(tb[k + 1]) for k in range(steps)]
    return tb[0].elapsed_time(tb[steps]) / steps, per, wall, step_ms


class MallScrub:
    """Defeats the 256 MB Infinity Cache (MALL) between timed launches: a device
    copy of 512 MiB evicts every line a launch could reuse, and a read-only
    pass over the copy's 512 MiB source then writes back the copy's dirty
    lines, so that the timed launch finds a cache of clean lines that hold none
    of its data, instead of paying the write-back of the scrub's own stores
    (the copy alone added 6 us to the 70B decode attention, 2 us to a 7B
    decode GEMM).  Both run outside the events of the launch being timed."""

    def __init__(self, torch, dev, mib=512):
        n = mib << 20
        self.torch = torch
        self.src = torch.empty(n, dtype=torch.uint8, device=dev)
        self.src.fill_(1)
        self.dst = torch.empty_like(self.src)
        self.words = self.src.view(torch.int32)
        self.acc = torch.empty((), dtype=torch.int32, device=dev)

    def __call__(self):
        self.dst.copy_(self.src)
        # a reduction over the 32-bit words as stored: it reads the 512 MiB and
        # writes one word (a dtype argument would first write a widened copy)
        self.torch.amax(self.words, dim=0, out=self.acc)


def run_cold(torch, launches, steps, warmup, scrub):
    """Per-launch times with the MALL scrubbed before every launch (outside its
    events): the launch's inputs and weights come from HBM, not from the
    Infinity Cache.  Returns per-launch medians over `steps` passes (ms)."""
    for _ in range(max(1, warmup)):
        for l in launches:
            l[4]()
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in launches] for _ in range(steps)]
    for k in range(steps):
        for i, l in enumerate(launches):
            scrub()
            ev[k][i][0].record()
            l[4]()
            ev[k][i][1].record()
    torch.cuda.synchronize()
    return [_median([ev[k][i][0].elapsed_time(ev[k][i][1]) for k in range(steps)])
            for i in range(len(launches))]


def run_graphed(torch, launches, steps, warmup, reps=20):
    """Timing for steps made of many short launches, where the host's launch
    latency would otherwise be measured instead of the kernels: each launch is
    captured REPS times into a HIP graph and replayed between two events, and
    the whole step is captured once and replayed STEPS times.  Every output is
    compared with the eager run's before timing."""
    for _ in range(max(1, warmup)):
        for l in launches:
            l[4]()
    torch.cuda.synchronize()
    eager = [[t.clone() for t in l[5]] for l in launches]
    step_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(step_graph):
        for l in launches:
            l[4]()
    for t_list in (l[5] for l in launches):
        for t in t_list:
            t.zero_()
    step_graph.replay()
    torch.cuda.synchronize()
    same = all(torch.equal(a, b) for l, e in zip(launches, eager) for a, b in zip(l[5], e))
    per = []
    for l in launches:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                l[4]()
        g.replay()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) / reps)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for _ in range(steps):
        step_graph.replay()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    return t0.elapsed_time(t1) / steps, per, wall, same


def kernel_totals(launches, per, kernel):
    ms = sum(p for l, p in zip(launches, per) if l[0] == kernel)
    nbytes = sum(l[2] for l in launches if l[0] == kernel)
    ops = sum(l[3] for l in launches if l[0] == kernel)
    n = sum(1 for l in launches if l[0] == kernel)
    return ms, nbytes, ops, n


def source_sha(kernel):
    return hashlib.sha256((CSRC / KERNEL_SOURCE[kernel]).read_bytes()).hexdigest()


def profiled_traffic(kernel, workload):
    """HBM bytes per launch from profiles/traffic_<kernel>_<workload>.txt, or None
    if that summary is missing or was taken on a different kernel source."""
    f = ROOT / "profiles" / f"traffic_{kernel}_{workload}.txt"
    if not f.exists():
        return None
    kv = {}
    for line in f.read_text().splitlines():
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_sha(kernel):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def calibrated_value(name, key):
    """A figure from a committed calibration summary profiles/<name>, or None if
    it is missing or was taken on a different calibration-kernel source."""
    f = ROOT / "profiles" / name
    if not f.exists():
        return None
    kv = {}
    for line in f.read_text().splitlines():
        if ":" in line and not line.startswith(("#", " ")):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    src = CSRC / "calibrate.hip"
    if not src.exists() or kv.get("source_sha256") != hashlib.sha256(src.read_bytes()).hexdigest():
        return None
    try:
        return float(kv[key])
    except (KeyError, ValueError):
        return None


def calibrated_stream_gbs():
    """Median rate of the 16:4 read/write stream (profiles/hbm_stream_calibration.txt)."""
    return calibrated_value("hbm_stream_calibration.txt", "median_gbs")


def calibrated_mfma_tops():
    """Steady-state rate of the register-only int8 MFMA loop, from the committed
    profiles/mfma_i8_calibration.txt (None if missing or taken on another source)."""
    v = calibrated_value("mfma_i8_calibration.txt", "steady_state_pops")
    return None if v is None else 1e3 * v


def roofline(kernel, workload, launches, per, bound):
    ms, nbytes, ops, n = kernel_totals(launches, per, kernel)
    tr = profiled_traffic(kernel, workload)
    if bound == "mfma":
        ach = ops / (ms * 1e-3) / 1e12
        cal = calibrated_mfma_tops()
        return {"bound": "mfma", "kernel": kernel, "launches_per_step": n,
                "achieved": round(ach, 1), "peak": INT8_PEAK_TOPS, "unit": "TFLOP/s",
                "op_note": "int8 MFMA operations (2 per multiply-accumulate) over the step's "
                           "launches of the kernel / their summed event time",
                "frac": round(ach / INT8_PEAK_TOPS, 4),
                "traffic": None if tr is None else round(tr),
                "practical_peak": None if cal is None else round(cal, 1),
                "practical_frac": None if cal is None else round(ach / cal, 4),
                "practical_note": "steady-state rate of the same MFMA instruction in a "
                                  "register-only loop at the chip's power limit "
                                  "(bench.py --mfma-calibration; profiles/mfma_i8_calibration.txt)"}
    ach = nbytes / (ms * 1e-3) / 1e9
    cal = calibrated_stream_gbs()
    return {"bound": "hbm", "kernel": kernel, "launches_per_step": n,
            "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None if tr is None else round(tr),
            "practical_peak": None if cal is None else round(cal, 1),
            "practical_frac": None if cal is None else round(ach / cal, 4),
            "practical_note": "rate of a plain non-temporal stream reading 16 bytes for every 4 "
                              "written (bench.py --stream-calibration; "
                              "profiles/hbm_stream_calibration.txt)"}


def copy_calibration():
    import torch
    dev = torch.device("cuda:0")
    n = (1 << 30) // 2
    a = torch.empty(n, dtype=torch.float16, device=dev).normal_()
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(11)]
    ev[0].record()
    for i in range(10):
        b.copy_(a)
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(10))
    med = 0.5 * (ms[4] + ms[5])
    print(json.dumps({"copy_calibration": True, "bytes_read_per_launch": 2 * n,
                      "bytes_written_per_launch": 2 * n, "launches": 10,
                      "copy_ms_median": round(med, 4),
                      "copy_GB/s_read_plus_write": round(4 * n / (med * 1e-3) / 1e9, 1)}),
          flush=True)
    return 0


def mfma_calibration():
    import numpy as np
    import torch

    import hadamard_rotation_int4_amd as qr
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(7)
    # 16 q, q uniform in -8..7: the values the GEMM's unpacked INT4 operands take
    frag = torch.from_numpy((16 * rng.integers(-8, 8, size=(64, 16))).astype(np.int8)).to(dev)
    grid, iters = 2048, 4096
    ops = 2.0 * 32 * 32 * 32 * 4 * iters * grid * 4
    qr.calibrate_mfma_i8(frag, grid, 16)
    torch.cuda.synchronize()
    # 16 launches back to back (about 40 ms, as long as a block step's GEMMs),
    # each bracketed by events and with its own clock counters
    nl = 16
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nl + 1)]
    outs = []
    ev[0].record()
    for i in range(nl):
        outs.append(qr.calibrate_mfma_i8(frag, grid, iters, clocks=True))
        ev[i + 1].record()
    torch.cuda.synchronize()
    runs = []
    for i, (chk, clk) in enumerate(outs):
        ms = ev[i].elapsed_time(ev[i + 1])
        c = clk.view(torch.int64).cpu().numpy().astype(np.float64)
        mhz = float(np.mean((c[:, 1] - c[:, 0]) / ((c[:, 3] - c[:, 2]) / 100.0)))
        pops = ops / (ms * 1e-3) / 1e15
        runs.append({"ms": round(ms, 3), "POP/s": round(pops, 3), "clock_MHz": round(mhz),
                     "frac_of_peak_at_clock": round(pops / (256 * 8192 * mhz * 1e6 / 1e15), 3)})
    # every wavefront's checksums against the exact sum (include/qr.h)
    f = frag.cpu().numpy().astype(np.int64)
    total = 0
    for j in range(4):
        b = f[(np.arange(64) + 7 + 16 * j) % 64]
        total += int((np.concatenate([f[:32], f[32:]], 1) @ np.concatenate([b[:32], b[32:]], 1).T).sum())
    exact = all(bool(((c.cpu().numpy().astype(np.int64).reshape(-1, 64).sum(1) % 2**32)
                      == (iters * total) % 2**32).all()) for c, _ in outs)
    pops = sorted(r["POP/s"] for r in runs)
    print(json.dumps({"mfma_calibration": True, "instruction": "v_mfma_i32_32x32x32_i8",
                      "grid": grid, "wavefronts_per_simd": grid * 4 // 1024, "iters": iters,
                      "int_ops_per_launch": ops, "checksums_exact": exact,
                      "median_POP/s": pops[len(pops) // 2], "min_POP/s": pops[0], "max_POP/s": pops[-1],
                      "median_clock_MHz": sorted(r["clock_MHz"] for r in runs)[len(runs) // 2],
                      "peak_POP/s": INT8_PEAK_TOPS / 1e3,
                      "runs": runs}), flush=True)
    return 0


def stream_calibration():
    import numpy as np
    import torch

    import hadamard_rotation_int4_amd as qr
    dev = torch.device("cuda:0")
    n16 = (1 << 30) // 16  # the input bytes of one d = 8192 rotate+quant launch at T = 65536
    src = torch.empty(n16 * 4, dtype=torch.int32, device=dev).random_()
    out = torch.empty(n16, dtype=torch.uint32, device=dev)
    grid = 2048
    qr.calibrate_stream(src, grid, out=out)
    torch.cuda.synchronize()
    nl = 16
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nl + 1)]
    ev[0].record()
    for i in range(nl):
        qr.calibrate_stream(src, grid, out=out)
        ev[i + 1].record()
    torch.cuda.synchronize()
    nbytes = n16 * 20
    runs = [round(nbytes / (ev[i].elapsed_time(ev[i + 1]) * 1e-3) / 1e9, 1) for i in range(nl)]
    sv = src[: 4 * 4096].view(4096, 4).cpu().numpy().astype(np.int64) & 0xFFFFFFFF
    ref = sv[:, 0] ^ sv[:, 1] ^ sv[:, 2] ^ sv[:, 3]
    exact = bool((out[:4096].cpu().numpy().astype(np.int64) == ref).all())
    srt = sorted(runs)
    print(json.dumps({"stream_calibration": True, "bytes_read_per_launch": n16 * 16,
                      "bytes_written_per_launch": n16 * 4, "grid": grid, "launches": nl,
                      "first_4096_outputs_exact": exact,
                      "median_GB/s": srt[nl // 2], "min_GB/s": srt[0], "max_GB/s": srt[-1],
                      "runs_GB/s": runs}), flush=True)
    return 0


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this path is measured on one GPU only (the per-GPU shard of "
                                   "a sharded run has the same shapes); run with --gpus 1",
                          "n_gpus": args.gpus}))
        return 2
    if args.copy_calibration:
        return copy_calibration()
    if args.mfma_calibration:
        return mfma_calibration()
    if args.stream_calibration:
        return stream_calibration()
    import torch

    import hadamard_rotation_int4_amd as qr
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wname = args.workload
    bits = 8 if wname.endswith("_w8a8") else 4
    quarot = wname in ("70b_block", "7b_block", "70b_block_w8a8", "7b_block_w8a8")
    W = wl.WORKLOADS[wname.replace("_w8a8", "").replace("block", "prefill") if quarot else wname]
    print(f"[bench] workload {W.name}{' (QuaRot online path)' if quarot else ''}", file=sys.stderr,
          flush=True)
    config = {"workload": None}
    if wname in ("70b_prefill", "7b_prefill") or quarot:
        T = W.tokens[0]
        group = args.group if wname in ("70b_prefill", "7b_prefill") else 0
        launches, lin, kvdesc = make_block(torch, qr, wl, W, T, dev, True, args.fp16_hadamard,
                                           quarot, bits, group)
        inputs_desc = ("RMSNorm (no scale) + INT4 before QKV and gate/up, Hadamard heads "
                       f"({W.hidden // 128} heads of 128) + INT4 before O, online Hadamard "
                       f"d = {lin['down'].k} + INT4 before down" if quarot
                       else "4 fused rotate+quant")
        if bits != 4:
            inputs_desc = f"{bits}-bit codes one per byte: " + inputs_desc.replace(" + INT4", "")
        if group:
            inputs_desc = (f"group-wise scales (group {group} along K) on both operands: 4 "
                           "rotate+quant")
        config.update({
            "workload": f"{W.name}{' (QuaRot online path)' if quarot else ''}: T={T} tokens, "
                        f"hidden {W.hidden}, FFN {lin['down'].k}, QKV {lin['qkv'].n}; "
                        f"{inputs_desc}, 5 W4A4 GEMMs, {kvdesc}",
            "tokens": T, "hidden": W.hidden, "ffn": lin["down"].k,
            "hadamard_arithmetic": (f"fp16 for d = {lin['down'].k}, fp32 otherwise"
                                    if args.fp16_hadamard else "fp32")})
        dominant, bound = ("w4a4_gemm_groups" if group else "w4a4_gemm" if bits == 4
                           else "w8a8_gemm"), "mfma"
    elif wname == "7b_decode":
        launches = []
        for T in W.tokens:
            L, lin, _ = make_block(torch, qr, wl, W, T, dev, False)
            launches += L
        config.update({
            "workload": f"{W.name}: T in {list(W.tokens)}; per T 4 fused rotate+quant (d = "
                        f"{W.hidden}, {lin['down'].k}) and the 5 W4A4 GEMMs (weight streaming)",
            "tokens": list(W.tokens), "hidden": W.hidden, "ffn": lin["down"].k})
        dominant, bound = "w4a4_gemm", "hbm"
    else:
        launches, desc = make_kv_decode(torch, qr, wl, W, dev)
        config.update({"workload": desc})
        dominant, bound = "kv_decode_attention", "hbm"
    torch.cuda.synchronize()

    graphed = wname in ("7b_decode", "70b_kv")
    step_ms = None
    if graphed:
        ms_step, per, wall, same = run_graphed(torch, launches, args.steps, args.warmup)
        if not same:
            print("[bench] graph replay differs from the eager run", file=sys.stderr, flush=True)
            return 1
    else:
        ms_step, per, wall, step_ms = run_timed(torch, launches, args.steps, args.warmup)
    # Workloads whose launches fit in the 256 MB Infinity Cache are timed per
    # launch a second time with the cache scrubbed before every launch: those
    # MALL-cold times are the ones reported against HBM; the warm ones are kept
    # beside them, labelled.
    cold = wname in SMALL_WORKING_SET
    per_warm = per
    if cold:
        per = run_cold(torch, launches, COLD_REPS, 1, MallScrub(torch, dev))
    total_ops = sum(l[3] for l in launches)
    total_bytes = sum(l[2] for l in launches)
    if bound == "mfma":
        value, unit = total_ops / (ms_step * 1e-3) / 1e12, "TOPS"
    else:
        value, unit = total_bytes / (ms_step * 1e-3) / 1e9, "GB/s"

    kernels = {}
    for l, p, pw in zip(launches, per, per_warm):
        kernels[f"{l[0]}:{l[1]}"] = {"ms": round(p, 4), "GB/s": round(l[2] / p / 1e6, 1),
                                     "TOPS": round(l[3] / p / 1e9, 1)}
        if cold:
            kernels[f"{l[0]}:{l[1]}"]["ms_mall_warm"] = round(pw, 4)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": config,
        "roofline": roofline(dominant, wname, launches, per, bound),
    }
    for k in ("hadamard_quant", "rmsnorm_quant", "hadamard_heads_quant", "hadamard_quant_i8",
              "rmsnorm_quant_i8", "hadamard_heads_quant_i8", "hadamard_quant_groups"):
        if any(l[0] == k for l in launches):
            out["roofline_" + k] = roofline(k, wname, launches, per, "hbm")
    if dominant != "kv_rotate_quant" and any(l[0] == "kv_rotate_quant" for l in launches):
        out["roofline_kv_rotate_quant"] = roofline("kv_rotate_quant", wname, launches, per, "hbm")
    out["kernels"] = kernels if len(kernels) <= 40 else {
        k: {"ms": round(sum(p for l, p in zip(launches, per) if l[0] == k), 4),
            "launches": sum(1 for l in launches if l[0] == k)}
        for k in sorted({l[0] for l in launches})}
    if wname in ("70b_prefill", "7b_prefill") and not args.no_context and not args.group:
        out["quality"] = quality_report(torch, qr, wl, W, dev)
    if quarot and not args.no_context:
        out["fp16_context"] = fp16_context(torch, wl, W, T, dev, launches, per, args)
    out["wall_s_timed"] = round(wall, 3)
    if step_ms:
        out["step_ms_median"] = round(_median(step_ms), 4)
        out["step_ms_min_max"] = [round(min(step_ms), 4), round(max(step_ms), 4)]
    out["timing"] = (("HIP graph replay of the step; " if graphed else
                      "eager launches, HIP events around each launch and each step on the "
                      "launch stream; ")
                     + (f"per-launch times (kernels, rooflines) are medians of {COLD_REPS} "
                        "passes with the Infinity Cache (MALL) scrubbed before every launch "
                        "(MALL-cold, against HBM); ms_mall_warm: "
                        + ("graphs of 20 back-to-back launches (outputs checked equal to the "
                           "eager run)" if graphed else "median over the timed steps")
                        if cold else "per-launch times are medians over the timed steps "
                        "(working sets of GBs: MALL-cold by size)"))
    if wname == "70b_prefill" and not args.no_configs and not args.group and not args.fp16_hadamard:
        del launches
        import gc
        gc.collect()
        torch.cuda.empty_cache()
        out["configs"] = config_summaries(torch, qr, wl, dev)
    if not args.no_cpu_baseline and wname in ("70b_prefill", "70b_block") and not args.group:
        out["cpu_baseline"] = cpu_baseline(W, args.cpu_sample_tokens, quarot=quarot)
    print(json.dumps(out), flush=True)
    return 0


def _gbs(nbytes, ms):
    return round(nbytes / (ms * 1e-3) / 1e9, 1)


def config_summaries(torch, qr, wl, dev):
    """Compact results of the four configurations the default (70B prefill)
    line does not time in full, each timed per launch MALL-cold (median of
    COLD_REPS passes with the Infinity Cache scrubbed before every launch) and
    reported against the roofline that bounds it.  Parity of these shapes is
    covered by the GPU tests."""
    import gc
    scrub = MallScrub(torch, dev)
    res = {}

    def frac(gbs):
        return round(gbs / HBM_PEAK_GBS, 4)

    # -- configuration 1: tiny W4A4 linear (X [32, 4096], W [4096, 4096]) --
    W = wl.WORKLOADS["tiny"]
    T, l = W.tokens[0], W.linears[0]
    x = wl.activations_torch(torch, dev, W.wid, 0, T, l.k, W.n_outliers, W.outlier_lo,
                             W.outlier_hi)
    s = torch.from_numpy(wl.signs(W.wid, l.k)).to(dev)
    w = wl.weights_torch(torch, dev, W.wid, 1, l.n, l.k)
    wq = qr.hadamard_quant(w, s, 1.0)
    del w
    qa = (torch.empty((T, l.k // 2), dtype=torch.uint8, device=dev),
          torch.empty((T,), dtype=torch.float16, device=dev))
    y = torch.empty((T, l.n), dtype=torch.float16, device=dev)
    L = [("hadamard_quant", "x", hq_bytes(T, l.k), 0,
          lambda: qr.hadamard_quant(x, s, 1.0, out=qa), qa),
         ("w4a4_gemm", "linear", gemm_bytes(T, l.n, l.k), gemm_ops(T, l.n, l.k),
          lambda: qr.w4a4_gemm(*qa, *wq, out=y), (y,))]
    ms_graph, per_warm, _, same = run_graphed(torch, L, 20, 3)
    per = run_cold(torch, L, COLD_REPS, 1, scrub)
    res["1_tiny_w4a4_linear"] = {
        "workload": "rotate+quant of X fp16 [32, 4096] (d = 4096) and the W4A4 GEMM "
                    "32 x 4096 x 4096 (weights prepared offline)",
        "step_us_graph_replay": round(ms_graph * 1e3, 2),
        "hadamard_quant_us": round(per[0] * 1e3, 2),
        "w4a4_gemm_us": round(per[1] * 1e3, 2),
        "w4a4_gemm_GB/s": _gbs(L[1][2], per[1]), "w4a4_gemm_frac_hbm": frac(_gbs(L[1][2], per[1])),
        "graph_replay_equals_eager": bool(same),
        "bound": "latency (1.1 us of HBM time at peak)"}
    del L, x, wq, qa, y
    gc.collect()

    # -- configuration 2: Llama-2-7B one-block prefill, T = 2048 --
    W = wl.WORKLOADS["7b_prefill"]
    T = W.tokens[0]
    L, lin, _ = make_block(torch, qr, wl, W, T, dev, False)
    ms_step, per_warm, _, _ = run_timed(torch, L, 10, 3)
    per = run_cold(torch, L, COLD_REPS, 1, scrub)
    g_ms, g_b, g_ops, _ = kernel_totals(L, per, "w4a4_gemm")
    h4 = [(l, p) for l, p in zip(L, per) if l[0] == "hadamard_quant" and "down_in" not in l[1]]
    hd = [(l, p) for l, p in zip(L, per) if l[0] == "hadamard_quant" and "down_in" in l[1]]
    tops = g_ops / (g_ms * 1e-3) / 1e12
    res["2_7b_prefill"] = {
        "workload": f"Llama-2-7B block, T = {T}: 4 rotate+quant (d = 4096 x 3, 11008) + 5 W4A4 "
                    "GEMMs (QKV 12288, O 4096, gate/up 11008, down 4096 x 11008)",
        "step_ms_mall_warm": round(ms_step, 4),
        "gemm_TOPS": round(tops, 1), "gemm_frac_int8_peak": round(tops / INT8_PEAK_TOPS, 4),
        "gemm_per_launch_TOPS": {l[1].split(":")[-1]: round(l[3] / p / 1e9, 1)
                                 for l, p in zip(L, per) if l[0] == "w4a4_gemm"},
        "hadamard_quant_d4096_us": round(1e3 * sum(p for _, p in h4) / len(h4), 2),
        "hadamard_quant_d4096_GB/s": _gbs(sum(l[2] for l, _ in h4), sum(p for _, p in h4)),
        "hadamard_quant_d11008_us": round(1e3 * hd[0][1], 2),
        "hadamard_quant_d11008_GB/s": _gbs(hd[0][0][2], hd[0][1]),
        "hadamard_quant_d11008_frac_hbm": frac(_gbs(hd[0][0][2], hd[0][1])),
        "note": "per-launch MALL-cold medians; the d = 11008 rotation is bound inside each "
                "row (its VALU and MFMA fractions are in the committed counter summary)"}
    del L, lin
    gc.collect()
    torch.cuda.empty_cache()

    # -- configuration 3: Llama-2-7B decode, T in {1, 8, 32, 64} --
    W = wl.WORKLOADS["7b_decode"]
    per_t = {}
    for T in W.tokens:
        L, lin, _ = make_block(torch, qr, wl, W, T, dev, False)
        per = run_cold(torch, L, COLD_REPS, 1, scrub)
        g_ms, g_b, _, _ = kernel_totals(L, per, "w4a4_gemm")
        hq = [(l, p) for l, p in zip(L, per) if l[0] == "hadamard_quant"]
        per_t[f"T{T}"] = {
            "gemm_us": round(g_ms * 1e3, 2), "gemm_GB/s": _gbs(g_b, g_ms),
            "gemm_frac_hbm": frac(_gbs(g_b, g_ms)),
            "hadamard_quant_us": {l[1].split(":")[-1]: round(p * 1e3, 2) for l, p in hq}}
        del L, lin
        gc.collect()
    res["3_7b_decode"] = {
        "workload": "Llama-2-7B decode shapes: per T the 4 rotate+quant launches and the 5 "
                    "weight-streaming W4A4 GEMMs (101 MB of INT4 weights)",
        "per_T": per_t,
        "note": "MALL-cold: weights and activations read from HBM (GB/s of the weight + "
                "activation + output streams over the 5 GEMMs' summed time)"}
    torch.cuda.empty_cache()

    # -- configuration 5: Llama-2-70B KV cache, Init + 50 x (Append, Decode) --
    W = wl.WORKLOADS["70b_kv"]
    L, _ = make_kv_decode(torch, qr, wl, W, dev)
    per = run_cold(torch, L, COLD_REPS, 1, scrub)
    init = [(l, p) for l, p in zip(L, per) if l[1] in ("k:init", "v:init")]
    dec = [(l, p) for l, p in zip(L, per) if l[0] == "kv_decode_attention"]
    app = [p for l, p in zip(L, per) if "append" in l[1]]
    qp = [(l, p) for l, p in zip(L, per) if l[1] == "q:prompt"]
    i_b, i_ms = sum(l[2] for l, _ in init), sum(p for _, p in init)
    d_b, d_ms = sum(l[2] for l, _ in dec), sum(p for _, p in dec)
    res["5_70b_kv"] = {
        "workload": "Llama-2-70B KV path: batch 32, 2048-token prompt + 50 decode steps, 8 KV "
                    "heads / 64 query heads of 128, group 128",
        "kv_init_us": round(i_ms * 1e3, 2), "kv_init_GB/s": _gbs(i_b, i_ms),
        "kv_init_frac_hbm": frac(_gbs(i_b, i_ms)),
        "q_prompt_rotation_GB/s": _gbs(qp[0][0][2], qp[0][1]),
        "decode_attention_us_median": round(1e3 * _median([p for _, p in dec]), 2),
        "decode_attention_GB/s": _gbs(d_b, d_ms),
        "decode_attention_frac_hbm": frac(_gbs(d_b, d_ms)),
        "append_us_median": round(1e3 * _median(app), 2),
        "note": "MALL-cold per launch (the 73 MB cache would otherwise stay in the Infinity "
                "Cache between decode steps)"}
    del L
    gc.collect()
    torch.cuda.empty_cache()
    return res


def fp16_context(torch, wl, W, T, dev, launches, per, args):
    """The five linear layers in fp16 against the same five in the 4-bit path
    (their input quantizers plus the W4A4 GEMMs); timed after the step, on
    their own.  Context for the pages' FP16-block speedups, not a target."""
    L = fp16_linears(torch, wl, W, T, dev)
    torch.cuda.synchronize()
    ms16, per16, _, _ = run_timed(torch, L, max(1, args.steps // 2), 1)
    del L
    lin_kernels = ("w4a4_gemm", "rmsnorm_quant", "hadamard_heads_quant", "hadamard_quant",
                   "w8a8_gemm", "rmsnorm_quant_i8", "hadamard_heads_quant_i8", "hadamard_quant_i8")
    ms4 = sum(p for l, p in zip(launches, per) if l[0] in lin_kernels)
    ops = 2 * T * sum(l.n * l.k for l in W.linears)
    # hipBLASLt's int8 GEMM (torch._int_mm, int32 out, no epilogue) at the same
    # shapes: what the vendor library reaches with the same int8 matrix cores
    Li = []
    for i, l in enumerate(W.linears):
        g = torch.Generator(device=dev)
        g.manual_seed(1000 + i)
        a = torch.randint(-8, 8, (T, l.k), generator=g, device=dev, dtype=torch.int8)
        b = torch.randint(-8, 8, (l.n, l.k), generator=g, device=dev, dtype=torch.int8)
        Li.append(("int8_gemm", l.name, 0, gemm_ops(T, l.n, l.k),
                   (lambda a=a, b=b: torch._int_mm(a, b.t())), ()))
    try:
        ms8, per8, _, _ = run_timed(torch, Li, max(1, args.steps // 2), 1)
        int8_ctx = {"hipblaslt_int8_linears_ms": round(ms8, 4),
                    "hipblaslt_int8_TOPS": round(ops / (ms8 * 1e-3) / 1e12, 1),
                    "hipblaslt_int8_per_gemm_TOPS": {l.name: round(gemm_ops(T, l.n, l.k) / p / 1e9, 1)
                                                      for l, p in zip(W.linears, per8)}}
    except RuntimeError as e:  # shapes the library does not take
        int8_ctx = {"hipblaslt_int8": f"unavailable: {e}"[:200]}
    del Li
    # prefill attention runs in fp16 on both sides (the pages use an off-the-shelf
    # flash attention on the unquantized Q/K/V): time it once and add it to both
    attn_ms = None
    try:
        Hq, Hkv, Dh = W.hidden // 128, (8 if W.hidden == 8192 else W.hidden // 128), 128
        B = 32 if T % 32 == 0 and T >= 32 * 128 else 1
        S = T // B
        g = torch.Generator(device=dev)
        g.manual_seed(77)
        q = torch.randn((B, Hq, S, Dh), generator=g, device=dev, dtype=torch.float16)
        k = torch.randn((B, Hkv, S, Dh), generator=g, device=dev, dtype=torch.float16)
        v = torch.randn((B, Hkv, S, Dh), generator=g, device=dev, dtype=torch.float16)
        k = k.repeat_interleave(Hq // Hkv, dim=1).contiguous()
        v = v.repeat_interleave(Hq // Hkv, dim=1).contiguous()
        La = [("fp16_attention", "sdpa", 0, 0,
               (lambda: torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)),
               ())]
        attn_ms, _, _, _ = run_timed(torch, La, max(1, args.steps // 2), 1)
        del q, k, v, La
    except RuntimeError as e:  # no attention kernel for these shapes
        attn_ms = f"unavailable: {e}"[:200]
    block = {}
    if isinstance(attn_ms, float):
        block = {"fp16_attention_ms": round(attn_ms, 4),
                 "block_speedup": round((ms16 + attn_ms) / (ms4 + attn_ms), 3),
                 "block_note": f"(fp16 linears + causal SDPA, B={B} x S={S}, {Hq} heads) vs "
                               "(4 quantizers + 5 quantized GEMMs + the same SDPA); KV "
                               "quantization and norms left out of both"}
    else:
        block = {"fp16_attention": attn_ms}
    return {"fp16_linears_ms": round(ms16, 4),
            "fp16_TFLOP/s": round(ops / (ms16 * 1e-3) / 1e12, 1),
            "fp16_per_gemm_ms": {l.name: round(p, 4) for l, p in zip(W.linears, per16)},
            "quantized_linears_ms": round(ms4, 4),
            "linears_speedup": round(ms16 / ms4, 3),
            **block,
            **int8_ctx,
            "note": "torch.matmul (hipBLASLt) fp16 GEMMs of the same shapes vs the 4 input "
                    "quantizers + 5 quantized GEMMs of the step; hipBLASLt int8 (torch._int_mm, "
                    "int32 output, no scales) at the same shapes for calibration"}


def quality_report(torch, qr, wl, W, dev, t=64, n=512):
    """SQNR of the W4A4 output against the unquantized product X W^T (float64 on
    the host) on a sample of the QKV GEMM: t tokens of its input, n output
    channels, with the randomized Hadamard and without it (quantization only).
    Reported, not a target: it shows what the rotation buys on outlier inputs."""
    import numpy as np
    lin = {l.name: l for l in W.linears}
    K = lin["qkv"].k
    x = wl.activations_torch(torch, dev, W.wid, 10, t, K, W.n_outliers, W.outlier_lo,
                             W.outlier_hi)
    w = wl.weights_torch(torch, dev, W.wid, 1, n, K)
    s = torch.from_numpy(wl.signs(W.wid, K)).to(dev)
    ref = x.double().cpu().numpy() @ w.double().cpu().numpy().T
    res = {}
    for rot in (True, False):
        qa, sa = qr.hadamard_quant(x, s, 1.0, rotate=rot)
        qw, sw = qr.hadamard_quant(w, s, 1.0, rotate=rot)
        y = qr.w4a4_gemm(qa, sa, qw, sw).double().cpu().numpy()
        res["sqnr_db_rotated" if rot else "sqnr_db_no_rotation"] = round(
            float(10 * np.log10(np.sum(ref ** 2) / np.sum((y - ref) ** 2))), 2)
    res["sample"] = (f"{t} tokens of the QKV input (outlier channels planted) x {n} output "
                     "channels, against float64 X W^T")
    return res


def cpu_baseline(W, t_sample, quarot=False):
    """Time the oracle (float64 rotation + quantization, exact GEMM via float64
    BLAS on the codes, KV quantization) on a bounded sample of the step:
    t_sample tokens against the first 1024 output channels of each GEMM.
    With quarot the GEMM inputs go through the block's own quantizers
    (RMSNorm + INT4, Hadamard heads + INT4, online Hadamard + INT4 before down).
    Reported as TOPS over the same GEMM operations (2 per MAC)."""
    import numpy as np

    import workloads as wl
    from oracle import block as ob
    from oracle import gemm as og
    from oracle import hadamard as oh
    from oracle import kv as okv
    from oracle import quant as oq

    cores = len(os.sched_getaffinity(0))
    lin = {l.name: l for l in W.linears}
    n_s = 1024
    xs = {name: wl.activations(W.wid, 10 + i, t_sample, (lin["down"].k if name == "down_in" else W.hidden))
          for i, name in enumerate(("attn_in", "o_in", "ffn_in", "down_in"))}
    ws = {name: wl.weights(W.wid, 1 + i, n_s, l.k) for i, (name, l) in enumerate(lin.items())}
    sg = {d: wl.signs(W.wid, d) for d in (W.hidden, lin["down"].k)}
    # weights are prepared offline (not timed), as on the GPU
    wq = {}
    for name, l in lin.items():
        q, s = oq.sym_quant_math(oh.rotate(ws[name].astype(np.float64), sg[l.k]))
        wq[name] = (oq.pack_int4(q), s)
    kx = wl.kv_tensor(5, 0, 1, t_sample, 8, 128)
    t0 = time.perf_counter()
    qa = {}
    for name, x in xs.items():
        if quarot and name in ("attn_in", "ffn_in"):
            q, s, _ = ob.rmsnorm_quant_math(x, 1e-5)
        elif quarot and name == "o_in":
            q, s, _ = ob.hadamard_heads_quant_math(x, W.hidden // 128)
        else:
            q, s = oq.sym_quant_math(oh.rotate(x.astype(np.float64), sg[x.shape[1]]))
        qa[name] = (oq.pack_int4(q), s)
    ops = 0
    for name, l in lin.items():
        ap, asc = qa[l.input]
        wp, wsc = wq[name]
        og.w4a4_gemm(ap, asc, wp, wsc)
        ops += 2 * t_sample * n_s * l.k
    for _ in range(2):  # K and V
        cq = np.zeros((1, 8, t_sample, 64), np.uint8)
        cm = np.zeros((1, 8, t_sample, 1, 2), np.float16)
        okv.kv_rotate_quant_cache(kx, wl.signs(5, 128), True, 128, 0.95, cq, cm, 0)
    dt = time.perf_counter() - t0
    try:
        blas = np.show_config(mode="dicts").get("Build Dependencies", {}).get("blas", {}).get("name")
    except Exception:  # noqa: BLE001
        blas = None
    try:  # the BLAS library numpy actually loaded, and its thread count
        from threadpoolctl import threadpool_info
        pools = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        blas_threads = max((p.get("num_threads", 0) for p in pools), default=None)
        if pools:
            blas = f"{pools[0].get('internal_api')} {pools[0].get('version')}"
    except Exception:  # noqa: BLE001
        blas_threads = None
    return {
        "value": round(ops / dt / 1e12, 6), "unit": "TOPS", "cores": blas_threads or cores,
        "kind": "oracle",
        "sample": f"{t_sample} tokens x first {n_s} output channels of each of the 5 GEMMs "
                  f"(full K), their 4 " + ("input quantizers (RMSNorm, Hadamard heads, online "
                                           "Hadamard)" if quarot else "fused rotate+quant inputs")
                  + f", K/V of {t_sample} tokens x 8 heads; float64 oracle, {dt:.2f} s",
        "seconds": round(dt, 3), "cpu": cpu_model(), "blas": blas, "blas_threads": blas_threads,
        "cores_available": cores,
    }


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


if __name__ == "__main__":
    sys.exit(main())
