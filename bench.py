"""Benchmark of the QuaRot online-rotation + INT4 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 70b_prefill|7b_prefill]
                    [--no-cpu-baseline]

One step is one pass of the whole hot path over one batch of synthetic input
(inputs already resident in HBM, weights prepared offline and not timed):
  * fused Hadamard rotation + per-token INT4 quantization of the four GEMM
    inputs of a Llama-2 block (attention input, attention output, FFN input --
    shared by gate and up -- and the down-projection input, d = K of its GEMM);
  * the five W4A4 GEMMs (QKV, O, gate, up, down) with the scale epilogue;
  * head-wise Hadamard + asymmetric 4-bit group-128 quantization of K and V
    into the packed cache (Init of the whole prompt), and the rotation of Q.
Prints one JSON line (rank 0).  ``value`` is the whole step's throughput in
TOPS (GEMM int ops per step / step time).  The ``roofline`` object is for the
dominant kernel (the W4A4 GEMM); ``roofline_hadamard_quant`` is the same for the
fused rotation + quantization kernel against the HBM roofline.  The
``cpu_baseline`` is the oracle timed on the host on a bounded sample.
"""
from __future__ import annotations

import argparse
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="70b_prefill", choices=["70b_prefill", "7b_prefill"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=2048)
    return ap.parse_args()


def hq_bytes(T, d):
    """Algorithmic HBM bytes of one fused rotate+quant launch: read fp16 x, write
    packed codes and the fp16 scale (signs are cache resident)."""
    return T * (2 * d + d // 2 + 2)


def gemm_ops(T, N, K):
    return 2 * T * N * K


def gemm_bytes(T, N, K):
    return T * K // 2 + N * K // 2 + 2 * T + 2 * N + 2 * T * N


def kv_bytes(rows, dh, group):
    return rows * (2 * dh + dh // 2 + 4 * (dh // group))


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU only; run with --gpus 1",
                          "n_gpus": args.gpus}))
        return 2
    import numpy as np
    import torch

    import hadamard_rotation_int4_amd as qr
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    W = wl.WORKLOADS[args.workload]
    T = W.tokens[0]
    H = W.hidden
    lin = {l.name: l for l in W.linears}
    ffn = lin["down"].k
    wid = W.wid
    print(f"[bench] workload {W.name}: T={T} hidden={H} ffn={ffn}", file=sys.stderr, flush=True)

    # ---- inputs resident in HBM ----
    inputs = {}
    for i, name in enumerate(("attn_in", "o_in", "ffn_in", "down_in")):
        d = ffn if name == "down_in" else H
        inputs[name] = wl.activations_torch(torch, dev, wid, 10 + i, T, d, W.n_outliers,
                                            W.outlier_lo, W.outlier_hi)
    signs = {d: torch.from_numpy(wl.signs(wid, d)).to(dev) for d in (H, ffn)}
    # ---- weights: random init, rotated by the same R_K and quantized per output channel
    #      with the library's own kernel (offline preparation, not timed) ----
    wq = {}
    for i, (name, l) in enumerate(lin.items()):
        w = wl.weights_torch(torch, dev, wid, 1 + i, l.n, l.k)
        wq[name] = qr.hadamard_quant(w, signs[l.k], 1.0)
        del w
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
    # ---- outputs ----
    qbuf = {name: (torch.empty((T, t.shape[1] // 2), dtype=torch.uint8, device=dev),
                   torch.empty((T,), dtype=torch.float16, device=dev))
            for name, t in inputs.items()}
    ybuf = {name: torch.empty((T, l.n), dtype=torch.float16, device=dev) for name, l in lin.items()}
    qout = torch.empty((T * Hq, Dh), dtype=torch.float16, device=dev)
    torch.cuda.synchronize()

    # ---- one step, each launch bracketed by events (same stream as the kernels) ----
    launches = []   # (kernel, label, algorithmic bytes, ops)
    for name, x in inputs.items():
        launches.append(("hadamard_quant", name, hq_bytes(T, x.shape[1]), 0))
    for name, l in lin.items():
        launches.append(("w4a4_gemm", name, gemm_bytes(T, l.n, l.k), gemm_ops(T, l.n, l.k)))
    launches.append(("kv_rotate_quant", "k", kv_bytes(T * Hkv, Dh, G), 0))
    launches.append(("kv_rotate_quant", "v", kv_bytes(T * Hkv, Dh, G), 0))
    launches.append(("hadamard", "q", T * Hq * Dh * 4, 0))

    def run_launch(i):
        kern, label = launches[i][0], launches[i][1]
        if kern == "hadamard_quant":
            x = inputs[label]
            qr.hadamard_quant(x, signs[x.shape[1]], 1.0, out=qbuf[label])
        elif kern == "w4a4_gemm":
            src = lin[label].input
            qa, sa = qbuf[src]
            qw, sw = wq[label]
            qr.w4a4_gemm(qa, sa, qw, sw, out=ybuf[label])
        elif kern == "kv_rotate_quant":
            x = k_in if label == "k" else v_in
            cq, cm = cache[label]
            qr.kv_rotate_quant(x, kv_signs if label == "k" else None, G, 0.95, cq, cm, 0,
                               rotate=(label == "k"))

    # the Q rotation writes into a preallocated output through the C entry point
    def run_q():
        code = qr._load().qr_hadamard(qr._ptr(q_in), q_in.shape[0], Dh, Dh, qr._ptr(kv_signs),
                                      qr._ptr(qout), 0, qr._stream(None))
        qr._check(code, "qr_hadamard")

    def step(events=None):
        for i in range(len(launches)):
            if events is not None:
                events[i][0].record()
            if launches[i][0] == "hadamard":
                run_q()
            else:
                run_launch(i)
            if events is not None:
                events[i][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in launches] for _ in range(K)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for k in range(K):
        step(ev[k])
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t0.elapsed_time(t1)
    ms_step = ms_total / K

    per = {}
    for i, (kern, label, nbytes, ops) in enumerate(launches):
        ms = sum(ev[k][i][0].elapsed_time(ev[k][i][1]) for k in range(K)) / K
        per[f"{kern}:{label}"] = dict(kernel=kern, ms=ms, bytes=nbytes, ops=ops,
                                      gbs=nbytes / ms / 1e6, tops=ops / ms / 1e9)
    total_ops = sum(l[3] for l in launches)
    value = total_ops / (ms_step * 1e-3) / 1e12

    gemm = [v for v in per.values() if v["kernel"] == "w4a4_gemm"]
    g_ms = sum(v["ms"] for v in gemm)
    g_ops = sum(v["ops"] for v in gemm)
    g_tops = g_ops / (g_ms * 1e-3) / 1e12
    hqk = [v for v in per.values() if v["kernel"] == "hadamard_quant"]
    h_ms = sum(v["ms"] for v in hqk)
    h_bytes = sum(v["bytes"] for v in hqk)
    h_gbs = h_bytes / (h_ms * 1e-3) / 1e9

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": f"{W.name}: T={T} tokens, hidden {H}, FFN {ffn}, QKV {lin['qkv'].n}; "
                        f"4 fused rotate+quant, 5 W4A4 GEMMs, K/V init into a 4-bit cache "
                        f"({B}x{S}x{Hkv}x{Dh}, group {G}), Q rotation ({Hq} heads)",
            "tokens": T, "hidden": H, "ffn": ffn,
        },
        "roofline": {
            "bound": "mfma", "kernel": "qr_w4a4_gemm (all five launches of a step)",
            "achieved": round(g_tops, 1), "peak": INT8_PEAK_TOPS, "unit": "TFLOP/s",
            "op_note": "int8 MFMA operations (2 per multiply-accumulate), dense peak 5.0 POP/s",
            "frac": round(g_tops / INT8_PEAK_TOPS, 4), "traffic": None,
        },
        "roofline_hadamard_quant": {
            "bound": "hbm", "kernel": "qr_hadamard_quant (four launches of a step)",
            "achieved": round(h_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(h_gbs / HBM_PEAK_GBS, 4), "traffic": None,
        },
        "kernels": {k: {"ms": round(v["ms"], 4), "GB/s": round(v["gbs"], 1),
                        "TOPS": round(v["tops"], 1)} for k, v in per.items()},
        "wall_s_timed": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(W, args.cpu_sample_tokens)
    print(json.dumps(out), flush=True)
    return 0


def cpu_baseline(W, t_sample):
    """Time the oracle (float64 rotation + quantization, exact GEMM via float64
    BLAS on the codes, KV quantization) on a bounded sample of the step:
    t_sample tokens against the first 1024 output channels of each GEMM.
    Reported as TOPS over the same GEMM operations (2 per MAC)."""
    import numpy as np

    import workloads as wl
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
        import numpy as _np
        blas = _np.show_config(mode="dicts").get("Build Dependencies", {}).get("blas", {}).get("name")
    except Exception:  # noqa: BLE001
        blas = None
    return {
        "value": round(ops / dt / 1e12, 6), "unit": "TOPS", "cores": cores, "kind": "oracle",
        "sample": f"{t_sample} tokens x first {n_s} output channels of each of the 5 GEMMs "
                  f"(full K), their 4 fused rotate+quant inputs, K/V of {t_sample} tokens x 8 heads; "
                  f"float64 oracle, {dt:.2f} s",
        "seconds": round(dt, 3), "cpu": platform.processor() or platform.machine(), "blas": blas,
    }


if __name__ == "__main__":
    sys.exit(main())
