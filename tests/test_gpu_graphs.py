"""Every entry point captured in one HIP graph: each replay, with eager work and
synchronizations between replays, reproduces the eager results bit for bit
(the library allocates, frees and clears nothing inside a call, so its
launches are capture-safe)."""
import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
qr = pytest.importorskip("hadamard_rotation_int4_amd")


def test_all_entry_points_replay_in_a_graph():
    dev = torch.device("cuda")
    T, d, N, ffn = 64, 4096, 512, 11008
    x = wl.activations_torch(torch, dev, 60, 0, T, d)
    xd = wl.activations_torch(torch, dev, 60, 1, T, ffn)
    w = wl.weights_torch(torch, dev, 60, 2, N, d)
    s = torch.from_numpy(wl.signs(60, d)).to(dev)
    sd = torch.from_numpy(wl.signs(60, ffn)).to(dev)
    B, H, Hq, Dh, S = 2, 2, 8, 128, 300
    kv = wl.kv_tensor_torch(torch, dev, 60, 3, B, S, H, Dh)
    ks = torch.from_numpy(wl.signs(60, Dh)).to(dev)
    qd = wl.activations_torch(torch, dev, 60, 4, B * Hq, Dh, 0)
    # weights prepared once (outside the graph)
    wq, wsc = qr.hadamard_quant(w, s, 1.0)
    w8, ws8 = qr.hadamard_quant_i8(w, s, 1.0, 8)
    cq = torch.zeros((B, H, S, Dh // 2), dtype=torch.uint8, device=dev)
    cm = torch.zeros((B, H, S, 1, 2), dtype=torch.float16, device=dev)
    vq, vm = torch.zeros_like(cq), torch.zeros_like(cm)
    ws = torch.empty((qr.kv_decode_workspace_bytes(B, Hq, H, Dh, S),), dtype=torch.uint8,
                     device=dev)
    outs = {
        "hq": (torch.empty((T, d // 2), dtype=torch.uint8, device=dev),
               torch.empty((T,), dtype=torch.float16, device=dev)),
        "hq_down": (torch.empty((T, ffn // 2), dtype=torch.uint8, device=dev),
                    torch.empty((T,), dtype=torch.float16, device=dev)),
        "rms": (torch.empty((T, d // 2), dtype=torch.uint8, device=dev),
                torch.empty((T,), dtype=torch.float16, device=dev)),
        "heads": (torch.empty((T, d // 2), dtype=torch.uint8, device=dev),
                  torch.empty((T,), dtype=torch.float16, device=dev)),
        "q8": (torch.empty((T, d), dtype=torch.int8, device=dev),
               torch.empty((T,), dtype=torch.float16, device=dev)),
        "rms8": (torch.empty((T, d), dtype=torch.int8, device=dev),
                 torch.empty((T,), dtype=torch.float16, device=dev)),
        "heads8": (torch.empty((T, d), dtype=torch.int8, device=dev),
                   torch.empty((T,), dtype=torch.float16, device=dev)),
        "y": torch.empty((T, N), dtype=torch.float16, device=dev),
        "y8": torch.empty((T, N), dtype=torch.float16, device=dev),
        "qrot": torch.empty((B * Hq, Dh), dtype=torch.float16, device=dev),
        "att": torch.empty((B, Hq, Dh), dtype=torch.float16, device=dev),
    }

    def step():
        qr.hadamard_quant(x, s, 1.0, out=outs["hq"])
        qr.hadamard_quant(xd, sd, 1.0, out=outs["hq_down"])
        qr.rmsnorm_quant(x, 1e-5, 1.0, out=outs["rms"])
        qr.hadamard_heads_quant(x, 32, 1.0, out=outs["heads"])
        qr.hadamard_quant_i8(x, s, 1.0, 8, out=outs["q8"])
        qr.rmsnorm_quant_i8(x, 1e-5, 1.0, 6, out=outs["rms8"])
        qr.hadamard_heads_quant_i8(x, 32, 1.0, 8, out=outs["heads8"])
        qr.w4a4_gemm(*outs["hq"], wq, wsc, out=outs["y"])
        qr.w8a8_gemm(*outs["q8"], w8, ws8, out=outs["y8"])
        qr.kv_rotate_quant(kv, ks, 128, 0.95, cq, cm, 0)
        qr.kv_rotate_quant(kv, None, 128, 0.95, vq, vm, 0, rotate=False, bits=3)
        qr.hadamard(qd, ks, torch.float16, out=outs["qrot"])
        qr.kv_decode_attention(outs["qrot"].view(B, Hq, Dh), cq, cm, vq, vm, S, 128,
                               1.0 / np.sqrt(Dh), out=outs["att"], workspace=ws)

    def snapshot():
        flat = []
        for v in outs.values():
            flat += list(v) if isinstance(v, tuple) else [v]
        return [t.clone() for t in flat + [cq, cm, vq, vm]]

    step()
    torch.cuda.synchronize()
    eager = snapshot()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        # eager work between replays: scribble over every output first
        for v in outs.values():
            for t in (v if isinstance(v, tuple) else (v,)):
                t.view(torch.uint8).fill_(0x5A)
        for t in (cq, cm, vq, vm):
            t.view(torch.uint8).fill_(0x33)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for i, (a, b) in enumerate(zip(eager, got)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep}, output {i}"


def test_threads_and_streams_in_parallel():
    # the entry points keep no global state: four host threads, each on its own
    # stream and buffers, get the same results as one thread running them in turn
    import threading
    dev = torch.device("cuda")
    T, d, N = 96, 8192, 768
    jobs = []
    for i in range(4):
        x = wl.activations_torch(torch, dev, 61, i, T, d)
        w = wl.weights_torch(torch, dev, 61, 10 + i, N, d)
        s = torch.from_numpy(wl.signs(61, d)).to(dev)
        jobs.append((x, w, s))

    def run(job, stream):
        x, w, s = job
        with torch.cuda.stream(stream):
            qw, sw = qr.hadamard_quant(w, s, 1.0)
            qa, sa = qr.rmsnorm_quant(x, 1e-5, 1.0)
            y = qr.w4a4_gemm(qa, sa, qw, sw)
            q8, s8 = qr.hadamard_heads_quant_i8(x, 64, 1.0, 8)
            w8, ws8 = qr.hadamard_quant_i8(w, s, 1.0, 8)
            y8 = qr.w8a8_gemm(q8, s8, w8, ws8)
        stream.synchronize()
        return y, y8

    ref = [run(j, torch.cuda.current_stream()) for j in jobs]
    results = [None] * len(jobs)
    streams = [torch.cuda.Stream() for _ in jobs]

    def worker(i):
        for _ in range(3):
            results[i] = run(jobs[i], streams[i])

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    for (y, y8), (ry, ry8) in zip(results, ref):
        assert torch.equal(y.view(torch.int16), ry.view(torch.int16))
        assert torch.equal(y8.view(torch.int16), ry8.view(torch.int16))
