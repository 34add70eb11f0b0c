#!/usr/bin/env python3
"""Benchmark of the VQ MoE expert matmul on one MI355X.

A step is one pass of the routed SwiGLU expert FFN (``vq_moe_ffn``: route
grouping, codebook staging, code unpacking, lookup-and-scale, the fused
dot products, SwiGLU, the down projection and the gate-weighted combine)
over one batch of synthetic input.  The default workload is the decode step
of a 128-expert, top-8 layer (hidden 2048, expert inter 768) with every
projection at d=4/K=512 (9-bit codes), one token per step.

Inputs are resident in HBM before timing starts.  Each step uses fresh
routes and activations, and steps rotate over several copies of the layer at
distinct addresses so the weights come from HBM, not from the 256 MB
Infinity Cache.  The K timed steps are captured once in a HIP graph and
replayed (the launches are the only thing a graph removes; every kernel runs).
``value`` is algorithmic bytes / wall time: the routed experts' packed codes,
scales and row maps, the codebooks, activations, outputs, ids and weights.

The JSON line also carries ``roofline`` for the dominant kernel (the fused
gate+up+SwiGLU launch, timed per launch with HIP events on its stream) and
``cpu_baseline`` (the CPU oracle timed on a bounded sample of the same
workload on the host's cores).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "VQ MoE expert GB/s (decode, % HBM peak) and TFLOP/s (prefill, % MFMA peak)"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA
MALL_BYTES = 256 << 20
DEFAULT_WORKLOAD = "moe_decode_e128_h2048_i768_d4k512_b1"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--layers", type=int, default=0, help="layer copies (0 = auto)")
    p.add_argument("--no-graph", action="store_true", help="time eager launches")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle baseline sample (0 = skip)")
    p.add_argument("--kernel-launches", type=int, default=100,
                   help="launches of the dominant kernel timed with HIP events")
    return p.parse_args()


def expert_bytes(T, e: int) -> int:
    """Stored bytes of one expert of one projection (codes, scales, row map)."""
    rows = T.expert_stored_rows(e)
    b = rows * (T.wpr * 4 + T.groups * 2)
    if T.row_map is not None:
        b += T.rows * 4
    return b


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported "
              "(the path is single-GPU; expert-parallel sharding is a design note only)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import vq_dequant_matmul_amd as vq

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    vq.load_library()

    wl = synth.WORKLOADS[args.workload]
    if wl.n_tok > 16:
        print(f"{args.workload}: prefill workloads are timed by the grouped-GEMM path",
              file=sys.stderr)
        sys.exit(2)
    K, W = args.steps, args.warmup
    n_steps = K + W

    # ---- layer, copies, per-step inputs (all resident before timing) ---------------
    t0 = time.perf_counter()
    gate_h, up_h, down_h = synth.make_moe_layer(wl)
    layer_bytes = sum(t.stored_bytes() for t in (gate_h, up_h, down_h))
    L = args.layers or max(2, math.ceil(4 * MALL_BYTES / layer_bytes))
    base = [vq.VQTensor.from_host(t) for t in (gate_h, up_h, down_h)]
    layers = [base] + [[t.clone() for t in base] for _ in range(L - 1)]
    xs, ids, ws = [], [], []
    for i in range(n_steps):
        x, r, w = synth.make_moe_inputs(wl, i)
        xs.append(x)
        ids.append(r)
        ws.append(w)
    x_dev = torch.from_numpy(np.stack(xs).view(np.int16)).view(torch.bfloat16).cuda()
    ids_dev = torch.from_numpy(np.stack(ids)).cuda()
    w_dev = torch.from_numpy(np.stack(ws)).cuda()
    y = torch.empty((wl.n_tok, wl.hidden), dtype=torch.float32, device="cuda")
    ws_bytes = vq.vq_moe_ffn_workspace_size(*base, wl.n_tok, wl.top_k)
    workspace = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    log(f"[bench] {args.workload}: {L} layer copies x {layer_bytes / 1e6:.1f} MB, "
        f"{n_steps} step inputs, setup {time.perf_counter() - t0:.1f}s")

    cb_bytes = sum(t.K * t.d * 2 for t in (gate_h, up_h, down_h))
    io_bytes = wl.n_tok * wl.hidden * (2 + 4) + wl.n_tok * wl.top_k * 8

    def step_bytes(i):
        uniq = np.unique(ids[i])
        return int(sum(expert_bytes(t, int(e)) for e in uniq for t in (gate_h, up_h, down_h))
                   + cb_bytes + io_bytes)

    def gate_up_bytes(i):
        uniq = np.unique(ids[i])
        return int(sum(expert_bytes(t, int(e)) for e in uniq for t in (gate_h, up_h))
                   + gate_h.K * gate_h.d * 2 + up_h.K * up_h.d * 2
                   + wl.n_tok * wl.hidden * 2 + wl.n_tok * wl.top_k * (4 + 4 * wl.inter))

    def step(i):
        G, U, D = layers[i % L]
        vq.vq_moe_ffn(G, U, D, x_dev[i], ids_dev[i], w_dev[i], out=y, workspace=workspace)

    # ---- warmup (eager: loads the kernels) -------------------------------------------
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    log(f"[bench] warmup {W} steps done")

    use_graph = not args.no_graph
    graph = None
    if use_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(W, n_steps):
                step(i)
        torch.cuda.synchronize()

    # ---- timed region: exactly K steps -----------------------------------------------
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    if use_graph:
        graph.replay()
    else:
        for i in range(W, n_steps):
            step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    log(f"[bench] timed {K} steps in {elapsed * 1e3:.2f} ms")

    # the graph's last step must equal an eager run of the same step, bit for bit
    y_graph = y.clone()
    step(n_steps - 1)
    torch.cuda.synchronize()
    graph_check = bool(torch.equal(y_graph.view(torch.int32), y.view(torch.int32)))
    if not graph_check:
        log("[bench] WARNING: graph replay differs from eager")

    total_bytes = sum(step_bytes(i) for i in range(W, n_steps))
    value = total_bytes / elapsed / 1e9
    ms_per_step = elapsed * 1e3 / K

    # ---- dominant kernel: fused gate+up+SwiGLU, per-launch HIP events -------------------
    n_k = max(1, args.kernel_launches)
    h_buf = torch.empty((wl.n_tok * wl.top_k, wl.inter), dtype=torch.float32, device="cuda")
    backlog = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_k)]
    torch.cuda.synchronize()
    for _ in range(48):           # keep the GPU busy while the launches are queued
        backlog.fill_(1.0)
    for j in range(n_k):
        i = W + (j % K)
        G, U, _ = layers[i % L]
        evs[j][0].record()
        vq.vq_moe_gate_up(G, U, x_dev[i], ids_dev[i], out=h_buf)
        evs[j][1].record()
    torch.cuda.synchronize()
    durs = np.array([a.elapsed_time(b) * 1e-3 for a, b in evs])       # seconds
    kbytes = np.array([gate_up_bytes(W + (j % K)) for j in range(n_k)])
    k_mean = float(durs.mean())
    achieved = float(kbytes.mean() / k_mean / 1e9)
    del backlog
    roofline = {
        "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
        "kernel": "vq::k_rows (gate+up+SwiGLU, fused)",
        "launch_us": round(k_mean * 1e6, 2), "bytes_per_launch": int(kbytes.mean()),
    }
    log(f"[bench] dominant kernel: {k_mean * 1e6:.2f} us/launch, {achieved:.0f} GB/s")

    # ---- CPU oracle on a bounded sample ------------------------------------------------
    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        oracle.build(force=False)
        cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        t_cpu, n_cpu, b_cpu = 0.0, 0, 0
        while t_cpu < args.cpu_seconds and n_cpu < n_steps:
            i = W + n_cpu % K
            c0 = time.perf_counter()
            oracle.moe_ffn(gate_h, up_h, down_h, xs[i], ids[i], ws[i])
            t_cpu += time.perf_counter() - c0
            b_cpu += step_bytes(i)
            n_cpu += 1
        cpu = {"value": round(b_cpu / t_cpu / 1e9, 4), "unit": "GB/s", "cores": cores,
               "kind": "oracle",
               "sample": f"{n_cpu} decode steps of the same workload ({wl.n_tok} token, "
                         f"{wl.top_k} routed experts each), {t_cpu:.1f}s"}
        log(f"[bench] cpu oracle: {n_cpu} steps in {t_cpu:.1f}s")

    rec = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16xf16->f32",
        "data": "synthetic",
        "config": {
            "workload": args.workload, "experts": wl.n_experts, "top_k": wl.top_k,
            "hidden": wl.hidden, "inter": wl.inter, "d": wl.d, "bits": wl.bits,
            "K": 1 << wl.bits, "tokens": wl.n_tok, "layer_copies": L,
            "hip_graph": use_graph, "graph_replay_bit_equal": graph_check,
            "hbm_frac": round(value / HBM_PEAK_GBS, 4),
            "bytes_per_step": int(total_bytes / K),
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
