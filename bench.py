#!/usr/bin/env python3
"""Benchmark of the VQ MoE expert matmul on one MI355X.

A step is one pass of the routed SwiGLU expert FFN (``vq_moe_ffn``: route
grouping, codebook staging, code unpacking, lookup-and-scale, the fused dot
products or MFMA tiles, SwiGLU, the down projection and the gate-weighted
combine) over one batch of synthetic input.  The default workload is the
largest one: prefill of 4096 tokens through a 512-expert, top-10 layer
(hidden 4096, expert inter 1024) with every projection at d=2/K=256 (8-bit
codes) and 12.43 % of the rows skip-zero; ``--workload`` selects the other
seeded layers (decode of 1 token on a 128-expert top-8 layer at d=4/K=512,
decode batches of 1 and 8 tokens on the 512-expert layer, prefill of 2048
tokens on a 128-expert layer at d=4/K=2048).

Inputs are resident in HBM before timing starts.  Each step uses fresh
routes and activations, and steps rotate over enough copies of the layer at
distinct addresses that a copy is used again only after four times the
256 MB Infinity Cache of other steps' bytes, so the weights come from HBM.
The K timed steps are captured once in a HIP graph and replayed (a graph
removes launch overhead only; every kernel runs).

Decode workloads report GB/s of algorithmic bytes (the routed experts'
packed codes, scales and row maps, the codebooks, activations, outputs, ids
and weights) against the 8 TB/s HBM peak; prefill workloads report TFLOP/s
of algorithmic flops (2 x live weight rows x columns per routed pair, over
the three projections) against the 2.5 PFLOP/s dense fp16 MFMA peak.

``roofline`` times the dominant kernel (the fused gate+up launch) per
launch with HIP events recorded on its own stream; ``cpu_baseline`` times
the CPU oracle on a bounded sample of the same workload on the host cores.

Three more workload families share the JSON line's format: ``moe_stack*``
(one token through a stack of 40 or 42 MoE layers with promoted layers,
``vq_moe_stack``), ``ple_gather*`` (rows of stacked VQ embedding tables,
``vq_row_gather``) and ``fit*`` (fitting the format to one projection's
bf16 weights, ``vq_fit``, reported in TFLOP/s of nearest-entry searches
against the fp32 vector peak).  ``--gpus`` above 1 is refused: the path
runs on one GPU.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "VQ MoE expert GB/s (decode, % HBM peak) and TFLOP/s (prefill, % MFMA peak)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA
MALL_BYTES = 256 << 20
MAX_COPY_BYTES = 120 << 30     # device memory spent on layer copies at most
DEFAULT_WORKLOAD = "moe_prefill_e512_h4096_i1024_d2k256_t4096_sz"
CSRC = os.path.join(ROOT, "vq_dequant_matmul_amd", "csrc")
TRAFFIC = os.path.join(ROOT, "profiles", "hbm_traffic.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None, help="timed steps (default 200 decode, 20 prefill)")
    p.add_argument("--warmup", type=int, default=None, help="untimed steps (default 20 / 3)")
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--layers", type=int, default=0, help="layer copies (0 = auto)")
    p.add_argument("--no-graph", action="store_true", help="time eager launches")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle baseline sample (0 = skip)")
    p.add_argument("--kernel-launches", type=int, default=None,
                   help="launches of the dominant kernel timed with HIP events")
    return p.parse_args()


class HipEvents:
    """hipEventCreate / hipEventElapsedTime through the HIP runtime."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self):
        ev = ctypes.c_void_p()
        rc = self.hip.hipEventCreate(ctypes.byref(ev))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return ev

    def record(self, ev, stream):
        rc = self.hip.hipEventRecord(ev, stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def destroy(self, ev):
        self.hip.hipEventDestroy(ev)


def kernel_source_hash(family: str) -> str:
    """Hash of the device sources that build one kernel family ("decode",
    "prefill", "gather": its own files and the shared device header);
    recorded counter traffic is valid only for that hash."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.startswith("vq_" + family) or name == "vq_common.hpp":
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, family: str):
    """HBM bytes per launch of the dominant kernel from the recorded
    rocprofv3 FETCH_SIZE / WRITE_SIZE passes (each scaled by what the counter
    reads for a device copy of known size), or None when no record matches the
    current kernel sources.  Record lines: workload, source hash, bytes per
    launch, then free text."""
    try:
        with open(TRAFFIC) as f:
            lines = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    except OSError:
        return None
    for ln in lines:
        if ln[0] == workload and ln[1] == kernel_source_hash(family):
            return int(ln[2])
    return None


def cpu_model() -> str:
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def oracle_baseline(run, budget_s: float, max_samples: int, scale: float, unit: str,
                    digits: int, what: str):
    """Time the CPU oracle on samples run(j) (each returns its algorithmic
    work) at all of the oracle's OpenMP threads until budget_s is spent, then
    the same samples again at one thread (at most a third of the budget).
    Returns the cpu_baseline record."""
    import oracle
    oracle.build(force=False)
    cores = oracle.threads()
    t_all, n, work = 0.0, 0, 0
    while t_all < budget_s and n < max_samples:
        c0 = time.perf_counter()
        w = run(n)
        t_all += time.perf_counter() - c0
        work += w
        n += 1
    oracle.set_threads(1)
    try:
        t_one, n1, work1 = 0.0, 0, 0
        while n1 < n and (n1 == 0 or t_one < budget_s / 3):
            c0 = time.perf_counter()
            w = run(n1)
            t_one += time.perf_counter() - c0
            work1 += w
            n1 += 1
    finally:
        oracle.set_threads(cores)
    log(f"[bench] cpu oracle: {n} samples in {t_all:.1f}s at {cores} threads, "
        f"{n1} in {t_one:.1f}s at 1 thread")
    return {"value": round(work / t_all / scale, digits), "unit": unit, "cores": cores,
            "kind": "oracle", "sample": f"{n} x {what}, {t_all:.1f}s",
            "cpu_model": cpu_model(),
            "one_thread": {"value": round(work1 / t_one / scale, digits), "unit": unit,
                           "cores": 1, "sample": f"{n1} x {what}, {t_one:.1f}s"}}


def launch_stats(durs) -> dict:
    """Mean, p10, p50 and p90 of per-launch durations (seconds) in us."""
    import numpy as np
    d = np.asarray(durs) * 1e6
    return {"mean": round(float(d.mean()), 2), "p10": round(float(np.percentile(d, 10)), 2),
            "p50": round(float(np.percentile(d, 50)), 2),
            "p90": round(float(np.percentile(d, 90)), 2), "n": int(d.size)}


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

    if args.workload in CEILINGS:
        return bench_ceiling(args)
    if args.workload in synth.GATHER_WORKLOADS:
        return bench_gather(args, synth.GATHER_WORKLOADS[args.workload])
    if args.workload in synth.STACK_WORKLOADS:
        return bench_stack(args, synth.STACK_WORKLOADS[args.workload])
    if args.workload in synth.FIT_WORKLOADS:
        return bench_fit(args, synth.FIT_WORKLOADS[args.workload])
    wl = synth.WORKLOADS[args.workload]

    # ---- layer, copies, per-step inputs (all resident before timing) ---------------
    # n_steps inputs for the timed steps, then n_k more for the dominant
    # kernel's timing loop (every launch there has its own routes too)
    t0 = time.perf_counter()
    gate_h, up_h, down_h = synth.make_moe_layer(wl)
    base = [vq.VQTensor.from_host(t) for t in (gate_h, up_h, down_h)]
    # the engine the library runs for this batch decides the metric
    prefill = vq.vq_moe_ffn_engine(*base, wl.n_tok, wl.top_k) == vq.VQ_ENGINE_MFMA
    family = "prefill" if prefill else "decode"
    K = args.steps if args.steps is not None else (20 if prefill else 200)
    W = args.warmup if args.warmup is not None else (3 if prefill else 20)
    n_k = args.kernel_launches if args.kernel_launches is not None else (10 if prefill else 100)
    n_steps = K + W
    layer_bytes = sum(t.stored_bytes() for t in (gate_h, up_h, down_h))
    xs, ids, ws = [], [], []
    for i in range(n_steps + n_k):
        x, r, w = synth.make_moe_inputs(wl, i)
        xs.append(x)
        ids.append(r)
        ws.append(w)

    # ---- algorithmic work -------------------------------------------------------------
    cb_bytes = sum(t.K * t.d * 2 for t in (gate_h, up_h, down_h))
    io_bytes = wl.n_tok * wl.hidden * (2 + 4) + wl.n_tok * wl.top_k * 8
    live = {id(t): np.array([t.expert_stored_rows(e) for e in range(wl.n_experts)])
            for t in (gate_h, up_h, down_h)}
    ebytes = {id(t): np.array([expert_bytes(t, e) for e in range(wl.n_experts)], dtype=np.int64)
              for t in (gate_h, up_h, down_h)}

    def step_bytes(i):
        uniq = np.unique(ids[i])
        return int(sum(ebytes[id(t)][uniq].sum() for t in (gate_h, up_h, down_h))
                   + cb_bytes + io_bytes)

    def gate_up_bytes(i):
        uniq = np.unique(ids[i])
        return int(sum(ebytes[id(t)][uniq].sum() for t in (gate_h, up_h))
                   + gate_h.K * gate_h.d * 2 + up_h.K * up_h.d * 2
                   + wl.n_tok * wl.hidden * 2 + wl.n_tok * wl.top_k * (4 + 4 * wl.inter))

    def gate_up_flops(i):
        r = ids[i].ravel()
        return int(2 * wl.hidden * (live[id(gate_h)][r].sum() + live[id(up_h)][r].sum()))

    def step_flops(i):
        r = ids[i].ravel()
        return gate_up_flops(i) + int(2 * wl.inter * live[id(down_h)][r].sum())

    # Layer copies: step i uses copy i % L, so a copy (and every byte of it)
    # is touched again only after L - 1 other steps; L makes those steps'
    # bytes at least four times the Infinity Cache (the smallest step counts).
    min_step = min(step_bytes(i) for i in range(n_steps + n_k))
    L = args.layers or max(2, math.ceil(4 * MALL_BYTES / layer_bytes),
                           1 + math.ceil(4 * MALL_BYTES / min_step))
    if not args.layers and L * layer_bytes > MAX_COPY_BYTES:
        L = max(2, MAX_COPY_BYTES // layer_bytes)
        log(f"[bench] WARNING: layer copies capped at {L} ({L * layer_bytes / 1e9:.1f} GB)")
    layers = [base] + [[t.clone() for t in base] for _ in range(L - 1)]
    x_dev = torch.from_numpy(np.stack(xs).view(np.int16)).view(torch.bfloat16).cuda()
    ids_dev = torch.from_numpy(np.stack(ids)).cuda()
    w_dev = torch.from_numpy(np.stack(ws)).cuda()
    y = torch.empty((wl.n_tok, wl.hidden), dtype=torch.float32, device="cuda")
    ws_bytes = vq.vq_moe_ffn_workspace_size(*base, wl.n_tok, wl.top_k)
    workspace = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    log(f"[bench] {args.workload}: {L} layer copies x {layer_bytes / 1e6:.1f} MB, "
        f"{n_steps} + {n_k} step inputs (smallest step {min_step / 1e6:.1f} MB), "
        f"workspace {ws_bytes / 1e6:.1f} MB, setup {time.perf_counter() - t0:.1f}s")

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

    if prefill:
        total = sum(step_flops(i) for i in range(W, n_steps))
        value, unit = total / elapsed / 1e12, "TFLOP/s"
        frac = value / MFMA_F16_PEAK_TFLOPS
    else:
        total = sum(step_bytes(i) for i in range(W, n_steps))
        value, unit = total / elapsed / 1e9, "GB/s"
        frac = value / HBM_PEAK_GBS
    ms_per_step = elapsed * 1e3 / K

    # ---- dominant kernel: fused gate+up launch, HIP events on its stream -------------
    # Launch j of the timing loop uses its own inputs (n_steps + j) and layer
    # copy (n_steps + j) % L.  A queue of 256 MiB device copies keeps the GPU
    # busy while the launches are queued, so the timed launches run back to
    # back; the copy is also the kernel of known size the HBM byte counters
    # are calibrated on.
    kidx = [n_steps + j for j in range(n_k)]
    hip = HipEvents()
    src = torch.ones(1 << 26, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()

    def queue_copies():
        for _ in range(48):
            dst.copy_(src)

    queue_copies()
    if prefill:
        # ~1 ms launches: an event pair around each one (the library records
        # them on its launch stream around the gate+up GEMM only)
        pairs = [(hip.create(), hip.create()) for _ in range(n_k)]
        for j, i in enumerate(kidx):
            vq.vq_set_kernel_events(pairs[j][0], pairs[j][1])
            step(i)
        vq.vq_set_kernel_events(None, None)
        torch.cuda.synchronize()
        durs = np.array([hip.elapsed_ms(a, b) * 1e-3 for a, b in pairs])     # seconds
        for a, b in pairs:
            hip.destroy(a)
            hip.destroy(b)
        k_mean = float(durs.mean())
        stats = launch_stats(durs)
        timing = f"HIP event pair around each of {n_k} launches"
    else:
        # ~10 us launches: per-launch event markers add a few us each, so
        # one event pair spans n_k back-to-back launches of the gate+up stage
        # alone for the mean; a second pass with a pair around each launch
        # gives the spread (p10/p50/p90 include the markers' cost)
        h = torch.empty((wl.n_tok * wl.top_k, wl.inter), dtype=torch.float32, device="cuda")
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

        def gate_up(i):
            G, U, _ = layers[i % L]
            vq.vq_moe_gate_up(G, U, x_dev[i], ids_dev[i], out=h)

        ev0, ev1 = hip.create(), hip.create()
        hip.record(ev0, stream)
        for i in kidx:
            gate_up(i)
        hip.record(ev1, stream)
        torch.cuda.synchronize()
        k_mean = hip.elapsed_ms(ev0, ev1) * 1e-3 / n_k
        hip.destroy(ev0)
        hip.destroy(ev1)
        queue_copies()
        pairs = [(hip.create(), hip.create()) for _ in range(n_k)]
        for j, i in enumerate(kidx):
            hip.record(pairs[j][0], stream)
            gate_up(i)
            hip.record(pairs[j][1], stream)
        torch.cuda.synchronize()
        durs = np.array([hip.elapsed_ms(a, b) * 1e-3 for a, b in pairs])
        for a, b in pairs:
            hip.destroy(a)
            hip.destroy(b)
        stats = launch_stats(durs)
        del h
        timing = (f"one HIP event pair around {n_k} back-to-back launches (mean); "
                  f"a pair around each launch for the percentiles")
    del src, dst
    if prefill:
        kwork = np.array([gate_up_flops(i) for i in kidx])
        achieved = float(kwork.mean() / k_mean / 1e12)
        roofline = {"bound": "mfma", "achieved": round(achieved, 1),
                    "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
                    "traffic": recorded_traffic(args.workload, family),
                    "kernel": "vq::k_gemm (gate+up grouped GEMM, SwiGLU epilogue)",
                    "launch_us": round(k_mean * 1e6, 2), "launch_us_stats": stats,
                    "flops_per_launch": int(kwork.mean()), "timing": timing}
    else:
        kwork = np.array([gate_up_bytes(i) for i in kidx])
        achieved = float(kwork.mean() / k_mean / 1e9)
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": recorded_traffic(args.workload, family),
                    "kernel": "vq::k_rows (gate+up+SwiGLU, fused)",
                    "launch_us": round(k_mean * 1e6, 2), "launch_us_stats": stats,
                    "bytes_per_launch": int(kwork.mean()), "timing": timing}
    log(f"[bench] dominant kernel: {k_mean * 1e6:.2f} us/launch "
        f"(p10 {stats['p10']}, p90 {stats['p90']}), {achieved:.1f} {roofline['unit']}")

    # ---- CPU oracle on a bounded sample ------------------------------------------------
    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        rng = np.random.default_rng(0)
        if prefill:
            # a few tokens of a step: each token's output is independent
            toks = [np.sort(rng.choice(wl.n_tok, size=2, replace=False)).astype(np.int32)
                    for _ in range(10 * n_steps)]

            def run(j):
                i = W + j % K
                oracle.moe_ffn(gate_h, up_h, down_h, xs[i], ids[i], ws[i], tokens=toks[j])
                r = ids[i][toks[j]].ravel()
                return int(2 * wl.hidden * (live[id(gate_h)][r].sum() + live[id(up_h)][r].sum())
                           + 2 * wl.inter * live[id(down_h)][r].sum())
            cpu = oracle_baseline(run, args.cpu_seconds, 10 * n_steps, 1e12, "TFLOP/s", 6,
                                  f"2 sampled tokens of a step ({wl.top_k} routed experts each)")
        else:
            def run(j):
                i = W + j % K
                oracle.moe_ffn(gate_h, up_h, down_h, xs[i], ids[i], ws[i])
                return step_bytes(i)
            cpu = oracle_baseline(run, args.cpu_seconds, 10 * n_steps, 1e9, "GB/s", 4,
                                  f"whole decode steps ({wl.n_tok} token(s), "
                                  f"{wl.top_k} routed experts each)")

    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16xf16->f32",
        "data": "synthetic",
        "config": {
            "workload": args.workload, "experts": wl.n_experts, "top_k": wl.top_k,
            "hidden": wl.hidden, "inter": wl.inter, "d": wl.d, "bits": wl.bits,
            "K": 1 << wl.bits, "tokens": wl.n_tok, "dead_row_fraction": wl.dead_frac,
            "engine": "mfma" if prefill else "decode", "layer_copies": L, "hip_graph": use_graph, "graph_replay_bit_equal": graph_check,
            "peak_frac": round(frac, 4),
            ("flops_per_step" if prefill else "bytes_per_step"): int(total / K),
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


CEILINGS = ("ceiling_read_hbm", "ceiling_mfma_f16")


def bench_ceiling(args):
    """The device's own ceilings beside the published peaks: a streaming read
    of a 6 GiB buffer (vq_probe_read) and an MFMA-only loop (vq_probe_mfma),
    each over a few launch shapes, best of 5 launches per shape, timed with
    HIP events on the launch stream."""
    import torch
    import vq_dequant_matmul_amd as vq
    hip = HipEvents()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    read = args.workload == "ceiling_read_hbm"
    shapes = (256, 512, 768, 1024, 2048) if read else (256, 512, 1024, 2048)
    out = torch.empty(max(shapes) * 256, dtype=torch.float32, device="cuda")
    if read:
        buf = torch.ones(6 << 28, dtype=torch.float32, device="cuda")   # 6 GiB
        work = buf.numel() * 4
        iters = 0
    else:
        iters = 20000
    results = {}
    for n_wg in shapes:
        def launch():
            if read:
                vq.vq_probe_read(buf, n_wg, out)
            else:
                vq.vq_probe_mfma(n_wg, iters, out)
        launch()
        torch.cuda.synchronize()
        best = None
        for _ in range(5):
            a, b = hip.create(), hip.create()
            hip.record(a, stream)
            launch()
            hip.record(b, stream)
            torch.cuda.synchronize()
            t = hip.elapsed_ms(a, b) * 1e-3
            hip.destroy(a)
            hip.destroy(b)
            best = t if best is None else min(best, t)
        if read:
            results[n_wg] = work / best / 1e9
        else:
            results[n_wg] = n_wg * 4 * iters * 4 * 32768 / best / 1e12
        log(f"[bench] {args.workload} workgroups={n_wg}: {results[n_wg]:.1f} "
            f"{'GB/s' if read else 'TFLOP/s'} ({best * 1e6:.1f} us)")
    top = max(results, key=results.get)
    peak = HBM_PEAK_GBS if read else MFMA_F16_PEAK_TFLOPS
    rec = {
        "metric": "device ceiling: " + ("streaming HBM read" if read else "fp16 MFMA, registers only"),
        "value": round(results[top], 1), "unit": "GB/s" if read else "TFLOP/s", "n_gpus": 1,
        "higher_is_better": True, "data": "synthetic",
        "dtype": "u32" if read else "f16xf16->f32",
        "config": {"workload": args.workload, "best_workgroups": top,
                   "by_workgroups": {str(k): round(v, 1) for k, v in results.items()},
                   "bytes" if read else "mfma_per_wave": work if read else iters * 4},
        "published_peak": peak, "frac_of_published_peak": round(results[top] / peak, 4),
    }
    print(json.dumps(rec), flush=True)


def bench_stack(args, sw):
    """One token through a stack of MoE layers with promoted layers: a step
    is one vq_moe_stack call (every layer's gate+up and down+combine, the
    hidden state updated in place) from a fresh hidden state and fresh
    routes for every layer."""
    import numpy as np
    import torch

    import synth
    import vq_dequant_matmul_amd as vq

    b = sw.base
    K = args.steps if args.steps is not None else 30
    W = args.warmup if args.warmup is not None else 3
    n_k = args.kernel_launches if args.kernel_launches is not None else 200
    n_steps = K + W

    t0 = time.perf_counter()
    # one host layer per geometry; every position of the stack gets a device
    # copy at its own address, with enough copies per geometry that a copy
    # is reused only after several times the Infinity Cache has streamed by
    geoms = sorted({sw.layer_bits(l) for l in range(sw.n_layers)})
    host = {bits: synth.make_stack_layer(
        sw, next(l for l in range(sw.n_layers) if sw.layer_bits(l) == bits)) for bits in geoms}
    layer_bytes = {bits: sum(t.stored_bytes() for t in host[bits]) for bits in geoms}
    copies = {bits: max(2, min(sum(sw.layer_bits(l) == bits for l in range(sw.n_layers)),
                               math.ceil(4 * MALL_BYTES / layer_bytes[bits])))
              for bits in geoms}
    dev = {bits: [[vq.VQTensor.from_host(t) for t in host[bits]]] for bits in geoms}
    for bits in geoms:
        dev[bits] += [[t.clone() for t in dev[bits][0]] for _ in range(copies[bits] - 1)]
    pos = {bits: 0 for bits in geoms}
    stack = []
    for l in range(sw.n_layers):
        bits = sw.layer_bits(l)
        stack.append(dev[bits][pos[bits] % copies[bits]])
        pos[bits] += 1
    xs, ids, ws = [], [], []
    for i in range(n_steps):
        x, r, w = synth.make_stack_inputs(sw, i)
        xs.append(x)
        ids.append(r)
        ws.append(w)
    x_dev = torch.from_numpy(np.stack(xs)).cuda()
    ids_dev = torch.from_numpy(np.stack(ids)).cuda()
    w_dev = torch.from_numpy(np.stack(ws)).cuda()
    hidden = torch.empty((b.n_tok, b.hidden), dtype=torch.float32, device="cuda")

    def layers_of(i):
        return [(*stack[l], ids_dev[i, l], w_dev[i, l]) for l in range(sw.n_layers)]
    step_layers = [layers_of(i) for i in range(n_steps)]
    ws_bytes = vq.vq_moe_stack_workspace_size(step_layers[0], b.n_tok, b.top_k)
    workspace = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    log(f"[bench] {sw.name}: geometries {geoms} with {copies} device copies, "
        f"{sum(layer_bytes[g] * copies[g] for g in geoms) / 1e9:.2f} GB of layers, "
        f"setup {time.perf_counter() - t0:.1f}s")

    hl = {bits: host[bits] for bits in geoms}
    io_bytes = b.n_tok * b.hidden * 4 * 3 + b.n_tok * b.top_k * 8

    def layer_bytes_of(i, l, projs=3):
        G, U, D = hl[sw.layer_bits(l)]
        uniq = np.unique(ids[i][l])
        ts = (G, U, D)[:projs]
        return int(sum(expert_bytes(t, int(e)) for e in uniq for t in ts)
                   + sum(t.K * t.d * 2 for t in ts) + io_bytes)

    def step_bytes(i):
        return sum(layer_bytes_of(i, l) for l in range(sw.n_layers))

    def step(i):
        hidden.copy_(x_dev[i])
        vq.vq_moe_stack(step_layers[i], hidden, workspace=workspace)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    log(f"[bench] warmup {W} steps done")
    use_graph = not args.no_graph
    if use_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(W, n_steps):
                step(i)
        torch.cuda.synchronize()
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
    h_graph = hidden.clone()
    step(n_steps - 1)
    torch.cuda.synchronize()
    graph_check = bool(torch.equal(h_graph.view(torch.int32), hidden.view(torch.int32)))
    if not graph_check:
        log("[bench] WARNING: graph replay differs from eager")
    total = sum(step_bytes(i) for i in range(W, n_steps))
    value = total / elapsed / 1e9

    # dominant kernel: the gate+up launch, over the stack's layers in order
    hip = HipEvents()
    src = torch.ones(1 << 26, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    h = torch.empty((b.n_tok * b.top_k, b.inter), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    for _ in range(48):
        dst.copy_(src)
    ev0, ev1 = hip.create(), hip.create()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    hip.record(ev0, stream)
    for j in range(n_k):
        i, l = W + (j // sw.n_layers) % K, j % sw.n_layers
        G, U, _ = stack[l]
        vq.vq_moe_gate_up(G, U, x_dev[i], ids_dev[i, l], out=h)
    hip.record(ev1, stream)
    torch.cuda.synchronize()
    k_mean = hip.elapsed_ms(ev0, ev1) * 1e-3 / n_k
    hip.destroy(ev0)
    hip.destroy(ev1)
    del src, dst, h
    kwork = np.array([layer_bytes_of(W + (j // sw.n_layers) % K, j % sw.n_layers, 2)
                      - b.n_tok * b.hidden * 8 + b.n_tok * b.top_k * b.inter * 4
                      for j in range(n_k)])
    achieved = float(kwork.mean() / k_mean / 1e9)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                # the record covers the 9-bit layers' kernel, not the mix timed here
                "traffic": None,
                "kernel": "vq::k_rows (gate+up+SwiGLU, fused), over the stack's layers",
                "launch_us": round(k_mean * 1e6, 2), "bytes_per_launch": int(kwork.mean()),
                "timing": f"one HIP event pair around {n_k} back-to-back launches"}
    log(f"[bench] gate+up: {k_mean * 1e6:.2f} us/launch, {achieved:.1f} GB/s")

    cpu = None
    if args.cpu_seconds > 0:
        import oracle

        def run(j):
            i = W + j % K
            layers = [(*hl[sw.layer_bits(l)], ids[i][l], ws[i][l]) for l in range(sw.n_layers)]
            oracle.moe_stack(layers, xs[i])
            return step_bytes(i)
        cpu = oracle_baseline(run, args.cpu_seconds, K, 1e9, "GB/s", 4,
                              f"whole steps of the same workload ({sw.n_layers} layers)")

    rec = {
        "metric": "VQ MoE layer stack GB/s (decode, % HBM peak)", "value": round(value, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(elapsed * 1e3 / K, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16xf16->f32", "data": "synthetic",
        "config": {
            "workload": sw.name, "layers": sw.n_layers, "promoted_layers": list(sw.promoted),
            "experts": b.n_experts, "top_k": b.top_k, "hidden": b.hidden, "inter": b.inter,
            "d": b.d, "bits": b.bits, "promoted_bits": sw.promoted_bits, "tokens": b.n_tok,
            "device_copies": {str(k): v for k, v in copies.items()}, "hip_graph": use_graph,
            "graph_replay_bit_equal": graph_check,
            "peak_frac": round(value / HBM_PEAK_GBS, 4), "bytes_per_step": int(total / K),
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


# The fit's rate limit: fp32 VALU operations issued one by one, neither fused
# (no multiply-add: the distances round every operation) nor packed.  A CU's
# four SIMDs each take a wave64 fp32 instruction every 2 cycles (32 lanes a
# cycle; the counters of the encode pass show 0.47 instructions per SIMD and
# cycle), so MI355X issues 256 x 4 x 32 x 2.4 GHz = 78.6 T such operations
# a second -- half its published 157.3 TFLOP/s, which counts a fused
# multiply-add as two flops.
VALU_F32_OPS_PEAK_T = 78.6


def bench_fit(args, fw):
    """Fitting the format to one projection's weights: a step is one vq_fit
    call (scales, the Lloyd iterations on the fit set, the fp16 codebook and
    the encode pass over every subvector)."""
    import numpy as np
    import torch

    import synth
    import vq_dequant_matmul_amd as vq

    K = args.steps if args.steps is not None else 5
    W = args.warmup if args.warmup is not None else 1
    n_k = args.kernel_launches if args.kernel_launches is not None else 5
    t0 = time.perf_counter()
    w = synth.make_fit_weights(fw.seed, fw.n_rows, fw.cols)
    sample, init = fw.draws()
    w_dev = torch.from_numpy(w.view(np.int16)).cuda().view(torch.bfloat16)
    s_dev, i_dev = torch.from_numpy(sample).cuda(), torch.from_numpy(init).cuda()
    ws_bytes = vq.load_library().vq_fit_workspace_size(fw.d, fw.K, fw.n_sample)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    log(f"[bench] {fw.name}: {fw.n_rows}x{fw.cols} bf16 weights, fit set {fw.n_sample}, "
        f"K={fw.K}, {fw.iters} iterations, setup {time.perf_counter() - t0:.1f}s")
    N = fw.n_rows * (fw.cols // fw.d)
    # per subvector-entry pair: d subtractions, d squares, d - 1 additions
    ops = 3 * fw.d - 1
    assign_flops = fw.iters * fw.n_sample * fw.K * ops
    encode_flops = N * fw.K * ops
    step_flops = assign_flops + encode_flops

    out = {}

    def step():
        out["r"] = vq.vq_fit(w_dev, fw.d, fw.bits, fw.K, s_dev, i_dev, fw.iters, workspace=ws)

    for _ in range(W):
        step()
    torch.cuda.synchronize()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    log(f"[bench] timed {K} fits in {elapsed * 1e3:.2f} ms")
    value = step_flops * K / elapsed / 1e12

    hip = HipEvents()
    # the device copies of known size that the HBM byte counters are
    # calibrated on (as for the other workloads)
    src = torch.ones(1 << 26, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(48):
        dst.copy_(src)
    del src, dst
    pairs = [(hip.create(), hip.create()) for _ in range(n_k)]
    for j in range(n_k):
        vq.vq_set_kernel_events(pairs[j][0], pairs[j][1])
        step()
    vq.vq_set_kernel_events(None, None)
    torch.cuda.synchronize()
    durs = np.array([hip.elapsed_ms(a, b) * 1e-3 for a, b in pairs])
    for a, b in pairs:
        hip.destroy(a)
        hip.destroy(b)
    k_mean = float(durs.mean())
    achieved = encode_flops / k_mean / 1e12
    roofline = {"bound": "alu", "achieved": round(achieved, 2),
                "peak": round(VALU_F32_OPS_PEAK_T, 1), "unit": "TFLOP/s",
                "frac": round(achieved / VALU_F32_OPS_PEAK_T, 4),
                "traffic": recorded_traffic(args.workload, "fit"),
                "kernel": "vq::k_fit_encode (nearest fp16 entry for every subvector, packed)",
                "launch_us": round(k_mean * 1e6, 2), "flops_per_launch": int(encode_flops),
                "timing": f"HIP event pair around each of {n_k} launches"}
    log(f"[bench] encode: {k_mean * 1e3:.3f} ms/launch, {achieved:.2f} TFLOP/s")

    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        # a bounded slice: the first rows of the tensor with a proportional
        # share of the fit set (its indices that fall in those rows)
        rows = 1024
        n_sub = fw.cols // fw.d
        sub_s = sample[sample < rows * n_sub]
        sub_i = init % (rows * n_sub)

        def run(j):
            oracle.fit(w[:rows], fw.d, fw.bits, fw.K, sub_s, sub_i, fw.iters)
            return (fw.iters * len(sub_s) + rows * n_sub) * fw.K * ops
        cpu = oracle_baseline(run, args.cpu_seconds, 1000, 1e12, "TFLOP/s", 6,
                              f"fits of the first {rows} rows with their share of the fit "
                              f"set ({len(sub_s)} subvectors)")

    rec = {
        "metric": "VQ codebook fit TFLOP/s (nearest-entry searches, % of the un-fused fp32 VALU rate)",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(elapsed * 1e3 / K, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {
            "workload": fw.name, "rows": fw.n_rows, "cols": fw.cols, "d": fw.d,
            "bits": fw.bits, "K": fw.K, "fit_set": fw.n_sample, "iterations": fw.iters,
            "seed": fw.seed, "subvectors": N, "flops_per_step": int(step_flops),
            "peak_frac": round(value / VALU_F32_OPS_PEAK_T, 4),
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def bench_gather(args, wl):
    """Row gather from the stacked VQ embedding tables: a step is one
    vq_row_gather launch over one batch of ids (tokens x tables rows)."""
    import numpy as np
    import torch

    import synth
    import vq_dequant_matmul_amd as vq

    K = args.steps if args.steps is not None else 200
    W = args.warmup if args.warmup is not None else 20
    n_k = args.kernel_launches if args.kernel_launches is not None else 100
    n_steps = K + W

    t0 = time.perf_counter()
    T = synth.make_gather_table(wl)
    Wd = vq.VQTensor.from_host(T)
    ids = [synth.make_gather_ids(wl, i) for i in range(n_steps)]
    ids_dev = torch.from_numpy(np.stack(ids)).cuda()
    y_bytes = wl.n_ids * wl.cols * 4
    # outputs rotate over buffers that together exceed the Infinity Cache, so
    # the stores reach HBM
    n_out = max(2, min(16, math.ceil(4 * MALL_BYTES / y_bytes)))
    ys = [torch.empty((wl.n_ids, wl.cols), dtype=torch.float32, device="cuda")
          for _ in range(n_out)]
    torch.cuda.synchronize()
    log(f"[bench] {wl.name}: table {T.stored_bytes() / 1e9:.2f} GB, {n_steps} id batches of "
        f"{wl.n_ids}, {n_out} output buffers, setup {time.perf_counter() - t0:.1f}s")

    # algorithmic bytes: per gathered row its codes, scales, id and fp32
    # output; per launch the codebook
    row_bytes = T.wpr * 4 + T.groups * 2 + 8 + wl.cols * 4
    step_bytes = wl.n_ids * row_bytes + T.K * T.d * 2

    def step(i):
        vq.vq_row_gather(Wd, ids_dev[i], out=ys[i % n_out])

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

    last = (n_steps - 1) % n_out
    y_graph = ys[last].clone()
    step(n_steps - 1)
    torch.cuda.synchronize()
    graph_check = bool(torch.equal(y_graph.view(torch.int32), ys[last].view(torch.int32)))
    if not graph_check:
        log("[bench] WARNING: graph replay differs from eager")
    del y_graph

    value = step_bytes * K / elapsed / 1e9
    frac = value / HBM_PEAK_GBS

    # the step is the one kernel: an event pair around n_k back-to-back
    # launches, behind a queue of device copies that keeps the GPU busy while
    # they are queued
    hip = HipEvents()
    src = torch.ones(1 << 26, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(48):
        dst.copy_(src)
    ev0, ev1 = hip.create(), hip.create()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    hip.record(ev0, stream)
    for j in range(n_k):
        step(W + (j % K))
    hip.record(ev1, stream)
    torch.cuda.synchronize()
    k_mean = hip.elapsed_ms(ev0, ev1) * 1e-3 / n_k
    hip.destroy(ev0)
    hip.destroy(ev1)
    del src, dst
    achieved = step_bytes / k_mean / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": recorded_traffic(wl.name, "gather"),
                "kernel": "vq::k_gather (row gather, exact fp32 rows)",
                "launch_us": round(k_mean * 1e6, 2), "bytes_per_launch": int(step_bytes),
                "timing": f"one HIP event pair around {n_k} back-to-back launches"}
    log(f"[bench] k_gather: {k_mean * 1e6:.2f} us/launch, {achieved:.1f} GB/s")

    cpu = None
    if args.cpu_seconds > 0:
        import oracle

        def run(j):
            oracle.gather(T, ids[W + j % K])
            return step_bytes
        cpu = oracle_baseline(run, args.cpu_seconds, 10 * n_steps, 1e9, "GB/s", 4,
                              f"whole steps of the same workload ({wl.n_ids} rows each)")

    rec = {
        "metric": "VQ embedding row gather GB/s (% HBM peak)", "value": round(value, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(elapsed * 1e3 / K, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16xf16->f32", "data": "synthetic",
        "config": {
            "workload": wl.name, "tables": wl.tables, "rows_per_table": wl.rows,
            "cols": wl.cols, "d": wl.d, "bits": wl.bits, "K": T.K, "tokens": wl.n_tok,
            "rows_per_step": wl.n_ids, "output_buffers": n_out, "hip_graph": use_graph,
            "graph_replay_bit_equal": graph_check, "peak_frac": round(frac, 4),
            "bytes_per_step": int(step_bytes),
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
