"""Benchmark of the fused MoE layer forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload decode|prefill|fp8|mxfp8|fp8t|router|tiny|...]
                    [--launch graph|eager] [--chain stages|persistent]

A step is one pass of the whole chain (route -> align -> [quant] -> Gate-Up ->
Down -> combine; router GEMM first for the router workload) over one batch of
seeded synthetic input already resident in HBM.  The timed steps are eager
launches on one stream with nothing else in between (with --launch graph the
chain is captured once as a HIP graph and every step is one replay; on
MI355X that measured no faster).  With --chain persistent a step is one
moe_forward_persistent call instead: the same stages as phases of one
persistent kernel chained by device-side ready flags.  Where that entry point
applies (bf16 weights, T*k <= 16*E) both chains are timed and reported under
layer.chain_ms, and their outputs are compared bit for bit.  A separate pass
with HIP events around every stage gives the per-kernel times.  Prints ONE
JSON line.

value = tokens per second of the whole layer (T tokens per step).  The
roofline object describes the dominant kernel (the Gate-Up GEMM): its
algorithmic bytes (or flops) per launch divided by its average launch time
measured with HIP events on the stream it runs on.  cpu_baseline times the
oracle on the host cores on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


CSRC = os.path.join(ROOT, "expert_layer_amd", "csrc")


def _include_closure(root):
    """root and every csrc header it includes, directly or not."""
    seen, todo = set(), [root]
    while todo:
        f = todo.pop()
        if f in seen or not os.path.exists(os.path.join(CSRC, f)):
            continue
        seen.add(f)
        with open(os.path.join(CSRC, f)) as fh:
            for line in fh:
                line = line.strip()
                if line.startswith("#include \""):
                    todo.append(line.split('"')[1])
    return sorted(seen)


def kernel_source_hash(root=None):
    """Hash of the kernel sources: with root (a .hip file of the library), of
    that file and the headers it includes; without, of every source.  Counter
    figures are reported only for the sources they were taken on."""
    files = _include_closure(root) if root else sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".hpp")))
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def gemm13_algorithmic(wl, counts):
    """Algorithmic bytes / flops of one Gate-Up launch.

    bytes: w1 + w3 of every expert with at least one row (plus the shared
    expert), one read of each gathered x row per slot, one write of h per slot
    (fp8: codes + per-128 scales; mxfp8: codes + one scale byte per 32;
    fp8t: codes, and h unquantised in fp32 since its scale needs all of h).
    flops: 4*H*I per slot row.
    """
    R = wl.T * wl.k + wl.shared * wl.T
    wb = 1 if wl.wtype in ("fp8", "mxfp8", "fp8t") else 2
    touched = int((counts > 0).sum()) + wl.shared
    weight = touched * 2 * wl.I * wl.H * wb
    if wl.wtype == "fp8":
        weight += touched * 2 * (wl.I // 128) * (wl.H // 128) * 4
        act = R * (wl.H + wl.H // 128 * 4) + R * (wl.I + wl.I // 128 * 4)
    elif wl.wtype == "mxfp8":
        weight += touched * 2 * wl.I * (wl.H // 32)
        act = R * (wl.H + wl.H // 32) + R * (wl.I + wl.I // 32)
    elif wl.wtype == "fp8t":
        act = R * wl.H + R * wl.I * 4
    else:
        act = R * wl.H * 2 + R * wl.I * 2
    flops = 4.0 * wl.H * wl.I * R
    return weight + act, flops, touched


def layer_flops(wl):
    f = 6.0 * wl.H * wl.I * wl.T * (wl.k + wl.shared)
    if wl.router:
        f += 4.0 * wl.T * wl.H * wl.E
    return f


def layer_floor_bytes(wl, counts):
    wb = 1 if wl.wtype in ("fp8", "mxfp8", "fp8t") else 2
    touched = int((counts > 0).sum()) + wl.shared
    b = touched * 3 * wl.I * wl.H * wb
    if wl.wtype == "fp8":
        b += touched * 3 * (wl.I // 128) * (wl.H // 128) * 4
    elif wl.wtype == "mxfp8":
        b += touched * 3 * wl.I * (wl.H // 32)
    b += wl.T * wl.H * 2 * 2  # x in, out
    b += wl.T * wl.E * 4 if not wl.router else wl.E * wl.H * 4
    return b


def load_traffic(name, src_hash):
    """HBM traffic of the dominant kernel from the committed rocprofv3 counter summary,
    only while the kernel sources are the ones the counters were taken on."""
    path = os.path.join(ROOT, "profiles", f"gemm13_{name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if "kernel_file" in t:   # the kernel's own file and its headers
        src_hash = kernel_source_hash(t["kernel_file"])
    if t.get("kernel_source_hash") != src_hash:
        return None
    return t.get("hbm_bytes_per_launch")


def host_cpu():
    """CPU model and the host's logical core count, from /proc/cpuinfo and the OS."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, os.cpu_count() or 1


def oracle_threads():
    """Threads for the oracle: every core this process may run on, at most 16
    (the GPU machine gives one GPU's job a 16-core share of the host)."""
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return max(1, min(16, avail))


def cpu_baseline(wl, d, b, budget_s):
    """The oracle as it stands, timed on the host cores on a bounded sample of
    the same workload, with all available threads and with one thread.

    Per-step work that depends on all tokens (routing and align, the x
    quantisation of the FP8 types) runs on every token; the expert FFN and the
    combine run on the first n tokens (n sized to the time budget), passed
    over again when one pass is short.  Weight quantisation is offline (done
    once per model) and not timed.  Per-tensor FP8 takes the h scale from the
    sampled pairs.  tokens/s = 1 / (FFN+combine time per token + all-token
    time / T)."""
    from oracle import oracle as orc
    nthreads = oracle_threads()
    model, ncores = host_cpu()
    host = workloads.bits
    x = host(d["x"])
    logits = host(d["logits"]) if not wl.router else host(b.logits)
    bias = host(d["bias"]) if d["bias"] is not None else None
    bias_rows = host(d["bias_rows"]) if d["bias_rows"] is not None else None

    t0 = time.perf_counter()
    ids, w = orc.route(logits, wl.k, bias, bias_rows)
    orc.align(ids, wl.E, wl.shared)
    xs = None
    if wl.wtype == "fp8":
        x, xs = orc.quant_rows_fp8(x)
    elif wl.wtype == "mxfp8":
        x, xs = orc.quant_rows_mx(x, nthreads=nthreads)
    elif wl.wtype == "fp8t":
        x, xs = orc.quant_tensor_fp8(x, nthreads=nthreads)
    t_all = time.perf_counter() - t0

    def layer_for(rows):
        """Oracle layer over the experts the given tokens use (weights quantised by the oracle, untimed)."""
        used = np.unique(ids[rows].ravel())
        remap = np.full(wl.E, -1, np.int32)
        remap[used] = np.arange(used.size, dtype=np.int32)
        ids_c = ids.copy()
        ids_c[rows] = remap[ids[rows]]
        idx = torch.from_numpy(used).to(d["w1"].device)
        mats = {n: host(d[n][idx]) for n in ("w1", "w3", "w2")}
        sh = {n: host(d[n]) if d[n] is not None else None for n in ("sw1", "sw3", "sw2")}
        if wl.wtype == "bf16":
            return orc.Layer(mats["w1"], mats["w3"], mats["w2"], sh["sw1"], sh["sw3"], sh["sw2"]), ids_c
        if wl.wtype == "fp8":
            qf = lambda a: orc.quant_blocks_fp8(a, nthreads=nthreads)          # noqa: E731
            wt = 1
        elif wl.wtype == "mxfp8":
            qf = lambda a: orc.quant_rows_mx(a, nthreads=nthreads)             # noqa: E731
            wt = 2
        else:
            qf = lambda a: orc.quant_tensor_fp8(a, mats=a.shape[0] if a.ndim == 3 else 1,  # noqa: E731
                                                nthreads=nthreads)
            wt = 3
        q = {n: qf(a) for n, a in mats.items()}
        qs = {n: (qf(a) if a is not None else (None, None)) for n, a in sh.items()}
        L = orc.Layer(q["w1"][0], q["w3"][0], q["w2"][0], qs["sw1"][0], qs["sw3"][0], qs["sw2"][0], wtype=wt,
                      s1=q["w1"][1], s3=q["w3"][1], s2=q["w2"][1], ss1=qs["sw1"][1], ss3=qs["sw3"][1],
                      ss2=qs["sw2"][1])
        return L, ids_c

    def timed_pass(threads, budget):
        # calibrate on 2 tokens, then size the sample to the budget
        rows = np.arange(min(2, wl.T), dtype=np.int64)
        L, ids_c = layer_for(rows)
        t0 = time.perf_counter()
        orc.layer_rows(L, x, ids_c, w, rows, xs=xs, nthreads=threads)
        per_tok = (time.perf_counter() - t0) / rows.size
        n = int(max(2, min(wl.T, budget / max(per_tok, 1e-9))))
        reps = int(max(1, min(64, budget / max(per_tok * n, 1e-9))))
        rows = np.arange(n, dtype=np.int64)
        L, ids_c = layer_for(rows)
        t0 = time.perf_counter()
        for _ in range(reps):
            orc.layer_rows(L, x, ids_c, w, rows, xs=xs, nthreads=threads)
        t = time.perf_counter() - t0
        return 1.0 / (t / (n * reps) + t_all / wl.T), n, reps, t

    v_n, n_n, r_n, t_n = timed_pass(nthreads, 0.6 * budget_s)
    v_1, n_1, r_1, t_1 = timed_pass(1, 0.4 * budget_s)
    prec = "fp64" if wl.wtype == "bf16" else "fp64 with the FP8 quantisation emulated exactly"
    return {"value": v_n, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "value_1thread": v_1, "host_cores": ncores, "cpu_model": model,
            "sample": f"per-step work over all {wl.T} tokens (route+align"
                      f"{', x quantisation' if wl.wtype != 'bf16' else ''}: {t_all:.2f}s); expert FFN + combine "
                      f"on the first {n_n} tokens x {r_n} passes ({t_n:.1f}s, {nthreads} threads) and the first "
                      f"{n_1} tokens x {r_1} passes ({t_1:.1f}s, 1 thread); {prec}"
                      + ("; h scale from the sampled pairs" if wl.wtype == "fp8t" else "")}


def router_gemm_only(T: int) -> None:
    """The split-BF16 router GEMM on its own: x [T, H] bf16 ~N(0, 1), router
    weights [E, H] fp32 ~N(0, 0.01) split on the device, H and E of the router
    workload; prints one JSON line with the average time per call."""
    import expert_layer_amd as moe
    wl = workloads.WORKLOADS["router"]
    H, E = wl.H, wl.E
    g = torch.Generator(device="cuda:0").manual_seed(wl.seed)
    x = torch.randn((T, H), generator=g, device="cuda:0").to(torch.bfloat16)
    w = 0.01 * torch.randn((E, H), generator=g, device="cuda:0")
    hi = torch.empty((E, H), dtype=torch.bfloat16, device="cuda:0")
    lo = torch.empty_like(hi)
    logits = torch.empty((T, E), device="cuda:0")
    moe.moe_router_split(w, hi, lo)
    for _ in range(3):
        moe.moe_router_gemm(x, hi, lo, logits)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 10
    t0.record()
    for _ in range(n):
        moe.moe_router_gemm(x, hi, lo, logits)
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1000.0 / n
    print(json.dumps({"router_gemm_us": round(us, 2), "T": T, "H": H, "E": E, "calls": n,
                      "tflops": round(2 * 2 * T * H * E / us / 1e6, 1),
                      "x_bytes": T * H * 2, "split_weight_bytes": 2 * E * H * 2}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode", choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--residual-norm", action="store_true",
                    help="fuse a residual add + RMSNorm into the combine stage (bf16 residual and weight)")
    ap.add_argument("--launch", choices=("eager", "graph"), default="eager",
                    help="time the chain as eager launches (default) or as one captured HIP graph per step")
    ap.add_argument("--chain", choices=("stages", "persistent"), default="stages",
                    help="a step is the five-stage chain (default) or one moe_forward_persistent call")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="instead of the layer, run a plain device copy of BYTES bytes 5 times (used to scale "
                         "the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--router-gemm", type=int, default=0, metavar="T",
                    help="instead of the layer, time the split-BF16 router GEMM alone on T tokens at the router "
                         "workload's hidden size and expert count (10 calls after 3 warm-up; for its counters)")
    args = ap.parse_args()
    if args.router_gemm:
        router_gemm_only(args.router_gemm)
        return
    if args.copy_calibration:
        n = args.copy_calibration
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel() * 4, "launches": 5}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer runs on a single MI355X, see the sharding notes in the design document)",
              file=sys.stderr)
        sys.exit(2)

    import expert_layer_amd as moe
    from expert_layer_amd.chain import Buffers, Layer, run_chain, split_router

    moe.lib()
    wl = workloads.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] workload {wl.name}: generating inputs")
    d = workloads.make_inputs(wl, device=dev)
    fp8 = wl.wtype in ("fp8", "mxfp8", "fp8t")
    layer = Layer.from_weights(d["w1"], d["w3"], d["w2"], d["sw1"], d["sw3"], d["sw2"], fp8=wl.wtype == "fp8",
                               mx=wl.wtype == "mxfp8", pt=wl.wtype == "fp8t")
    y_dtype = torch.float32 if wl.T * (wl.k + wl.shared) * wl.H <= (1 << 24) else torch.bfloat16
    b = Buffers(layer, wl.T, wl.k, y_dtype=y_dtype, router=wl.router)
    hi = lo = None
    if wl.router:
        hi, lo = split_router(d["router_w"])
    kw = dict(logits=None if wl.router else d["logits"], router_hi=hi, router_lo=lo, bias=d["bias"],
              bias_rows=d["bias_rows"])
    if args.residual_norm:
        g = torch.Generator(device=dev).manual_seed(wl.seed + 17)
        kw["residual"] = torch.randn((wl.T, wl.H), generator=g, device=dev).to(torch.bfloat16)
        kw["norm_weight"] = (1.0 + 0.1 * torch.randn(wl.H, generator=g, device=dev)).to(torch.bfloat16)
    stream = torch.cuda.current_stream()
    names = (["router"] if wl.router else []) + ["route", "align"] + (["quant"] if fp8 else []) + \
        ["gemm13"] + (["hquant"] if wl.wtype == "fp8t" else []) + ["gemm2", "combine"]
    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        run_chain(layer, b, d["x"], wl.k, **kw)
    torch.cuda.synchronize()
    counts = b.counts.cpu().numpy()

    # per-stage times: eager launches with events around every stage
    ev = [{n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for n in names}
          for _ in range(args.steps)]
    log(f"[bench] per-stage pass, {args.steps} steps")
    for i in range(args.steps):
        run_chain(layer, b, d["x"], wl.k, stages=ev[i], **kw)
    torch.cuda.synchronize()
    stage_ms = {n: float(np.mean([e[n][0].elapsed_time(e[n][1]) for e in ev])) for n in names}

    # whole-chain steps: eager launches, or the chain captured once as a HIP
    # graph and replayed (the kernels and buffers are the same)
    def timed(fn, label):
        if args.launch == "graph":
            side = torch.cuda.Stream()
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                fn()
            stream.wait_stream(side)
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                fn()
            graph.replay()
            step = graph.replay
        else:
            step = fn
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        log(f"[bench] timing {args.steps} steps ({label}, {args.launch})")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record(stream)
        for _ in range(args.steps):
            step()
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return start.elapsed_time(end) / args.steps, wall * 1e3 / args.steps

    pers_ok = wl.wtype == "bf16" and wl.T * wl.k <= 16 * wl.E and not args.residual_norm
    if args.chain == "persistent" and not pers_ok:
        print("--chain persistent needs bf16 weights, T*k <= 16*E and no --residual-norm", file=sys.stderr)
        sys.exit(2)
    chain_ms = {}
    pers_same = None
    if pers_ok:
        ydt = moe.MOE_DTYPE_F32 if y_dtype == torch.float32 else moe.MOE_DTYPE_BF16
        pws = torch.empty(moe.moe_forward_workspace_bytes(layer.experts, wl.T, wl.k, ydt), dtype=torch.uint8,
                          device=dev)
        pout = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=dev)

        def persistent():
            moe.moe_forward_persistent(layer.experts, d["x"], wl.k, pout, pws, logits=kw["logits"], router_hi=hi,
                                       router_lo=lo, bias=d["bias"], bias_rows=d["bias_rows"], y_dtype=ydt)
        for _ in range(args.warmup):
            persistent()
        chain_ms["persistent"], pers_wall = timed(persistent, "persistent")
        moe.moe_forward_persistent_status(pws)
    chain_ms["stages"], stages_wall = timed(lambda: run_chain(layer, b, d["x"], wl.k, **kw), "stages")
    if pers_ok:
        pers_same = bool(torch.equal(pout, b.out))
        if not pers_same:
            log("[bench] WARNING: persistent chain output differs from the five-stage chain")
    ms_step = chain_ms[args.chain]
    wall_ms = pers_wall if args.chain == "persistent" else stages_wall
    log("[bench] per-stage ms: " + ", ".join(f"{n}={v:.4f}" for n, v in stage_ms.items()) +
        f"; step {ms_step:.4f} ms (wall {wall_ms:.4f} ms, {args.chain}, {args.launch})" +
        (f"; persistent {chain_ms['persistent']:.4f} ms, stages {chain_ms['stages']:.4f} ms" if pers_ok else ""))

    value = wl.T / (ms_step * 1e-3)
    g13_bytes, g13_flops, touched = gemm13_algorithmic(wl, counts)
    g13_s = stage_ms["gemm13"] * 1e-3
    src_hash = kernel_source_hash()
    if wl.T * wl.k <= 16 * wl.E:   # small groups: the weight stream bounds the layer
        achieved = g13_bytes / g13_s / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": load_traffic(wl.name, src_hash)}
    else:
        peak = MFMA_PEAK_TFLOPS["fp8" if fp8 else "bf16"]
        achieved = g13_flops / g13_s / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak, "traffic": load_traffic(wl.name, src_hash)}
    if roof["traffic"] is not None:
        roof["traffic_source"] = (f"profiles/gemm13_{wl.name}_traffic.json: rocprofv3 FETCH_SIZE + WRITE_SIZE of "
                                  "this kernel, calibrated on a device copy, taken on this kernel's current "
                                  "source file and headers (not measured in this run)")
    roof["kernel"] = "gemm13"
    roof["per_launch"] = {"bytes": g13_bytes, "flops": g13_flops, "touched_experts": touched,
                          "avg_ms": stage_ms["gemm13"]}
    floor = layer_floor_bytes(wl, counts)
    lf = layer_flops(wl)
    layer_info = {"ms": ms_step, "tflops": lf / (ms_step * 1e-3) / 1e12,
                  "hbm_floor_gbs": floor / (ms_step * 1e-3) / 1e9,
                  "hbm_frac": floor / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                  "mfma_frac": lf / (ms_step * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS["fp8" if fp8 else "bf16"],
                  "stage_ms": stage_ms, "chain_ms": chain_ms, "persistent_matches_stages": pers_same}

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        try:
            cpu = cpu_baseline(wl, d, b, args.cpu_budget)
        except MemoryError:
            cpu = None

    rec = {"metric": "MoE layer tokens/s + % of HBM (decode) / MFMA (prefill) roofline, 1 GPU",
           "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "fp8" if fp8 else "bf16", "data": "synthetic",
           "config": {"workload": wl.name, "T": wl.T, "H": wl.H, "E": wl.E, "k": wl.k, "I": wl.I,
                      "shared": wl.shared, "weights": wl.wtype, "router": wl.router,
                      "y_dtype": "f32" if y_dtype == torch.float32 else "bf16", "seed": wl.seed,
                      "launch": args.launch, "chain": args.chain, "residual_norm": bool(args.residual_norm)},
           "roofline": roof, "layer": layer_info, "cpu_baseline": cpu,
           "kernel_source_hash": src_hash}
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
