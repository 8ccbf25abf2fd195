#!/usr/bin/env python3
"""Throughput of the WUSH W4A4 layer path on one MI355X.

One step = the online hot path over one batch: transform + quantize the
activations (wush_transform_quant), then the W4A4 matmul against the
offline-packed weights (wush_w4a4_gemm).  Inputs are seeded synthetic tensors
already resident in HBM; to keep the 256 MB Infinity Cache from serving them,
each step uses the next of `--rotate` copies of the activations and of the
packed weights.

Prints one JSON line (rank 0, one GPU):
  value        whole-step layer throughput, 2*M*N*K / step time, in TFLOP/s
  quant_GBps   algorithmic bytes of transform+quantize / its time
  roofline     the dominant kernel (the matmul) against the dense MXFP4 peak
  tq_roofline  transform+quantize against its own bound
  cpu_baseline the oracle timed on a bounded sample on this host's cores

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published peaks
HBM_GBPS = 8000.0
MXFP4_TFLOPS = 10100.0      # dense FP4 matrix
FP16_TFLOPS = 2500.0        # dense fp16 matrix (NVFP4 path)
INT8_TOPS = 5000.0          # dense int8 matrix
# fp32 FMA on the vector ALU without packed math: 256 CU x 4 SIMD x 16 lanes x 2 flop x 2.4 GHz
VALU_FP32_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
# vector-ALU lane operations: 256 CU x 4 SIMD x 16 lanes x 2.4 GHz
VALU_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
FP64_TFLOPS = 78.6          # fp64 vector FMA
MFMA_FP32_TFLOPS = 157.3    # dense fp32 matrix (the dense transforms run on v_mfma_f32_16x16x4_f32)
# INT4 matmul: per output and 32-group, convert + multiply + fma on the vector ALU
INT4_RESCALE_OPS = 3

METRIC = "W4A4 layer TFLOPS (transform+quant+GEMM) & quant GB/s, % roofline"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="qwen3_14b",
                    choices=["qwen3_14b", "qwen3_8b_up", "tiny", "square_sweep", "had256", "moments", "build",
                             "mfma_ceiling"],
                    help="default: the Qwen3-14B MLP pair (up 5120->17408, down 17408->5120) at 16384 tokens, "
                         "the largest configuration that fits one GPU")
    ap.add_argument("--fmt", default=None, help="square_sweep: mxfp4 | nvfp4 | int4")
    ap.add_argument("--kind", default=None,
                    help="identity | hadamard | wus | wush, or hd (the Hadamard-diagonal variant)")
    ap.add_argument("--batch", type=int, default=1, help="had256: batch 1..16")
    ap.add_argument("--rotate", type=int, default=8)
    ap.add_argument("--row-major-scales", action="store_true",
                    help="MXFP4: wush_transform_quant + wush_w4a4_gemm (scale pre-pass per call) instead of the "
                         "plane-ordered scale path")
    ap.add_argument("--shared", type=int, default=0, metavar="G",
                    help="wus/wush: share one matrix per group of nblk/G adjacent blocks (shared-transform variant)")
    ap.add_argument("--sweep", action="store_true",
                    help="square_sweep: every format x transform in turn, one JSON line each, with the layer loss")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=16.0, help="target wall time of the oracle sample")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="processes for the oracle's transform+quantize leg (default: the host cores this process "
                         "may use, at most 16)")
    ap.add_argument("--copy-reference", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-sized buffer --steps times (calibrates HBM byte counters)")
    return ap.parse_args()


# ----------------------------------------------------------------------------- setup


class Layer:
    """One quantized linear layer, device resident, with `rotate` copies of its inputs."""

    def __init__(self, wl, fmt, kind, rotate, W, torch, Wt, X, shared=0, planes=True):
        from synth.gen import bf16_bits
        self.wl, self.fmt, self.kind = wl, fmt, kind
        self.bs = W.BLOCK[fmt]
        self.M, self.K, self.N = wl.n, wl.d_in, wl.d_out
        t0 = time.time()
        nblk = self.K // self.bs
        # offline: moments and transforms on the host (library C++ builder)
        Sx = np.empty((nblk, self.bs, self.bs), np.float32)
        W.wush_block_moments(self.bs, X, Sx)
        self.hd = kind == "hd"
        # shared-transform variant: G groups of adjacent blocks
        self.group = (np.arange(nblk) * shared // nblk).astype(np.int32) if shared and kind in ("wus", "wush") else None
        self.ngroups = shared
        dev = "cuda"
        sdt = torch.int16 if fmt == "int4" else torch.uint8
        Wd = torch.from_numpy(Wt).to(dev)
        wc = torch.empty((self.N, self.K // 2), dtype=torch.uint8, device=dev)
        wsc = torch.empty((self.N, nblk), dtype=sdt, device=dev)
        if wl.dtype == "bf16":
            xd = torch.from_numpy(bf16_bits(X).view(np.int16)).to(dev).view(torch.bfloat16)
        else:
            xd = torch.from_numpy(X).to(dev)
        if self.hd:
            # Hadamard-diagonal variant: per-channel scales instead of block matrices
            Tx = np.empty(self.K, np.float32)
            Tw = np.empty(self.K, np.float32)
            W.wush_build_hd(self.bs, Wt, Sx, Tx, Tw)
            self.Tx = torch.from_numpy(Tx).to(dev)
            self.w_g = W.wush_pack_weights_hd(fmt, Wd, torch.from_numpy(Tw).to(dev), wc, wsc)
            self.x_g = W.wush_nvfp4_global_scale_hd(xd, self.Tx) if fmt == "nvfp4" else 1.0
        elif self.group is not None:
            Tx, Tw = W.wush_build_shared(kind, Wt, Sx, self.bs, self.group, shared)
            self.Tx = torch.from_numpy(Tx).to(dev)
            self.gdev = torch.from_numpy(self.group).to(dev)
            self.w_g = W.wush_pack_weights_shared(fmt, Wd, torch.from_numpy(Tw).to(dev), self.gdev, wc, wsc)
            self.x_g = W.wush_nvfp4_global_scale_shared(xd, self.Tx, self.gdev) if fmt == "nvfp4" else 1.0
        else:
            Tx = np.empty_like(Sx)
            Tw = np.empty_like(Sx)
            W.wush_build_transforms(kind, self.bs, Wt if kind in ("wus", "wush") else None,
                                    Sx if kind in ("wus", "wush") else None, Tx, Tw)
            ident = kind == "identity"
            self.Tx = None if ident else torch.from_numpy(Tx).to(dev)
            Twd = None if ident else torch.from_numpy(Tw).to(dev)
            self.w_g = W.wush_pack_weights(fmt, Wd, Twd, wc, wsc)
            self.x_g = W.wush_nvfp4_global_scale(xd, self.Tx) if fmt == "nvfp4" else 1.0
        del Wd
        self.X = [xd] + [xd.clone() for _ in range(rotate - 1)]
        self.wc = [wc] + [wc.clone() for _ in range(rotate - 1)]
        self.wsc = [wsc] + [wsc.clone() for _ in range(rotate - 1)]
        self.xc = torch.empty((self.M, self.K // 2), dtype=torch.uint8, device=dev)
        self.xsc = torch.empty((self.M, nblk), dtype=sdt, device=dev)
        self.Y = torch.empty((self.M, self.N), dtype=torch.float32, device=dev)
        # MXFP4 with a dense transform: scales in the matmul's plane order, the
        # weights' converted once here, the activations' written by the step
        self.planes = (planes and fmt == "mxfp4" and kind in ("hadamard", "wus", "wush") and not self.hd
                       and self.group is None and self.K % 256 == 0)
        if self.planes:
            self.pa = torch.empty(W.wush_mxfp4_planes_bytes(self.M, self.K), dtype=torch.uint8, device=dev)
            self.pb = []
            for r in range(rotate):
                pb = torch.empty(W.wush_mxfp4_planes_bytes(self.N, self.K), dtype=torch.uint8, device=dev)
                W.wush_mxfp4_scale_planes(self.wsc[r], pb, self.K)
                self.pb.append(pb)
        wsb = W.wush_w4a4_gemm_ws_bytes(fmt, self.M, self.N, self.K)
        self.ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev) if wsb else None
        self.x_elem_bytes = 2 if wl.dtype == "bf16" else 4
        self.host = (Wt, X, Tx, Tw)
        self.setup_s = time.time() - t0

    # algorithmic work
    def tq_bytes(self):
        el = self.M * self.K
        sbytes = {"mxfp4": 1.0 / 32, "nvfp4": 1.0 / 16, "int4": 2.0 / 32}[self.fmt]
        if self.hd:
            tbytes = self.K * 4
        else:
            tbytes = 0 if self.kind == "identity" else (self.K // self.bs) * self.bs * self.bs * 4
        return el * (self.x_elem_bytes + 0.5 + sbytes) + tbytes

    def tq_flops(self):
        if self.hd:   # one product and log2(bs) butterfly adds per element
            return (1.0 + np.log2(self.bs)) * self.M * self.K
        return 0.0 if self.kind == "identity" else 2.0 * self.bs * self.M * self.K

    def gemm_flops(self):
        return 2.0 * self.M * self.N * self.K

    def gemm_bytes(self):
        sb = {"mxfp4": 1.0 / 32, "nvfp4": 1.0 / 16, "int4": 2.0 / 32}[self.fmt]
        return (self.M + self.N) * self.K * (0.5 + sb) + self.M * self.N * 4


def tq_engine(L):
    """(bound, peak TFLOP/s) of the unit the layer's transform+quantize kernel computes on.

    Mirrors the library's dispatch: the dense transforms run on the fp32 matrix
    cores (v_mfma_f32_16x16x4_f32) for bf16 and fp32 activations alike; the
    Hadamard-diagonal variant runs one product and log2(bs) adds per element
    on the vector ALU (one lane operation each); identity has no arithmetic.
    """
    if L.hd:
        return "alu", VALU_TOPS
    return "mfma", MFMA_FP32_TFLOPS


def run_layer_steps(layers, W, torch, steps, warmup, rotate):
    """Warm up, then time `steps` steps; per-kernel HIP events on the launch stream."""
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        r = i % rotate
        for li, L in enumerate(layers):
            if ev is not None:
                ev[li][0].record(stream)
            if L.hd:
                W.wush_transform_quant_hd(L.fmt, L.X[r], L.Tx, L.xc, L.xsc, g=L.x_g)
            elif L.group is not None:
                W.wush_transform_quant_shared(L.fmt, L.X[r], L.Tx, L.gdev, L.xc, L.xsc, g=L.x_g)
            elif L.planes:
                W.wush_transform_quant_mx_planes(L.X[r], L.Tx, L.xc, L.pa)
            else:
                W.wush_transform_quant(L.fmt, L.X[r], L.Tx, L.xc, L.xsc, g=L.x_g)
            if ev is not None:
                ev[li][1].record(stream)
            if L.planes:
                W.wush_w4a4_gemm_mx_planes(L.xc, L.pa, L.wc[r], L.pb[r], L.Y)
            else:
                W.wush_w4a4_gemm(L.fmt, L.xc, L.xsc, L.wc[r], L.wsc[r], L.Y, a_g=L.x_g, b_g=L.w_g, ws=L.ws)
            if ev is not None:
                ev[li][2].record(stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # whole-step timing: no per-kernel events inside
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / steps
    # per-kernel durations: events between launches on the same stream
    n_ev = min(steps, 50)
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in layers] for _ in range(n_ev)]
    for i in range(n_ev):
        step(i, evs[i])
    torch.cuda.synchronize()
    tq_ms = [float(np.mean([evs[i][li][0].elapsed_time(evs[i][li][1]) for i in range(n_ev)])) for li in range(len(layers))]
    gm_ms = [float(np.mean([evs[i][li][1].elapsed_time(evs[i][li][2]) for i in range(n_ev)])) for li in range(len(layers))]
    return ms_step, tq_ms, gm_ms


# ----------------------------------------------------------------------------- HBM traffic


def measured_traffic(kernel, layer_names):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None.

    Records are keyed "<entry point>@<layer workload>" and hold the kernel
    source's sha256 prefix at measurement time; once the source has changed
    the figure no longer describes this kernel and None is reported.  With
    several layers in the step the figure is the mean over their launches
    (matching `achieved`, which is per launch on average too).
    """
    import hashlib
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            recs = json.load(f)
        total = 0.0
        for name in layer_names:
            rec = recs[kernel + "@" + name]
            with open(os.path.join(ROOT, rec["source"]), "rb") as f:
                if hashlib.sha256(f.read()).hexdigest()[:16] != rec["sha256_prefix"]:
                    return None
            total += (rec["fetch_kib"] * rec["fetch_factor"] + rec["write_kib"] * rec["write_factor"]) * 1024
    except (OSError, KeyError, ValueError):
        return None
    return round(total / len(layer_names))


# ----------------------------------------------------------------------------- CPU baseline


def host_workers(requested=0):
    """Processes for the oracle's pooled leg: the cores this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(requested or 16, n))


# State the forked workers of the oracle's transform+quantize leg read (set
# before the pool is created, inherited by fork; never touched by the GPU path).
_CPU_LEG = {}


def _oracle_tq_rows(bounds):
    lo, hi = bounds
    st = _CPU_LEG
    return st["fn"](st["T"], st["rows"][lo:hi], st["g"])


def _oracle_tq_pool(fn, T, rows, g, workers):
    """Oracle transform+quantize of `rows` split over `workers` forked processes."""
    import multiprocessing as mp
    _CPU_LEG.update(fn=fn, T=T, rows=rows, g=g)
    n = rows.shape[0]
    step = -(-n // workers)
    chunks = [(lo, min(n, lo + step)) for lo in range(0, n, step)]
    with mp.get_context("fork").Pool(len(chunks)) as pool:
        parts = pool.map(_oracle_tq_rows, chunks)
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def cpu_baseline(cases, fmt, kind, shared, target_s, workers):
    """The oracle timed on a bounded sample of the same step, scaled to TFLOP/s.

    Runs before the process touches the GPU (its transform+quantize leg forks
    worker processes).  Per layer: the oracle builds its own transforms from
    the seeded inputs (untimed); transform+quantize of `mt` activation rows
    runs over `workers` processes (wall time); the matmul leg decodes and
    multiplies `ms` of those rows against `ns` weight rows in fp64 with
    `workers` BLAS threads (weight codes prepared untimed).  The step time is
    the sum over layers of (tq wall per row x M) + (matmul time per flop x 2MNK).
    """
    from threadpoolctl import threadpool_limits
    from oracle import quant, gemm, transforms
    bs = {"mxfp4": 32, "nvfp4": 16, "int4": 32}[fmt]
    step_s, flops, notes = 0.0, 0.0, []
    for wl, Wt, X in cases:
        M, K, N = X.shape[0], X.shape[1], Wt.shape[0]
        with threadpool_limits(workers):
            Sx = transforms.activation_moments(X, bs).astype(np.float32)
            if kind == "hd":
                Tx, Tw, _, _ = transforms.build_hd(Wt, Sx, bs)

                def tq(T, rows, gg):
                    return quant.transform_quant_hd(fmt, T, rows, g=gg)
                apply = quant.apply_hd
            elif shared and kind in ("wus", "wush"):
                nblk = K // bs
                group = (np.arange(nblk) * shared // nblk).astype(np.int32)
                Tg, Twg, _, _ = transforms.build_shared(kind, Wt, Sx, bs, group, shared)
                Tx, Tw = transforms.expand_shared(Tg, group), transforms.expand_shared(Twg, group)

                def tq(T, rows, gg):
                    return quant.transform_quant(fmt, T, rows, g=gg)
                apply = quant.apply_transform
            else:
                Tx, Tw, _, _ = transforms.build_transforms(kind, Wt, Sx, bs)
                ident = kind == "identity"

                def tq(T, rows, gg):
                    return quant.transform_quant(fmt, T, rows, g=gg, identity=ident)

                def apply(T, rows):
                    return quant.apply_transform(T, rows, identity=ident)
        # size the sample from a short pooled run: about half the target per layer for this leg
        cal = min(M, 32 * workers)
        gx = quant.nvfp4_tensor_scale(apply(Tx, X[:cal])) if fmt == "nvfp4" else None
        t0 = time.perf_counter()
        _oracle_tq_pool(tq, Tx, X[:cal], gx, workers)
        per_row = (time.perf_counter() - t0) / cal
        budget = 0.5 * target_s / len(cases)
        mt = int(max(cal, min(M, budget / max(per_row, 1e-9))))
        if fmt == "nvfp4":   # the oracle's own tensor scale of the sample (untimed)
            gx = quant.nvfp4_tensor_scale(apply(Tx, X[:mt]))
        t0 = time.perf_counter()
        ca, sa = _oracle_tq_pool(tq, Tx, X[:mt], gx, workers)
        t_tq = time.perf_counter() - t0
        ns = min(N, 1024)
        gw = quant.nvfp4_tensor_scale(apply(Tw, Wt[:ns])) if fmt == "nvfp4" else None
        cw, sw = _oracle_tq_pool(tq, Tw, Wt[:ns], gw, workers)     # untimed prep
        ms = min(mt, 256)
        with threadpool_limits(workers):
            t0 = time.perf_counter()
            gemm.w4a4_gemm(fmt, ca[:ms], sa[:ms], cw, sw, gx, gw)
            t_g0 = time.perf_counter() - t0
            reps = int(max(1, min(50, 0.5 * budget / max(t_g0, 1e-9))))
            t0 = time.perf_counter()
            for _ in range(reps):
                gemm.w4a4_gemm(fmt, ca[:ms], sa[:ms], cw, sw, gx, gw)
            t_g = (time.perf_counter() - t0) / reps
        layer_flops = 2.0 * M * N * K
        layer_s = (t_tq / mt) * M + t_g / (2.0 * ms * ns * K) * layer_flops
        step_s += layer_s
        flops += layer_flops
        notes.append(f"{wl.name}: transform+quantize of {mt} of {M} tokens over {workers} processes "
                     f"({t_tq:.1f} s wall); decode+fp64 matmul of {ms} tokens x {ns} weight rows x K={K} "
                     f"({reps} reps, {t_g:.3f} s each, {workers} BLAS threads); scaled to the layer "
                     f"({layer_s:.0f} s)")
    return {
        "value": flops / step_s / 1e12,
        "unit": "TFLOP/s",
        "cores": workers,
        "kind": "oracle",
        "sample": "; ".join(notes) + f"; whole step {step_s:.0f} s",
        "host_cpus": os.cpu_count(),
    }


# ----------------------------------------------------------------------------- main


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from synth.gen import CONFIGS, make_weights, make_activations

    layer_workload = args.workload not in ("had256", "moments", "build", "mfma_ceiling") and not args.copy_reference
    if layer_workload:
        if args.workload == "qwen3_14b":
            wls = [CONFIGS["qwen3_14b_up"], CONFIGS["qwen3_14b_down"]]
        else:
            wls = [CONFIGS[args.workload]]
        fmt = args.fmt or wls[0].formats[0]
        kind = args.kind or ("wush" if "wush" in wls[0].kinds else wls[0].kinds[-1])
        cases = [(wl, make_weights(wl), make_activations(wl)) for wl in wls]
        # the oracle's timing forks worker processes, so it runs before anything touches the GPU
        cpu = None
        if not args.no_cpu_baseline and not args.sweep:
            cpu = cpu_baseline(cases, fmt, kind, args.shared, args.cpu_seconds, host_workers(args.cpu_workers))

    import aware_block_transforms_amd as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.copy_reference:
        n = args.copy_reference << 18          # MiB -> float32 elements
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_reference_bytes": n * 4, "copies": args.steps}), flush=True)
        return

    if args.workload == "had256":
        return bench_had256(args, W, torch)
    if args.workload == "moments":
        return bench_moments(args, W, torch)
    if args.workload == "build":
        return bench_build(args, W, torch)
    if args.workload == "mfma_ceiling":
        return bench_mfma_ceiling(args, torch)

    if args.sweep:
        return bench_sweep(args, W, torch, cases[0])

    layers = [Layer(wl, fmt, kind, args.rotate, W, torch, Wt, X, shared=args.shared,
                    planes=not args.row_major_scales) for wl, Wt, X in cases]
    del cases

    ms_step, tq_ms, gm_ms = run_layer_steps(layers, W, torch, args.steps, args.warmup, args.rotate)

    flops = sum(L.gemm_flops() for L in layers)
    tq_bytes = sum(L.tq_bytes() for L in layers)
    tq_flops = sum(L.tq_flops() for L in layers)
    tq_t = sum(tq_ms) / 1e3
    gm_t = sum(gm_ms) / 1e3
    gemm_peak = {"mxfp4": MXFP4_TFLOPS, "nvfp4": FP16_TFLOPS, "int4": INT8_TOPS}[fmt]
    gemm_achieved = flops / gm_t / 1e12
    tq_alu = tq_flops / tq_t / 1e12
    tq_gbps = tq_bytes / tq_t / 1e9
    x_dtype = wls[0].dtype
    # dominant kernel by measured time
    dom_gemm = gm_t >= tq_t
    wname = "+".join(L.wl.name for L in layers)
    gemm_name = "wush_w4a4_gemm_mx_planes" if layers[0].planes else "wush_w4a4_gemm"
    roof_gemm = {"kernel": gemm_name, "bound": "mfma", "achieved": round(gemm_achieved, 2),
                 "peak": gemm_peak, "unit": "TFLOP/s", "frac": round(gemm_achieved / gemm_peak, 4),
                 "traffic": measured_traffic(gemm_name, [L.wl.name for L in layers]) if fmt == "mxfp4" else None,
                 "algorithmic_bytes": round(sum(L.gemm_bytes() for L in layers) / len(layers)),
                 "avg_us": round(gm_t * 1e6 / len(layers), 2)}
    if fmt == "int4":
        # the per-group fp32 rescale on the vector ALU bounds the INT4 matmul
        rescale = sum(INT4_RESCALE_OPS * L.M * L.N * (L.K // 32) for L in layers) / gm_t / 1e12
        roof_gemm.update({"bound": "alu", "achieved": round(rescale, 2), "peak": round(VALU_TOPS, 1),
                          "unit": "Top/s", "frac": round(rescale / VALU_TOPS, 4),
                          "int8_TOPS": round(gemm_achieved, 2), "int8_frac": round(gemm_achieved / INT8_TOPS, 4)})
    tq_name = ("wush_transform_quant_hd" if layers[0].hd else
               "wush_transform_quant_shared" if layers[0].group is not None else
               "wush_transform_quant_mx_planes" if layers[0].planes else "wush_transform_quant")
    # Each layer's transform+quantize is priced on the engine its kernel runs on
    # (tq_engine) and on HBM; the step's bound is the slower of the two summed
    # over layers.
    engines = [tq_engine(L) for L in layers]
    t_alu = sum(L.tq_flops() / (peak * 1e12) for L, (_, peak) in zip(layers, engines))
    t_hbm = tq_bytes / (HBM_GBPS * 1e9)
    tq_bound, tq_peak = engines[0]
    lnames = [L.wl.name for L in layers]
    if t_alu > t_hbm:
        roof_tq = {"kernel": tq_name, "bound": tq_bound, "achieved": round(tq_alu, 2),
                   "peak": round(tq_peak, 1), "unit": "TFLOP/s", "frac": round(t_alu / tq_t, 4),
                   "traffic": measured_traffic(tq_name, lnames) if fmt == "mxfp4" else None,
                   "algorithmic_bytes": round(tq_bytes / len(layers)), "avg_us": round(tq_t * 1e6 / len(layers), 2),
                   "hbm_GBps": round(tq_gbps, 1), "hbm_frac": round(tq_gbps / HBM_GBPS, 4)}
    else:
        roof_tq = {"kernel": tq_name, "bound": "hbm", "achieved": round(tq_gbps, 1),
                   "peak": HBM_GBPS, "unit": "GB/s", "frac": round(tq_gbps / HBM_GBPS, 4),
                   "traffic": measured_traffic(tq_name, lnames) if fmt == "mxfp4" else None,
                   "algorithmic_bytes": round(tq_bytes / len(layers)), "avg_us": round(tq_t * 1e6 / len(layers), 2),
                   **({"engine": tq_bound, "engine_frac": round(t_alu / tq_t, 4)} if t_alu > 0 else {})}
    if len(layers) > 1:
        roof_tq["per_layer_us"] = [round(t * 1e3, 2) for t in tq_ms]
        roof_gemm["per_layer_us"] = [round(t * 1e3, 2) for t in gm_ms]
        roof_gemm["per_layer_frac"] = [round(L.gemm_flops() / (t / 1e3) / 1e12 / gemm_peak, 4)
                                       for L, t in zip(layers, gm_ms)]
    out = {
        "metric": METRIC,
        "value": round(flops / (ms_step / 1e3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": fmt,
        "data": "synthetic",
        "config": {"workload": wname, "transform": kind, "format": fmt,
                   "x_dtype": x_dtype, "tokens": layers[0].M,
                   "layers": [[L.K, L.N] for L in layers], "rotate_buffers": args.rotate,
                   **({"shared_groups": args.shared} if layers[0].group is not None else {}),
                   "mx_scale_layout": "planes" if layers[0].planes else "row-major"},
        "quant_GBps": round(tq_gbps, 1),
        "tq_us": round(tq_t * 1e6, 2),
        "gemm_us": round(gm_t * 1e6, 2),
        "roofline": roof_gemm if dom_gemm else roof_tq,
        "tq_roofline": roof_tq,
        "gemm_roofline": roof_gemm,
    }
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


def bench_sweep(args, W, torch, case):
    """Every format x transform of one workload (the square sweep): one JSON line each.

    Each line times the step as the main bench does (transform+quantize, then
    the matmul, rotated buffers) and reports the layer loss of the pages'
    problem statement, sum((Yhat - W^T X)^2) / (d_out n), computed on the GPU by
    wush_layer_loss against W^T X taken in fp64 on the host (numpy) from the same
    seeded W and X.
    """
    wl, Wt, X = case
    t0 = time.time()
    Yref = (X.astype(np.float64) @ Wt.astype(np.float64).T).astype(np.float32)
    ref_s = time.time() - t0
    Yref_d = torch.from_numpy(Yref).cuda()
    del Yref
    lws = torch.empty(max(8, W.wush_loss_ws_bytes(wl.n, wl.d_out)) // 8, dtype=torch.float64, device="cuda")
    loss = torch.empty(1, dtype=torch.float64, device="cuda")
    results = []
    for fmt in wl.formats:
        for kind in wl.kinds:
            L = Layer(wl, fmt, kind, args.rotate, W, torch, Wt, X)
            ms_step, tq_ms, gm_ms = run_layer_steps([L], W, torch, args.steps, args.warmup, args.rotate)
            W.wush_layer_loss(L.Y, Yref_d, loss, lws)
            torch.cuda.synchronize()
            flops = L.gemm_flops()
            gm_t, tq_t = gm_ms[0] / 1e3, tq_ms[0] / 1e3
            bound, peak = tq_engine(L)
            t_alu = L.tq_flops() / (peak * 1e12)
            gemm_peak = {"mxfp4": MXFP4_TFLOPS, "nvfp4": FP16_TFLOPS, "int4": INT8_TOPS}[fmt]
            line = {"metric": METRIC, "value": round(flops / (ms_step / 1e3) / 1e12, 2), "unit": "TFLOP/s",
                    "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
                    "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": fmt,
                    "data": "synthetic",
                    "config": {"workload": wl.name, "transform": kind, "format": fmt, "x_dtype": wl.dtype,
                               "tokens": wl.n, "mx_scale_layout": "planes" if L.planes else "row-major"},
                    "layer_loss": loss.item(),
                    "tq_us": round(tq_t * 1e6, 2), "gemm_us": round(gm_t * 1e6, 2),
                    "quant_GBps": round(L.tq_bytes() / tq_t / 1e9, 1),
                    "tq_hbm_frac": round(L.tq_bytes() / tq_t / 1e9 / HBM_GBPS, 4),
                    "tq_engine_frac": round(t_alu / tq_t, 4) if t_alu else None,
                    "gemm_frac": round(flops / gm_t / 1e12 / gemm_peak, 4), "gemm_peak": gemm_peak}
            if fmt == "int4":
                rescale = INT4_RESCALE_OPS * L.M * L.N * (L.K // 32) / gm_t / 1e12
                line["gemm_rescale_frac"] = round(rescale / VALU_TOPS, 4)
            print(json.dumps(line), flush=True)
            results.append((fmt, kind, loss.item()))
            del L
            torch.cuda.empty_cache()
    print(json.dumps({"sweep_losses": {f"{f}/{k}": v for f, k, v in results}, "reference_s": round(ref_s, 1)}),
          flush=True)


def bench_had256(args, W, torch):
    from synth.gen import CONFIGS, make_weights, bf16_bits, bf16_round
    wl = CONFIGS["had256"]
    B = args.batch
    Wt = make_weights(wl)
    d_out, d_in = Wt.shape
    dev = "cuda"
    packed = torch.empty((W.wush_had256_packed_bytes(d_out, d_in),), dtype=torch.uint8, device=dev)
    W.wush_had256_pack_weights(torch.from_numpy(Wt).to(dev), packed)
    x = bf16_round(np.random.default_rng([5, 1]).standard_normal((B, d_in)).astype(np.float32))
    xd = torch.from_numpy(bf16_bits(x).view(np.int16)).to(dev)
    # enough weight copies that they overflow the 256 MB Infinity Cache twice
    # over, so every step streams its weights from HBM
    wbytes = packed.numel()
    nrot = max(args.rotate, -(-2 * 256 * 2**20 // wbytes))
    P = [packed] + [packed.clone() for _ in range(nrot - 1)]
    y = torch.empty((B, d_out), dtype=torch.float32, device=dev)
    ws = torch.empty(W.wush_had256_gemv_ws_bytes(B, d_in), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        W.wush_had256_gemv(xd, P[i % nrot], y, ws=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        W.wush_had256_gemv(xd, P[i % nrot], y, ws=ws)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    byts = wbytes + B * d_in * 2 + B * d_out * 4
    gbps = byts / (ms / 1e3) / 1e9
    flops = 2.0 * B * d_out * d_in
    out = {"metric": "Hadamard-256 3-bit GEMV weight stream GB/s", "value": round(gbps, 1), "unit": "GB/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int3+fp32",
           "data": "synthetic",
           "config": {"workload": wl.name, "batch": B, "d_in": d_in, "d_out": d_out, "weight_copies": nrot},
           "tflops": round(flops / (ms / 1e3) / 1e12, 3),
           "roofline": {"kernel": "wush_had256_gemv", "bound": "hbm", "achieved": round(gbps, 1),
                        "peak": HBM_GBPS, "unit": "GB/s", "frac": round(gbps / HBM_GBPS, 4),
                        "traffic": measured_traffic("wush_had256_gemv_b%d" % B, [wl.name]),
                        "avg_us": round(ms * 1e3, 2)}}
    print(json.dumps(out), flush=True)


def bench_moments(args, W, torch):
    """Calibration block moments on the GPU for the Qwen3-8B up-projection's activations (bs 32)."""
    from synth.gen import CONFIGS, make_activations, bf16_bits
    wl = CONFIGS["qwen3_8b_up"]
    X = make_activations(wl)
    n, d_in = X.shape
    bs = 32
    dev = "cuda"
    xd = torch.from_numpy(bf16_bits(X).view(np.int16)).to(dev).view(torch.bfloat16)
    Xs = [xd] + [xd.clone() for _ in range(args.rotate - 1)]
    Sx = torch.empty((d_in // bs, bs, bs), dtype=torch.float32, device=dev)
    ws = torch.empty(W.wush_block_moments_dev_ws_bytes(bs, n, d_in), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        W.wush_block_moments_dev(bs, Xs[i % args.rotate], Sx, ws=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        W.wush_block_moments_dev(bs, Xs[i % args.rotate], Sx, ws=ws)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    flops = 2.0 * n * d_in * bs            # the full bs x bs product per block and token
    tflops = flops / (ms / 1e3) / 1e12
    out = {"metric": "calibration block moments TFLOP/s (fp64 accumulation)", "value": round(tflops, 3),
           "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f64",
           "data": "synthetic", "config": {"workload": wl.name + "-moments", "tokens": n, "d_in": d_in, "bs": bs},
           "roofline": {"kernel": "wush_block_moments_dev", "bound": "alu", "achieved": round(tflops, 3),
                        "peak": FP64_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / FP64_TFLOPS, 4),
                        "traffic": None, "avg_us": round(ms * 1e3, 2)}}
    print(json.dumps(out), flush=True)


def bench_build(args, W, torch):
    """The offline transform builder on the GPU for the Qwen3-8B up-projection (WUSH, bs 32), next to the host one."""
    from synth.gen import CONFIGS, make_weights, make_activations
    wl = CONFIGS["qwen3_8b_up"]
    Wt, X = make_weights(wl), make_activations(wl)
    d_out, d_in = Wt.shape
    bs, nblk = 32, d_in // 32
    Sx = np.empty((nblk, bs, bs), np.float32)
    W.wush_block_moments(bs, X, Sx)
    dev = "cuda"
    Wd, Sd = torch.from_numpy(Wt).to(dev), torch.from_numpy(Sx).to(dev)
    Tx = torch.empty((nblk, bs, bs), dtype=torch.float32, device=dev)
    Tw = torch.empty_like(Tx)
    ws = torch.empty(W.wush_build_transforms_dev_ws_bytes(bs, d_in), dtype=torch.uint8, device=dev)
    for _ in range(max(1, args.warmup // 5)):
        W.wush_build_transforms_dev("wush", bs, Wd, Sd, Tx, Tw, ws=ws)
    steps = max(1, args.steps // 10)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        W.wush_build_transforms_dev("wush", bs, Wd, Sd, Tx, Tw, ws=ws)   # synchronises
    ms = (time.perf_counter() - t0) * 1e3 / steps
    hx, hw = np.empty((nblk, bs, bs), np.float32), np.empty((nblk, bs, bs), np.float32)
    t0 = time.perf_counter()
    W.wush_build_transforms("wush", bs, Wt, Sx, hx, hw)
    host_ms = (time.perf_counter() - t0) * 1e3
    same = bool(np.array_equal(Tx.cpu().numpy(), hx) and np.array_equal(Tw.cpu().numpy(), hw))
    moment_flops = 2.0 * d_out * nblk * bs * (bs + 1) / 2        # the weight moments dominate the arithmetic
    tflops = moment_flops / (ms / 1e3) / 1e12
    out = {"metric": "transform builder blocks/s (offline, fp64)", "value": round(nblk / (ms / 1e3), 1),
           "unit": "blocks/s", "n_gpus": 1, "steps": steps, "warmup": max(1, args.warmup // 5),
           "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f64", "data": "synthetic",
           "config": {"workload": wl.name + "-build", "d_out": d_out, "d_in": d_in, "bs": bs, "kind": "wush"},
           "host_builder_ms": round(host_ms, 2), "host_threads": os.cpu_count(), "identical_to_host": same,
           "roofline": {"kernel": "wush_build_transforms_dev", "bound": "alu", "achieved": round(tflops, 4),
                        "peak": FP64_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / FP64_TFLOPS, 5),
                        "traffic": None, "avg_us": round(ms * 1e3, 1)}}
    print(json.dumps(out), flush=True)


def bench_mfma_ceiling(args, torch):
    """Matrix-core rates with operands in registers (libwush_ceiling.so).

    FP4 block-scaled MFMA streams (the W4A4 matmul's instruction) on random and
    on zero operand bits, one wave per SIMD, and on random operands that change
    every MFMA as in the matmul; fp32 16x16x4 MFMA (the dense
    transform's instruction) as 2 or 8 accumulation chains of 8 steps, at one
    and four waves per SIMD, alone and with independent vector FMAs between the
    MFMAs, plus the vector FMAs alone.  The value is the random-operand FP4
    rate of the 16x16x128 instruction.
    """
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "aware_block_transforms_amd", "libwush_ceiling.so"))
    lib.wush_ceiling_fp4.argtypes = [ctypes.c_int] * 3 + [ctypes.c_void_p] * 3
    lib.wush_ceiling_f32.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p] * 3
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    rng = np.random.default_rng([7, 7])
    rand_bits = torch.from_numpy(rng.integers(0, 2**32, 1024 * 16, dtype=np.uint64).astype(np.uint32).view(np.int32)).cuda()
    zero_bits = torch.zeros(1024 * 16, dtype=torch.int32, device="cuda")
    f32_src = torch.from_numpy(rng.standard_normal(1024 * 16).astype(np.float32)).cuda()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(cus * 4 * 256, dtype=torch.float32, device="cuda")

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        best = None
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) / 1e3
            best = t if best is None else min(best, t)
        return best

    res = {}
    it4 = 4000
    for which, name, per_instr, nacc in ((0, "16x16x128", 16 * 16 * 128 * 2, 8), (1, "32x32x64", 32 * 32 * 64 * 2, 4)):
        for label, bits in (("random", rand_bits), ("zero", zero_bits)):
            def run(w=which, b=bits):
                assert lib.wush_ceiling_fp4(w, cus, it4, b.data_ptr(), out.data_ptr(), sp) == 0
            t = timed(run)
            res[f"fp4_{name}_{label}_TFLOPs"] = round(cus * 4 * it4 * nacc * per_instr / t / 1e12, 1)
    # operands that change every MFMA, in the matmul's order (64 MFMAs per iteration)
    it_vary = it4 // 8

    def run_vary():
        assert lib.wush_ceiling_fp4(2, cus, it_vary, rand_bits.data_ptr(), out.data_ptr(), sp) == 0
    t = timed(run_vary)
    res["fp4_16x16x128_random_varying_TFLOPs"] = round(cus * 4 * it_vary * 64 * 16 * 16 * 128 * 2 / t / 1e12, 1)
    it32 = 4000
    for wps in (1, 4):
        for nchain, nvalu in ((2, 0), (8, 0), (2, 4), (2, 8), (8, 8), (0, 8)):
            def run(c=nchain, v=nvalu, w=wps):
                assert lib.wush_ceiling_f32(c, v, cus * w, it32, f32_src.data_ptr(), out.data_ptr(), sp) == 0
            t = timed(run)
            key = f"f32_{wps}w_chains{nchain}_valu{nvalu}"
            res[key + "_us"] = round(t * 1e6, 1)
            if nchain:
                res[key + "_TFLOPs"] = round(cus * 4 * wps * it32 * nchain * 8 * 2048 / t / 1e12, 1)
    # HBM read rate of the transform step's tile pattern against flat reads of
    # the same bytes (the Qwen3-14B down-projection's bf16 activations)
    lib.wush_ceiling_read.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    rows, row_bytes = 16384, 17408 * 2
    nbuf = 3
    bufs = [torch.empty(rows * row_bytes, dtype=torch.uint8, device="cuda") for _ in range(nbuf)]
    for b in bufs:
        b.fill_(1)
    rout = torch.empty(16 << 20, dtype=torch.int32, device="cuda")
    for pattern, name, blocks, tpw in ((0, "flat", cus * 8, 0), (1, "tiles_upw16", 0, 16), (1, "tiles_upw64", 0, 64)):
        state = {"i": 0}

        def run(p=pattern, bl=blocks, t=tpw, st=state):
            b = bufs[st["i"] % nbuf]
            st["i"] += 1
            assert lib.wush_ceiling_read(p, b.data_ptr(), rows, row_bytes, bl, t, rout.data_ptr(), sp) == 0
        t = timed(run)
        res[f"read_{name}_GBps"] = round(rows * row_bytes / t / 1e9, 1)
    del bufs
    v = res["fp4_16x16x128_random_TFLOPs"]
    print(json.dumps({"metric": "matrix-core ceiling, operands in registers", "value": v, "unit": "TFLOP/s",
                      "n_gpus": 1, "steps": 5, "warmup": 1, "ms_per_step": None, "higher_is_better": True,
                      "scaling": "weak", "vs_baseline": None, "dtype": "fp4", "data": "synthetic",
                      "config": {"workload": "mfma-ceiling", "cus": cus},
                      "roofline": {"kernel": "fp4_stream 16x16x128", "bound": "mfma", "achieved": v,
                                   "peak": MXFP4_TFLOPS, "unit": "TFLOP/s", "frac": round(v / MXFP4_TFLOPS, 4),
                                   "traffic": None},
                      "rates": res}), flush=True)


if __name__ == "__main__":
    main()
