"""Throughput of the block-scaled FP8 GEMM (NT, E4M3, FP32 g x g block scales,
BF16 out) on one MI355X, printed as one JSON line.

A step is one call of dg_gemm_fp8_nt over one input set: the whole method
(tile schedule, HBM->LDS staging, scale fetch, FP8 MFMA partials, per-segment
FP32 promotion, BF16 epilogue) runs inside that one kernel launch.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--fmt e4m3|e5m2|e4m3xe5m2|e5m2xe4m3] [--gran 64|128|256]
                  [--bias] [--act none|relu|gelu] [--sa-rows 1] [--layout nt|nn|tt|tn]
                  [--workspace]

--fmt and --gran run the same workload with the operands in another FP8
format or with another block granularity (default: E4M3 and the workload's
own g); --bias and --act add the fused epilogue out = act(C + bias) (bias a
seeded N(0, 0.5) vector); --sa-rows 1 scales A per row and K segment (1 x g
blocks, quantised by dg_quantize_fp8_rows) instead of per g x g block;
--layout stores A as [K,M] (tt, tn) and/or B as [K,N] (nn, tn), transposed
on the GPU before timing, and calls dg_gemm_fp8_layout; --workspace calls
dg_gemm_fp8_ws with a workspace instead (small-M shapes may then split K over
workgroups); the default run is the E4M3 NT workload as specified.

Inputs: FP32 matrices drawn from the seeded generators in ``synth`` (the
workload's shapes and value distributions), copied to the GPU and block
quantised there by the library's own quantiser (dg_quantize_fp8_blocks), so
every byte the GEMM reads is resident in HBM before the timed region. Input
sets are cloned so that consecutive steps rotate over enough distinct
buffers (> 2x the 256 MB Infinity Cache) that the operands come from HBM,
not from the last-level cache.

Timing: W untimed warm-up steps (eager calls), then K steps between two HIP
events on the stream the GEMM is launched on, bracketed by
torch.cuda.synchronize(). The K steps are replays of a HIP graph that
captures L consecutive launches (L the largest divisor of K up to 100; the
graph is replayed once untimed first, and its outputs are checked bit for bit
against the eager calls'), so the host's per-call cost does not sit between
kernels of a few microseconds. value = 2*M*N*K / (time per step) in TFLOP/s.

Sustained clock: after the timed steps the same graph replays for
--clock-window seconds (default 3, untimed) while a host thread samples
`amd-smi metric --clock --power`; config.sustained_clock gives the median of
the samples' mean gfx clock over the XCDs and of the socket power (null
without amd-smi). It says at what clock the measured rate was reached.

roofline: the GEMM kernel is the only kernel of a step. Its average launch
duration is the timed region / K. achieved = algorithmic FLOPs (MFMA-bound
shapes) or algorithmic bytes (HBM-bound shapes) per launch / that duration,
against MI355X's published dense FP8 MFMA peak (5.0 PFLOP/s) or HBM
bandwidth (8 TB/s). Algorithmic bytes = M*K + N*K (FP8 operands, once) +
4*(ceil(M/g) + ceil(N/g))*K/g (FP32 scales) + 2*M*N (BF16 out).

cpu_baseline: the CPU oracle (plain FP64, test infrastructure) timed on the
host's cores over a bounded sample of the same workload: whole output rows,
as many as fit in about 10 s, or the whole output repeated for that long.
"""

from __future__ import annotations

import argparse
import json
import math
import statistics
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402  (seeded inputs only; no GEMM arithmetic)

PEAK_FP8_TFLOPS = 5000.0  # MI355X dense FP8 MFMA (published)
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E (published)
MALL_BYTES = 256 << 20    # Infinity Cache
DEFAULT_WORKLOAD = 4      # large square M=N=K=8192, g=128: the largest shape, MFMA-bound

# HBM traffic of the GEMM kernel per launch, from rocprofv3 --pmc FETCH_SIZE and
# WRITE_SIZE (each scaled by the copy-kernel calibration factor), keyed by
# workload and tagged with the hash of the sources of the kernel class that
# workload runs (KERNEL_SOURCES) as they were when the counters were taken. A
# different hash means the kernel changed since: traffic is null.
TRAFFIC = {
    "square8192": {"src": "bb28682c6310a4e5", "bytes": 940560677},
    "prefill_m4096_n7168_k2048": {"src": "bb28682c6310a4e5", "bytes": 151255113},
    "longk_m2000_n4000_k16384_g64": {"src": "bb28682c6310a4e5", "bytes": 278791791},
    "decode_m64_n4096_k7168": {"src": "86e89fe55db16f3c", "bytes": 33667236},
}

# Sources that make up each workload's kernel: its class's device code, the
# shared device header, the argument header and the host dispatch.
_COMMON_SOURCES = ("gemm_common.h", "gemm_fp8_nt.h", "dg_host.hip")
KERNEL_SOURCES = {
    "decode_m64_n4096_k7168": ("gemm_fp8_stream.hip",) + _COMMON_SOURCES,
    "square8192": ("gemm_fp8_big.h", "gemm_fp8_nt_big.hip") + _COMMON_SOURCES,
    "prefill_m4096_n7168_k2048": ("gemm_fp8_big.h", "gemm_fp8_nt_big.hip") + _COMMON_SOURCES,
    "longk_m2000_n4000_k16384_g64": ("gemm_fp8_big.h", "gemm_fp8_nt_big.hip") + _COMMON_SOURCES,
}


def kernel_source_hash(workload: str) -> str | None:
    import hashlib

    names = KERNEL_SOURCES.get(workload)
    if names is None:
        return None
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "fp8_block_scaled_scales_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def workload_by_name(key: str) -> int:
    for c, w in synth.WORKLOADS.items():
        if key in (str(c), w["name"]):
            return c
    raise SystemExit("unknown workload %r; choose one of %s" % (
        key, ", ".join("%d=%s" % (c, w["name"]) for c, w in synth.WORKLOADS.items())))


FORMATS = {"e4m3": (0, 0), "e5m2": (1, 1), "e4m3xe5m2": (0, 1), "e5m2xe4m3": (1, 0)}
ACTS = {"none": 0, "relu": 1, "gelu": 2}
BIAS_SEED = 9901


def make_bias(N: int):
    return synth.normal(BIAS_SEED, (N,), sigma=0.5).astype("float32")


def algorithmic(w, g=None, sa_rows=None) -> tuple[float, float]:
    M, N, K = w["M"], w["N"], w["K"]
    g = g or w["g"]
    ra = sa_rows or g  # A rows per factor
    flops = 2.0 * M * N * K
    nbytes = M * K + N * K + 4 * (math.ceil(M / ra) + math.ceil(N / g)) * (K // g) + 2 * M * N
    return flops, float(nbytes)


def bound_of(w) -> str:
    flops, nbytes = algorithmic(w)
    # machine balance 5.0e15 / 8e12 = 625 FLOP/B
    return "hbm" if flops / nbytes < PEAK_FP8_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9) else "mfma"


def make_inputs(c: int, dev, g: int, fa: int = 0, fb: int = 0, sa_rows: int | None = None):
    """Quantised GPU inputs of workload c at granularity g, formats fa/fb: (a8, sa, b8, sb)."""
    import torch

    import fp8_block_scaled_scales_amd as dg

    xa = torch.from_numpy(synth.make_a(c)).to(dev)
    if sa_rows == 1:
        a8, sa = dg.dg_quantize_fp8_rows(xa, gran=g, fmt=fa)
    else:
        a8, sa = dg.dg_quantize_fp8_blocks(xa, gran=g, fmt=fa)
    del xa
    xb = torch.from_numpy(synth.make_b(c)).to(dev)
    b8, sb = dg.dg_quantize_fp8_blocks(xb, gran=g, fmt=fb)
    del xb
    torch.cuda.synchronize(dev)
    return a8, sa, b8, sb


LAYOUTS = {"nt": 0, "nn": 1, "tt": 2, "tn": 3}


def gpu_leg(c: int, steps: int, warmup: int, sets: int | None, g: int, fa: int = 0, fb: int = 0,
            bias: bool = False, act: int = 0, sa_rows: int | None = None, layout: int = 0, ws: bool = False):
    import torch

    import fp8_block_scaled_scales_amd as dg

    w = synth.WORKLOADS[c]
    M, N, K = w["M"], w["N"], w["K"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    a8, sa, b8, sb = make_inputs(c, dev, g, fa, fb, sa_rows)
    if layout & 2:
        a8 = a8.t().contiguous()  # A stored [K, M]
    if layout & 1:
        b8 = b8.t().contiguous()  # B stored [K, N]
    set_bytes = a8.numel() + b8.numel() + 4 * (sa.numel() + sb.numel()) + 2 * M * N
    if sets is None:
        sets = max(2, min(64, math.ceil(2 * MALL_BYTES / set_bytes) + 1))
    bufs = [(a8, sa, b8, sb, torch.empty((M, N), dtype=torch.bfloat16, device=dev))]
    for _ in range(sets - 1):
        bufs.append((a8.clone(), sa.clone(), b8.clone(), sb.clone(),
                     torch.empty((M, N), dtype=torch.bfloat16, device=dev)))
    stream = torch.cuda.current_stream(dev)
    print("bench: workload %d %s, %d input sets of %.1f MB, tile %s" % (
        c, w["name"], sets, set_bytes / 1e6, dg.dg_query_tile(M, N, K, g, layout, workspace=ws)), file=sys.stderr,
        flush=True)

    tbias = torch.from_numpy(make_bias(N)).to(dev) if bias else None
    # one workspace for every call: they all run on one stream
    wsbuf = dg.dg_workspace(M, N, K, g, layout, device=dev) if ws else None

    def launch(i, st):
        x = bufs[i % sets]
        if ws:
            dg.dg_gemm_fp8_ws(x[0], x[2], x[1], x[3], out=x[4], gran=g, layout=layout, sa_rows=sa_rows, fmt_a=fa,
                              fmt_b=fb, bias=tbias, act=act, workspace=wsbuf, stream=st)
        elif layout and sa_rows == 1:
            # per-row A factors with a transposed layout: the workspace call, without a workspace
            dg.dg_gemm_fp8_ws(x[0], x[2], x[1], x[3], out=x[4], gran=g, layout=layout, sa_rows=1, fmt_a=fa, fmt_b=fb,
                              bias=tbias, act=act, stream=st)
        elif layout:
            dg.dg_gemm_fp8_layout(x[0], x[2], x[1], x[3], out=x[4], gran=g, layout=layout, fmt_a=fa, fmt_b=fb,
                                  bias=tbias, act=act, stream=st)
        elif sa_rows == 1:
            dg.dg_gemm_fp8_nt_ex(x[0], x[2], x[1], x[3], out=x[4], gran=g, sa_rows=1, fmt_a=fa, fmt_b=fb, bias=tbias,
                                 act=act, stream=st)
        elif bias or act:
            dg.dg_gemm_fp8_nt_epi(x[0], x[2], x[1], x[3], out=x[4], gran=g, fmt_a=fa, fmt_b=fb, bias=tbias, act=act,
                                  stream=st)
        elif fa == 0 and fb == 0:
            dg.dg_gemm_fp8_nt(x[0], x[2], x[1], x[3], out=x[4], gran=g, stream=st)
        else:
            dg.dg_gemm_fp8_nt_fmt(x[0], x[2], x[1], x[3], out=x[4], gran=g, fmt_a=fa, fmt_b=fb, stream=st)

    # Warm-up, eager: also allocates the library's split-K workspace and runs
    # its one-time device check, neither of which may happen under capture.
    for i in range(max(1, warmup)):
        launch(i, stream)
    torch.cuda.synchronize(dev)
    eager = bufs[0][4].clone()  # every set holds the same inputs, so every output must match it

    # The timed steps are replays of a captured graph of L launches (L divides
    # K), so the host's per-call cost does not starve the GPU between these
    # few-microsecond kernels. The graph holds kernel launches only.
    L = max(d for d in range(1, min(steps, 100) + 1) if steps % d == 0)
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for i in range(L):
                launch(i, cap)
    torch.cuda.synchronize(dev)
    for x in bufs:
        x[4].zero_()  # so the check below sees what the replay wrote
    graph.replay()  # untimed: uploads the graph; replays run on the current stream
    torch.cuda.synchronize(dev)
    assert torch.cuda.current_stream(dev) == stream
    for i in range(min(sets, L)):
        if not torch.equal(bufs[i][4].view(torch.int16), eager.view(torch.int16)):
            raise SystemExit("graph replay output differs from the eager call's")
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    # The timed region is the K steps between start and end; events between
    # the replays split it into up to five trials of whole replays, for the
    # spread of the per-call time (the value is the whole region's).
    reps = steps // L
    cuts = sorted({round(i * reps / 5) for i in range(6)})
    marks = [torch.cuda.Event(enable_timing=True) for _ in cuts[1:-1]]
    start.record(stream)
    for r in range(reps):
        if r in cuts[1:-1]:
            marks[cuts.index(r) - 1].record(stream)
        graph.replay()
    end.record(stream)
    torch.cuda.synchronize(dev)
    ms = start.elapsed_time(end) / steps
    bounds = [start] + marks + [end]
    trials = [bounds[i].elapsed_time(bounds[i + 1]) / ((cuts[i + 1] - cuts[i]) * L) for i in range(len(bounds) - 1)]
    finite = bool(torch.isfinite(bufs[(steps - 1) % sets][4].float()).all().item())
    clock = clock_window(graph, dev, ms * L) if clock_s > 0 else None
    return ms, sets, finite, L, trials, clock


def _smi_sample():
    """One amd-smi reading of GPU 0: (mean gfx clock over the XCDs in MHz,
    socket power in W), or None when amd-smi is missing or says nothing."""
    try:
        res = subprocess.run(["amd-smi", "metric", "-g", "0", "--clock", "--power", "--json"], capture_output=True,
                             text=True, timeout=20)
        txt = res.stdout
        starts = [i for i in (txt.find("{"), txt.find("[")) if i >= 0]
        d = json.loads(txt[min(starts):])
        g = d["gpu_data"][0] if isinstance(d, dict) else d[0]
        clks = [v["clk"]["value"] for k, v in g["clock"].items()
                if k.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict)]
        pw = g.get("power", {}).get("socket_power", {})
        return (sum(clks) / len(clks) if clks else None), (pw.get("value") if isinstance(pw, dict) else None)
    except Exception:
        return None


clock_s = 3.0  # length of the untimed clock window after the timed steps (0: none)


def clock_window(graph, dev, graph_ms: float):
    """The sustained gfx clock under this load: after the timed steps, the
    same graph replays for about clock_s seconds (untimed) while a host thread
    samples amd-smi; returns the median of the samples' mean gfx clock over
    the XCDs and of the socket power, or None without amd-smi."""
    import threading

    import torch

    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            r = _smi_sample()
            if r is None:
                return
            samples.append(r)

    reps = max(1, int(clock_s * 1e3 / max(graph_ms, 1e-3)))
    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    for r in range(reps):
        graph.replay()
        if r % 16 == 15:
            torch.cuda.synchronize(dev)  # keep the queue short, so the window lasts as long as the replays
    torch.cuda.synchronize(dev)
    stop.set()
    th.join(timeout=30)
    clk = [c for c, _ in samples if c]
    pw = [p for _, p in samples if p]
    if not clk:
        return None
    return {"gfx_mhz_median": round(statistics.median(clk), 1), "socket_power_w_median": statistics.median(pw) if pw else None,
            "samples": len(clk), "source": "amd-smi metric --clock --power, sampled while the graph replayed for %.1f s "
                                            "after the timed steps (untimed)" % clock_s}


QUANT_IN = {"f32": 4, "bf16": 2, "f16": 2}  # input element kinds of the quantiser and their bytes


def quant_leg(c: int, operand: str, steps: int, warmup: int, sets: int | None, g: int, fmt: int, per_row: bool,
              in_kind: str = "f32"):
    """The GPU quantiser on workload c's A or B (FP32, or rounded to BF16 / FP16 before the timed region):
    per-call time over rotating input sets."""
    import torch

    import fp8_block_scaled_scales_amd as dg

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = torch.from_numpy(synth.make_a(c) if operand == "a" else synth.make_b(c)).to(dev)
    if in_kind != "f32":
        x = x.to(torch.bfloat16 if in_kind == "bf16" else torch.float16)
    rows, cols = x.shape
    nblocks = (rows if per_row else math.ceil(rows / g)) * (cols // g)
    set_bytes = (QUANT_IN[in_kind] + 1) * rows * cols + 4 * nblocks  # input in, FP8 codes and FP32 factors out
    if sets is None:
        sets = max(2, min(64, math.ceil(2 * MALL_BYTES / set_bytes) + 1))
    bufs = [(x if i == 0 else x.clone(), torch.empty((rows, cols), dtype=torch.uint8, device=dev),
             torch.empty(nblocks, dtype=torch.float32, device=dev)) for i in range(sets)]
    if in_kind == "f32":
        fn = dg.dg_quantize_fp8_rows if per_row else dg.dg_quantize_fp8_blocks
    else:
        fn = dg.dg_quantize_fp8_rows_typed if per_row else dg.dg_quantize_fp8_blocks_typed
    stream = torch.cuda.current_stream(dev)

    def launch(i, st):
        xx, q, sc = bufs[i % sets]
        fn(xx, gran=g, fmt=fmt, q=q, scales=sc.view(-1, cols // g), stream=st)

    for i in range(max(1, warmup)):
        launch(i, stream)
    torch.cuda.synchronize(dev)
    eager = (bufs[0][1].clone(), bufs[0][2].clone())
    L = max(d for d in range(1, min(steps, 100) + 1) if steps % d == 0)
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for i in range(L):
                launch(i, cap)
    torch.cuda.synchronize(dev)
    for _, q, sc in bufs:
        q.zero_()
        sc.zero_()
    graph.replay()
    torch.cuda.synchronize(dev)
    for i in range(min(sets, L)):  # every set holds the same input
        if not (torch.equal(bufs[i][1], eager[0]) and torch.equal(bufs[i][2].view(torch.int32), eager[1].view(torch.int32))):
            raise SystemExit("graph replay output differs from the eager call's")
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps // L):
        graph.replay()
    end.record(stream)
    torch.cuda.synchronize(dev)
    ms = start.elapsed_time(end) / steps
    return ms, sets, L, rows, cols, nblocks


def pipeline_leg(c: int, steps: int, warmup: int, sets: int | None, g: int):
    """Workload c as a layer runs it (DeepGEMM实战 §4.4: weights quantised offline, activations online): per
    step, A in BF16 quantised on the GPU with 1 x g factors, then the GEMM against B quantised once beforehand.
    Times the pipeline, the quantiser alone and the GEMM alone, each as replays of its own graph."""
    import torch

    import fp8_block_scaled_scales_amd as dg

    w = synth.WORKLOADS[c]
    M, N, K = w["M"], w["N"], w["K"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    a16 = torch.from_numpy(synth.make_a(c)).to(dev).to(torch.bfloat16)
    xb = torch.from_numpy(synth.make_b(c)).to(dev)
    b8, sb = dg.dg_quantize_fp8_blocks(xb, gran=g)  # the weights, quantised once (untimed)
    del xb
    set_bytes = 2 * M * K + M * K + 4 * M * (K // g) + b8.numel() + 4 * sb.numel() + 2 * M * N
    if sets is None:
        sets = max(2, min(64, math.ceil(2 * MALL_BYTES / set_bytes) + 1))
    bufs = []
    for i in range(sets):
        bufs.append((a16 if i == 0 else a16.clone(), torch.empty((M, K), dtype=torch.uint8, device=dev),
                     torch.empty((M, K // g), dtype=torch.float32, device=dev), b8 if i == 0 else b8.clone(),
                     sb if i == 0 else sb.clone(), torch.empty((M, N), dtype=torch.bfloat16, device=dev)))
    stream = torch.cuda.current_stream(dev)

    def quant(i, st):
        x = bufs[i % sets]
        dg.dg_quantize_fp8_rows_typed(x[0], gran=g, q=x[1], scales=x[2], stream=st)

    def gemm(i, st):
        x = bufs[i % sets]
        dg.dg_gemm_fp8_nt_ex(x[1], x[3], x[2], x[4], out=x[5], gran=g, sa_rows=1, stream=st)

    def both(i, st):
        quant(i, st)
        gemm(i, st)

    for i in range(max(1, warmup)):
        both(i, stream)
    torch.cuda.synchronize(dev)
    eager = bufs[0][5].clone()
    L = max(d for d in range(1, min(steps, 100) + 1) if steps % d == 0)

    def timed(fn):
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream(dev)
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            with torch.cuda.graph(graph, stream=cap):
                for i in range(L):
                    fn(i, cap)
        torch.cuda.synchronize(dev)
        graph.replay()  # untimed: uploads the graph
        torch.cuda.synchronize(dev)
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(steps // L):
            graph.replay()
        end.record(stream)
        torch.cuda.synchronize(dev)
        return start.elapsed_time(end) / steps

    for x in bufs:
        x[5].zero_()
    ms_pipe = timed(both)
    for i in range(min(sets, L)):
        if not torch.equal(bufs[i][5].view(torch.int16), eager.view(torch.int16)):
            raise SystemExit("graph replay output differs from the eager pipeline's")
    ms_quant = timed(quant)
    ms_gemm = timed(gemm)
    return ms_pipe, ms_quant, ms_gemm, sets, L


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def cpu_leg(c: int, g: int, fa: int = 0, fb: int = 0, bias: bool = False, act: int = 0, budget_s: float = 10.0,
            sa_rows: int | None = None, layout: int = 0):
    """The oracle on a bounded sample of workload c, in TFLOP/s (FP64 on the host)."""
    import numpy as np

    import oracle

    w = synth.WORKLOADS[c]
    M, N, K = w["M"], w["N"], w["K"]
    threads = oracle.default_threads()
    if sa_rows == 1:
        a8, sa = oracle.quantize_rows_fmt(synth.make_a(c), g, fa)
    else:
        a8, sa = oracle.quantize_blocks_fmt(synth.make_a(c), g, fa)
    b8, sb = oracle.quantize_blocks_fmt(synth.make_b(c), g, fb)

    bvec = make_bias(N) if bias else None

    a_st = np.ascontiguousarray(a8.T) if layout & 2 else a8
    b_st = np.ascontiguousarray(b8.T) if layout & 1 else b8

    def ref(rows=None):
        if sa_rows == 1:
            # per-row A factors: the oracle on the logical operands (the stored layout changes no product)
            r = oracle.gemm_ref_rowa(a8, b8, sa, sb, g, fa, fb, rows=rows)
        elif layout:
            r = oracle.gemm_ref_layout(a_st, b_st, sa, sb, g, layout, M, N, K, fa, fb, rows=rows)
        elif fa == 0 and fb == 0:
            r = oracle.gemm_ref(a8, b8, sa, sb, g, rows=rows)
        else:
            r = oracle.gemm_ref_fmt(a8, b8, sa, sb, g, fa, fb, rows=rows)
        return oracle.epilogue(r, bvec, act) if (bias or act) else r

    # probe: one row per thread
    probe = np.arange(min(M, threads), dtype=np.int64)
    t0 = time.perf_counter()
    ref(probe)
    per_row = (time.perf_counter() - t0) / probe.size
    rows = int(budget_s / max(per_row, 1e-9))
    rows = max(threads, (rows // threads) * threads)
    if rows < M:
        sel = np.linspace(0, M - 1, rows).astype(np.int64)
        t0 = time.perf_counter()
        ref(sel)
        dt = time.perf_counter() - t0
        done = 2.0 * rows * N * K
        sample = "%d of %d output rows (evenly spaced) x all %d columns, K=%d" % (rows, M, N, K)
    else:
        reps, dt, done = 0, 0.0, 0.0
        t0 = time.perf_counter()
        while dt < budget_s:
            ref()
            reps += 1
            dt = time.perf_counter() - t0
        done = 2.0 * M * N * K * reps
        sample = "the whole %dx%d output, %d times, K=%d" % (M, N, reps, K)
    return {"value": done / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": sample + " (FP64, %.1f s; %d threads of the host's %d hardware threads, within its CPU "
                               "quota of %s and one GPU's CPU share of %d; %s)" % (
                dt, threads, oracle.host_threads(), oracle.cpu_quota(), oracle.CPU_SHARE, _cpu_model())}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=str(DEFAULT_WORKLOAD),
                    help="workload number or name (default: the large square M=N=K=8192)")
    ap.add_argument("--sets", type=int, default=None, help="input sets rotated over (default: defeat the MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fmt", default="e4m3", choices=sorted(FORMATS),
                    help="operand formats, A x B (default e4m3: both E4M3FN)")
    ap.add_argument("--gran", type=int, default=None, choices=(64, 128, 256),
                    help="block granularity (default: the workload's)")
    ap.add_argument("--bias", action="store_true", help="fused epilogue: add a bias vector")
    ap.add_argument("--act", default="none", choices=sorted(ACTS), help="fused epilogue activation")
    ap.add_argument("--layout", default="nt", choices=sorted(LAYOUTS),
                    help="operand storage: A [M,K] or [K,M] (first letter n / t), B [N,K] or [K,N] (t / n)")
    ap.add_argument("--clock-window", type=float, default=3.0, metavar="S",
                    help="after the timed steps, keep replaying for S seconds (untimed) while sampling the gfx "
                         "clock and power with amd-smi (0: skip)")
    ap.add_argument("--workspace", action="store_true",
                    help="call dg_gemm_fp8_ws with a workspace (small-M shapes may then split K over workgroups)")
    ap.add_argument("--sa-rows", type=int, default=None, choices=(1,),
                    help="1: per-row A factors (1 x g blocks) instead of g x g blocks")
    ap.add_argument("--quant", default=None, choices=("a", "b"),
                    help="time the GPU quantiser on the workload's A or B instead of the GEMM (g x g "
                         "blocks, or 1 x g with --sa-rows 1; format from the first letter pair of --fmt)")
    ap.add_argument("--quant-in", default="f32", choices=tuple(QUANT_IN),
                    help="with --quant: the operand's element type as the quantiser reads it")
    ap.add_argument("--pipeline", action="store_true",
                    help="time the workload as a layer runs it: A in BF16 quantised per row (1 x g) on the GPU, "
                         "then the GEMM against B quantised beforehand; reports the quantiser's share")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MB",
                    help="only run a plain device copy of MB megabytes three times (calibrates the HBM "
                         "byte counters of a profiler run) and exit")
    args = ap.parse_args()
    global clock_s
    clock_s = max(0.0, args.clock_window)

    if args.copy_probe:
        import torch

        n = args.copy_probe << 20
        x = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "repeats": 3}), flush=True)
        return

    if args.gpus != 1:
        sys.stderr.write("bench.py measures one GPU only: the GEMM runs whole on a single MI355X and "
                         "nothing here launches or coordinates more than one (asked for --gpus %d)\n" % args.gpus)
        raise SystemExit(2)
    if args.steps < 1 or args.warmup < 0:
        raise SystemExit("--steps must be >= 1 and --warmup >= 0")

    c = workload_by_name(args.workload)
    w = synth.WORKLOADS[c]
    g = args.gran or w["g"]
    if w["K"] % g:
        raise SystemExit("--gran %d does not divide K = %d" % (g, w["K"]))
    fa, fb = FORMATS[args.fmt]
    if args.pipeline:
        flops, gemm_bytes = algorithmic(w, g, 1)
        M_, K_ = w["M"], w["K"]
        # the quantiser reads A in BF16 and writes its codes and factors, which the GEMM reads back
        pipe_bytes = gemm_bytes + 2.0 * M_ * K_ + M_ * K_ + 4.0 * M_ * (K_ // g)
        ms, mq, mg, sets, glen = pipeline_leg(c, args.steps, args.warmup, args.sets, g)
        tflops = flops / (ms * 1e-3) / 1e12
        if bound_of(w) == "mfma":
            roof = {"bound": "mfma", "achieved": round(tflops, 3), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tflops / PEAK_FP8_TFLOPS, 4), "traffic": None}
        else:
            gbs = pipe_bytes / (ms * 1e-3) / 1e9
            roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None}
        print(json.dumps({
            "metric": "FP8 block-scaled GEMM TFLOPS with the activation quantised on the GPU in each step (1 GPU)",
            "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "fp8_e4m3", "data": "synthetic",
            "config": {"workload": w["name"], "M": w["M"], "N": w["N"], "K": w["K"], "gran": g,
                       "a_input": "bf16, quantised per step with 1x%d factors" % g,
                       "b_input": "e4m3 with %dx%d factors, quantised before the timed steps" % (g, g),
                       "input_sets": sets, "quant_us": round(mq * 1e3, 3), "gemm_us": round(mg * 1e3, 3),
                       "quant_share": round(mq / ms, 4),
                       "launch": "hipGraph of %d quantise + GEMM pairs, replayed %d times" % (glen, args.steps // glen)},
            "roofline": roof, "cpu_baseline": None}), flush=True)
        return
    if args.quant:
        fmt = fa if args.quant == "a" else fb
        ms, sets, glen, rows, cols, nblocks = quant_leg(c, args.quant, args.steps, args.warmup, args.sets, g, fmt,
                                                        args.sa_rows == 1, args.quant_in)
        qbytes = (QUANT_IN[args.quant_in] + 1.0) * rows * cols + 4.0 * nblocks
        gbs = qbytes / (ms * 1e-3) / 1e9
        print(json.dumps({
            "metric": "FP8 block quantiser throughput (%s in, FP8 codes and FP32 factors out; 1 GPU)"
                      % args.quant_in.upper(),
            "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "f32", "data": "synthetic",
            "config": {"workload": w["name"], "operand": args.quant.upper(), "input": args.quant_in, "rows": rows,
                       "cols": cols, "gran": g,
                       "blocks": "1x%d" % g if args.sa_rows == 1 else "%dx%d" % (g, g),
                       "fmt": "e5m2" if fmt else "e4m3", "input_sets": sets,
                       "launch": "hipGraph of %d launches, replayed %d times" % (glen, args.steps // glen)},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None},
            "cpu_baseline": None}), flush=True)
        return
    flops, nbytes = algorithmic(w, g, args.sa_rows)
    act = ACTS[args.act]
    layout = LAYOUTS[args.layout]
    ms, sets, finite, glen, trials, clock = gpu_leg(c, args.steps, args.warmup, args.sets, g, fa, fb, args.bias, act,
                                                    args.sa_rows, layout, args.workspace)
    if not finite:
        raise SystemExit("GEMM output holds non-finite values")
    sec = ms * 1e-3
    tflops = flops / sec / 1e12
    bound = bound_of(w)
    if bound == "mfma":
        achieved, peak, unit = tflops, PEAK_FP8_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = nbytes / sec / 1e9, PEAK_HBM_GBS, "GB/s"
    default_variant = (fa, fb, g, args.bias, act, args.sa_rows, layout, args.sets, args.workspace) == \
        (0, 0, w["g"], False, 0, None, 0, None, False)
    tr = TRAFFIC.get(w["name"]) if default_variant else None
    traffic = tr["bytes"] if tr and tr["src"] == kernel_source_hash(w["name"]) else None

    cpu = None if args.no_cpu_baseline else cpu_leg(c, g, fa, fb, args.bias, act, sa_rows=args.sa_rows, layout=layout)

    line = {
        "metric": "FP8 block-scaled GEMM TFLOPS and % of MI355X dense FP8 peak (1 GPU)",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3" if args.fmt == "e4m3" else "fp8_" + args.fmt,
        "data": "synthetic",
        "config": {"workload": w["name"], "M": w["M"], "N": w["N"], "K": w["K"], "gran": g, "fmt": args.fmt,
                   "epilogue": ("bias+" if args.bias else "") + args.act,
                   "a_scales": "1x%d" % g if args.sa_rows == 1 else "%dx%d" % (g, g),
                   "layout": args.layout.upper(), "out": "bf16", "input_sets": sets,
                   "entry": "dg_gemm_fp8_ws (workspace)" if args.workspace else "without workspace",
                   "launch": "hipGraph of %d launches, replayed %d times" % (glen, args.steps // glen),
                   "trials_us": {"n": len(trials), "median": round(statistics.median(trials) * 1e3, 3),
                                 "min": round(min(trials) * 1e3, 3), "max": round(max(trials) * 1e3, 3)},
                   "pct_fp8_peak": round(100.0 * tflops / PEAK_FP8_TFLOPS, 2),
                   "sustained_clock": clock,
                   "alg_GBps": round(nbytes / sec / 1e9, 1)},
        "roofline": {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": traffic},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
