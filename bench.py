"""Benchmark of the W4A4 MXFP4 linear layer on one MI355X.

One step is the whole hot path over one batch: online quantization of the
activations (with the workload's block rotation) followed by the MXFP4 GEMM
against pre-quantized weights (weight quantization is offline and untimed).
Both operands use the library's GEMM-native tiled layout: the quantizer
writes X's codes and scales tiled, and W is quantized to it offline.
Inputs are seeded synthetic tensors of the workload's shape, resident in HBM
before the timed region; the step cycles through enough buffer sets (X, W,
codes, scales, Y) that the working set exceeds the 256 MB Infinity Cache.

Prints one JSON line:
  value       2*M*N*K / (time of one step), TFLOP/s, from HIP events around
              the whole loop of K steps (no event markers between launches),
              after --settle-ms of untimed steps and the W warm-up steps (the
              engine clock dips for the first ~17 ms of load after an idle
              gap; settle_ms in the line).
              A step is one quantize + GEMM.  For decode shapes (M <= 64,
              bf16 activations) both that and one launch of the fused layer
              (mxfp4_linear_small) are timed.  Each path is timed launched
              eagerly and replayed from HIP graphs (one graph per cycle of
              steps over the buffer sets: the same kernels, with one host
              launch per cycle); the fastest is the step (config.path, config.launch),
              all four are in `launch`, and the other path is reported beside
              it (`split` or `fused`)
  roofline    the dominant kernel (the GEMM, or the fused layer for decode
              shapes, bytes = bf16 X + MXFP4 W + Y), its launch time the mean
              over at least max(K, 200) launches of that kernel alone (`launches`), back
              to back over the buffer sets, as whole replays of a HIP graph of
              at least 64 launches after untimed ones, with HIP events on the
              launch stream around the loop.  `us_marked` gives the mean, median and min of a loop of
              the K steps with events around every launch (each marker adds a
              dispatch gap, which inflates short kernels).  Large M: the
              MFMA-bound large-tile kernel, algorithmic FLOPs per launch / its
              mean launch time, against the dense MXFP4 MFMA peak.  M <= 64
              (decode): the HBM-bound small-M kernel, algorithmic bytes (both
              operands' codes and scales read once, Y written) / launch time,
              against HBM.  `traffic` = HBM bytes per launch from rocprofv3
              counters (profiles/), or null if the kernel source changed since
  quantize    the quantizer kernel: algorithmic bytes (X read, codes and
              scales written) per launch / its mean launch time, against HBM
              and against the device copy measured in the same run
              (frac_of_copy); launch time and `us_marked` as for roofline
  transforms  each block transform (none, Hadamard-32, Kronecker 4x8,
              per-channel smoothing) on this workload: the quantizer alone,
              and the linear step (quantize + GEMM against weights folded with
              that transform, a copy per buffer set) replayed from a cycle
              graph; for decode shapes also the fused layer's step
  smooth_vs_kron  the smoothed step over the Kronecker step (the pages'
              SmoothQuant comparison, as context)
  read_ceiling  a bare streaming kernel (libmxfp4_ceiling.so) over the same
              byte counts and buffer rotation: the quantizer's pattern, and
              for decode shapes the weight stream; `frac_of_read_ceiling` in
              `quantize` and `roofline` is its time over the kernel's
  power       board power and engine clock (amd-smi, sampled from a side
              thread) while the step's dominant kernel, and the MFMA loop,
              run back to back for --power-seconds each, beside idle
  parity      the timed configuration's outputs against the oracle on the
              CPU sample's rows: codes and scales bit-exact, fp32 Y within
              the 1e-5 normalized bound (the run exits 1 otherwise)
  weight_fit  offline weight quantization with the E8M0 rule and with fitted
              block exponents: time, and the squared error of each against the
              weight-side transformed fp32 weights
  mxfp4_out   the same GEMM writing MXFP4 (mxfp4_gemm_requant, Y requantized
              per 32-block in the epilogue) beside the bf16-output GEMM, both
              timed back to back over the buffer sets
  copy_gbps   a plain device copy in the same run (practical HBM ceiling)
  mfma_ceiling  the scaled FP4 MFMA alone, every SIMD issuing back to back
              with no memory traffic (libmxfp4_ceiling.so): TFLOP/s, the
              engine clock it held, and the GEMM's rate as a fraction of it
  cpu_baseline  the CPU oracle on the same workload (all rows by default, at
              most 8192): the layer in TFLOP/s, and the quantizer alone in
              GB/s single-threaded and over every host thread

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--cpu-rows R] [--power-seconds S]
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np

import workloads

METRIC = "MXFP4 GEMM TFLOPS @ M=3584,K=3072,N=12288 (% peak); quantize GB/s (% HBM)"
PEAK_MXFP4_TFLOPS = 10100.0     # MI355X dense FP4/FP6 MFMA
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
CACHE_BUST_BYTES = 600 << 20    # working set per cycle of buffer sets (> 256 MB)
SETTLE_S = 0.05                 # untimed runs of the work before each timed loop (--settle-ms)
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "mxfp4_w4a4_quantized_amd", "csrc")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def source_digest(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel: str, workload: str, digest: str):
    """HBM bytes per launch recorded from rocprofv3 FETCH_SIZE/WRITE_SIZE runs
    in profiles/<kernel>_<workload>_traffic.md, if they were taken on the
    current kernel source (same digest); else None."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    d = re.search(r"^source_digest:\s*(\w+)", text, re.M)
    t = re.search(r"^traffic_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not d or not t or d.group(1) != digest:
        return None
    return float(t.group(1))


# ------------------------------------------------------ measurement helpers ---

def _dequant(codes, scales):
    """MXFP4 (row-major) -> fp32 on the device with torch ops (for error
    figures only)."""
    import torch
    lut = torch.tensor([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6],
                       dtype=torch.float32, device=codes.device)
    c = torch.stack([codes & 15, codes >> 4], dim=-1).reshape(codes.shape[0], -1).long()
    v = lut[c]
    e = torch.exp2(scales.float() - 127).repeat_interleave(32, dim=1)
    return v * e


def _rotated(w, rot):
    """Weights after the weight-side transform (fp32, for error figures)."""
    import torch
    import mxfp4_w4a4_quantized_amd as mx
    if rot == "h32":
        import math
        blocks = w.reshape(w.shape[0], -1, 32).double()
        h = torch.ones(1, 1, dtype=torch.float64, device=w.device)
        for _ in range(5):
            h = torch.cat([torch.cat([h, h], 1), torch.cat([h, -h], 1)], 0)
        return (blocks @ h.T / math.sqrt(32)).reshape(w.shape).float()
    if isinstance(rot, mx.Smooth):
        return w * rot.r[None, :]
    if isinstance(rot, mx.Kron):
        t = torch.kron(rot.a.double(), rot.b.double())
        return (w.reshape(w.shape[0], -1, 32).double() @ t.T).reshape(w.shape).float()
    return w


def _sse(codes, scales, ref):
    return float(((_dequant(codes, scales).double() - ref.double()) ** 2).sum())


# ----------------------------------------------------------------- GPU leg ---

def gpu_leg(name: str, steps: int, warmup: int, power_seconds: float = 0.0, settle_s: float = SETTLE_S):
    import torch
    import mxfp4_w4a4_quantized_amd as mx

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = workloads.make(name)
    wl = inp["wl"]
    m, n, k = wl.m, wl.n, wl.k
    bf16_in = wl.x_dtype == "bf16"
    out_dtype = torch.bfloat16 if wl.out_dtype == "bf16" else torch.float32
    if bf16_in:
        x0 = torch.from_numpy(inp["x"].view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        x0 = torch.from_numpy(inp["x"]).to(dev)
    if wl.rot == "h32":
        rot = mx.HADAMARD32
    elif wl.rot == "kron":
        rot = mx.Kron.from_host(inp["a"], inp["b"], dev)
    else:
        rot = None
    lay = mx.TILED
    wc0, ws0 = mx.quantize_weight(torch.from_numpy(inp["w"]).to(dev), rot, layout=lay)   # offline
    torch.cuda.synchronize()

    mp = mx.padded_rows(m)
    set_bytes = (x0.numel() * x0.element_size() + mp * k // 2 + mp * k // 32 +
                 wc0.numel() + ws0.numel() + m * n * (2 if out_dtype == torch.bfloat16 else 4))
    nsets = max(2, -(-CACHE_BUST_BYTES // set_bytes))
    sets = []
    for _ in range(nsets):
        sets.append(dict(
            x=x0.clone(), wc=wc0.clone(), ws=ws0.clone(),
            xc=torch.empty((mp, k // 2), dtype=torch.uint8, device=dev),
            xs=torch.empty((mp, k // 32), dtype=torch.uint8, device=dev),
            y=torch.empty((m, n), dtype=out_dtype, device=dev)))
    del x0, wc0, ws0
    torch.cuda.synchronize()
    log(f"workload {name}: M={m} N={n} K={k} rot={wl.rot} x={wl.x_dtype} y={wl.out_dtype}; "
        f"{nsets} buffer sets of {set_bytes / 2**20:.1f} MiB")

    split = [lambda s: mx.quantize_rotate(s["x"], rot, s["xc"], s["xs"], layout=lay),
             lambda s: mx.gemm(s["xc"], s["xs"], s["wc"], s["ws"], out_dtype, s["y"], layout=lay)]
    # decode shapes: the fused layer (activation quantization inside the GEMM, one launch)
    use_fused = (m <= mx.LINEAR_SMALL_MAX_M and bf16_in and (wl.rot != "kron" or 2 <= wl.p <= 16))
    fused = [lambda s: mx.linear_small(s["x"], s["wc"], s["ws"], rot, out_dtype, s["y"], layout=lay, n=n)]

    stream = torch.cuda.current_stream(dev)   # the stream every launch goes to

    def settle(run_once):
        """Untimed runs of the work about to be timed, for settle_s seconds,
        right before its warm-up steps: after an idle gap (the host's set-up,
        a graph capture) the engine clock first overshoots downwards, and the
        first ~17 ms of flux_up steps ran ~10% slower than the rest (88-90 vs
        79 us per step in 200-step windows after 1 s idle, then flat for the
        next 0.6 s).  The timed loop then measures the rate the load settles
        to, as a serving loop sees it."""
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        n = 0
        while n < 2 or time.perf_counter() - t_start < settle_s:
            run_once()
            n += 1
            if n % 8 == 0:
                torch.cuda.synchronize()   # the host stays a few launches ahead, no more
        torch.cuda.synchronize()

    def time_loop(parts, marks):
        """Time `steps` steps with HIP events on the launch stream around the
        whole loop; with `marks`, also around every part of every step.  An
        event marker between two launches makes the command processor finish
        the first before it stamps the time, which removes the overlap of one
        launch's start with the previous one's end: the step time comes from a
        loop without them, the per-launch durations from a second loop with
        them."""
        cyc = [0]

        def one_step():
            s_ = sets[cyc[0] % nsets]
            cyc[0] += 1
            for f in parts:
                f(s_)
        settle(one_step)
        for i in range(warmup):
            for f in parts:
                f(sets[i % nsets])
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(parts) + 1)] for _ in range(steps)] \
            if marks else None
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        t0.record(stream)
        for i in range(steps):
            s = sets[i % nsets]
            if marks:
                e = ev[i]
                e[0].record(stream)
                for j, f in enumerate(parts):
                    f(s)
                    e[j + 1].record(stream)
            else:
                for f in parts:
                    f(s)
        t1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        per = [np.array([e[j].elapsed_time(e[j + 1]) for e in ev]) for j in range(len(parts))] if marks else None
        return t0.elapsed_time(t1), wall, per

    total_ms, wall, _ = time_loop(split, False)
    _, _, (q_ms, g_ms) = time_loop(split, True)
    fused_res = None
    if use_fused:
        f_total, f_wall, _ = time_loop(fused, False)
        _, _, (f_ms,) = time_loop(fused, True)
        fused_res = dict(total_ms=f_total, wall_s=f_wall, ms=f_ms)

    # The same steps replayed from HIP graphs: one graph holds a whole cycle
    # of steps, one per buffer set in order (a serving loop captures many
    # layers the same way), so the host pays one graph launch per cycle
    # instead of one launch per kernel; a second graph holds the first
    # `steps % nsets` steps.  Exactly `steps` steps are timed, with events
    # around the whole replay loop.  The captured work is the eager steps',
    # kernel for kernel.
    def capture(parts, count):
        """One graph of `count` steps of `parts`, cycling over the buffer sets."""
        seq = [sets[i % nsets] for i in range(count)]
        for s in seq[:nsets]:
            for f in parts:
                f(s)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for s in seq:
                for f in parts:
                    f(s)
        torch.cuda.synchronize()
        return gr

    def time_graph(parts, per_replay=None):
        per = per_replay or nsets
        cycle = capture(parts, per)
        rest = steps % per
        tail = capture(parts, rest) if rest else None
        settle(cycle.replay)
        for _ in range(max(1, warmup // per)):
            cycle.replay()
        if tail is not None:   # a graph's first replay is slower: not in the timed loop
            tail.replay()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(steps // per):
            cycle.replay()
        if tail is not None:
            tail.replay()
        t1.record(stream)
        torch.cuda.synchronize()
        del cycle, tail
        return t0.elapsed_time(t1)

    graph_ms = {"quantize+gemm": time_graph(split)}
    if use_fused:
        graph_ms["fused"] = time_graph(fused)

    # Per-launch duration of one kernel: launches of it alone, back to back
    # over the buffer sets, as whole replays of one graph of at least 64
    # launches (so that the host's graph-launch cost stays hidden behind the
    # GPU work even for a few-microsecond kernel), at least max(steps, 200)
    # launches in all, after untimed replays; HIP events on the launch stream
    # around the whole loop and none between launches: the kernel's duration
    # plus the dispatch gap between two launches, without the gap each event
    # marker adds (which dominates short kernels).  A kernel property, so its
    # window does not shrink with --steps: at --steps 20, exactly 20 launches
    # (one replay of a fresh 20-launch graph) read 81 us per flux_up GEMM,
    # and one replay of 80 launches 79.6-80.8 us, against 76.7 us over 240
    # (the first launches after a change of kernel run slower).
    alone_per_replay = nsets * -(-64 // nsets)
    alone_reps = max(1, -(-max(steps, 200) // alone_per_replay))
    alone_launches = alone_reps * alone_per_replay

    def time_alone_ms(parts):
        cycle = capture(parts, alone_per_replay)
        settle(cycle.replay)
        for _ in range(max(1, warmup // alone_per_replay)):
            cycle.replay()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(alone_reps):
            cycle.replay()
        t1.record(stream)
        torch.cuda.synchronize()
        del cycle
        return t0.elapsed_time(t1) / alone_launches

    def time_alone(f):
        return time_alone_ms([f])

    q_alone, g_alone = time_alone(split[0]), time_alone(split[1])
    if use_fused:
        fused_res["alone"] = time_alone(fused[0])

    # --- the transforms side by side on this workload's activations: the
    # quantizer alone (the GEMM does not depend on the transform)
    def time_parts(fn):
        """ms per launch of one kernel, timed like time_alone."""
        return time_alone(fn)

    trng = np.random.default_rng(1)
    tkinds = {"none": None, "h32": mx.HADAMARD32,
              "kron4x8": mx.Kron.from_host((np.eye(4) + 0.1 * trng.standard_normal((4, 4))).astype(np.float32),
                                           (np.eye(8) + 0.1 * trng.standard_normal((8, 8))).astype(np.float32), dev),
              "smooth": mx.Smooth.from_host((0.5 + trng.random(k)).astype(np.float32), dev)}
    transforms = {}
    for tname, trot in tkinds.items():
        tms = time_parts(lambda s_, r_=trot: mx.quantize_rotate(s_["x"], r_, s_["xc"], s_["xs"], layout=lay))
        transforms[tname] = {"quantize_ms": tms}

    # --- the linear step with each transform: quantize (activation side) +
    # GEMM against weights folded with that transform's weight side (a copy
    # per buffer set, so the weights stream as in the step above), replayed
    # from a cycle graph; for decode shapes also the fused layer
    w32 = torch.from_numpy(inp["w"]).to(dev)
    for tname, trot in tkinds.items():
        twc, tws = mx.quantize_weight(w32, trot, layout=lay)
        tsets = [dict(s_, wc=twc.clone(), ws=tws.clone()) for s_ in sets]
        del twc, tws
        tparts = [lambda s_, r_=trot: mx.quantize_rotate(s_["x"], r_, s_["xc"], s_["xs"], layout=lay),
                  lambda s_: mx.gemm(s_["xc"], s_["xs"], s_["wc"], s_["ws"], out_dtype, s_["y"], layout=lay)]
        saved, sets[:] = list(sets), tsets
        transforms[tname]["step_ms"] = time_graph(tparts) / steps
        if use_fused and (not isinstance(trot, mx.Kron) or 2 <= trot.a.shape[0] <= 16):
            transforms[tname]["fused_step_ms"] = time_graph(
                [lambda s_, r_=trot: mx.linear_small(s_["x"], s_["wc"], s_["ws"], r_, out_dtype, s_["y"], layout=lay,
                                                     n=n)]) / steps
        sets[:] = saved
        del tsets, saved
    torch.cuda.empty_cache()

    # --- the streaming-read ceiling (libmxfp4_ceiling.so) on the same byte
    # counts and the same rotation over buffer sets: the quantizer's pattern
    # (4 KiB read and 1 KiB written per wave), and for decode shapes the
    # weight stream (16 KiB read per wave, nothing written)
    read_ceiling = {}
    sl = stream_lib()
    x_bytes_dev = sets[0]["x"].numel() * sets[0]["x"].element_size()
    cases = [("quantize", x_bytes_dev, 4, 1)]
    if m <= 64:
        cases.append(("weights", sets[0]["wc"].numel() + sets[0]["ws"].numel(), 16, 0))
    for cname, rbytes, rk, wk in cases:
        waves = rbytes // (rk * 1024)
        if waves < 1:
            continue
        # random bytes, like the operands (constant bytes streamed about 1% faster)
        gen = torch.Generator(device=dev)
        gen.manual_seed(11)
        bufs = [dict(src=torch.randint(0, 256, (waves * rk * 1024,), dtype=torch.uint8, device=dev, generator=gen),
                     dst=torch.empty(max(waves * wk, 1) * 1024, dtype=torch.uint8, device=dev)) for _ in range(nsets)]

        def launch(b_, rk_=rk, wk_=wk, waves_=waves):
            # torch's current stream at call time: the capture stream inside a graph capture
            st = sl.mxfp4_ceiling_stream(b_["src"].data_ptr(), b_["dst"].data_ptr(), waves_, rk_, wk_,
                                         torch.cuda.current_stream(dev).cuda_stream)
            if st != 0:
                raise RuntimeError(f"mxfp4_ceiling_stream failed: HIP error {st}")
        saved, sets[:] = list(sets), bufs
        ms = time_alone_ms([launch])
        sets[:] = saved
        moved = waves * (rk + wk) * 1024
        read_ceiling[cname] = {"us_per_launch": ms * 1e3, "bytes": moved, "gbps": moved / (ms * 1e-3) / 1e9}
        del bufs, saved
    torch.cuda.empty_cache()

    # --- the same GEMM with an MXFP4 output (requantized in the epilogue)
    requant_ms = None
    if not use_fused and n % 256 == 0 and k % 128 == 0:
        qc_out = torch.empty((mx.padded_rows(m), n // 2), dtype=torch.uint8, device=dev)
        qs_out = torch.empty((mx.padded_rows(m), n // 32), dtype=torch.uint8, device=dev)
        requant_ms = time_parts(lambda s_: mx.gemm_requant(s_["xc"], s_["xs"], s_["wc"], s_["ws"], layout=lay,
                                                             out_layout=lay, m=m, n=n, y_codes=qc_out,
                                                             y_scales=qs_out))
        gemm_ms = time_parts(lambda s_: mx.gemm(s_["xc"], s_["xs"], s_["wc"], s_["ws"], out_dtype, s_["y"],
                                                 layout=lay))
        requant_ms = (requant_ms, gemm_ms)
        del qc_out, qs_out

    # --- offline weight quantization: plain E8M0 rule vs fitted exponents, and
    # the squared error of each against the (transformed) fp32 weights
    w32 = torch.from_numpy(inp["w"]).to(dev)
    wrot = rot.weight_side() if isinstance(rot, (mx.Kron, mx.Smooth)) else rot
    wfit = {}
    for fit in (False, True):
        for _ in range(2):
            wc_, ws_ = mx.quantize_rotate(w32, wrot, fit=fit)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(5):
            wc_, ws_ = mx.quantize_rotate(w32, wrot, fit=fit)
        e1.record(stream)
        torch.cuda.synchronize()
        wfit["fit" if fit else "plain"] = dict(ms=e0.elapsed_time(e1) / 5, codes=wc_, scales=ws_)
    wref = w32 if wrot is None else _rotated(w32, wrot)
    for v in wfit.values():
        v["sse"] = _sse(v.pop("codes"), v.pop("scales"), wref)
    del w32, wref

    # plain device copy of 1 GiB: the practical HBM ceiling in this run
    nb = 1 << 30
    src = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    reps = 10
    c0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * nb * reps / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst

    props = torch.cuda.get_device_properties(dev)
    ceiling = mfma_ceiling(dev, stream, props.multi_processor_count)

    # --- outputs of the timed configuration for the parity check against the
    # oracle (untimed): X's codes and scales (untiled on the host), the GEMM's
    # fp32 Y, and for decode shapes the fused layer's fp32 Y
    s0 = sets[0]
    mx.quantize_rotate(s0["x"], rot, s0["xc"], s0["xs"], layout=lay)
    y32 = mx.gemm(s0["xc"], s0["xs"], s0["wc"], s0["ws"], torch.float32, layout=lay, m=m, n=n)
    yf32 = mx.linear_small(s0["x"], s0["wc"], s0["ws"], rot, torch.float32, layout=lay, n=n) if use_fused else None
    torch.cuda.synchronize()
    hxc, hxs = mx.untile_host(s0["xc"].cpu().numpy(), s0["xs"].cpu().numpy(), m)
    outputs = dict(xc=hxc, xs=hxs, y32=y32.cpu().numpy(), yf32=None if yf32 is None else yf32.cpu().numpy())
    del y32, yf32

    # --- engine clock and board power while the step's dominant kernel runs
    # back to back for a few seconds, and while the MFMA loop does
    power = None
    if power_seconds > 0:
        dom = (lambda s_: mx.linear_small(s_["x"], s_["wc"], s_["ws"], rot, out_dtype, s_["y"], layout=lay, n=n)) \
            if use_fused and fused_res["alone"] < g_alone else split[1]
        power = power_trace(dev, props, stream, [("gemm" if dom is split[1] else "fused", dom)], sets, power_seconds)
    return dict(ceiling=ceiling, m=m, n=n, k=k, wl=wl, total_ms=total_ms, wall_s=wall, q_ms=q_ms, g_ms=g_ms,
                q_alone=q_alone, g_alone=g_alone, graph_ms=graph_ms, read_ceiling=read_ceiling, outputs=outputs,
                power=power, fused=fused_res, copy_gbps=copy_gbps, transforms=transforms, wfit=wfit,
                requant=requant_ms, nsets=nsets, alone_launches=alone_launches, device=props.name,
                cus=props.multi_processor_count, arch=getattr(props, "gcnArchName", ""))


def stream_lib():
    """libmxfp4_ceiling.so with the streaming probe's signature."""
    import ctypes
    from mxfp4_w4a4_quantized_amd import build as hip_build
    if not os.path.exists(hip_build.CEILING_LIB):
        raise RuntimeError(f"{hip_build.CEILING_LIB} is missing: build it with python -m mxfp4_w4a4_quantized_amd.build")
    L = ctypes.CDLL(hip_build.CEILING_LIB)
    L.mxfp4_ceiling_stream.restype = ctypes.c_int
    L.mxfp4_ceiling_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_void_p]
    L.mxfp4_ceiling_mfma.restype = ctypes.c_int
    L.mxfp4_ceiling_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    return L


def _smi_index(props):
    """amd-smi's index of this device (matched by PCI bus), or 0."""
    import subprocess
    bus = getattr(props, "pci_bus_id", None)
    try:
        r = subprocess.run(["amd-smi", "list", "--json"], capture_output=True, text=True, timeout=20)
        for e in json.loads(r.stdout):
            bdf = str(e.get("bdf", ""))
            if bus is not None and bdf.count(":") == 2 and int(bdf.split(":")[1], 16) == int(bus):
                return int(e["gpu"])
    except Exception:
        pass
    return 0


def _smi_sample(index):
    """(socket power W, mean engine clock MHz over the XCDs) from amd-smi."""
    import subprocess
    r = subprocess.run(["amd-smi", "metric", "-g", str(index), "-p", "-c", "--json"], capture_output=True, text=True,
                       timeout=10)
    d = json.loads(r.stdout)
    g = d["gpu_data"][0] if isinstance(d, dict) else d[0]
    pw = float(g["power"]["socket_power"]["value"])
    clk = [float(v["clk"]["value"]) for kname, v in g["clock"].items()
           if kname.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict)
           and v["clk"]["value"] not in ("N/A", None)]
    return pw, sum(clk) / len(clk), clk


def power_trace(dev, props, stream, phases, sets, seconds):
    """Board power and engine clock (amd-smi, sampled from a side thread) while
    each phase's kernel is replayed back to back over the buffer sets for
    `seconds`, beside idle and the MFMA loop of libmxfp4_ceiling.so; the
    kernel's mean launch time during the phase.  None if amd-smi is absent."""
    import shutil
    import threading

    import torch
    if shutil.which("amd-smi") is None:
        return None
    idx = _smi_index(props)
    L = stream_lib()
    cus = props.multi_processor_count
    out = torch.empty(cus * 256, dtype=torch.float32, device=dev)
    cyc = torch.zeros(cus * 4, dtype=torch.int64, device=dev)

    def ceiling(_s):   # on torch's current stream: the capture stream inside a graph capture
        L.mxfp4_ceiling_mfma(cus, 4096, out.data_ptr(), cyc.data_ptr(), torch.cuda.current_stream(dev).cuda_stream)
    res = {}

    def sample_while(flag, bag):
        while not flag.is_set():
            try:
                bag.append((time.perf_counter(),) + _smi_sample(idx))
            except Exception:
                time.sleep(0.1)

    def phase(name, fn):
        per = len(sets) * max(1, 40 // len(sets))
        if fn is not None:
            for s_ in sets:
                fn(s_)
            torch.cuda.synchronize()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                for i in range(per):
                    fn(sets[i % len(sets)])
            gr.replay()
            torch.cuda.synchronize()
        bag, flag = [], threading.Event()
        th = threading.Thread(target=sample_while, args=(flag, bag))
        t0 = time.perf_counter()
        th.start()
        reps = 0
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        while time.perf_counter() - t0 < seconds:
            if fn is None:
                time.sleep(0.05)
                continue
            for _ in range(5):
                gr.replay()
            torch.cuda.synchronize()
            reps += 5 * per
        e1.record(stream)
        torch.cuda.synchronize()
        flag.set()
        th.join()
        keep = [b for b in bag if b[0] - t0 > 0.5]      # past the clock ramp
        if not keep:
            return
        res[name] = {"samples": len(keep), "socket_w": round(sum(b[1] for b in keep) / len(keep), 1),
                     "gfx_mhz": round(sum(b[2] for b in keep) / len(keep), 1),
                     "gfx_mhz_per_xcd": [round(sum(b[3][j] for b in keep) / len(keep)) for j in range(len(keep[0][3]))],
                     "us_per_launch": None if fn is None else round(e0.elapsed_time(e1) * 1e3 / max(reps, 1), 2)}
    try:
        phase("idle", None)
        for name, fn in phases:
            phase(name, fn)
        phase("mfma_ceiling", ceiling)
    except Exception as e:   # a missing or failing amd-smi leaves the measurement out
        log(f"power trace skipped: {e}")
        return None
    return res or None


def mfma_ceiling(dev, stream, cus: int):
    """The block-scaled FP4 MFMA alone (libmxfp4_ceiling.so): one workgroup
    per CU, every SIMD issuing independent MFMAs back to back, no memory
    traffic.  Returns its TFLOP/s after a warm-up long enough for the clock to
    settle, and the engine clock it ran at (wave cycles / launch time)."""
    import ctypes

    import torch
    from mxfp4_w4a4_quantized_amd import build as hip_build
    if not os.path.exists(hip_build.CEILING_LIB):
        raise RuntimeError(f"{hip_build.CEILING_LIB} is missing: build it with python -m mxfp4_w4a4_quantized_amd.build")
    L = ctypes.CDLL(hip_build.CEILING_LIB)
    L.mxfp4_ceiling_mfma.restype = ctypes.c_int
    L.mxfp4_ceiling_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    iters = 4096
    out = torch.empty(cus * 256, dtype=torch.float32, device=dev)
    cyc = torch.zeros(cus * 4, dtype=torch.int64, device=dev)

    def launch():
        st = L.mxfp4_ceiling_mfma(cus, iters, out.data_ptr(), cyc.data_ptr(), stream.cuda_stream)
        if st != 0:
            raise RuntimeError(f"mxfp4_ceiling_mfma failed: HIP error {st}")

    for _ in range(20):
        launch()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record(stream)
    for _ in range(reps):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    s_per = e0.elapsed_time(e1) * 1e-3 / reps
    flops = 2.0 * 32 * 32 * 64 * 8 * iters * 4 * cus
    clock = float(cyc.double().mean()) / s_per / 1e9
    return dict(tflops=flops / s_per / 1e12, clock_ghz=clock)


# ----------------------------------------------------------------- CPU leg ---

def cpu_leg(name: str, rows: int, gpu_out=None):
    """The oracle, as it stands, on the first `rows` rows of X: quantize them
    (with the workload's rotation) and compute their GEMM against the full
    weight matrix (the oracle dequantizes both operands and multiplies in
    binary64).  Weight quantization is offline on both sides and untimed.
    The quantizer alone is also timed on the same rows single-threaded and
    split over the host's threads (the C oracle releases the GIL; it is the
    same function on row blocks).  With `gpu_out` (the timed configuration's
    outputs) the GPU's codes and scales must equal the oracle's on those rows
    and its fp32 Y must meet the 1e-5 normalized bound there."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from threadpoolctl import threadpool_info

    inp = workloads.make(name)
    wl = inp["wl"]
    rows = min(rows, wl.m)
    if wl.rot == "h32":
        xrot = wrot = "h32"
    elif wl.rot == "kron":
        xrot = ("kron", inp["a"], inp["b"])
        wrot = ("kron", oracle.inverse_transpose(inp["a"]), oracle.inverse_transpose(inp["b"]))
    else:
        xrot = wrot = None
    bf16 = wl.x_dtype == "bf16"
    wc, ws = oracle.quantize(inp["w"], rot=wrot)
    xs_in = np.ascontiguousarray(inp["x"][:rows])
    t = time.perf_counter()
    xc, xs = oracle.quantize(xs_in, rot=xrot, bf16=bf16)
    y = oracle.gemm(xc, xs, wc, ws)
    dt = time.perf_counter() - t
    assert y.shape == (rows, wl.n)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    flops = 2.0 * rows * wl.n * wl.k
    # the quantizer alone: one thread, then row blocks on every host thread
    qbytes = xs_in.nbytes + rows * wl.k // 2 + rows * wl.k // 32
    t = time.perf_counter()
    oracle.quantize(xs_in, rot=xrot, bf16=bf16)
    q1 = time.perf_counter() - t
    nthr = os.cpu_count() or 1
    cuts = [rows * i // nthr for i in range(nthr + 1)]
    t = time.perf_counter()
    with ThreadPoolExecutor(nthr) as ex:
        list(ex.map(lambda i: oracle.quantize(xs_in[cuts[i]:cuts[i + 1]], rot=xrot, bf16=bf16), range(nthr)))
    qn = time.perf_counter() - t
    parity = None
    if gpu_out is not None:
        codes_ok = bool(np.array_equal(gpu_out["xc"][:rows], xc) and np.array_equal(gpu_out["xs"][:rows], xs))
        na = np.sqrt((oracle.dequantize(xc, xs) ** 2).sum(1))
        nb = np.sqrt((oracle.dequantize(wc, ws) ** 2).sum(1))

        def nerr(got):
            diff = np.abs(got.astype(np.float64) - y)
            den = np.outer(na, nb)
            with np.errstate(divide="ignore", invalid="ignore"):
                rel = np.where(den > 0, diff / den, np.where(diff == 0, 0.0, np.inf))
            return float(rel.max())
        parity = {"rows": rows, "codes_bit_exact": codes_ok, "max_normalized_error": nerr(gpu_out["y32"][:rows])}
        if gpu_out["yf32"] is not None:
            parity["fused_max_normalized_error"] = nerr(gpu_out["yf32"][:rows])
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=threads, kind="oracle",
                sample=(f"{rows} of {wl.m} rows of X: quantize (single-threaded C) + GEMM "
                        f"against all {wl.n} weight rows (dequantize in single-threaded C, "
                        f"binary64 matmul on {threads} BLAS threads); {dt:.2f} s; host has "
                        f"{os.cpu_count()} logical CPUs"),
                quantize={"single_thread_gbps": round(qbytes / q1 / 1e9, 4),
                          "all_threads_gbps": round(qbytes / qn / 1e9, 4), "threads": nthr,
                          "bytes": qbytes},
                seconds=dt, parity=parity)


# -------------------------------------------------------------------- main ---

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="flux_up", choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--cpu-rows", type=int, default=-1,
                    help="rows of X in the oracle's CPU sample (-1: all rows, at most 8192; 0 skips the CPU leg)")
    ap.add_argument("--power-seconds", type=float, default=3.0,
                    help="seconds of back-to-back launches per phase of the clock and power trace (0 skips it)")
    ap.add_argument("--settle-ms", type=float, default=SETTLE_S * 1e3,
                    help="untimed runs of the timed work before its warm-up steps, in ms, so that the timed "
                         "loop runs at the clock the load settles to (0: only the warm-up steps)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(no sharding, no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0 or args.settle_ms < 0:
        ap.error("--steps must be >= 1, --warmup >= 0 and --settle-ms >= 0")

    g = gpu_leg(args.workload, args.steps, args.warmup, args.power_seconds, args.settle_ms * 1e-3)
    m, n, k, wl = g["m"], g["n"], g["k"], g["wl"]
    flops = 2.0 * m * n * k
    # the step: the fastest of the two-launch path and the fused layer, each
    # launched eagerly or replayed from HIP graphs
    cands = {("quantize+gemm", "eager"): g["total_ms"], ("quantize+gemm", "graph"): g["graph_ms"]["quantize+gemm"]}
    if g["fused"] is not None:
        cands[("fused", "eager")] = g["fused"]["total_ms"]
        cands[("fused", "graph")] = g["graph_ms"]["fused"]
    best_path, best_launch = min(cands, key=cands.get)
    ms_step = cands[(best_path, best_launch)] / args.steps
    per_path = {}
    for (p, lch), v in cands.items():
        per_path.setdefault(p, {})[lch] = round(v / args.steps, 5)
    # per-launch durations: each kernel launched back to back on its own;
    # the statistics of the loop with an event marker around every launch
    # (each marker adds a dispatch gap) are reported beside them
    g_us = g["g_alone"] * 1e3
    q_us = g["q_alone"] * 1e3

    def marked(ms):
        return {"mean": round(float(np.mean(ms)) * 1e3, 2), "median": round(float(np.median(ms)) * 1e3, 2),
                "min": round(float(np.min(ms)) * 1e3, 2)}
    g_tflops = flops / (g_us * 1e-6) / 1e12
    x_bytes = m * k * (2 if wl.x_dtype == "bf16" else 4)
    q_bytes = x_bytes + m * k // 2 + m * k // 32
    q_gbps = q_bytes / (q_us * 1e-6) / 1e9
    y_bytes = m * n * (2 if wl.out_dtype == "bf16" else 4)
    g_bytes = (m + n) * (k // 2 + k // 32) + y_bytes
    # the kernel mxfp4_gemm routes the shape to: the small-M kernel for decode
    # shapes (m <= 64) and for fewer than 8 output tiles of 256 x 256, else the
    # large-tile kernel; the bound follows from the arithmetic intensity
    small_m = m <= 64 or (-(-m // 256)) * (-(-n // 256)) < 8
    hbm_bound = flops / g_bytes < PEAK_MXFP4_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)
    g_src = ("gemm.hip", "gemm_small.hip", "block_quant.h", "internal.h") if small_m else ("gemm.hip", "gemm_large.hip", "internal.h")
    traffic = recorded_traffic("gemm", args.workload, source_digest(*g_src))
    q_traffic = recorded_traffic("quantize", args.workload, source_digest("quantize.hip", "block_quant.h", "internal.h"))
    rc_ = g["read_ceiling"]
    gkernel = "gemm_small" if small_m else "gemm_large"
    if hbm_bound:
        g_gbps = g_bytes / (g_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(g_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(g_gbps / PEAK_HBM_GBPS, 4), "frac_of_copy": round(g_gbps / g["copy_gbps"], 4),
                "kernel": gkernel}
        if "weights" in rc_:   # the streaming probe over the weight bytes, time ratio
            roof["frac_of_read_ceiling"] = round(rc_["weights"]["us_per_launch"] / g_us, 4)
    else:
        roof = {"bound": "mfma", "achieved": round(g_tflops, 1), "peak": PEAK_MXFP4_TFLOPS,
                "unit": "TFLOP/s", "frac": round(g_tflops / PEAK_MXFP4_TFLOPS, 4), "kernel": gkernel}
    roof.update({"traffic": traffic, "us_per_launch": round(g_us, 2), "launches": g["alone_launches"],
                 "us_marked": marked(g["g_ms"]), "algorithmic_bytes": g_bytes, "algorithmic_flops": flops})
    split_info = {"ms_per_step": per_path["quantize+gemm"], "quantize_us": round(q_us, 2), "gemm_us": round(g_us, 2)}
    fz = g["fused"]
    if best_path != "fused":
        # the two-launch path is the step; the fused figures, if any, are reported beside it
        fused_only = None if fz is None else {"ms_per_step": per_path["fused"],
                                              "us_per_launch": round(fz["alone"] * 1e3, 2)}
        fz = None
    else:
        fused_only = None
    if fz is not None:
        # the step is the fused layer: one launch reads bf16 X and the MXFP4 weights, writes Y
        f_us = fz["alone"] * 1e3
        f_bytes = x_bytes + n * (k // 2 + k // 32) + y_bytes
        f_gbps = f_bytes / (f_us * 1e-6) / 1e9
        f_traffic = recorded_traffic("linear_small", args.workload,
                                     source_digest("gemm_small.hip", "block_quant.h", "internal.h"))
        split_info["gemm_roofline"] = roof
        roof = {"bound": "hbm", "achieved": round(f_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(f_gbps / PEAK_HBM_GBPS, 4), "frac_of_copy": round(f_gbps / g["copy_gbps"], 4),
                "kernel": "linear_small", "traffic": f_traffic,
                "us_per_launch": round(f_us, 2), "launches": g["alone_launches"], "us_marked": marked(fz["ms"]),
                "algorithmic_bytes": f_bytes, "algorithmic_flops": flops}
    metric = METRIC if args.workload == "flux_up" else \
        f"MXFP4 GEMM TFLOPS @ M={m},K={k},N={n} (% peak); quantize GB/s (% HBM)"

    out = {
        "metric": metric,
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": args.workload, "m": m, "n": n, "k": k, "x_dtype": wl.x_dtype,
                   "rotation": wl.rot or "none", "out_dtype": wl.out_dtype, "layout": "tiled",
                   "path": best_path, "launch": best_launch,
                   "buffer_sets": g["nsets"], "parallelism": "single-gpu"},
        "roofline": roof,
        "quantize": {"bound": "hbm", "achieved": round(q_gbps, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(q_gbps / PEAK_HBM_GBPS, 4),
                     "frac_of_copy": round(q_gbps / g["copy_gbps"], 4),
                     "frac_of_read_ceiling": (round(rc_["quantize"]["us_per_launch"] / q_us, 4)
                                              if "quantize" in rc_ else None),
                     "traffic": q_traffic, "us_per_launch": round(q_us, 2), "launches": g["alone_launches"],
                     "us_marked": marked(g["q_ms"]),
                     "algorithmic_bytes": q_bytes},
        "split": split_info if fz is not None else None,
        "fused": fused_only,
        "launch": per_path,
        "transforms": {t: dict({"quantize_us": round(v["quantize_ms"] * 1e3, 2),
                                "quantize_gbps": round(q_bytes / (v["quantize_ms"] * 1e-3) / 1e9, 1),
                                "step_us": round(v["step_ms"] * 1e3, 2)},
                               **({"fused_step_us": round(v["fused_step_ms"] * 1e3, 2)} if "fused_step_ms" in v else {}))
                       for t, v in g["transforms"].items()},
        "smooth_vs_kron": {
            "step_ratio": round(g["transforms"]["smooth"]["step_ms"] / g["transforms"]["kron4x8"]["step_ms"], 4),
            "fused_step_ratio": (round(g["transforms"]["smooth"]["fused_step_ms"] / g["transforms"]["kron4x8"]["fused_step_ms"], 4)
                                 if "fused_step_ms" in g["transforms"]["kron4x8"] else None),
            "note": "smoothed linear step time / Kronecker linear step time; the pages report Kronecker 14% faster than SmoothQuant on MI350 (context)"},
        "read_ceiling": {c: {"us_per_launch": round(v["us_per_launch"], 2), "gbps": round(v["gbps"], 1),
                             "bytes": v["bytes"]} for c, v in rc_.items()},
        "power": g["power"],
        "weight_fit": {"plain_ms": round(g["wfit"]["plain"]["ms"], 3), "fit_ms": round(g["wfit"]["fit"]["ms"], 3),
                       "sse_plain": g["wfit"]["plain"]["sse"], "sse_fit": g["wfit"]["fit"]["sse"],
                       "sse_ratio": round(g["wfit"]["fit"]["sse"] / max(g["wfit"]["plain"]["sse"], 1e-300), 4)},
        "mxfp4_out": None if g["requant"] is None else {
            "us_per_launch": round(g["requant"][0] * 1e3, 2),
            "same_gemm_bf16_out_us": round(g["requant"][1] * 1e3, 2),
            "y_bytes": m * (n // 2 + n // 32), "y_bytes_bf16": m * n * 2},
        "copy_gbps": round(g["copy_gbps"], 1),
        "mfma_ceiling": {"tflops": round(g["ceiling"]["tflops"], 1),
                         "frac_of_peak": round(g["ceiling"]["tflops"] / PEAK_MXFP4_TFLOPS, 4),
                         "clock_ghz": round(g["ceiling"]["clock_ghz"], 3),
                         "gemm_frac_of_ceiling": None if hbm_bound else round(g_tflops / g["ceiling"]["tflops"], 4)},
        "device": {"name": g["device"], "arch": g["arch"], "cus": g["cus"]},
    }
    parity_ok = True
    if args.cpu_rows != 0:
        rows = min(m, 8192) if args.cpu_rows < 0 else args.cpu_rows
        log(f"CPU oracle on {rows} rows ...")
        cb = cpu_leg(args.workload, rows, g["outputs"])
        cb.pop("seconds")
        par = cb.pop("parity")
        cb["value"] = round(cb["value"], 6)
        out["cpu_baseline"] = cb
        out["parity"] = par
        parity_ok = par["codes_bit_exact"] and par["max_normalized_error"] <= 1e-5 and \
            par.get("fused_max_normalized_error", 0.0) <= 1e-5
    else:
        out["cpu_baseline"] = None
        out["parity"] = None
    print(json.dumps(out), flush=True)
    if not parity_ok:
        log(f"PARITY FAILURE against the oracle: {out['parity']}")
        sys.exit(1)


if __name__ == "__main__":
    main()
