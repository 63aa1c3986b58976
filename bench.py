"""Benchmark of the W4A8 integer-scale linear layer on one MI355X.

Default workload (the decode-regime sweep): the K=4096, N=22016 layer with
group 128 and amplifier 1024; one step is one pass of the hot path for every
M in {1, 4, 16, 64, 256}: per-token int8 quantization of X (M x 4096 fp32)
followed by the integer-scale W4A8 GEMM. Weights are packed once before
timing (the offline step) and then replicated into R buffers whose total
exceeds twice the 256 MB Infinity Cache; consecutive GEMMs read different
buffers, so weight bytes come from HBM. Each timed step is replayed from a
HIP graph (all K timed steps captured into one graph, replayed once; the
warm-up steps into another), the way a serving loop replays a captured decode
step; the same steps run first with every launch issued from Python, and that
rate is reported alongside ("eager"; --launch eager makes it the reported
one). Per-launch GEMM durations come from a graph of 2R back-to-back GEMM
launches at one M, timed with two events around its replays.

value = algorithmic bytes of one step / step time (GB/s); the per-launch
algorithmic bytes of a W4A8 GEMM are N*K/2 (packed int4) + 4*G*N (integer
scales) + M*K (int8 codes) + 4*M (token scales) + 4*M*N (fp32 output), and
5*M*K + 4*M for the activation quantizer.

Each M runs through the fused entry point bgt_w4a8_linear_is: one launch that
quantizes and multiplies for M <= 4, the quantizer and the GEMM otherwise
(--no-fused-quant: always the two calls).

--iscale-bits 8 or 16 stores the integer scales as uint8 / uint16 (the same
values, narrowed offline) and counts their bytes at that width.

Other workloads: --workload prefill (M in 512..4096, integer- and
float-scale GEMMs side by side; value in TOPS); --workload w8a8 (the
asymmetric W8A8 control with zero-point correction at M=256, K=N=4096;
activation quantization per step, weights quantized offline; value in GB/s
with algorithmic bytes N*K + M*K + 12*(M+N) + 4*M*N, plus 5*M*K + 12*M for
the activation quantizer); --workload w8is (fine-grained W8A8 with integer
scales at the LLaMA-3-8B down projection K=14336, N=4096, alpha=2^16: a
decode step over M in {1,4,16,64} in GB/s with algorithmic bytes
N*K + 4*G*N + M*K + 4*M + 4*M*N per GEMM, plus per-launch GEMM rates at
M in {256,1024,4096}); --workload moe (the grouped W4A8-IS GEMM at the
Mixtral-8x7B expert w1 shape, 8 experts, top-2 routing: a decode step over
T in {1,4,16,64} tokens in GB/s, with algorithmic bytes the active experts'
weights and scales + T*K + 4*T + routing + 4*R*N per launch, plus per-launch
rates at T in {512,4096}).

The default line also carries the compute-bound half of the metric: `prefill`
(the integer-scale GEMM and its float-scale control at M in {512, 1024, 2048,
4096} on the same layer, median / p10 / p90 of event-bracketed launches) with
its own `roofline_prefill` (int8 MFMA bound), a measured device-copy rate
(`copy_sanity`) and, in `kernels`, a roofline for every kernel the decode step
launches (the fused quantize+GEMM launches of M <= 4 under their own name);
`roofline` is the one with the largest summed time.

--workload block: the seven linears of a LLaMA-2-7B-shaped decoder block at
M = 1 (GB/s) and M = 512 (TOPS); --workload single: one 16 x 4096 x 4096 GEMM.

Profiling aids (not benchmark lines): --profile-m M runs only the
quantizer and the integer-scale GEMM at that M (decode layer shape) for
--steps iterations; --copy-probe-mb S copies an S MiB buffer --steps times
(a plain copy of known size, to calibrate the HBM byte counters).

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, TOP/s
MALL_BYTES = 256 << 20
METRIC = "W4A8 integer-scale GEMM TOPS + HBM GB/s, K=4096 N=22016, M=1..4096"


# HBM bytes per GEMM launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE
# (each scaled by the factor a plain copy of known size gives;
# profiles/*hbm_bytes.txt), keyed by (kernel, M). They hold only for the
# kernel sources they were taken on: when a source file differs from the one
# measured (sha256 prefix below), traffic is reported as null.
TRAFFIC_SRC_SHA = {"gemm.hip": "7c95a1badb659f9e", "gemm_wide.hip": "6b38f7952bb95fee",
                   "gemm_w8is.hip": "1301029dd06003ab"}
# sources of the launches one call makes (the wide path also runs the 256 x 128
# kernel over the last round's columns)
TRAFFIC_SRC = {"k_w4a8_decode<IS>": ("gemm.hip",), "k_w4a8_prefill<4,2,2,2,IS>": ("gemm.hip",),
               "k_w4a8_wide<IS>": ("gemm.hip", "gemm_wide.hip"), "k_w8a8_zp<9,32>": ("gemm.hip",),
               "k_w8is_split": ("gemm_w8is.hip",)}
TRAFFIC = {
    ("k_w4a8_decode<IS>", 1): 48194641,
    ("k_w4a8_decode<IS>", 4): 48561393,
    ("k_w4a8_decode<IS>", 16): 50010826,
    ("k_w4a8_decode<IS>", 64): 58482425,
    ("k_w4a8_prefill<4,2,2,2,IS>", 256): 79241723,
    ("k_w4a8_wide<IS>", 512): 149896694,
    ("k_w4a8_wide<IS>", 1024): 207369511,
    ("k_w4a8_wide<IS>", 2048): 384209919,
    ("k_w4a8_wide<IS>", 4096): 754830981,
    ("k_w8a8_zp<9,32>", 256): 29681405,
    ("k_w8is_split", 1): 62568942,
    ("k_w8is_split", 4): 62961976,
    ("k_w8is_split", 16): 64534582,
    ("k_w8is_split", 64): 69604498,
}


def measured_traffic(kernel, Ms):
    import hashlib
    names = TRAFFIC_SRC.get(kernel)
    if names is None:
        return None
    for name in names:
        with open(os.path.join(ROOT, "bit_gemm_token_amd", "csrc", name), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest()[:16] != TRAFFIC_SRC_SHA[name]:
                return None
    vals = [TRAFFIC.get((kernel, M)) for M in Ms]
    return None if any(v is None for v in vals) else int(np.mean(vals))


def gemm_bytes(M, N, K, scale_bytes=4, out_bytes=4):
    G = K // 128
    return N * K // 2 + scale_bytes * G * N + M * K + 4 * M + out_bytes * M * N


def quant_bytes(M, K):
    return 5 * M * K + 4 * M


def gemm_ops(M, N, K):
    return 2 * M * N * K


def pct(vals, q):
    return round(float(np.percentile(np.asarray(vals, dtype=np.float64), q)), 3)


def spread(vals):
    """median / p10 / p90 of a list of per-launch durations (us)."""
    return {"us_median": pct(vals, 50), "us_p10": pct(vals, 10), "us_p90": pct(vals, 90)}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def copy_sanity(torch, dev, mib=512, reps=10):
    """A plain device-to-device copy of `mib` MiB (torch), timed with events:
    the practical HBM rate on this machine (read + write bytes / time)."""
    n = (mib << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    ts = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        ts.append((e0, e1))
    torch.cuda.synchronize()
    us = [x.elapsed_time(y) * 1e3 for x, y in ts]
    med = float(np.median(us))
    del a, b
    return {"bytes_each_way": n * 4, "us_median": round(med, 2),
            "GBps": round(2 * n * 4 / med / 1e3, 1), "kind": "torch copy_ (read + write)"}


# --------------------------------------------------------------------- CPU side
def cpu_baseline(x, w, Ms=None, min_seconds=10.0, unit="GB/s"):
    """Time the oracle (as it stands) on the decode step: per-token
    quantization plus the integer-scale GEMM over all columns for every M of
    the step, repeated until at least min_seconds of CPU work have run; in
    GB/s of the step's algorithmic bytes, or TOPS of its GEMM ops.

    Offline weight packing is excluded, as it is on the GPU side.
    """
    import oracle
    oracle.build()
    Ms = list(synth.DECODE_M) if Ms is None else Ms
    K, N = x.shape[1], w.shape[1]
    pw = oracle.pack_weights(w, 128, 1024)
    xs = {M: np.ascontiguousarray(x[:M]) for M in Ms}
    step_bytes = sum(quant_bytes(M, K) + gemm_bytes(M, N, K) for M in Ms)
    step_ops = sum(gemm_ops(M, N, K) for M in Ms)
    steps = 0
    t0 = time.perf_counter()
    while True:
        for M in Ms:
            q, s = oracle.quant_sym_i8(xs[M])
            oracle.w4a8_gemm_is(q, s, pw["codes"], pw["iscale"], pw["alpha"])
        steps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    value = steps * step_bytes / el / 1e9 if unit == "GB/s" else steps * step_ops / el / 1e12
    return {
        "value": round(value, 4),
        "unit": unit,
        "cores": cores,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"{steps} passes of quant_act + w4a8_gemm_is at M in {Ms}, K={K}, N={N} "
                  f"in {el:.1f} s; offline packing excluded",
    }


# --------------------------------------------------------------------- GPU side
class Rotor:
    """R copies of the packed weights and integer scales (same values, distinct memory)."""

    def __init__(self, torch, packed, iscale, fscale, min_bytes=2 * MALL_BYTES):
        per = packed.numel() + iscale.numel() * 4 + fscale.numel() * 4
        self.R = max(2, math.ceil(min_bytes / per))
        self.bufs = [(packed.clone(), iscale.clone(), fscale.clone()) for _ in range(self.R)]
        self.i = 0

    def next(self):
        b = self.bufs[self.i % self.R]
        self.i += 1
        return b

    def get(self, i):
        return self.bufs[i % self.R]


def graph_steps(torch, step, steps, warmup):
    """Capture step(k) for k < steps into one HIP graph (and `warmup` steps
    into another), replay the warm-up graph untimed, then time one replay of
    the K-step graph; returns ms per step. One graph for the whole timed region
    keeps host-side launch cost out of short steps."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g_warm = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_warm):
        for k in range(max(1, warmup)):
            step(k)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for k in range(steps):
            step(k)
    g_warm.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def graph_launch_us(torch, launch, n, reps=5):
    """Per-launch duration of launch(j), j < n, captured back to back in one HIP
    graph and replayed `reps` times between two events on the stream the
    kernels run on; returns one duration (us) per replay. One eager launch
    first: a GEMM that splits K allocates its workspace on first use, which it
    does not do under capture (it would run unsplit)."""
    launch(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for j in range(n):
            launch(j)
    g.replay()
    ev = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        ev.append((e0, e1))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 / n for a, b in ev]


def run_decode(args, torch, bgt, dev):
    K, N = synth.K_LAYER, synth.N_LAYER
    Ms = list(synth.DECODE_M)
    x, w = synth.layer_inputs(0, M=max(Ms), K=K, N=N)
    xd = torch.from_numpy(x).to(dev)
    xs = {M: xd[:M].contiguous() for M in Ms}
    pw = bgt.pack_weights_int4(torch.from_numpy(w).to(dev), alpha=synth.ALPHA)
    sb = args.iscale_bits // 8                     # bytes per stored integer scale
    if sb != 4:                                    # offline: narrow storage, same values
        pw["iscale"] = bgt.narrow_iscale(pw["iscale"], sb)
    rot = Rotor(torch, pw["packed"], pw["iscale"], pw["fscale"])
    qbuf = {M: (torch.empty((M, K), dtype=torch.int8, device=dev),
                torch.empty(M, dtype=torch.float32, device=dev)) for M in Ms}
    ybuf = {M: torch.empty((M, N), dtype=torch.float32, device=dev) for M in Ms}

    def linear(M, packed, iscale):
        """Per-token quantization of X then the integer-scale GEMM: one call of
        the fused entry point (a single launch for M <= 4), or the quantizer and
        the GEMM as two calls with --no-fused-quant."""
        q, s = qbuf[M]
        if args.fused_quant:
            bgt.w4a8_linear_is(xs[M], packed, iscale, pw["alpha"], N, qx=q, sx=s, y=ybuf[M])
        else:
            bgt.quantize_act(xs[M], q=q, scale=s)
            bgt.w4a8_gemm_is_narrow(q, s, packed, iscale, pw["alpha"], N, y=ybuf[M])

    def step(k, events=None):
        """Step k: quantization + GEMM per M; the GEMMs of step k read weight
        copies k*len(Ms) .. k*len(Ms)+len(Ms)-1 (mod R), so consecutive GEMMs
        never share a copy."""
        for i, M in enumerate(Ms):
            packed, iscale, _ = rot.get(k * len(Ms) + i)
            if events is not None:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
            linear(M, packed, iscale)
            if events is not None:
                e1.record()
                events.append((M, e0, e1))

    # eager launches: every call issued from Python as the step runs
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    eager_events = []
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k, eager_events)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / args.steps

    # HIP graphs: step k captured once, then replayed; the timed region
    # replays each step's graph exactly once
    ms_step = graph_steps(torch, step, args.steps, args.warmup) if args.launch == "graph" else eager_ms

    # per-launch GEMM duration (and quantization + GEMM duration): back-to-back
    # launches at one M, weight copies rotating as in the step; ten replays of
    # the graph give ten samples (each the mean over 2R launches)
    per_m, lin_m = {}, {}
    for M in Ms:
        q, s = qbuf[M]

        def launch(j, q=q, s=s, M=M):
            packed, iscale, _ = rot.get(j)
            bgt.w4a8_gemm_is_narrow(q, s, packed, iscale, pw["alpha"], N, y=ybuf[M])

        def launch_lin(j, M=M):
            packed, iscale, _ = rot.get(j)
            linear(M, packed, iscale)
        per_m[M] = graph_launch_us(torch, launch, 2 * rot.R, reps=10)
        lin_m[M] = graph_launch_us(torch, launch_lin, 2 * rot.R, reps=10)

    eager_per_m = {M: [] for M in Ms}
    for M, e0, e1 in eager_events:
        eager_per_m[M].append(e0.elapsed_time(e1) * 1e3)     # us
    step_bytes = sum(gemm_bytes(M, N, K, sb) + quant_bytes(M, K) for M in Ms)

    # what the step launches at each M: one fused kernel (quantization in the
    # GEMM's prologue: reads the fp32 rows, writes codes and token scales), or
    # the quantizer and then the GEMM kernel
    fused = {M: bool(args.fused_quant and bgt.w4a8_linear_fused(xs[M])) for M in Ms}
    launches = []                                   # (kernel, M, durations, bytes, ops)
    for M in Ms:
        if fused[M]:
            launches.append((bgt.w4a8_kernel_name(M, N, K) + "+fused-quant", M, lin_m[M],
                             gemm_bytes(M, N, K, sb) + 4 * M * K, gemm_ops(M, N, K)))
        else:
            launches.append((bgt.w4a8_kernel_name(M, N, K), M, per_m[M], gemm_bytes(M, N, K, sb),
                             gemm_ops(M, N, K)))
    sweep = {}
    for M in Ms:
        us = float(np.mean(per_m[M]))
        b = gemm_bytes(M, N, K, sb)
        sweep[str(M)] = {"gemm_us": round(us, 3), **{"gemm_" + k: v for k, v in spread(per_m[M]).items()},
                         "gemm_GBps": round(b / us / 1e3, 1),
                         "gemm_TOPS": round(gemm_ops(M, N, K) / us / 1e6, 2),
                         "hbm_frac": round(b / us / 1e3 / HBM_PEAK_GBS, 4),
                         "mfma_frac": round(gemm_ops(M, N, K) / us / 1e6 / INT8_PEAK_TOPS, 4),
                         "quant_gemm_us": round(float(np.mean(lin_m[M])), 3),
                         **{"quant_gemm_" + k: v for k, v in spread(lin_m[M]).items()},
                         "quant_gemm_launches": 1 if fused[M] else 2,
                         "eager_quant_gemm_us_median": round(float(np.median(eager_per_m[M])), 3),
                         "kernel": bgt.w4a8_kernel_name(M, N, K) + ("+fused-quant" if fused[M] else "")}
    kernels = kernel_rooflines(launches)
    dom = max(kernels, key=lambda k: k["total_us"])
    roof = dict(dom["roofline"])
    roof["traffic"] = measured_traffic(dom["kernel"], dom["launch_M"]) if sb == 4 else None
    out = {
        "metric": METRIC, "value": round(step_bytes / (ms_step * 1e-3) / 1e9, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8xint4->int32",
        "data": "synthetic (seeded; X ~N(0,1) + 1% channels x20, W ~N(0,0.02) + 0.1% x10)",
        "config": {"workload": "decode sweep: W4A8-IS quant_act + GEMM, K=4096 N=22016 g=128 "
                               "alpha=1024, M in {1,4,16,64,256} per step",
                   "launch": "hip_graph" if args.launch == "graph" else "eager",
                   "iscale_storage": {4: "int32", 2: "uint16", 1: "uint8"}[sb],
                   "quantization": "fused into the GEMM for M <= 4" if args.fused_quant else "separate launch",
                   "weight_buffers_rotated": rot.R},
        "eager": {"ms_per_step": round(eager_ms, 4),
                  "value": round(step_bytes / (eager_ms * 1e-3) / 1e9, 1)},
        "roofline": roof, "kernels": [{k: v for k, v in e.items() if k != "roofline"} | e["roofline"]
                                      for e in kernels],
        "sweep": sweep,
    }
    return out, (x, w), (pw, rot)


def kernel_rooflines(launches):
    """Group timed launches by kernel; per kernel the summed mean duration, and a
    roofline over its launches: the bound is whichever of the HBM time
    (algorithmic bytes / 8 TB/s) and the MFMA time (ops / 5 POP/s) is larger
    summed over them; achieved = mean bytes (or ops) per launch / mean launch
    duration."""
    by = {}
    for name, M, durs, b, ops in launches:
        by.setdefault(name, []).append((M, durs, b, ops))
    out = []
    for name, items in by.items():
        Ms = [m for m, _, _, _ in items]
        durs = [u for _, d, _, _ in items for u in d]
        avg_us = float(np.mean(durs))
        mb = float(np.mean([b for _, _, b, _ in items]))
        mo = float(np.mean([o for _, _, _, o in items]))
        t_hbm = sum(b for _, _, b, _ in items) / HBM_PEAK_GBS
        t_mfma = sum(o for _, _, _, o in items) / INT8_PEAK_TOPS / 1e3
        if t_hbm >= t_mfma:
            ach = mb / avg_us / 1e3
            r = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "frac": round(ach / HBM_PEAK_GBS, 4)}
        else:
            ach = mo / avg_us / 1e6
            r = {"bound": "mfma", "achieved": round(ach, 1), "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                 "frac": round(ach / INT8_PEAK_TOPS, 4)}
        r.update({"traffic": None, "kernel": name, "launch_M": Ms, "avg_launch_us": round(avg_us, 3),
                  "bytes_per_launch": int(mb), "ops_per_launch": int(mo)})
        out.append({"kernel": name, "launch_M": Ms,
                    "total_us": round(sum(float(np.mean(d)) for _, d, _, _ in items), 3), "roofline": r})
    return out


def prefill_sweep(torch, bgt, dev, xd, pw, rot, Ms, warmup=3, timed=10, out_dtype=None):
    """Per-launch durations of the integer-scale GEMM and its float-scale
    control at each M (K=4096, N=22016), weight copies rotating; median, p10,
    p90 over `timed` event-bracketed launches."""
    K, N = synth.K_LAYER, synth.N_LAYER
    qs = {M: bgt.quantize_act(xd[:M].contiguous())[:2] for M in Ms}
    odt = out_dtype or torch.float32
    res = {}
    for fs in (False, True):
        for M in Ms:
            q, s = qs[M]
            y = torch.empty((M, N), dtype=odt, device=dev)
            ts = []
            for it in range(warmup + timed):
                packed, iscale, fscale = rot.next()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                if fs:
                    bgt.w4a8_gemm_fs(q, s, packed, fscale, N, y=y)
                else:
                    bgt.w4a8_gemm_is_narrow(q, s, packed, iscale, pw["alpha"], N, y=y)
                e1.record()
                if it >= warmup:
                    ts.append((e0, e1))
            torch.cuda.synchronize()
            us = [a.elapsed_time(b) * 1e3 for a, b in ts]
            med = float(np.median(us))
            tops = gemm_ops(M, N, K) / med / 1e6
            res[("fs" if fs else "is") + str(M)] = {
                **spread(us), "TOPS": round(tops, 1), "mfma_frac": round(tops / INT8_PEAK_TOPS, 4),
                "GBps": round(gemm_bytes(M, N, K, out_bytes=2 if out_dtype is not None and out_dtype != torch.float32 else 4) / med / 1e3, 1),
                "kernel": bgt.w4a8_kernel_name(M, N, K, fs)}
            del y
    big = max(Ms)
    r = res["is%d" % big]
    roof = {"bound": "mfma", "achieved": r["TOPS"], "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
            "frac": r["mfma_frac"],
            "traffic": measured_traffic(r["kernel"], [big]) if out_dtype in (None, torch.float32) else None,
            "kernel": r["kernel"], "launch_M": [big], "avg_launch_us": r["us_median"],
            "ops_per_launch": gemm_ops(big, N, K), "timing": "median of event-bracketed launches"}
    return res, roof


def run_prefill(args, torch, bgt, dev):
    """The compute-bound half on its own: the integer-scale GEMM and its
    float-scale control at M in {512, 1024, 2048, 4096} (value: TOPS of the
    integer-scale GEMMs over the sweep)."""
    K, N = synth.K_LAYER, synth.N_LAYER
    Ms = list(synth.PREFILL_M)
    x, w = synth.layer_inputs(0, M=max(Ms), K=K, N=N)
    xd = torch.from_numpy(x).to(dev)
    pw = bgt.pack_weights_int4(torch.from_numpy(w).to(dev), alpha=synth.ALPHA)
    rot = Rotor(torch, pw["packed"], pw["iscale"], pw["fscale"])
    odt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[args.out_dtype]
    res, roof = prefill_sweep(torch, bgt, dev, xd, pw, rot, Ms, warmup=args.warmup, timed=args.steps,
                              out_dtype=odt)
    tot_ops = sum(gemm_ops(M, N, K) for M in Ms)
    tot_us = sum(res["is%d" % M]["us_median"] for M in Ms)
    out = {
        "metric": METRIC, "value": round(tot_ops / tot_us / 1e6, 1), "unit": "TOPS",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(tot_us / 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8xint4->int32", "data": "synthetic (seeded)",
        "config": {"workload": "prefill sweep: W4A8-IS GEMM K=4096 N=22016, M in {512,1024,2048,4096}",
                   "output": {"f32": "float32", "f16": "float16", "bf16": "bfloat16"}[args.out_dtype]},
        "roofline": roof,
        "sweep": res,
    }
    return out, (x, w)


def linear_workload(args, torch, bgt, dev, layers, Ms, fused_quant=True):
    """Quantizer + integer-scale GEMM for each (name, K, N, packed weights) of
    `layers` at each M: a step per M (all layers in order, graph-replayed),
    weight copies rotating so weight bytes come from HBM; per-launch durations
    of what each step launches. Returns per-M step times and launch records."""
    per_layer = [p["packed"].numel() + p["iscale"].numel() * 4 for _, _, _, p, _ in layers]
    R = max(2, math.ceil(2 * MALL_BYTES / sum(per_layer)))
    rot = [[(p["packed"].clone(), p["iscale"].clone()) for _, _, _, p, _ in layers] for _ in range(R)]
    res = {}
    for M in Ms:
        bufs = []
        for name, K, N, p, xs in layers:
            xd = torch.from_numpy(np.ascontiguousarray(xs[:M])).to(dev)
            bufs.append((xd, torch.empty((M, K), dtype=torch.int8, device=dev),
                         torch.empty(M, dtype=torch.float32, device=dev),
                         torch.empty((M, N), dtype=torch.float32, device=dev)))

        def lin(i, r, M=M, bufs=bufs):
            name, K, N, p, _ = layers[i]
            xd, q, sc, y = bufs[i]
            pk, isc = rot[r % R][i]
            if fused_quant:
                bgt.w4a8_linear_is(xd, pk, isc, p["alpha"], N, qx=q, sx=sc, y=y)
            else:
                bgt.quantize_act(xd, q=q, scale=sc)
                bgt.w4a8_gemm_is(q, sc, pk, isc, p["alpha"], N, y=y)

        def gemm(i, r, M=M, bufs=bufs):
            name, K, N, p, _ = layers[i]
            xd, q, sc, y = bufs[i]
            pk, isc = rot[r % R][i]
            bgt.w4a8_gemm_is(q, sc, pk, isc, p["alpha"], N, y=y)

        def step(k):
            for i in range(len(layers)):
                lin(i, k)
        for k in range(args.warmup):
            step(k)
        torch.cuda.synchronize()
        ms_step = graph_steps(torch, step, args.steps, args.warmup)
        n = 2 * R if M <= 64 else R
        launches = []
        layer_res = {}
        for i, (name, K, N, p, _) in enumerate(layers):
            fused = bool(fused_quant and bgt.w4a8_linear_fused(bufs[i][0]))
            d_lin = graph_launch_us(torch, lambda j, i=i: lin(i, j), n, reps=10 if M <= 64 else 5)
            d_gemm = graph_launch_us(torch, lambda j, i=i: gemm(i, j), n, reps=10 if M <= 64 else 5)
            kname = bgt.w4a8_kernel_name(M, N, K) + ("+fused-quant" if fused else "")
            b = gemm_bytes(M, N, K) + (4 * M * K if fused else 0)
            launches.append((kname, M, d_lin if fused else d_gemm, b, gemm_ops(M, N, K)))
            layer_res[name] = {"K": K, "N": N, "kernel": kname,
                               "quant_gemm_us": round(float(np.mean(d_lin)), 3),
                               "gemm_us": round(float(np.mean(d_gemm)), 3),
                               **{"gemm_" + k: v for k, v in spread(d_gemm).items()},
                               "quant_gemm_launches": 1 if fused else 2}
        step_bytes = sum(gemm_bytes(M, N, K) + quant_bytes(M, K) for _, K, N, _, _ in layers)
        step_ops = sum(gemm_ops(M, N, K) for _, K, N, _, _ in layers)
        kernels = kernel_rooflines(launches)
        dom = max(kernels, key=lambda k: k["total_us"])
        res[M] = {"ms_per_step": round(ms_step, 4),
                  "GBps": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
                  "TOPS": round(step_ops / (ms_step * 1e-3) / 1e12, 2),
                  "step_bytes": step_bytes, "step_ops": step_ops, "layers": layer_res,
                  "roofline": dom["roofline"],
                  "kernels": [{k: v for k, v in e.items() if k != "roofline"} | e["roofline"]
                              for e in kernels]}
        del bufs
    return res, R


def run_block(args, torch, bgt, dev):
    """The seven linears of a LLaMA-2-7B-shaped decoder block (q, k, v, o
    4096 -> 4096; gate, up 4096 -> 11008; down 11008 -> 4096), all W4A8
    integer-scale, group 128, amplifier 1024, random N(0, 0.02) weights; one
    step is quant_act + GEMM for every linear. M = 1 (decode: value in GB/s of
    the block's algorithmic bytes) and M = 512 (prefill: TOPS)."""
    Ms = (1, 512)
    layers = []
    for name, x, w in synth.block_inputs(0, max(Ms)):
        K, N = w.shape
        p = bgt.pack_weights_int4(torch.from_numpy(w).to(dev), alpha=synth.ALPHA)
        layers.append((name, K, N, p, x))
        del w
    res, R = linear_workload(args, torch, bgt, dev, layers, Ms, fused_quant=args.fused_quant)
    r1, r512 = res[1], res[512]
    return {
        "metric": "LLaMA-2-7B block linears, W4A8 integer-scale: GB/s at M=1, TOPS at M=512",
        "value": r1["GBps"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": r1["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8xint4->int32",
        "data": "synthetic (seeded; X ~N(0,1) + 1% channels x20, W ~N(0,0.02))",
        "config": {"workload": "LLaMA-2-7B block: q,k,v,o 4096x4096, gate,up 4096x11008, down "
                               "11008x4096; quant_act + W4A8-IS GEMM per linear, g=128 alpha=1024; "
                               "value at M=1, M=512 in `prefill`",
                   "launch": "hip_graph", "weight_buffers_rotated": R},
        "roofline": r1["roofline"], "decode": r1,
        "prefill": {k: v for k, v in r512.items()},
        "roofline_prefill": r512["roofline"],
    }, (None, None)


def run_single(args, torch, bgt, dev):
    """One W4A8 integer-scale GEMM: X 16 x 4096 N(0,1) with 1% channels x20,
    W 4096 x 4096 N(0, 0.02), alpha 1024, seed 0; a step is quant_act + GEMM."""
    x, w = synth.single_gemm_inputs(0)
    K, N = w.shape
    p = bgt.pack_weights_int4(torch.from_numpy(w).to(dev), alpha=synth.ALPHA)
    res, R = linear_workload(args, torch, bgt, dev, [("single", K, N, p, x)], (16,),
                             fused_quant=args.fused_quant)
    r = res[16]
    return {
        "metric": "single W4A8 integer-scale GEMM M=16 K=4096 N=4096, HBM GB/s",
        "value": r["GBps"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8xint4->int32",
        "data": "synthetic (seed 0; X ~N(0,1) + 1% channels x20, W ~N(0,0.02))",
        "config": {"workload": "single layer: quant_act + W4A8-IS GEMM, M=16 K=4096 N=4096, g=128, "
                               "alpha=1024", "launch": "hip_graph", "weight_buffers_rotated": R},
        "roofline": r["roofline"], "detail": r,
    }, (None, None)


def run_w8a8(args, torch, bgt, dev):
    """Asymmetric W8A8 control: per-token uint8 X with zero points, per-channel W."""
    M, K, N = 256, 4096, 4096
    x, w = synth.w8a8_inputs(0, M, K, N)
    xd = torch.from_numpy(x).to(dev)
    wt = torch.from_numpy(np.ascontiguousarray(w.T)).to(dev)
    qw, sw, zw, cw = bgt.quantize_act(wt, mode="asym")          # offline
    rot = [(qw.clone(), sw.clone(), zw.clone(), cw.clone())
           for _ in range(max(2, math.ceil(2 * MALL_BYTES / qw.numel())))]
    qx = torch.empty((M, K), dtype=torch.uint8, device=dev)
    sx = torch.empty(M, dtype=torch.float32, device=dev)
    zx = torch.empty(M, dtype=torch.int32, device=dev)
    rx = torch.empty(M, dtype=torch.int32, device=dev)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    gb = N * K + M * K + 12 * (M + N) + 4 * M * N
    qb = 5 * M * K + 12 * M

    def step(k, events=None):
        bgt.quantize_act(xd, mode="asym", q=qx, scale=sx, zero=zx, rowsum=rx)
        a, b, c, d = rot[k % len(rot)]
        if events is not None:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
        bgt.w8a8_gemm_zp(qx, sx, zx, rx, a, b, c, d, y=y)
        if events is not None:
            e1.record()
            events.append((e0, e1))

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    ts = []
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k, ts)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    eager_us = float(np.median([a.elapsed_time(b) * 1e3 for a, b in ts]))
    ms_step = graph_steps(torch, step, args.steps, args.warmup) if args.launch == "graph" else eager_ms

    def launch(j):
        a, b, c, d = rot[j % len(rot)]
        bgt.w8a8_gemm_zp(qx, sx, zx, rx, a, b, c, d, y=y)
    durs = graph_launch_us(torch, launch, 2 * len(rot))
    avg = float(np.mean(durs))
    achieved = gb / avg / 1e3
    return {
        "metric": METRIC, "value": round((gb + qb) / (ms_step * 1e-3) / 1e9, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8xu8->int32",
        "data": "synthetic (seeded; X ~N(0.5,1), W ~N(0,0.02))",
        "config": {"workload": "W8A8 asymmetric control: quant_act(asym) + w8a8_gemm_zp, M=256 K=4096 N=4096",
                   "launch": "hip_graph" if args.launch == "graph" else "eager",
                   "weight_buffers_rotated": len(rot)},
        "eager": {"ms_per_step": round(eager_ms, 4), "value": round((gb + qb) / (eager_ms * 1e-3) / 1e9, 1),
                  "gemm_us_median": round(eager_us, 3)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("k_w8a8_zp<9,32>", [M]),
                     "kernel": "k_w8a8_zp<9,32>", "launch_M": [M], "avg_launch_us": round(avg, 3),
                     "bytes_per_launch": gb},
        "sweep": {"gemm_us": round(avg, 3), "gemm_TOPS": round(2 * M * N * K / avg / 1e6, 2)},
    }, (x, w)


W8IS_K, W8IS_N, W8IS_ALPHA = 14336, 4096, 1 << 16
W8IS_DECODE_M = (1, 4, 16, 64)
W8IS_PREFILL_M = (256, 1024, 4096)


def w8is_bytes(M, N, K, scale_bytes=4, out_bytes=4):
    G = K // 128
    return N * K + scale_bytes * G * N + M * K + 4 * M + out_bytes * M * N


def run_w8is(args, torch, bgt, dev):
    """Fine-grained W8A8 with integer scales at the LLaMA-3-8B down projection
    (K=14336, N=4096, g=128, alpha=2^16): one step is quant_act + GEMM for each
    M in {1, 4, 16, 64} (value in GB/s, as the decode workload); per-launch
    GEMM durations for those M and for M in {256, 1024, 4096} (TOPS)."""
    K, N, alpha = W8IS_K, W8IS_N, W8IS_ALPHA
    Ms = list(W8IS_DECODE_M)
    Ps = list(W8IS_PREFILL_M)
    x = synth.activations(900, max(Ps), K)
    w = synth.weights(901, K, N, std=0.02, outlier_prob=0.001)
    xd = torch.from_numpy(x).to(dev)
    pw = bgt.pack_weights_int8(torch.from_numpy(w).to(dev), alpha=alpha)
    assert pw["alpha"] == alpha
    sb = args.iscale_bits // 8
    isc0 = pw["iscale"] if sb == 4 else bgt.narrow_iscale(pw["iscale"], sb)
    per = pw["qw"].numel() + isc0.numel() * sb
    R = max(2, math.ceil(2 * MALL_BYTES / per))
    rot = [(pw["qw"].clone(), isc0.clone()) for _ in range(R)]
    xs = {M: xd[:M].contiguous() for M in Ms + Ps}
    qbuf = {M: (torch.empty((M, K), dtype=torch.int8, device=dev),
                torch.empty(M, dtype=torch.float32, device=dev)) for M in Ms + Ps}
    ybuf = {M: torch.empty((M, N), dtype=torch.float32, device=dev) for M in Ms + Ps}
    for M in Ps:
        bgt.quantize_act(xs[M], q=qbuf[M][0], scale=qbuf[M][1])

    def step(k):
        for i, M in enumerate(Ms):
            qw, isc = rot[(k * len(Ms) + i) % R]
            q, s = qbuf[M]
            bgt.quantize_act(xs[M], q=q, scale=s)
            bgt.w8a8_gemm_is(q, s, qw, isc, alpha, N, y=ybuf[M])

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ms_step = graph_steps(torch, step, args.steps, args.warmup) if args.launch == "graph" else eager_ms

    per_m = {}
    for M in Ms + Ps:
        q, s = qbuf[M]
        if M in Ms:
            bgt.quantize_act(xs[M], q=q, scale=s)

        def launch(j, q=q, s=s, M=M):
            qw, isc = rot[j % R]
            bgt.w8a8_gemm_is(q, s, qw, isc, alpha, N, y=ybuf[M])
        per_m[M] = graph_launch_us(torch, launch, 2 * R if M <= 256 else R, reps=3 if M > 256 else 5)
    sweep = {}
    for M in Ms + Ps:
        us = float(np.mean(per_m[M]))
        b = w8is_bytes(M, N, K, sb)
        sweep[str(M)] = {"gemm_us": round(us, 3), "gemm_GBps": round(b / us / 1e3, 1),
                         "gemm_TOPS": round(gemm_ops(M, N, K) / us / 1e6, 2),
                         "hbm_frac": round(b / us / 1e3 / HBM_PEAK_GBS, 4),
                         "mfma_frac": round(gemm_ops(M, N, K) / us / 1e6 / INT8_PEAK_TOPS, 4),
                         "kernel": bgt.w8a8_is_kernel_name(M, N, K)}
    step_bytes = sum(w8is_bytes(M, N, K, sb) + quant_bytes(M, K) for M in Ms)
    durs = [u for M in Ms for u in per_m[M]]
    avg_us = float(np.mean(durs))
    avg_bytes = float(np.mean([w8is_bytes(M, N, K, sb) for M in Ms]))
    achieved = avg_bytes / avg_us / 1e3
    kern = bgt.w8a8_is_kernel_name(1, N, K)
    return {
        "metric": "fine-grained W8A8 integer-scale GEMM HBM GB/s, K=14336 N=4096",
        "value": round(step_bytes / (ms_step * 1e-3) / 1e9, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8xint8->int32",
        "data": "synthetic (seeded; X ~N(0,1) + 1% channels x20, W ~N(0,0.02) + 0.1% x10)",
        "config": {"workload": "W8A8-IS decode sweep (LLaMA-3-8B down_proj): quant_act + GEMM, "
                               "K=14336 N=4096 g=128 alpha=2^16, M in {1,4,16,64} per step",
                   "launch": "hip_graph" if args.launch == "graph" else "eager",
                   "iscale_storage": {4: "int32", 2: "uint16", 1: "uint8"}[sb],
                   "weight_buffers_rotated": R},
        "eager": {"ms_per_step": round(eager_ms, 4),
                  "value": round(step_bytes / (eager_ms * 1e-3) / 1e9, 1)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(kern, Ms) if sb == 4 else None,
                     "kernel": kern, "launch_M": Ms, "avg_launch_us": round(avg_us, 3),
                     "bytes_per_launch": int(avg_bytes)},
        "sweep": sweep,
    }, (x, w)


MOE_K, MOE_N, MOE_E, MOE_TOPK = synth.MIXTRAL_HIDDEN, synth.MIXTRAL_FFN, synth.MIXTRAL_E, synth.MIXTRAL_TOPK
MOE_DECODE_T = (1, 4, 16, 64)
MOE_PREFILL_T = (512, 4096)


def moe_bytes(T, R, n_active, N, K, E):
    """Algorithmic bytes of one grouped launch: the weights and scales of the
    experts that receive tokens, each token's codes and scale once, the
    routing, and the R x N fp32 output."""
    G = K // 128
    return n_active * (N * K // 2 + 4 * G * N) + T * K + 4 * T + 4 * (E + 1) + 4 * R + 4 * R * N


def run_moe(args, torch, bgt, dev):
    """Grouped W4A8-IS GEMM at the Mixtral-8x7B expert w1/w3 shape (8 experts,
    top-2, K=4096, N=14336, alpha 1024): one step is quant_act + grouped GEMM
    for each T in {1, 4, 16, 64} tokens (GB/s); per-launch rates also at
    T in {512, 4096} (TOPS)."""
    K, N, E, topk = MOE_K, MOE_N, MOE_E, MOE_TOPK
    if args.moe_linear == "w2":
        K, N = N, K
    Ts, Ps = list(MOE_DECODE_T), list(MOE_PREFILL_T)
    x = synth.activations(700, max(Ps), K)
    w = synth.expert_weights(701, E, K, N)
    xd = torch.from_numpy(x).to(dev)
    G = K // 128
    packed = torch.empty((E, N * K // 2), dtype=torch.uint8, device=dev)
    isc = torch.empty((E, G, N), dtype=torch.int32, device=dev)
    fsc = torch.empty((E, G, N), dtype=torch.float32, device=dev)
    for e in range(E):
        bgt.pack_weights_int4(torch.from_numpy(w[e]).to(dev), alpha=synth.ALPHA, packed=packed[e],
                              fscale=fsc[e], iscale=isc[e])
    del w
    per = packed.numel() + isc.numel() * 4
    Rr = max(2, math.ceil(2 * MALL_BYTES / per))
    rot = [(packed.clone(), isc.clone()) for _ in range(Rr)]
    route = {}
    for T in Ts + Ps:
        offs, tok = synth.route_by_expert(synth.moe_routing(700 + T, T, E, topk), E)
        route[T] = (torch.from_numpy(offs).to(dev), torch.from_numpy(tok).to(dev),
                    int((np.diff(offs) > 0).sum()), len(tok))
    xs = {T: xd[:T].contiguous() for T in Ts + Ps}
    qbuf = {T: (torch.empty((T, K), dtype=torch.int8, device=dev),
                torch.empty(T, dtype=torch.float32, device=dev)) for T in Ts + Ps}
    ybuf = {T: torch.empty((route[T][3], N), dtype=torch.float32, device=dev) for T in Ts + Ps}
    for T in Ts + Ps:
        bgt.quantize_act(xs[T], q=qbuf[T][0], scale=qbuf[T][1])

    def gemm(T, j):
        pk, ic = rot[j % Rr]
        offs, tok, _, _ = route[T]
        q, s = qbuf[T]
        bgt.w4a8_moe_gemm_is(q, s, offs, tok, pk, ic, synth.ALPHA, N, y=ybuf[T])

    def step(k):
        for i, T in enumerate(Ts):
            q, s = qbuf[T]
            bgt.quantize_act(xs[T], q=q, scale=s)
            gemm(T, k * len(Ts) + i)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ms_step = graph_steps(torch, step, args.steps, args.warmup) if args.launch == "graph" else eager_ms

    per_t = {T: graph_launch_us(torch, lambda j, T=T: gemm(T, j), 2 * Rr if T <= 64 else Rr,
                                reps=5 if T <= 64 else 3) for T in Ts + Ps}
    sweep = {}
    for T in Ts + Ps:
        us = float(np.mean(per_t[T]))
        _, _, na, R = route[T]
        b = moe_bytes(T, R, na, N, K, E)
        sweep[str(T)] = {"gemm_us": round(us, 3), "experts_active": na, "slots": R,
                         "gemm_GBps": round(b / us / 1e3, 1),
                         "gemm_TOPS": round(2 * R * N * K / us / 1e6, 2),
                         "hbm_frac": round(b / us / 1e3 / HBM_PEAK_GBS, 4),
                         "mfma_frac": round(2 * R * N * K / us / 1e6 / INT8_PEAK_TOPS, 4),
                         "kernel": bgt.w4a8_moe_kernel_name(T, E, route[T][3], K)}
    step_bytes = sum(moe_bytes(T, route[T][3], route[T][2], N, K, E) + quant_bytes(T, K) for T in Ts)
    durs = [u for T in Ts for u in per_t[T]]
    avg_us = float(np.mean(durs))
    avg_bytes = float(np.mean([moe_bytes(T, route[T][3], route[T][2], N, K, E) for T in Ts]))
    achieved = avg_bytes / avg_us / 1e3
    return {
        "metric": f"grouped (MoE) W4A8 integer-scale GEMM HBM GB/s, Mixtral-8x7B {args.moe_linear} "
                  f"K={K} N={N} E=8 top-2",
        "value": round(step_bytes / (ms_step * 1e-3) / 1e9, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8xint4->int32",
        "data": "synthetic (seeded; X ~N(0,1) + 1% channels x20, W ~N(0,0.02) + 0.1% x10, "
                "top-2 of biased normal router logits)",
        "config": {"workload": f"MoE decode sweep: quant_act + grouped W4A8-IS GEMM, Mixtral-8x7B "
                               f"experts ({args.moe_linear}: K={K} N={N}, E=8, top-2), "
                               "T in {1,4,16,64} tokens per step",
                   "launch": "hip_graph" if args.launch == "graph" else "eager",
                   "weight_buffers_rotated": Rr},
        "eager": {"ms_per_step": round(eager_ms, 4),
                  "value": round(step_bytes / (eager_ms * 1e-3) / 1e9, 1)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     # counters were taken on the w1 shape only
                     "traffic": (measured_traffic(bgt.w4a8_moe_kernel_name(1, E, route[1][3], K), Ts)
                                 if args.moe_linear == "w1" else None),
                     "kernel": bgt.w4a8_moe_kernel_name(1, E, route[1][3], K), "launch_T": Ts,
                     "avg_launch_us": round(avg_us, 3), "bytes_per_launch": int(avg_bytes)},
        "sweep": sweep,
    }, (x, None)


def run_profile_m(args, torch, bgt, dev, M):
    """Quantizer + integer-scale GEMM at one M of the workload's layer, nothing
    else (decode: W4A8 K=4096 N=22016; w8is: W8A8 K=14336 N=4096; moe: the
    grouped GEMM at M tokens, Mixtral w1 shape)."""
    if args.workload == "w8is":
        K, N = W8IS_K, W8IS_N
        x = synth.activations(900, M, K)
        w = synth.weights(901, K, N, std=0.02, outlier_prob=0.001)
        pw = bgt.pack_weights_int8(torch.from_numpy(w).to(dev), alpha=W8IS_ALPHA)
        xd = torch.from_numpy(x).to(dev)
        q = torch.empty((M, K), dtype=torch.int8, device=dev)
        s = torch.empty(M, dtype=torch.float32, device=dev)
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        for _ in range(args.warmup + args.steps):
            bgt.quantize_act(xd, q=q, scale=s)
            bgt.w8a8_gemm_is(q, s, pw["qw"], pw["iscale"], W8IS_ALPHA, N, y=y)
        torch.cuda.synchronize()
        return {"profile_m": M, "launches": args.warmup + args.steps,
                "kernel": bgt.w8a8_is_kernel_name(M, N, K), "gemm_bytes": w8is_bytes(M, N, K)}
    if args.workload == "moe":
        K, N, E = MOE_K, MOE_N, MOE_E
        x = synth.activations(700, M, K)
        w = synth.expert_weights(701, E, K, N)
        packed = torch.empty((E, N * K // 2), dtype=torch.uint8, device=dev)
        isc = torch.empty((E, K // 128, N), dtype=torch.int32, device=dev)
        fsc = torch.empty((E, K // 128, N), dtype=torch.float32, device=dev)
        for e in range(E):
            bgt.pack_weights_int4(torch.from_numpy(w[e]).to(dev), alpha=synth.ALPHA,
                                  packed=packed[e], fscale=fsc[e], iscale=isc[e])
        offs, tok = synth.route_by_expert(synth.moe_routing(700 + M, M, E, MOE_TOPK), E)
        od, td = torch.from_numpy(offs).to(dev), torch.from_numpy(tok).to(dev)
        xd = torch.from_numpy(x).to(dev)
        q = torch.empty((M, K), dtype=torch.int8, device=dev)
        s = torch.empty(M, dtype=torch.float32, device=dev)
        y = torch.empty((len(tok), N), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        for _ in range(args.warmup + args.steps):
            bgt.quantize_act(xd, q=q, scale=s)
            bgt.w4a8_moe_gemm_is(q, s, od, td, packed, isc, synth.ALPHA, N, y=y)
        torch.cuda.synchronize()
        na = int((np.diff(offs) > 0).sum())
        return {"profile_m": M, "launches": args.warmup + args.steps,
                "kernel": bgt.w4a8_moe_kernel_name(M, E, len(tok), K),
                "gemm_bytes": moe_bytes(M, len(tok), na, N, K, E)}
    K, N = synth.K_LAYER, synth.N_LAYER
    x, w = synth.layer_inputs(0, M=M, K=K, N=N)
    xd = torch.from_numpy(x).to(dev)
    pw = bgt.pack_weights_int4(torch.from_numpy(w).to(dev), alpha=synth.ALPHA)
    q = torch.empty((M, K), dtype=torch.int8, device=dev)
    s = torch.empty(M, dtype=torch.float32, device=dev)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    for _ in range(args.warmup + args.steps):
        bgt.quantize_act(xd, q=q, scale=s)
        bgt.w4a8_gemm_is(q, s, pw["packed"], pw["iscale"], pw["alpha"], N, y=y)
    torch.cuda.synchronize()
    return {"profile_m": M, "launches": args.warmup + args.steps,
            "kernel": bgt.w4a8_kernel_name(M, N, K), "gemm_bytes": gemm_bytes(M, N, K)}


def run_copy_probe(args, torch, dev, mib):
    """A plain device copy of known size (read mib MiB, write mib MiB) per launch."""
    n = (mib << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(args.warmup + args.steps):
        b.copy_(a)
    torch.cuda.synchronize()
    return {"copy_probe_bytes_each_way": n * 4, "launches": args.warmup + args.steps}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "prefill", "w8a8", "w8is", "moe", "block", "single"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="decode workload: leave out the prefill sweep (M = 512..4096) of the same layer")
    ap.add_argument("--iscale-bits", type=int, default=32, choices=[8, 16, 32],
                    help="decode workload: integer scales stored as uint8 / uint16 / int32 "
                         "(same values; bytes counted at the stored width)")
    ap.add_argument("--no-fused-quant", dest="fused_quant", action="store_false",
                    help="decode workload: run the quantizer and the GEMM as two calls for "
                         "every M (default: the fused entry point, one launch for M <= 4)")
    ap.add_argument("--out-dtype", default="f32", choices=["f32", "f16", "bf16"],
                    help="prefill workload: element type of y (fp32 result rounded once)")
    ap.add_argument("--launch", default="graph", choices=["graph", "eager"],
                    help="decode workload: replay each step from a HIP graph (default) or "
                         "issue every launch from Python")
    ap.add_argument("--moe-linear", default="w1", choices=["w1", "w2"],
                    help="moe workload: the expert linear (w1/w3: 4096 -> 14336, w2: 14336 -> 4096)")
    ap.add_argument("--profile-m", type=int, default=0)
    ap.add_argument("--copy-probe-mb", type=int, default=0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer would shard column-parallel over N, with no exchange between GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_gemm_token_amd as bgt
    bgt.lib()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.profile_m or args.copy_probe_mb:
        r = (run_profile_m(args, torch, bgt, dev, args.profile_m) if args.profile_m
             else run_copy_probe(args, torch, dev, args.copy_probe_mb))
        print(json.dumps(r), flush=True)
        return
    if args.workload == "decode":
        out, (x, w), (pw, rot) = run_decode(args, torch, bgt, dev)
        if not args.no_prefill:
            # the compute-bound half of the metric (M = 512 .. 4096) on the same
            # layer and weight copies
            Ms = list(synth.PREFILL_M)
            xp = torch.from_numpy(synth.activations(0, max(Ms), synth.K_LAYER)).to(dev)
            res, roof = prefill_sweep(torch, bgt, dev, xp, pw, rot, Ms)
            del xp
            out["prefill"] = {"workload": "W4A8-IS GEMM and its float-scale control, K=4096 N=22016, "
                                          "M in {512,1024,2048,4096}, fp32 y",
                              "sweep": res}
            out["roofline_prefill"] = roof
        out["copy_sanity"] = copy_sanity(torch, dev)
    elif args.workload == "prefill":
        out, (x, w) = run_prefill(args, torch, bgt, dev)
    elif args.workload == "w8is":
        out, (x, w) = run_w8is(args, torch, bgt, dev)
    elif args.workload == "moe":
        out, (x, w) = run_moe(args, torch, bgt, dev)
    elif args.workload == "block":
        out, (x, w) = run_block(args, torch, bgt, dev)
    elif args.workload == "single":
        out, (x, w) = run_single(args, torch, bgt, dev)
    else:
        out, (x, w) = run_w8a8(args, torch, bgt, dev)
    if not args.no_cpu_baseline and args.workload in ("decode", "prefill"):
        out["cpu_baseline"] = (cpu_baseline(x, w) if args.workload == "decode"
                               else cpu_baseline(x, w, Ms=[256], unit="TOPS"))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
