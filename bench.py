"""Benchmark: one BitLinear forward + STE backward step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--rotate R] [--no-cpu-baseline]

A step is the whole hot path on one batch: ternarize + pack the master
weights and int8-quantize the activations (one bitnet_quantize call), the
INT8 forward GEMM, and the two bf16 STE backward GEMMs (dX and dW, one
bitlinear_bwd call), all through the C ABI of libbitnet.so on torch's current
stream. Inputs are seeded synthetic tensors of the 4096 x 2560 -> 6912 layer
(x, dY ~ N(0,1) bf16, W ~ U(+-1/sqrt(2560)) bf16), resident in HBM before
timing starts. R independent copies of all buffers are rotated step by step
so that the working set (~240 MB per copy) does not sit in the 256 MB
Infinity Cache between steps (the cold figure); the warm figure repeats one
copy.

Clock ramp: after the GPU has idled, its power management raises the
clocks over some tens of milliseconds of work (measured at the headline
workload: graph-replayed steps take 0.42 ms in the first 7 ms of work after
2 s idle, 0.37 ms by 20 ms and 0.355-0.36 ms from about 50 ms on). A
training loop runs in the settled state, so every timed region here is
preceded by at least --ramp-ms (default 200) milliseconds of untimed
repetitions of the same work, after the W warm-up steps; the K timed steps
are unchanged. --ramp-ms 0 measures straight after the warm-up steps.

Prints one JSON line: throughput in effective TOPS (6*M*N*K per step), the
step time (replays of the step captured in HIP graphs), per-call times (the
median of `steps` eager calls timed with HIP events on the launch stream,
enqueued behind about 30 ms of step replays so that the GPU never waits on
the host inside a timed call),
each call's fraction of the published peak and of the ceiling measured in
the same run (a plain device copy; register-only MFMA chains), the combined
GEMM fraction of the MFMA peak, the same summary for the other layer
workloads and the 8-layer stack (with its peak allocated bytes), and the CPU
oracle timed on a bounded sample of the headline workload.
"""

import argparse
import hashlib
import itertools
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "BitLinear fwd+bwd ms & TOPS at 4096×2560→6912; % of MFMA peak"
# MI355X published dense peaks (no sparsity).
PEAK_BF16_TFLOPS = 2500.0
PEAK_INT8_TOPS = 5000.0
PEAK_HBM_GBS = 8000.0
# Effective TOPS of the pages' fused kernel at this workload on an NVIDIA L4
# (8.80 ms for 6*M*N*K ops; context, other hardware).
PAGES_L4_TOPS = 49.4
HEADLINE = "c2_up_4096x2560x6912"

KERNEL_SOURCES = ["gemm_kernels.hip", "skinny_kernels.hip", "quant_kernels.hip", "device_common.h"]
# the other layer workloads reported in the same line, and the 8-layer stack
OTHER_WORKLOADS = ["c1_small", "c3_down_4096x6912x2560", "c5_skinny_32x6912x2560"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default=HEADLINE)
    p.add_argument("--rotate", type=int, default=4)
    p.add_argument("--ramp-ms", type=float, default=200.0,
                   help="untimed repetitions of the timed work before each timed region, in milliseconds of GPU "
                        "time, so that the clocks have left the idle state (0: none)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--stack-memory", action="store_true",
                   help="only measure the 8-layer stack's peak allocated bytes (run in a child process)")
    p.add_argument("--only-headline", action="store_true",
                   help="skip the other workloads and the stack (e.g. under a profiler)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain device copy of known size (for counter calibration)")
    p.add_argument("--vendor-gemms", action="store_true",
                   help="time the library GEMMs torch dispatches (hipBLASLt) on plain operands of the workload's "
                        "three products, for comparison (no conversion work; not part of the path)")
    p.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR", "CAL_WRITE_DIR"),
                   help="turn rocprofv3 FETCH_SIZE / WRITE_SIZE runs of the bench and of --copy-calibration "
                        "into profiles/pmc_traffic.json (no GPU needed)")
    return p.parse_args()


# bench kernel name -> substrings of the device kernel names it launches
KERNEL_MATCH = {
    # the one-pass launch with activation rows (its weight-only form is bitnet_ternarize_pack's), else the two
    # launches of the two-pass path
    "quantize": ["quant_onepass_kernel<17, true", "quant_onepass_kernel<24, true", "quant_front_kernel",
                 "ternarize_pack_kernel"],
    "fwd_i8": ["MfmaI8"],
    "bwd_bf16": ["bwd_prep_kernel", "wt_fp4_kernel", "xhat_kernel", "gemm_pair_kernel"],
}
COPY_BYTES = 256 << 20


def copy_calibration():
    """A plain device-to-device copy of COPY_BYTES, three times: the
    counters of this kernel calibrate FETCH_SIZE / WRITE_SIZE (it must read
    and write exactly COPY_BYTES each)."""
    import torch

    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 3}), flush=True)


def vendor_gemms(inp, steps, warmup):
    """The three products of one layer as plain library GEMMs through torch
    (hipBLASLt on this image): the INT8 forward (torch._int_mm, x_q [M][K] by
    the codes as int8 [K][N]), dX = dY [M][N] . W [N][K] and dW = dY^T . x
    in bf16, all operands contiguous (dY^T stored transposed); next to them,
    this library's calls on the workload's own inputs: bitlinear_fwd and
    bitlinear_bwd with dX only, dW only (each with its pre-pass) and both.
    Medians of `steps` back-to-back calls timed with HIP events after
    `warmup` calls and the clock ramp; the library GEMMs do none of the
    path's conversion work."""
    import torch

    from ternary_weight_quantization_amd import binding as B

    M, K, N = inp["M"], inp["K"], inp["N"]
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    xq = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=dev, generator=g)
    wq = torch.randint(-1, 2, (N, K), dtype=torch.int8, device=dev, generator=g)
    wq_t = wq.t().contiguous()
    dY = torch.randn((M, N), dtype=torch.bfloat16, device=dev, generator=g)
    W = torch.randn((N, K), dtype=torch.bfloat16, device=dev, generator=g)
    x = torch.randn((M, K), dtype=torch.bfloat16, device=dev, generator=g)
    dYt = dY.t().contiguous()
    cases = {
        "fwd_int8 x_q[M,K] @ q[K,N] (torch._int_mm)": lambda: torch._int_mm(xq, wq_t),
        "dX_bf16 dY[M,N] @ W[N,K]": lambda: dY @ W,
        "dW_bf16 dY^T[N,M] @ x[M,K]": lambda: dYt @ x,
    }
    # this library on the workload's inputs
    Kp = B.bitnet_k_pad(K)
    wdt = torch.bfloat16 if inp["w_dtype"] == "bf16" else torch.float32
    t = dict(W=_to_dev(inp["W"], wdt, dev), x=_to_dev(inp["x"], torch.bfloat16, dev),
             dY=_to_dev(inp["dY"], torch.bfloat16, dev),
             w_packed=torch.empty((N, Kp // 4), dtype=torch.uint8, device=dev),
             gamma=torch.empty((1,), dtype=torch.float32, device=dev),
             ws=torch.empty((B.bitnet_ternarize_workspace_bytes(N, K),), dtype=torch.uint8, device=dev),
             x_q=torch.empty((M, Kp), dtype=torch.int8, device=dev),
             s_x=torch.empty((M,), dtype=torch.float32, device=dev),
             y=torch.empty((M, N), dtype=torch.bfloat16, device=dev),
             dX=torch.empty((M, K), dtype=torch.bfloat16, device=dev),
             dW=torch.empty((N, K), dtype=wdt, device=dev))
    B.bitnet_quantize(t["W"], t["x"], t["w_packed"], t["gamma"], t["x_q"], t["s_x"], t["ws"])
    here = {
        "fwd (bitlinear_fwd)": lambda: B.bitlinear_fwd(t["x_q"], t["s_x"], t["w_packed"], t["gamma"], K, t["y"]),
        "dX (bitlinear_bwd, dX only)": lambda: B.bitlinear_bwd(t["dY"], t["x_q"], t["s_x"], t["w_packed"],
                                                               t["gamma"], K, dX=t["dX"]),
        "dW (bitlinear_bwd, dW only)": lambda: B.bitlinear_bwd(t["dY"], t["x_q"], t["s_x"], t["w_packed"],
                                                               t["gamma"], K, dW=t["dW"]),
        "dX + dW (bitlinear_bwd, one call)": lambda: B.bitlinear_bwd(t["dY"], t["x_q"], t["s_x"], t["w_packed"],
                                                                     t["gamma"], K, dX=t["dX"], dW=t["dW"]),
    }

    def med_us(f):
        for _ in range(warmup):
            f()
        ramp(f)
        torch.cuda.synchronize()
        evs = []
        for _ in range(steps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            f()
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        return _median_ms(evs) * 1e3

    flops = 2.0 * M * N * K
    out = {}
    for name, f in cases.items():
        us = med_us(f)
        out[name] = {"us": round(us, 1), "rate": round(flops / (us * 1e-6) / 1e12, 1),
                     "unit": "TOP/s" if "int8" in name else "TFLOP/s"}
    ours = {}
    for name, f in here.items():
        us = med_us(f)
        work = flops * (2 if "+" in name else 1)
        ours[name] = {"us": round(us, 1), "rate": round(work / (us * 1e-6) / 1e12, 1),
                      "unit": "TOP/s" if name.startswith("fwd") else "TFLOP/s"}
    return {"workload": f"{M}x{K}x{N}", "gemms": out, "here": ours}


def _pmc_rows(d):
    import glob
    import sqlite3

    rows = []
    for db in sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True)):
        con = sqlite3.connect(db)
        rows += list(con.execute("select name, counter_name, counter_value from pmc_events"))
        con.close()
    if not rows:
        raise SystemExit(f"no pmc_events in {d}")
    return rows


# kernels of calls outside the step (the sign-output backward, the forward with a
# bias, the TTQ backward's pair launch)
KERNEL_EXCLUDE = ["Sign1Epilogue", "FwdEpilogue<true>", "TtqDwEpilogue"]


def _per_dispatch_mean(rows, counter, match):
    vals = [v for name, cn, v in rows if cn == counter and any(m in name for m in match)
            and not any(x in name for x in KERNEL_EXCLUDE)]
    return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)


def summarize_pmc(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of each bench kernel,
    scaled by copy_bytes / (the copy kernel's reading): HBM bytes per launch."""
    cal = {}
    for counter, d in (("FETCH_SIZE", cal_fetch_dir), ("WRITE_SIZE", cal_write_dir)):
        rows = _pmc_rows(d)
        # torch's same-dtype device copy runs the runtime's copy kernel
        vals = [v for name, cn, v in rows if cn == counter and "copyBuffer" in name]
        if not vals:
            raise SystemExit(f"no copy kernel counters in {d}")
        name = next(n for n, cn, _ in rows if cn == counter and "copyBuffer" in n)
        kib = sum(vals) / len(vals)
        cal[counter] = {"kernel": name[:120], "kib_per_dispatch": kib, "factor": COPY_BYTES / (kib * 1024.0)}
    fetch_rows, write_rows = _pmc_rows(fetch_dir), _pmc_rows(write_dir)
    kernels = {}
    for bname, match in KERNEL_MATCH.items():
        # a bench call may launch several kernels: sum their per-dispatch means
        f_total = w_total = 0.0
        n_f = n_w = 0
        for m in match:
            # the list names every kernel the call may launch; a shape runs a subset
            f, nf = _per_dispatch_mean(fetch_rows, "FETCH_SIZE", [m])
            w, nw = _per_dispatch_mean(write_rows, "WRITE_SIZE", [m])
            if f is None or w is None:
                continue
            f_total += f * 1024.0 * cal["FETCH_SIZE"]["factor"]
            w_total += w * 1024.0 * cal["WRITE_SIZE"]["factor"]
            n_f += nf
            n_w += nw
        if n_f == 0 or n_w == 0:
            raise SystemExit(f"no counters for any kernel of {bname}")
        kernels[bname] = {"fetch_bytes": round(f_total), "write_bytes": round(w_total),
                          "hbm_bytes_per_launch": round(f_total + w_total), "dispatches": [n_f, n_w]}
    return {"source_hash": source_hash(), "calibration": cal, "kernels": kernels}


def source_hash():
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "ternary_weight_quantization_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_path(workload):
    return os.path.join(ROOT, "profiles", f"pmc_traffic_{workload}.json")


def load_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel sources; else None."""
    path = traffic_path(workload)
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_hash") != source_hash():
        return None
    e = d.get("kernels", {}).get(kernel)
    return None if e is None else e.get("hbm_bytes_per_launch")


def cpu_baseline(inp, target_s=12.0, chunk=256):
    """The oracle (as it stands) timed on a bounded sample of the workload.
    The sample is whole steps repeated: each pass ternarizes the full weight
    and then runs the M tokens, `chunk` rows at a time, through act-quant,
    forward and both backward products (dW summed over the chunks). Timing
    stops at the first chunk boundary after `target_s` seconds, so the
    sample is bounded on any host; the rate counts 6*rows*N*K ops for the
    rows processed."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle as O
    from oracle import compare as C
    from ternary_weight_quantization_amd import workloads as WL

    M, K, N = inp["M"], inp["K"], inp["N"]
    Kp = O.k_pad(K)
    w = WL.bf16_bits_to_f32(inp["W"]).astype(np.float64) if inp["w_dtype"] == "bf16" \
        else np.asarray(inp["W"], dtype=np.float64)
    rows_done = passes = 0
    t0 = time.perf_counter()
    while True:
        gamma = O.absmean_gamma(w)
        q = O.ternary_codes(w, gamma)
        O.pack_codes(q, Kp)
        dW = np.zeros((N, K))
        passes += 1
        for r0 in range(0, M, chunk):
            x = WL.bf16_bits_to_f32(inp["x"][r0:r0 + chunk]).astype(np.float64)
            dY = WL.bf16_bits_to_f32(inp["dY"][r0:r0 + chunk]).astype(np.float64)
            x_q, sx = O.act_quant(x, Kp)
            O.forward_y(O.forward_acc(x_q, q), sx, gamma)
            _, dW_part = O.backward(dY, x_q, sx, q, gamma)
            dW += dW_part
            rows_done += x.shape[0]
            if time.perf_counter() - t0 >= target_s:
                break
        if time.perf_counter() - t0 >= target_s:
            break
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    ops = 6.0 * rows_done * N * K
    # untimed: the elements of the whole workload within one fp32 ulp of a
    # rounding boundary (weights at gamma/2, scaled activations at a
    # half-integer); the GPU matches them bit for bit like every other
    gamma = O.absmean_gamma(w)
    x_all = WL.bf16_bits_to_f32(inp["x"]).astype(np.float64)
    _, s_all = O.act_quant(x_all, Kp)
    near = {"weights": C.near_boundary_weights(w, gamma), "activations": C.near_boundary_acts(x_all, s_all)}
    return {
        "value": ops / dt / 1e12,
        "unit": "TOPS",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{passes} pass(es) of the step (full {N}x{K} weight ternarization + the {M} tokens in "
                  f"chunks of {chunk} through act-quant, forward and STE backward), stopped after "
                  f"{rows_done} token rows; {dt:.2f} s wall, {ops / 1e9:.1f} G ops (6*rows*N*K), numpy fp64 "
                  f"with {threads} BLAS threads on {os.cpu_count()} visible cpus",
        "seconds": round(dt, 3),
        "near_boundary": near,
    }


# milliseconds of untimed work before each timed region (--ramp-ms)
RAMP_MS = 200.0
# GPU time enqueued ahead of each timed region of eager calls (lead())
LEAD_MS = 30.0


def ramp(f, ramp_ms=None):
    """Runs f() untimed, in batches of 4 calls, until ramp_ms milliseconds
    of GPU time have passed since the first call (at least one batch)."""
    import torch

    ramp_ms = RAMP_MS if ramp_ms is None else ramp_ms
    if ramp_ms <= 0:
        return
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    while True:
        for _ in range(4):
            f()
        b.record()
        b.synchronize()
        if a.elapsed_time(b) >= ramp_ms:
            return


def _median_ms(evs):
    import numpy as np

    return float(np.median([a.elapsed_time(b) for a, b in evs]))


def measure_ceilings(dev):
    """Ceilings measured in the same run: a plain 256 MiB device copy (HBM
    read + write) and the MFMA probe (register-only chains on every SIMD)
    for bf16 and int8; medians of 5 timed launches after 2 untimed."""
    import torch

    from ternary_weight_quantization_amd import binding as B

    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)

    def timed(f, n=5, warm=2):
        for _ in range(warm):
            f()
        ramp(f)
        evs = []
        for _ in range(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            f()
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        return _median_ms(evs)

    copy_ms = timed(lambda: dst.copy_(src))
    sink = torch.zeros((2048,), dtype=torch.float32, device=dev)
    out = {"copy_GBps": round(2 * COPY_BYTES / (copy_ms * 1e-3) / 1e9, 1)}
    for name, i8 in (("bf16_TFLOPs", False), ("int8_TOPs", True)):
        ops = B.bitnet_debug_mfma_probe(i8, 4000, sink)
        ms = timed(lambda: B.bitnet_debug_mfma_probe(i8, 4000, sink))
        out[name] = round(ops / (ms * 1e-3) / 1e12, 1)
    del src, dst
    torch.cuda.synchronize()
    return out


def _to_dev(a, dtype, dev):
    import numpy as np
    import torch

    if dtype == torch.bfloat16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def layer_bench(inp, steps, warmup, rotate, dev, extra=False):
    """One layer workload: per-call medians, the step time from graph
    replays over `rotate` buffer sets (cold) and over one set (warm)."""
    import numpy as np
    import torch

    from ternary_weight_quantization_amd import binding as B

    M, K, N = inp["M"], inp["K"], inp["N"]
    Kp = B.bitnet_k_pad(K)
    wdt = torch.bfloat16 if inp["w_dtype"] == "bf16" else torch.float32
    base = dict(x=_to_dev(inp["x"], torch.bfloat16, dev), W=_to_dev(inp["W"], wdt, dev),
                dY=_to_dev(inp["dY"], torch.bfloat16, dev))
    sets = []
    for _ in range(rotate):
        s = {k: v.clone() for k, v in base.items()}
        s.update(
            w_packed=torch.empty((N, Kp // 4), dtype=torch.uint8, device=dev),
            gamma=torch.empty((1,), dtype=torch.float32, device=dev),
            ws=torch.empty((B.bitnet_ternarize_workspace_bytes(N, K),), dtype=torch.uint8, device=dev),
            x_q=torch.empty((M, Kp), dtype=torch.int8, device=dev),
            s_x=torch.empty((M,), dtype=torch.float32, device=dev),
            y=torch.empty((M, N), dtype=torch.bfloat16, device=dev),
            dX=torch.empty((M, K), dtype=torch.bfloat16, device=dev),
            dW=torch.empty((N, K), dtype=wdt, device=dev),
        )
        sets.append(s)
    del base
    torch.cuda.synchronize()

    calls = {
        "quantize": lambda s: B.bitnet_quantize(s["W"], s["x"], s["w_packed"], s["gamma"], s["x_q"], s["s_x"], s["ws"]),
        "fwd_i8": lambda s: B.bitlinear_fwd(s["x_q"], s["s_x"], s["w_packed"], s["gamma"], K, s["y"]),
        "bwd_bf16": lambda s: B.bitlinear_bwd(s["dY"], s["x_q"], s["s_x"], s["w_packed"], s["gamma"], K,
                                              dX=s["dX"], dW=s["dW"]),
    }
    names = list(calls)

    def step(s, ev=None):
        for i, n in enumerate(names):
            if ev is not None:
                ev[i][0].record()
            calls[n](s)
            if ev is not None:
                ev[i][1].record()

    for i in range(warmup):
        step(sets[i % len(sets)])
    nxt = itertools.count()
    ramp(lambda: step(sets[next(nxt) % len(sets)]))
    for s in sets:  # every set's outputs from an eager step, the replays' reference
        step(s)
    torch.cuda.synchronize()

    # Step time: graph replays (host call overhead out of the timed region;
    # the same kernels and work as the eager step). One graph holds a step
    # on each buffer set in turn (a training loop captures many layers in
    # one graph); every replay is first checked against the eager outputs.
    outs = ("y", "dX", "dW", "x_q", "w_packed")
    ref = [{k: s[k].clone() for k in outs} for s in sets]

    def graph_of(ss):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for s in ss:
                step(s)
        return g

    def replay_ms(g, per_graph, n_steps):
        reps = max(1, n_steps // per_graph)
        for _ in range(max(1, warmup // per_graph)):
            g.replay()
        ramp(g.replay)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / (reps * per_graph)

    cold = graph_of(sets)
    for s in sets:
        for k in ("y", "dX", "dW"):
            s[k].zero_()
    cold.replay()
    torch.cuda.synchronize()
    for i, s in enumerate(sets):
        for k in outs:
            if not torch.equal(s[k], ref[i][k]):
                raise SystemExit(f"bench.py: graph replay differs from the eager step in {k} (set {i})")
    cold_ms = replay_ms(cold, len(sets), steps)
    warm = graph_of([sets[0]] * 4)
    warm_ms = replay_ms(warm, 4, steps)
    del warm

    def lead():
        # Replays of the step enqueued ahead of a timed region of eager
        # calls (about LEAD_MS of GPU time, enqueued in far less host time),
        # so that the host has launched every timed call before the GPU
        # reaches it: each event pair then spans that call's own GPU work
        # with the clocks in the state the step keeps, and no host launch
        # time. Without it, a host slower than the GPU between two calls
        # shows up in the later call's time.
        for _ in range(max(1, int(LEAD_MS / (cold_ms * len(sets))) + 1)):
            cold.replay()

    # Per-call times inside whole eager steps (the calls in step order),
    # after the lead: medians of `steps` steps.
    evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in names]
           for _ in range(steps)]
    torch.cuda.synchronize()
    lead()
    for i in range(steps):
        step(sets[i % len(sets)], evs[i])
    torch.cuda.synchronize()
    per_call = {n: _median_ms([tuple(evs[i][j]) for i in range(steps)]) for j, n in enumerate(names)}
    per_call_mean = {n: float(np.mean([evs[i][j][0].elapsed_time(evs[i][j][1]) for i in range(steps)]))
                     for j, n in enumerate(names)}
    out = dict(M=M, K=K, N=N, w_dtype=inp["w_dtype"], per_call=per_call, per_call_mean=per_call_mean,
               ms_per_step=cold_ms, ms_per_step_warm=warm_ms, sets=sets, lead=lead)
    if extra:
        # the separate quantization entry points (their own rows), per call
        ex = {
            "ternarize_pack": lambda s: B.bitnet_ternarize_pack(s["W"], s["w_packed"], s["gamma"], s["ws"]),
            "act_quant": lambda s: B.bitnet_act_quant(s["x"], s["x_q"], s["s_x"]),
        }
        out["per_call"].update({n: per_call_ms(f, sets, steps, warmup, lead) for n, f in ex.items()})
    if not extra:
        del out["sets"], out["lead"]
    return out


def per_call_ms(f, sets, steps, warmup, lead):
    """Median of `steps` back-to-back calls of f, each between two HIP
    events, enqueued behind `lead` (GPU work that keeps the GPU busy and
    its clocks in the step's state while the host launches them)."""
    import torch

    for i in range(warmup):
        f(sets[i % len(sets)])
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    lead()
    for i, (a, b) in enumerate(evs):
        a.record()
        f(sets[i % len(sets)])
        b.record()
    torch.cuda.synchronize()
    return _median_ms(evs)


def weight_reads(N, K, w_dtype, with_rows):
    """How often the weight quantization reads W: once where the library
    runs its one-pass launch (bf16 W, K a multiple of 64, W held in
    registers: N*K up to 17 vectors of 8 per thread of the 256 x 512 grid,
    or up to 24 when the call has no activation rows or K <= 3072; with
    activation rows K <= 7168), else twice (a reduction pass, then the
    ternarize + pack pass, which needs the finished gamma)."""
    grid = 256 * 512
    if w_dtype != "bf16" or K % 64 != 0 or (with_rows and K > 7168):
        return 2
    nvec = N * K // 8
    if nvec <= 17 * grid or (nvec <= 24 * grid and (not with_rows or K <= 3072)):
        return 1
    return 2


def layer_roofline(r, ceil):
    """Per-call rates against the published peaks and the measured ceilings.
    Quantization bytes count W as often as the path must read it (once for
    the one-pass launch), the codes, x, x_q and s."""
    M, K, N = r["M"], r["K"], r["N"]
    Kp = (K + 63) // 64 * 64
    w_bytes = 2 if r["w_dtype"] == "bf16" else 4
    gemm = 2.0 * M * N * K
    tern_b = weight_reads(N, K, r["w_dtype"], False) * w_bytes * N * K + N * Kp / 4
    quant_tern_b = weight_reads(N, K, r["w_dtype"], True) * w_bytes * N * K + N * Kp / 4
    aq_b = 2.0 * M * K + M * Kp + 4 * M
    work = {
        "quantize": ("hbm", (quant_tern_b + aq_b) / 1e9, PEAK_HBM_GBS, ceil["copy_GBps"], "GB/s"),
        "fwd_i8": ("mfma", gemm / 1e12, PEAK_INT8_TOPS, ceil["int8_TOPs"], "TOP/s"),
        "bwd_bf16": ("mfma", 2 * gemm / 1e12, PEAK_BF16_TFLOPS, ceil["bf16_TFLOPs"], "TFLOP/s"),
        "ternarize_pack": ("hbm", tern_b / 1e9, PEAK_HBM_GBS, ceil["copy_GBps"], "GB/s"),
        "act_quant": ("hbm", aq_b / 1e9, PEAK_HBM_GBS, ceil["copy_GBps"], "GB/s"),
    }
    out = {}
    for n, ms in r["per_call"].items():
        bound, w, peak, meas, unit = work[n]
        ach = w / (ms * 1e-3)
        out[n] = {"ms": round(ms, 4), "bound": bound, "achieved": round(ach, 2), "unit": unit,
                  "frac": round(ach / peak, 4), "frac_of_measured": round(ach / meas, 4)}
    t = r["per_call"]["fwd_i8"] + r["per_call"]["bwd_bf16"]
    # the survey's combined figure: ideal GEMM time at the dtype peaks / measured GEMM time
    ideal = gemm / (PEAK_INT8_TOPS * 1e12) + 2 * gemm / (PEAK_BF16_TFLOPS * 1e12)
    ideal_meas = gemm / (ceil["int8_TOPs"] * 1e12) + 2 * gemm / (ceil["bf16_TFLOPs"] * 1e12)
    return out, round(ideal / (t * 1e-3), 4), round(ideal_meas / (t * 1e-3), 4)


def stack_bench(steps, warmup, dev):
    """The 8-layer 2560 <-> 6912 stack at 4x512 tokens: step time of the
    forward chain (bitnet_quantize + bitlinear_fwd per layer, each layer's
    bf16 output the next one's input) and the STE backward chain (one
    bitlinear_bwd per layer, dX feeding the previous layer) as graph replays
    through the C ABI; and the peak allocated bytes of one forward + backward
    of the training module (QATBitLinear, bf16 masters, no retained
    activations) from a reset of torch's peak statistics (stack_memory, in a
    fresh process)."""
    import torch

    from ternary_weight_quantization_amd import binding as B
    from ternary_weight_quantization_amd import workloads as WL

    d = WL.stack_inputs(seed=0)
    M, dims = d["M"], d["dims"]
    L = len(dims) - 1
    Ws = [_to_dev(w, torch.bfloat16, dev) for w in d["Ws"]]
    x0 = _to_dev(d["x"], torch.bfloat16, dev)
    dY = _to_dev(d["dY"], torch.bfloat16, dev)
    st = []
    for i in range(L):
        K, N = dims[i], dims[i + 1]
        Kp = B.bitnet_k_pad(K)
        st.append(dict(K=K, N=N, w_packed=torch.empty((N, Kp // 4), dtype=torch.uint8, device=dev),
                       gamma=torch.empty((1,), dtype=torch.float32, device=dev),
                       ws=torch.empty((B.bitnet_ternarize_workspace_bytes(N, K),), dtype=torch.uint8, device=dev),
                       x_q=torch.empty((M, Kp), dtype=torch.int8, device=dev),
                       s_x=torch.empty((M,), dtype=torch.float32, device=dev),
                       y=torch.empty((M, N), dtype=torch.bfloat16, device=dev),
                       dX=torch.empty((M, K), dtype=torch.bfloat16, device=dev),
                       dW=torch.empty((N, K), dtype=torch.bfloat16, device=dev)))

    def step():
        a = x0
        for i, s in enumerate(st):
            B.bitnet_quantize(Ws[i], a, s["w_packed"], s["gamma"], s["x_q"], s["s_x"], s["ws"])
            B.bitlinear_fwd(s["x_q"], s["s_x"], s["w_packed"], s["gamma"], s["K"], s["y"])
            a = s["y"]
        g = dY
        for i in range(L - 1, -1, -1):
            s = st[i]
            B.bitlinear_bwd(g, s["x_q"], s["s_x"], s["w_packed"], s["gamma"], s["K"], dX=s["dX"], dW=s["dW"])
            g = s["dX"]

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ref = [(s["y"].clone(), s["dX"].clone(), s["dW"].clone()) for s in st]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for s in st:
        s["y"].zero_()
        s["dX"].zero_()
    g.replay()
    torch.cuda.synchronize()
    for i, s in enumerate(st):
        if not (torch.equal(s["y"], ref[i][0]) and torch.equal(s["dX"], ref[i][1]) and torch.equal(s["dW"], ref[i][2])):
            raise SystemExit(f"bench.py: stack graph replay differs from the eager step (layer {i})")
    for _ in range(max(1, warmup)):
        g.replay()
    ramp(g.replay)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(steps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    ops = sum(6.0 * M * dims[i] * dims[i + 1] for i in range(L))
    del g, st, Ws, ref
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    out = {
        "workload": f"stack_8x_{dims[0]}_{dims[1]}_M{M}",
        "ms_per_step": round(ms, 4),
        "tops": round(ops / (ms * 1e-3) / 1e12, 2),
    }
    return out


def stack_memory(dev):
    """Peak allocated bytes of one forward + backward of the 8-layer training
    module (QATBitLinear, bf16 masters, no retained activations), measured
    from a reset of torch's peak statistics in a fresh process (bench.py
    --stack-memory), after one untimed step that loads the library."""
    import torch

    from ternary_weight_quantization_amd import binding as B
    from ternary_weight_quantization_amd import layer as LY
    from ternary_weight_quantization_amd import workloads as WL

    d = WL.stack_inputs(seed=0)
    M, dims = d["M"], d["dims"]
    L = len(dims) - 1
    x0 = _to_dev(d["x"], torch.bfloat16, dev)
    dY = _to_dev(d["dY"], torch.bfloat16, dev)
    layers = [LY.QATBitLinear(dims[i], dims[i + 1], device=dev) for i in range(L)]
    with torch.no_grad():
        for lay, w in zip(layers, d["Ws"]):
            lay.weight.copy_(_to_dev(w, torch.bfloat16, dev))
    h = x0
    for lay in layers:
        h = lay(h)
    h.backward(dY)
    for lay in layers:
        lay.weight.grad = None
    del h
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    before = torch.cuda.memory_allocated()
    h = x0
    for lay in layers:
        h = lay(h)
    after_fwd = torch.cuda.memory_allocated()
    h.backward(dY)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated()
    masters = sum(lay.weight.numel() * lay.weight.element_size() for lay in layers)
    saved = sum(M * B.bitnet_k_pad(dims[i]) + 4 * M + dims[i + 1] * B.bitnet_k_pad(dims[i]) // 4 + 4
                for i in range(L))
    ws_max = max(max(B.bitlinear_fwd_workspace_bytes(M, dims[i + 1], dims[i]),
                     B.bitlinear_bwd_workspace_bytes(M, dims[i + 1], dims[i])) for i in range(L))
    return {
        "peak_allocated_bytes": int(peak),
        "peak_allocated_MB": round(peak / 1e6, 1),
        "breakdown_MB": {
            "before the step (bf16 masters, x, dY)": round(before / 1e6, 1),
            "masters": round(masters / 1e6, 1),
            "grads (bf16, as the masters)": round(masters / 1e6, 1),
            "saved state after the forward (int8 x_q + s, 2-bit codes + gamma)": round(saved / 1e6, 1),
            "allocated after the forward": round(after_fwd / 1e6, 1),
            "largest library workspace of one call": round(ws_max / 1e6, 1),
        },
        "pages_peak_MB": {"fused": 1151, "eager": 1887},
    }


def main():
    args = parse()
    global RAMP_MS
    RAMP_MS = args.ramp_ms
    if args.summarize_pmc:
        out = summarize_pmc(*args.summarize_pmc)
        out["workload"] = args.workload
        out["command"] = " ".join(sys.argv)
        with open(traffic_path(args.workload), "w") as f:
            json.dump(out, f, indent=1)
        print(json.dumps(out["kernels"]))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only (the layer is not sharded); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    if args.vendor_gemms:
        from ternary_weight_quantization_amd import workloads as WL

        print(json.dumps(vendor_gemms(WL.layer_inputs(args.workload, seed=0), args.steps, args.warmup)), flush=True)
        return
    if args.copy_calibration:
        copy_calibration()
        return

    import torch

    from ternary_weight_quantization_amd import binding as B
    from ternary_weight_quantization_amd import workloads as WL

    B.lib()
    dev = torch.device("cuda:0")
    if args.stack_memory:
        print(json.dumps(stack_memory(dev)), flush=True)
        return
    ceil = measure_ceilings(dev)
    inp = WL.layer_inputs(args.workload, seed=0)
    M, K, N = inp["M"], inp["K"], inp["N"]
    Kp = B.bitnet_k_pad(K)
    r = layer_bench(inp, args.steps, args.warmup, args.rotate, dev, extra=True)
    sets = r.pop("sets")
    lead = r.pop("lead")
    kernels, gemm_frac, gemm_frac_meas = layer_roofline(r, ceil)
    wdt = torch.bfloat16 if inp["w_dtype"] == "bf16" else torch.float32

    # Calls outside the step, timed per call the same way (medians).
    for s in sets:
        s["dW_sign1"] = torch.empty((N, Kp // 8), dtype=torch.uint8, device=dev)
        s["bias"] = torch.zeros((N,), dtype=torch.bfloat16, device=dev)
        s["db"] = torch.empty((N,), dtype=torch.float32, device=dev)
        s["ttq_params"] = torch.empty((3,), dtype=torch.float32, device=dev)
        B.ttq_init(s["W"], s["ttq_params"], s["ws"])
        s["ttq_codes"] = torch.empty((N, Kp // 4), dtype=torch.uint8, device=dev)
        s["ttq_wt"] = torch.empty((N, Kp), dtype=torch.bfloat16, device=dev)
        s["ttq_grads"] = torch.empty((2,), dtype=torch.float32, device=dev)
    ttq_ws = torch.empty((max(B.ttq_workspace_bytes(M, N, K), 1),), dtype=torch.uint8, device=dev)
    ttq_codes_ws = torch.empty((max(B.ttq_fwd_codes_workspace_bytes(M, N, K), 1),), dtype=torch.uint8, device=dev)
    for s in sets:
        B.ttq_quantize(s["W"], s["ttq_params"], s["ttq_codes"], s["ttq_wt"])
    torch.cuda.synchronize()
    xc = {
        # the backward with dW as 1-bit signs for a sign-based optimiser
        "bwd_sign1": lambda s: B.bitlinear_bwd(s["dY"], s["x_q"], s["s_x"], s["w_packed"], s["gamma"], K,
                                               dX=s["dX"], dW=s["dW_sign1"]),
        # the layer's optional bias
        "fwd_bias": lambda s: B.bitlinear_fwd(s["x_q"], s["s_x"], s["w_packed"], s["gamma"], K, s["y"],
                                              bias=s["bias"]),
        "bias_grad": lambda s: B.bitlinear_bias_grad(s["dY"], s["db"]),
        # the TTQ variant on the same shape, parameters from its initialization
        "ttq_quantize": lambda s: B.ttq_quantize(s["W"], s["ttq_params"], s["ttq_codes"], s["ttq_wt"]),
        "ttq_fwd": lambda s: B.ttq_fwd(s["x"], s["ttq_wt"], s["y"], workspace=ttq_ws),
        "ttq_fwd_codes": lambda s: B.ttq_fwd_codes(s["x"], s["ttq_codes"], s["ttq_params"], s["y"],
                                                   workspace=ttq_codes_ws),
        "ttq_bwd": lambda s: B.ttq_bwd(s["dY"], s["x"], s["ttq_wt"], s["ttq_codes"], K, dX=s["dX"], dW=s["dW"],
                                       grads=s["ttq_grads"], workspace=ttq_ws),
    }
    xms = {n: per_call_ms(f, sets, args.steps, args.warmup, lead) for n, f in xc.items()}
    # shares of -1 / 0 / +1 in the ternary weight ("bitlinear.py", ternary_stats),
    # from the packed codes of the step (exact counts on the GPU)
    counts = torch.empty((2,), dtype=torch.int64, device=dev)
    B.bitnet_code_counts(sets[0]["w_packed"], K, counts)
    neg, pos = (int(v) for v in counts.cpu())
    ternary = {"minus_one": round(neg / (N * K), 6), "zero": round((N * K - neg - pos) / (N * K), 6),
               "plus_one": round(pos / (N * K), 6)}
    del sets, lead
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    gemm_ops = 2.0 * M * N * K
    w_bytes = 2 if wdt == torch.bfloat16 else 4

    def rate(ms, work, peak, bound, unit, **kw):
        ach = work / (ms * 1e-3)
        return dict(ms=round(ms, 4), bound=bound, unit=unit, achieved=round(ach, 2), frac=round(ach / peak, 4), **kw)

    extra_calls = {
        "bwd_sign1": rate(xms["bwd_sign1"], 2 * gemm_ops / 1e12, PEAK_BF16_TFLOPS, "mfma", "TFLOP/s",
                          dW_bytes_written=N * Kp // 8),
        "fwd_bias": rate(xms["fwd_bias"], gemm_ops / 1e12, PEAK_INT8_TOPS, "mfma", "TOP/s"),
        "bias_grad": rate(xms["bias_grad"], (2.0 * M * N + 4 * N) / 1e9, PEAK_HBM_GBS, "hbm", "GB/s"),
        # read W, write the codes and the bf16 weight
        "ttq_quantize": rate(xms["ttq_quantize"], (w_bytes * N * K + N * Kp / 4 + 2 * N * Kp) / 1e9, PEAK_HBM_GBS,
                             "hbm", "GB/s"),
        "ttq_fwd": rate(xms["ttq_fwd"], gemm_ops / 1e12, PEAK_BF16_TFLOPS, "mfma", "TFLOP/s"),
        "ttq_fwd_codes": rate(xms["ttq_fwd_codes"], gemm_ops / 1e12, PEAK_BF16_TFLOPS, "mfma", "TFLOP/s"),
        "ttq_bwd": rate(xms["ttq_bwd"], 2 * gemm_ops / 1e12, PEAK_BF16_TFLOPS, "mfma", "TFLOP/s"),
    }

    ms_per_step = r["ms_per_step"]
    tops = 3 * gemm_ops / (ms_per_step * 1e-3) / 1e12
    step_calls = ("quantize", "fwd_i8", "bwd_bf16")
    dom = max(step_calls, key=lambda n: kernels[n]["ms"])
    d = kernels[dom]
    peak = {"quantize": PEAK_HBM_GBS, "fwd_i8": PEAK_INT8_TOPS, "bwd_bf16": PEAK_BF16_TFLOPS}[dom]
    roofline = {"kernel": dom, "bound": d["bound"], "achieved": d["achieved"], "peak": peak, "unit": d["unit"],
                "frac": d["frac"], "traffic": load_traffic(dom, args.workload)}

    out = {
        "metric": METRIC if args.workload == HEADLINE else METRIC.replace("4096×2560→6912", f"{M}×{K}→{N}"),
        "value": round(tops, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        # the pages' figure is for the headline shape only
        "vs_baseline": round(tops / PAGES_L4_TOPS, 3) if args.workload == HEADLINE else None,
        "dtype": "int8+bf16",
        "data": "synthetic",
        "config": {"workload": f"bitlinear_fwd_bwd_{M}x{K}x{N}", "M": M, "K": K, "N": N,
                   "w_dtype": inp["w_dtype"], "rotating_buffer_sets": args.rotate},
        "roofline": roofline,
        "ms_per_step_warm": round(r["ms_per_step_warm"], 4),
        "ramp_ms": RAMP_MS,
        "ternary_fractions": ternary,
        "gemm_mfma_frac": gemm_frac,
        "gemm_mfma_frac_of_measured": gemm_frac_meas,
        "measured_ceilings": ceil,
        "kernels": kernels,
        "per_call_mean_ms": {n: round(v, 4) for n, v in r["per_call_mean"].items()},
        "extra_calls": extra_calls,
        "cpu_baseline": None,
    }

    if not args.only_headline:
        configs = {}
        for name in OTHER_WORKLOADS:
            ci = WL.layer_inputs(name, seed=0)
            cr = layer_bench(ci, args.steps, args.warmup, 4 if ci["M"] * ci["K"] < 1 << 24 else 2, dev)
            ck, cf, cfm = layer_roofline(cr, ceil)
            cM, cK, cN = cr["M"], cr["K"], cr["N"]
            e = {"ms_per_step": round(cr["ms_per_step"], 4), "ms_per_step_warm": round(cr["ms_per_step_warm"], 4),
                 "tops": round(6.0 * cM * cN * cK / (cr["ms_per_step"] * 1e-3) / 1e12, 2),
                 "gemm_mfma_frac": cf, "kernels": ck}
            if name.startswith("c5"):
                # few tokens: the step is bound by moving the weight-sized data
                cKp = B.bitnet_k_pad(cK)
                wb = 2 * cN * cK
                step_bytes = (weight_reads(cN, cK, ci["w_dtype"], True) * wb + cN * cKp / 4  # W (once or twice), codes
                              + 2 * cM * cK + cM * cKp + 4 * cM          # act-quant
                              + cN * cKp / 4 + cM * cKp + 2 * cM * cN    # forward: codes, x_q, y
                              + cKp * ((cN + 63) // 64 * 32) + 2 * cM * cN + 2 * cM * cK  # dX: codes, dY, dX
                              + cM * cKp + 2 * cM * cN + wb)             # dW: x_q, dY, dW
                e["step_bytes"] = int(step_bytes)
                e["hbm_frac"] = round(step_bytes / (cr["ms_per_step"] * 1e-3) / (PEAK_HBM_GBS * 1e9), 4)
                e["hbm_frac_of_measured"] = round(step_bytes / (cr["ms_per_step"] * 1e-3) / (ceil["copy_GBps"] * 1e9),
                                                  4)
            configs[f"{name}"] = e
            torch.cuda.empty_cache()
        configs["c4_stack"] = stack_bench(args.steps, args.warmup, dev)
        # the peak bytes in a fresh process, so that no buffer of this one counts
        import subprocess

        try:
            r_ = subprocess.run([sys.executable, os.path.abspath(__file__), "--stack-memory"], capture_output=True,
                                text=True, timeout=600)
            lines = [ln for ln in r_.stdout.splitlines() if ln.startswith("{")]
            if r_.returncode != 0 or not lines:
                raise RuntimeError(f"exit {r_.returncode}: {r_.stderr[-500:]}")
            configs["c4_stack"].update(json.loads(lines[-1]))
        except (RuntimeError, OSError, ValueError, subprocess.TimeoutExpired) as e:
            # the timed figures stand; the memory figure is reported as missing
            print(f"bench.py: --stack-memory failed: {e}", file=sys.stderr)
            configs["c4_stack"]["peak_allocated_error"] = str(e)[:300]
        out["configs"] = configs

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp)
        out["cpu_baseline"]["value"] = round(out["cpu_baseline"]["value"], 6)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
