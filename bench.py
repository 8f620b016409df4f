"""Benchmark: one BitLinear forward + STE backward step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--rotate R] [--no-cpu-baseline]

A step is the whole hot path on one batch: ternarize + pack the master
weights, int8-quantize the activations, the INT8 forward GEMM, and the two
bf16 STE backward GEMMs (dX and dW, one bitlinear_bwd call), all through
the C ABI of libbitnet.so on torch's current stream. Inputs are seeded synthetic tensors of the
4096 x 2560 -> 6912 layer (x, dY ~ N(0,1) bf16, W ~ U(+-1/sqrt(2560)) bf16),
resident in HBM before timing starts. R independent copies of all buffers
are rotated step by step so that the working set (~240 MB per copy) does not
sit in the 256 MB Infinity Cache between steps.

Prints one JSON line: throughput in effective TOPS (6*M*N*K per step), the
step time (replays of the step captured in HIP graphs, one per buffer set),
per-call times from HIP events recorded on the launch stream around eager calls,
the roofline of the dominant kernel, and the CPU oracle timed on a bounded
sample of the same workload (rank 0 only).
"""

import argparse
import hashlib
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


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default=HEADLINE)
    p.add_argument("--rotate", type=int, default=4)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain device copy of known size (for counter calibration)")
    p.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR", "CAL_WRITE_DIR"),
                   help="turn rocprofv3 FETCH_SIZE / WRITE_SIZE runs of the bench and of --copy-calibration "
                        "into profiles/pmc_traffic.json (no GPU needed)")
    return p.parse_args()


# bench kernel name -> substrings of the device kernel names it launches
KERNEL_MATCH = {
    "ternarize_pack": ["absmean_partials_kernel", "ternarize_pack_kernel"],
    "act_quant": ["act_quant"],
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
    }


def main():
    args = parse()
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

    if args.copy_calibration:
        copy_calibration()
        return

    import numpy as np
    import torch

    from ternary_weight_quantization_amd import binding as B
    from ternary_weight_quantization_amd import workloads as WL

    B.lib()
    dev = torch.device("cuda:0")
    inp = WL.layer_inputs(args.workload, seed=0)
    M, K, N = inp["M"], inp["K"], inp["N"]
    Kp = B.bitnet_k_pad(K)
    wdt = torch.bfloat16 if inp["w_dtype"] == "bf16" else torch.float32

    def to_dev(a, dtype):
        if dtype == torch.bfloat16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    sets = []
    base = dict(x=to_dev(inp["x"], torch.bfloat16), W=to_dev(inp["W"], wdt), dY=to_dev(inp["dY"], torch.bfloat16))
    for r in range(args.rotate):
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

    names = ["ternarize_pack", "act_quant", "fwd_i8", "bwd_bf16"]

    def step(s, ev=None):
        calls = [
            lambda: B.bitnet_ternarize_pack(s["W"], s["w_packed"], s["gamma"], s["ws"]),
            lambda: B.bitnet_act_quant(s["x"], s["x_q"], s["s_x"]),
            lambda: B.bitlinear_fwd(s["x_q"], s["s_x"], s["w_packed"], s["gamma"], K, s["y"]),
            lambda: B.bitlinear_bwd(s["dY"], s["x_q"], s["s_x"], s["w_packed"], s["gamma"], K, dX=s["dX"], dW=s["dW"]),
        ]
        for i, c in enumerate(calls):
            if ev is not None:
                ev[i][0].record()
            c()
            if ev is not None:
                ev[i][1].record()

    for i in range(args.warmup):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()

    # Per-call times: eager steps with HIP events around each call, on the
    # stream the library launches on.
    evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in names]
           for _ in range(args.steps)]
    for i in range(args.steps):
        step(sets[i % len(sets)], evs[i])
    torch.cuda.synchronize()
    per_kernel = {n: float(np.mean([evs[i][j][0].elapsed_time(evs[i][j][1]) for i in range(args.steps)]))
                  for j, n in enumerate(names)}

    # Step time: graph replays, so that host-side call overhead stays out of
    # the timed region (the same kernels and work as the eager step). When
    # the step count is a multiple of the number of buffer sets, one graph
    # holds one step on each set in turn (a training loop captures many
    # layers in one graph, and this keeps the per-launch gap of a graph out
    # of every step); otherwise each set's step is its own graph. Every
    # replay pattern is first checked to reproduce the eager outputs bit for
    # bit.
    outs = ("y", "dX", "dW")
    ref = [{k: s[k].clone() for k in outs} for s in sets]
    R = len(sets)
    chained = args.steps % R == 0
    graphs = []
    if chained:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for s in sets:
                step(s)
        graphs.append(g)
    else:
        for s in sets:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(s)
            graphs.append(g)
    for s in sets:
        for k in outs:
            s[k].zero_()
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    for i, s in enumerate(sets):
        for k in outs:
            if not torch.equal(s[k], ref[i][k]):
                raise SystemExit(f"bench.py: graph replay differs from the eager step in {k} (set {i})")
    replays = args.steps // R if chained else args.steps
    for i in range(max(1, args.warmup // R) if chained else args.warmup):
        graphs[i % len(graphs)].replay()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(replays):
        graphs[i % len(graphs)].replay()
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps

    # The backward with dW as 1-bit signs for a sign-based optimiser (dX and
    # the dW signs in one call; no bf16 dW is written), timed per call like
    # the step's calls. Not part of the step.
    for s in sets:
        s["dW_sign1"] = torch.empty((N, Kp // 8), dtype=torch.uint8, device=dev)

    def bwd_sign1(s):
        B.bitlinear_bwd(s["dY"], s["x_q"], s["s_x"], s["w_packed"], s["gamma"], K, dX=s["dX"], dW=s["dW_sign1"])

    # The forward with a bias and the bias gradient (the layer's optional
    # bias), timed the same way; not part of the step.
    for s in sets:
        s["bias"] = torch.zeros((N,), dtype=torch.bfloat16, device=dev)
        s["db"] = torch.empty((N,), dtype=torch.float32, device=dev)

    def fwd_bias(s):
        B.bitlinear_fwd(s["x_q"], s["s_x"], s["w_packed"], s["gamma"], K, s["y"], bias=s["bias"])

    def bias_grad(s):
        B.bitlinear_bias_grad(s["dY"], s["db"])

    # The TTQ variant on the same shape ("TTQ_VERIFICATION.md": bf16
    # activations, a bf16 weight of {Wp, 0, -Wn}): quantize, forward, and the
    # backward with dX, dW and the two scale gradients; parameters from its
    # initialization. Timed the same way; not part of the step.
    for s in sets:
        s["ttq_params"] = torch.empty((3,), dtype=torch.float32, device=dev)
        B.ttq_init(s["W"], s["ttq_params"], s["ws"])
        s["ttq_codes"] = torch.empty((N, Kp // 4), dtype=torch.uint8, device=dev)
        s["ttq_wt"] = torch.empty((N, Kp), dtype=torch.bfloat16, device=dev)
        s["ttq_grads"] = torch.empty((2,), dtype=torch.float32, device=dev)
    ttq_ws = torch.empty((max(B.ttq_workspace_bytes(M, N, K), 1),), dtype=torch.uint8, device=dev)

    def ttq_quantize(s):
        B.ttq_quantize(s["W"], s["ttq_params"], s["ttq_codes"], s["ttq_wt"])

    def ttq_fwd(s):
        B.ttq_fwd(s["x"], s["ttq_wt"], s["y"], workspace=ttq_ws)

    # the forward from the stored codes and params (the exported state): the
    # few-token kernel at M <= 64, else the codes expanded and the GEMM
    ttq_codes_ws = torch.empty((max(B.ttq_fwd_codes_workspace_bytes(M, N, K), 1),), dtype=torch.uint8, device=dev)

    def ttq_fwd_codes(s):
        B.ttq_fwd_codes(s["x"], s["ttq_codes"], s["ttq_params"], s["y"], workspace=ttq_codes_ws)

    def ttq_bwd(s):
        B.ttq_bwd(s["dY"], s["x"], s["ttq_wt"], s["ttq_codes"], K, dX=s["dX"], dW=s["dW"], grads=s["ttq_grads"],
                  workspace=ttq_ws)

    def per_call_ms(f):
        for i in range(args.warmup):
            f(sets[i % len(sets)])
        ev1 = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
               for _ in range(args.steps)]
        for i in range(args.steps):
            ev1[i][0].record()
            f(sets[i % len(sets)])
            ev1[i][1].record()
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in ev1]))

    sign1_ms = per_call_ms(bwd_sign1)
    fwd_bias_ms = per_call_ms(fwd_bias)
    bias_grad_ms = per_call_ms(bias_grad)
    ttq_quantize(sets[0])
    torch.cuda.synchronize()
    ttq_ms = {n: per_call_ms(f) for n, f in (("quantize", ttq_quantize), ("fwd", ttq_fwd), ("bwd", ttq_bwd),
                                              ("fwd_codes", ttq_fwd_codes))}

    gemm_ops = 2.0 * M * N * K
    tops = 3 * gemm_ops / (ms_per_step * 1e-3) / 1e12
    # roofline of each kernel (algorithmic work per launch)
    w_bytes = 2 if wdt == torch.bfloat16 else 4
    roof = {
        "fwd_i8": ("mfma", gemm_ops / 1e12, PEAK_INT8_TOPS, "TOP/s"),
        # dX and dW in one call (two products)
        "bwd_bf16": ("mfma", 2 * gemm_ops / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"),
        # two reads of W plus the 2-bit write
        "ternarize_pack": ("hbm", (2 * w_bytes * N * K + N * Kp / 4) / 1e9, PEAK_HBM_GBS, "GB/s"),
        # read x (bf16), write x_q (int8, padded) and s
        "act_quant": ("hbm", (2.0 * M * K + M * Kp + 4 * M) / 1e9, PEAK_HBM_GBS, "GB/s"),
    }
    fracs = {}
    for n, (bound, work, peak, unit) in roof.items():
        achieved = work / (per_kernel[n] * 1e-3)
        fracs[n] = dict(bound=bound, achieved=achieved, peak=peak, unit=unit, frac=achieved / peak,
                        ms=per_kernel[n])
    dom = max(per_kernel, key=per_kernel.get)
    d = fracs[dom]
    traffic = load_traffic(dom, args.workload)
    roofline = {"kernel": dom, "bound": d["bound"], "achieved": round(d["achieved"], 3), "peak": d["peak"],
                "unit": d["unit"], "frac": round(d["frac"], 4), "traffic": traffic}

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
        "kernels": {n: {"ms": round(f["ms"], 4), "frac": round(f["frac"], 4), "bound": f["bound"],
                        "achieved": round(f["achieved"], 2), "unit": f["unit"]} for n, f in fracs.items()},
        "extra_calls": {"bwd_sign1": {
            "ms": round(sign1_ms, 4), "bound": "mfma", "unit": "TFLOP/s",
            "achieved": round(2 * gemm_ops / 1e12 / (sign1_ms * 1e-3), 2),
            "frac": round(2 * gemm_ops / 1e12 / (sign1_ms * 1e-3) / PEAK_BF16_TFLOPS, 4),
            "dW_bytes_written": N * Kp // 8},
            "fwd_bias": {
                "ms": round(fwd_bias_ms, 4), "bound": "mfma", "unit": "TOP/s",
                "achieved": round(gemm_ops / 1e12 / (fwd_bias_ms * 1e-3), 2),
                "frac": round(gemm_ops / 1e12 / (fwd_bias_ms * 1e-3) / PEAK_INT8_TOPS, 4)},
            "bias_grad": {
                "ms": round(bias_grad_ms, 4), "bound": "hbm", "unit": "GB/s",
                "achieved": round((2.0 * M * N + 4 * N) / 1e9 / (bias_grad_ms * 1e-3), 2),
                "frac": round((2.0 * M * N + 4 * N) / 1e9 / (bias_grad_ms * 1e-3) / PEAK_HBM_GBS, 4)},
            # read W, write the codes and the bf16 weight
            "ttq_quantize": {
                "ms": round(ttq_ms["quantize"], 4), "bound": "hbm", "unit": "GB/s",
                "achieved": round((w_bytes * N * K + N * Kp / 4 + 2 * N * Kp) / 1e9 / (ttq_ms["quantize"] * 1e-3), 2),
                "frac": round((w_bytes * N * K + N * Kp / 4 + 2 * N * Kp) / 1e9 / (ttq_ms["quantize"] * 1e-3)
                              / PEAK_HBM_GBS, 4)},
            "ttq_fwd": {
                "ms": round(ttq_ms["fwd"], 4), "bound": "mfma", "unit": "TFLOP/s",
                "achieved": round(gemm_ops / 1e12 / (ttq_ms["fwd"] * 1e-3), 2),
                "frac": round(gemm_ops / 1e12 / (ttq_ms["fwd"] * 1e-3) / PEAK_BF16_TFLOPS, 4)},
            # rate on the forward's flops; at few tokens the bound is reading
            # the codes (N * Kp / 4 bytes) and x
            "ttq_fwd_codes": {
                "ms": round(ttq_ms["fwd_codes"], 4), "bound": "mfma", "unit": "TFLOP/s",
                "achieved": round(gemm_ops / 1e12 / (ttq_ms["fwd_codes"] * 1e-3), 2),
                "frac": round(gemm_ops / 1e12 / (ttq_ms["fwd_codes"] * 1e-3) / PEAK_BF16_TFLOPS, 4),
                "codes_GB_per_s": round((N * Kp / 4 + 2.0 * M * K + 2.0 * M * N) / 1e9 / (ttq_ms["fwd_codes"] * 1e-3),
                                        2)},
            "ttq_bwd": {
                "ms": round(ttq_ms["bwd"], 4), "bound": "mfma", "unit": "TFLOP/s",
                "achieved": round(2 * gemm_ops / 1e12 / (ttq_ms["bwd"] * 1e-3), 2),
                "frac": round(2 * gemm_ops / 1e12 / (ttq_ms["bwd"] * 1e-3) / PEAK_BF16_TFLOPS, 4)}},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp)
        out["cpu_baseline"]["value"] = round(out["cpu_baseline"]["value"], 6)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
