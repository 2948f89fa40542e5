"""Benchmark of the quantized MoE hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input
resident in HBM: routing + block alignment, activation quantization (fp8
formats), the grouped GEMM with its fused scale / router-weight epilogue, and
the per-token combine (MXFP8: quantization + grouped GEMM).

Default workload: the mistral-7B-shaped up projection in fp8 W8A8, M=4096
tokens, K=4096, N=28672, E=8, top_k=2 (the first row of the FP8_W8A8 "Model
Results" on "Tianxing/moe quantization"; the largest E=8, top_k=2
configuration on one GPU, bound by the fp8 MFMA peak).  The same run also
times the int8 W8A16 decode shape (M=64, K=4096, N=14336, bound by HBM) and
reports it under "decode".  ``--workload`` selects one other workload (names
in quantized_moe_grouped_top_amd.synth.WORKLOADS) and times only that.

The expert weights exist in several copies that the steps rotate through, so
that no step finds its weights in the 256 MB Infinity Cache or in L2 from the
step before.

Prints one JSON line: value = whole-step throughput in algorithmic HBM GB/s
(the byte count of the "Tianxing/moe quantization" tables: activations +
expert weights + scales + per-slot bf16 outputs), plus the TFLOPS of the
step, the roofline of the dominant kernel (the grouped GEMM: after the timed
steps, as many back-to-back launches of it on the steps' buffers, weights
still rotated, bracketed by a pair of HIP events on the stream it runs on,
torch's current stream) and the CPU oracle timed on the host.
"""

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"fp8": 5033.0, "mxfp8": 5033.0, "bf16": 2516.0, "int8": 5033.0}
DEFAULT_WORKLOAD = "mistral7b_up_fp8_m4096_k4096_n28672"
DECODE_WORKLOAD = "int8w8a16_m64_k4096_n14336"


def alg_bytes(wl, active_experts=None):
    """Algorithmic bytes of one grouped GEMM call: every activation, weight
    and scale byte read once, every per-slot output written once as bf16."""
    E = wl.E if active_experts is None else active_experts
    M, K, N = wl.M, wl.K, wl.N
    if wl.fmt.startswith("act_"):
        # fused activation + quantization: the bf16 input [M, K] read once, the
        # codes [M, N] and the scales written once (MXFP8: per-expert padded
        # scale rows of N/32 bytes; fp8: one float)
        sf = 4 if wl.fmt == "act_fp8" else sum(-(-m // 128) * 128 for m in wl.seg) * (N // 32)
        return 2 * M * K + M * N + sf
    if wl.fmt == "fp8":
        return M * K + E * N * K + 4 * (E + 1) + M * wl.top_k * N * 2
    if wl.fmt in ("int8", "fp8wo"):   # bf16 rows, one-byte weights + channel scales
        return 2 * M * K + E * N * K + 4 * E * N + M * wl.top_k * N * 2
    if wl.fmt == "int4wo":            # bf16 rows, half-byte weights + channel scales
        return 2 * M * K + E * N * K // 2 + 4 * E * N + M * wl.top_k * N * 2
    if wl.fmt == "int8dq":      # int8 rows + one scale per token, int8 weights + channel scales
        return M * K + 4 * M + E * N * K + 4 * E * N + M * wl.top_k * N * 2
    if wl.fmt == "mxfp8_dgrad":       # dy codes + scales, weights along N, bf16 dx [M, K]
        return M * N * (1 + 1 / 32) + E * N * K * (1 + 1 / 32) + 2 * M * K
    if wl.fmt == "mxfp8_wgrad":       # columnwise dy and x (padded rows), bf16 dw [E, N, K]
        P = sum(-(-m // 128) * 128 for m in wl.seg)
        return (N + K) * P * (1 + 1 / 32) + 2 * E * N * K
    # MXFP8: data + e8m0 scales of both operands, bf16 output rows
    return M * K * (1 + 1 / 32) + E * N * K * (1 + 1 / 32) + 2 * M * N


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default=None,
                   help=f"one workload to time (default: {DEFAULT_WORKLOAD}, plus "
                        f"{DECODE_WORKLOAD} reported under 'decode')")
    p.add_argument("--copies", type=int, default=0,
                   help="weight copies rotated over (0: enough for >= 1 GiB of weights)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="target CPU time of the oracle baseline")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device-to-device copy 10 times (the known-size "
                        "kernel that scales the FETCH_SIZE / WRITE_SIZE counters)")
    return p.parse_args()


GEMM_SOURCES = ("qmoe_gemm.hip", "qmoe_gemm_tile.hip", "qmoe_device.h", "qmoe_internal.h")
ACT_SOURCES = ("qmoe_quant.hip", "qmoe_internal.h")


def _code_only(text):
    """C++ source without its comments and with whitespace runs collapsed
    (string and character literals kept as they are)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash(workload=None):
    """sha256 over the code (comments and layout left out) of the sources of
    the workload's timed kernel (the grouped GEMM, or the fused activation
    quantization): a recorded HBM traffic figure is only valid for the code
    it was counted on."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "quantized_moe_grouped_top_amd", "csrc")
    act = workload is not None and workload.startswith(("swiglu_", "srelu_"))
    for name in ACT_SOURCES if act else GEMM_SOURCES:
        with open(os.path.join(d, name), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()


def recorded_traffic(workload):
    """HBM bytes per grouped-GEMM launch counted by rocprofv3 (FETCH_SIZE +
    WRITE_SIZE, scaled by the copy-kernel factor) for this workload, read from
    the traffic summaries under profiles/; None when there is none or when the
    kernel sources changed since the counters were taken."""
    want = kernel_source_hash(workload)
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*traffic*.md"))):
        text = open(path).read()
        fields = dict(re.findall(r"^- (\w+): `([^`]*)`", text, re.M))
        if fields.get("workload") == workload and fields.get("kernel_source_sha256") == want:
            return int(fields["traffic_bytes_per_launch"])
    return None


def copy_calibration():
    """One elementwise kernel over 1 GiB of float32 (read once, written once),
    launched 10 times: torch's own element-wise kernel, not a DMA blit."""
    import torch
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(10):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"kernel": "torch.neg float32", "bytes_read": 4 * n,
                                           "bytes_written": 4 * n, "launches": 10}}), flush=True)


def _sample_weights(O, w, fmt, cols):
    """Oracle weight quantization of the output channels `cols` of every
    expert (an expert's per-tensor fp8 scale still comes from its whole
    matrix): offline, outside the timed region."""
    import numpy as np
    rows = w[:, cols]
    if fmt == "fp8":
        s = np.array([O.fp8_tensor_scale(w[e]) for e in range(w.shape[0])], np.float32)
        q = np.stack([O.fp8_quantize_with_scale(rows[e], s[e]) for e in range(w.shape[0])])
        return q, s
    return {"fp8wo": O.quantize_weight_fp8_rows, "int4wo": O.quantize_weight_int4}.get(
        fmt, O.quantize_weight_int8)(rows)


def cpu_baseline(wl, case, target_s):
    """The CPU oracle on the same workload, timed on the host, on a bounded
    sample: the whole step (routing, alignment, activation quantization,
    grouped GEMM, combine) repeated until target_s seconds have passed (at
    least once).  Weight quantization is offline and not timed.  Routed
    workloads above 0.25 TFLOP run the step over every token
    but only the first n_s output columns, and the time is scaled by N / n_s."""
    import numpy as np
    from oracle import formats as F
    from oracle import moe as O

    x = case["x"].view(__import__("torch").int16).cpu().numpy().view(np.uint16)
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    if wl.fmt.startswith("act_"):
        act = O.ACT_SWIGLU if wl.act == "swiglu" else O.ACT_SRELU
        rows = max(1, min(wl.M, 2000))            # a bounded sample of whole rows
        reps, t0 = 0, time.perf_counter()
        while True:
            if wl.fmt == "act_mxfp8":
                O.act_quantize_mxfp8(x[:rows], [0, rows], act)
            else:
                O.act_quantize_fp8(x[:rows], act)
            reps += 1
            el = time.perf_counter() - t0
            if el >= target_s:
                break
        per = el / reps * wl.M / rows
        return {"value": round(alg_bytes(wl) / per / 1e9, 3), "unit": "GB/s", "cores": threads,
                "kind": "oracle",
                "sample": f"the first {rows} of {wl.M} rows, {reps} time(s) in {el:.1f} s, "
                          f"scaled to the whole input (numpy float64)"}
    w = case["w"].cpu().numpy()
    if wl.fmt in ("mxfp8_dgrad", "mxfp8_wgrad"):
        mo = case["m_offsets"].cpu().numpy()
        dy = case["dy"].view(__import__("torch").int16).cpu().numpy().view(np.uint16)
        wq, wsf = O.quantize_weight_mxfp8_colwise(w) if wl.fmt == "mxfp8_dgrad" else (None, None)
        del w
        reps, t0 = 0, time.perf_counter()
        while True:
            if wl.fmt == "mxfp8_dgrad":
                dq, dsf = O.quantize_act_mxfp8(dy, mo)
                O.grouped_linear_dgrad_mxfp8(dq, dsf, wq, wsf, mo)
            else:
                dT, dTsf = O.quantize_act_mxfp8_colwise(dy, mo)
                xT, xTsf = O.quantize_act_mxfp8_colwise(x, mo)
                O.grouped_linear_wgrad_mxfp8(dT, dTsf, xT, xTsf, mo, wl.N, wl.K)
            reps += 1
            el = time.perf_counter() - t0
            if el >= target_s:
                break
        per = el / reps
        return {"value": round(alg_bytes(wl) / per / 1e9, 3), "unit": "GB/s", "cores": threads,
                "kind": "oracle", "tflops": round(wl.flops / per / 1e12, 6),
                "sample": f"whole workload, {reps} step(s) in {el:.1f} s "
                          f"(numpy float64; BLAS threads = OMP_NUM_THREADS or all cores)"}
    n_s = wl.N
    if wl.fmt == "mxfp8":
        wq, wsf = O.quantize_weight_mxfp8(w)
        mo = case["m_offsets"].cpu().numpy()
    else:
        budget = 2.5e11                             # flops of the sampled step
        if wl.flops > budget:
            n_s = max(256, min(wl.N, int(wl.N * budget / wl.flops) // 256 * 256))
        wq, ws = _sample_weights(O, w, wl.fmt, np.arange(n_s))
        lg = case["logits"].cpu().numpy()
    del w
    reps, t0 = 0, time.perf_counter()
    while True:
        if wl.fmt == "mxfp8":
            aq, asf = O.quantize_act_mxfp8(x, mo)
            O.grouped_gemm_mxfp8(aq, asf, wq, wsf, mo)
        else:
            ids, wts = O.route_topk(lg, wl.top_k)
            O.align_block_size(ids, wl.E, 16)
            if wl.fmt == "fp8":
                aq, sa = O.quantize_act_fp8(x)
                y = O.grouped_gemm_fp8w8a8(aq, sa, wq, ws, ids, wts)
            elif wl.fmt == "int8dq":
                aq, sa = O.quantize_act_int8_rows(x)
                y = O.grouped_gemm_int8w8a8(aq, sa, wq, ws, ids, wts)
            elif wl.fmt == "fp8wo":
                y = O.grouped_gemm_fp8w8a16(x, wq, ws, ids, wts)
            elif wl.fmt == "int4wo":
                y = O.grouped_gemm_int4w16(x, wq, ws, ids, wts)
            else:
                y = O.grouped_gemm_int8w8a16(x, wq, ws, ids, wts)
            O.combine(F.bf16_decode(O.slot_results_bf16(y)), wl.top_k)
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s:
            break
    per = el / reps * wl.N / n_s
    what = ("whole workload" if n_s == wl.N else
            f"every token, output columns 0..{n_s - 1} of {wl.N}, time scaled by N / {n_s}")
    return {"value": round(alg_bytes(wl) / per / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "tflops": round(wl.flops / per / 1e12, 6),
            "sample": f"{what}; {reps} step(s) in {el:.1f} s "
                      f"(numpy float64; BLAS threads = OMP_NUM_THREADS or all cores)"}


def measure(wl, args):
    """Time `args.steps` steps of one workload after `args.warmup` untimed
    ones.  Returns (fields of the JSON line, the inputs, the layer object)."""
    import torch

    import quantized_moe_grouped_top_amd as qm
    from quantized_moe_grouped_top_amd import runner, synth

    case = synth.make_case(wl, 0, device="cuda")
    layout = None
    # step(i): one pass of the whole path; kernel(i): the timed kernel alone,
    # on the buffers the steps leave behind (inputs rotated the same way)
    if wl.fmt.startswith("act_"):
        # input copies rotate so that no step finds its input in a cache
        copies = args.copies or max(2, -(-(1 << 30) // (2 * case["x"].numel())))
        xs = [case["x"]] + [case["x"].clone() for _ in range(copies - 1)]
        moe = runner.ActQuant(wl.M, wl.N, wl.E, wl.act, wl.fmt[4:])
        mo = case["m_offsets"]

        def kernel(i):
            moe(xs[i % copies], mo)

        step = kernel
    elif wl.fmt == "mxfp8_wgrad":
        copies = 1                             # operands are made from x and dy every step
        moe = runner.MxWgrad(wl.M, wl.K, wl.N, wl.E, wl.seg)
        mo = case["m_offsets"]

        def kernel(i):
            moe.gemm()

        def step(i):
            moe.quantize(case["dy"], case["x"], mo)
            moe.gemm()
    else:
        w_q, w_s = runner.quantize_weights(
            case["w"], "mxfp8_colwise" if wl.fmt == "mxfp8_dgrad" else wl.fmt)
        if not wl.fmt.startswith("mxfp8"):
            # decode (block_m 16): fragment-ordered weights, one contiguous 1 KB
            # read per MFMA operand; otherwise tiles of one 8 KB block per stage
            layout = (qm.MOE_W_FRAG if qm.moe_recommended_block_m(wl.M, wl.E, wl.top_k) == 16
                      else qm.MOE_W_TILED)
            w_q = runner.pack_weights(w_q, layout)
        copies = args.copies or max(2, -(-(1 << 30) // w_q.numel()))
        weights = [(w_q, w_s)] + [(w_q.clone(), w_s.clone()) for _ in range(copies - 1)]
        if wl.fmt in ("mxfp8_dgrad", "mxfp8"):
            # dgrad: the output gradient [M, N] against the weights along N: dx [M, K]
            if wl.fmt == "mxfp8_dgrad":
                moe, src = runner.MxMoE(wl.M, wl.N, wl.K, wl.E), case["dy"]
            else:
                moe, src = runner.MxMoE(wl.M, wl.K, wl.N, wl.E), case["x"]
            mo = case["m_offsets"]

            def kernel(i):
                q, s = weights[i % copies]
                moe.gemm(q, s, mo)

            def step(i):
                moe.quantize(src, mo)
                kernel(i)
        else:
            moe = runner.RoutedMoE(wl.fmt, wl.M, wl.K, wl.N, wl.E, wl.top_k, w_layout=layout)

            def kernel(i):
                q, s = weights[i % copies]
                moe.gemm(case["x"], q, s)

            def step(i):
                moe.route(case["logits"])
                moe.quantize(case["x"])
                kernel(i)
                moe.combine()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # The timed kernel's mean launch duration: HIP events on the stream the
    # library launches on (torch's current stream) around the same number of
    # back-to-back launches, with the weights (or inputs) still rotated.
    # Events around each launch inside the steps would also count the
    # dispatch after an event marker (~6 us per launch at decode, where
    # rocprofv3's kernel duration is 76.8 us and such events read 82.8 us).
    # One untimed launch goes first, so that the GPU is busy when the first
    # event is reached and the host's launch latency stays outside the events;
    # short kernels get more launches (about 20 ms of them: a window of a few
    # milliseconds varies by ~10% from run to run on the device's clocks).
    n_kernel = max(args.steps, min(2000, int(20.0 / max(elapsed * 1e3 / args.steps, 1e-3))))
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    kernel(args.warmup + args.steps)
    ev0.record()
    for i in range(n_kernel):
        kernel(args.warmup + args.steps + 1 + i)
    ev1.record()
    torch.cuda.synchronize()
    gemm_ms = ev0.elapsed_time(ev1) / n_kernel

    active = wl.E
    if wl.fmt in ("fp8", "int8", "int8dq", "fp8wo", "int4wo"):
        ids = moe.topk_ids.cpu()
        active = int(torch.unique(ids).numel())
    nbytes = alg_bytes(wl, active)
    ms = elapsed * 1e3 / args.steps
    dtype = {"fp8": "fp8", "int8": "bf16", "int8dq": "int8", "fp8wo": "bf16", "int4wo": "bf16",
             "mxfp8": "mxfp8", "mxfp8_dgrad": "mxfp8", "mxfp8_wgrad": "mxfp8", "act_fp8": "fp8",
             "act_mxfp8": "mxfp8"}[wl.fmt]
    is_act = wl.fmt.startswith("act_")
    bound = "hbm" if is_act or wl.flops / nbytes < 600 else "mfma"
    if bound == "hbm":
        achieved = nbytes / (gemm_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = wl.flops / (gemm_ms * 1e-3) / 1e12
        peak = MFMA_PEAK_TFLOPS[dtype]
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4)}
    roof.update({"traffic": recorded_traffic(wl.name),
                 "kernel": "fused activation + quantization" if is_act else "grouped GEMM",
                 "kernel_us": round(gemm_ms * 1e3, 2), "kernel_launches": n_kernel,
                 "alg_bytes": int(nbytes),
                 "flops": None if is_act else int(wl.flops)})
    fields = {
        "value": round(nbytes / (ms * 1e-3) / 1e9, 2),
        "tflops": None if is_act else round(wl.flops / (ms * 1e-3) / 1e12, 3),
        "ms_per_step": round(ms, 5),
        "dtype": dtype,
        "config": {"workload": wl.name, "format": wl.fmt, "M": wl.M, "K": wl.K, "N": wl.N,
                   "E": wl.E, "top_k": wl.top_k,
                   ("input_copies" if is_act else "weight_copies"): copies,
                   "block_m": getattr(moe, "block_m", None),
                   "weight_layout": None if layout is None else
                   {qm.MOE_W_TILED: "tiled", qm.MOE_W_FRAG: "frag"}.get(layout, "rowmajor")},
        "roofline": roof,
    }
    return fields, case, moe


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported "
              f"(the library runs the hot path on one MI355X).", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import torch

    import quantized_moe_grouped_top_amd as qm
    from quantized_moe_grouped_top_amd import synth

    qm.lib()                                   # fail loudly if the library is missing
    torch.cuda.set_device(0)
    wl = synth.WORKLOADS[args.workload or DEFAULT_WORKLOAD]
    fields, case, moe = measure(wl, args)
    del moe
    line = {
        "metric": "TFLOPS and HBM GB/s (% of MI355X roofline) for quantized MoE GEMM, E=8 top_k=2",
        "value": fields["value"],
        "unit": "GB/s",
        "tflops": fields["tflops"],
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": fields["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": fields["dtype"],
        "data": "synthetic (seeded N(0,1) activations and logits, N(0,1/sqrt(K)) weights)",
        "config": fields["config"],
        "roofline": fields["roofline"],
    }
    if args.workload is None:
        # the HBM-bound decode shape, timed in the same run (no CPU baseline),
        # right after the first workload while the GPU is still busy (an idle
        # GPU, e.g. during the CPU baseline, lowers its clocks first)
        torch.cuda.empty_cache()
        dargs = argparse.Namespace(**vars(args))
        dargs.warmup = max(args.warmup, 100)
        dfields, _, _ = measure(synth.WORKLOADS[DECODE_WORKLOAD], dargs)
        line["decode"] = {"workload": DECODE_WORKLOAD, "ms_per_step": dfields["ms_per_step"],
                          "value": dfields["value"], "unit": "GB/s",
                          "gemm_us": dfields["roofline"]["kernel_us"],
                          "roofline": dfields["roofline"]}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, case, args.cpu_seconds)
    del case
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
