#!/usr/bin/env python3
"""Benchmark of the Nyström self-attention forward on one MI355X.

One step = one ``nystrom_attn_fwd`` call over a whole batch (segment means,
landmark softmaxes, pseudoinverse, B~V, W, output with the conv skip).  The
default workload is batch 2 x 12 heads, n = 8192, d = 64, m = 64, bf16 I/O,
6 iterations, conv kernel 33.

Inputs are seeded synthetic tensors already resident in HBM.  The timed steps
rotate over several independent input/output sets whose total exceeds the
256 MB last-level cache, so every call reads its inputs from HBM.

Prints one JSON line.  ``value`` is tokens/s (batch * n per step; with
``--lengths``, a batch of right-padded sequences, the real tokens) over exactly
``--steps`` calls timed with two events on the launch stream; a second pass
records an event between calls (``per_call_us``: median, p10, p90) and a
third has the library bracket every kernel with events.  ``roofline`` is for
the kernel with the largest share of GPU time: its algorithmic bytes per
launch divided by its mean event-timed duration; ``traffic`` is that
kernel's scaled HBM bytes per launch from the committed counter summary
``profiles/hbm_traffic_<workload>.txt`` when it was made from the current
kernel sources, else null.  ``cpu_baseline`` is the fp64 CPU oracle timed on
the host on whole calls of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix cores, TFLOP/s
FP32_VECTOR_PEAK_TFLOPS = 157.3  # fp32 vector ALUs, TFLOP/s
METRIC = "Nyström attention fwd tokens/s at n=8192,m=64,d=64; % of HBM roofline"

# Context from the paper's efficiency table (GTX 1080Ti, self-attention module
# only, random inputs, precision and head shape not stated): at n = 8192 the
# 64-landmark variant took 12.3 ms and 450 MB against 155.4 ms and 10,233 MB
# for standard attention.
PAGES_CONTEXT = {"hardware": "GTX 1080Ti (not comparable)", "n": 8192, "nystrom64_ms": 12.3,
                 "standard_ms": 155.4, "nystrom64_MB": 450, "standard_MB": 10233,
                 "speedup_vs_standard": 12.7, "memory_reduction_vs_standard": 22.8}


def algorithmic_bytes(wl, kernel: str, token_rows=None) -> int:
    """Bytes each kernel must move per launch: the per-row figure times the
    token rows over all heads (batch * heads * n, or the sum of the
    per-sequence lengths times heads with a key-padding mask)."""
    e = wl.elem_bytes
    all_rows = wl.batch * wl.heads * wl.n
    rows = all_rows if token_rows is None else token_rows
    row = wl.d * e
    convw = 4 * wl.heads * wl.d * wl.conv_k
    if kernel == "segment_mean":
        return 2 * row * rows                  # read Q and K
    if kernel in ("landmark_bv", "landmark_pass"):
        return 2 * row * rows                  # read K and V (the m x m pseudoinverse beside it moves no n-sized data)
    if kernel == "apply":
        return (2 * rows + all_rows) * row + convw  # read Q, V (token rows); write every row of O
    return 0


def backward_flops(wl, kernel: str) -> float:
    """Flops each backward kernel performs per launch (2 per multiply-add;
    per-row figure x rows over all heads)."""
    rows = float(wl.batch * wl.heads * wl.n)
    md, kd = wl.m * wl.d, wl.conv_k * wl.d
    # bf16 I/O at d = 32, 64: matrix-core passes, with the skip in kernels of its own.
    mm = wl.dtype == "bf16" and wl.d in (32, 64)
    if kernel == "bwd_rows_reduce":
        return rows * 2 * 4 * md           # scores, dO W^T, F^T dO, dS^T Q
    if kernel == "bwd_keys":
        # scores, dBV V^T, dS^T Qt, B^T dBV, dS K; the vector path also runs
        # the skip's transpose and filter gradient here
        return rows * 2 * (5 * md + (0 if mm else 2 * kd))
    if kernel == "bwd_skip_grad":
        return rows * 2 * kd               # filter gradient
    if kernel == "dconv":
        return rows * 2 * kd               # the skip's transpose (the forward's convolution)
    if kernel == "bwd_rows_dq":
        return rows * 2 * 3 * md           # scores, dO W^T, dS Kt
    if kernel == "bwd_land_prep":
        return wl.batch * wl.heads * 2.0 * wl.m * wl.m * wl.d  # dBV = Z^T dW
    if kernel == "bwd_landmarks":
        # per head: 8 products per step of the reverse pass (m x m x m each;
        # the forward steps are saved by the recomputed forward), dZ, dQt_A,
        # dKt_A (m x m x d each)
        m3, steps = float(wl.m) ** 3, wl.iters
        per_head = 2 * m3 * 8 * steps + 6.0 * wl.m * wl.m * wl.d
        return wl.batch * wl.heads * per_head
    return 0.0


def pinv_flops(wl) -> float:
    return float(wl.batch * wl.heads) * (wl.iters * 8.0 * wl.m ** 3 + 2.0 * wl.m * wl.m * wl.d)


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        info = [x for x in threadpool_info() if x.get("user_api") == "blas"]
        if info:
            return int(max(x.get("num_threads", 1) for x in info))
    except Exception:
        pass
    return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


def measured_copy_gbs(torch, dev, stream) -> float:
    """Device copy bandwidth (GB/s, bytes read + written) of a plain 256 MiB
    fp32 copy, best of five timed launches: the practical ceiling the HBM
    fraction is also quoted against."""
    src = torch.ones(64 * 2 ** 20, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = float("inf")
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) / 1e3)
    del src, dst
    return 2 * 256 * 2 ** 20 / best / 1e9


def single_thread_oracle(wl, host0, lengths, budget_s: float):
    """Tokens/s of the oracle with its BLAS limited to one thread, on the
    first (batch, head) slice of the workload (the oracle's work is per
    slice), or None where threadpoolctl is missing."""
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:
        return None
    from oracle import nystrom_attention
    q, k, v = (host0[x][:1, :1] for x in ("Q", "K", "V"))
    w = None if host0["conv_w"] is None else host0["conv_w"][:1]
    ln = None if lengths is None else lengths[:1]
    rows = wl.n if ln is None else min(max(ln[0], 0), wl.n)
    reps = 0
    with threadpool_limits(limits=1, user_api="blas"):
        c0 = time.perf_counter()
        while True:
            nystrom_attention(q, k, v, wl.m, wl.iters, w, lengths=ln)
            reps += 1
            if time.perf_counter() - c0 >= budget_s:
                break
        dt = time.perf_counter() - c0
    # A token of the workload needs every head's work: one slice covers
    # `rows` tokens of one head, so whole-workload tokens/s divides by heads.
    return {"value": round(rows * reps / dt / wl.heads, 1), "unit": "tokens/s", "cores": 1,
            "sample": f"{reps} call(s) on one (batch, head) slice, n={wl.n}, {dt:.1f} s, "
                      f"scaled to whole tokens ({wl.heads} heads)"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="headline")
    ap.add_argument("--sets", type=int, default=0, help="input sets rotated in the timed loop (0: enough to exceed 512 MiB)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="wall time budget of the CPU-oracle leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--lengths", default=None,
                    help="tokens of each batch entry, comma-separated: a batch of right-padded sequences "
                         "(key-padding mask, nystrom_attn_fwd_masked); value then counts real tokens")
    ap.add_argument("--backward", action="store_true",
                    help="time nystrom_attn_bwd (gradients of Q, K, V and the filters) instead of the forward")
    ap.add_argument("--layer", action="store_true",
                    help="time nystrom_layer_fwd (QKV projection, heads, attention, output projection) on "
                         "X [batch][n][heads*d]")
    ap.add_argument("--error", action="store_true",
                    help="time nystrom_attn_error (per-head error of the method against exact attention, on device)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of known size (for HBM counter scaling)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the forward pass is independent per (batch, head), so a "
              "multi-GPU run would only split the heads; run with --gpus 1.", file=sys.stderr)
        return 2

    import torch  # noqa: E402  (imported before the library so it binds torch's HIP runtime)
    from efficient_transformer_attention_mean_amd import _lib
    from efficient_transformer_attention_mean_amd.workloads import WORKLOADS, bf16_bits, bf16_bits_to_f32, make_inputs

    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.backward:
        return backward_bench(args, wl, dev)
    if args.layer:
        return layer_bench(args, wl, dev)
    if args.error:
        return error_bench(args, wl, dev)
    lengths = None
    eff = [wl.n] * wl.batch
    if args.lengths:
        lengths = [int(x) for x in args.lengths.split(",")]
        if len(lengths) != wl.batch:
            print(f"--lengths needs {wl.batch} values for workload {wl.name}", file=sys.stderr)
            return 2
        eff = [min(max(x, 0), wl.n) for x in lengths]
    token_rows = sum(eff) * wl.heads
    # Read Q, K, V token rows once, write every row of O once, plus the filters.
    io_bytes = wl.compulsory_bytes() - 3 * (wl.batch * wl.n * wl.heads - token_rows) * wl.d * wl.elem_bytes
    sets = args.sets or max(2, int(np.ceil(512 * 2 ** 20 / io_bytes)) + 1)

    def to_dev(x):
        if wl.dtype == "bf16":
            return torch.from_numpy(bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev)

    host0 = None
    bufs = []
    for i in range(sets):
        inp = make_inputs(wl, seed=wl.seed + 1000 * i)
        if i == 0:
            host0 = inp
        Q, K, V = (to_dev(inp[k]) for k in ("Q", "K", "V"))
        W = None if inp["conv_w"] is None else torch.from_numpy(inp["conv_w"]).to(dev)
        bufs.append((Q, K, V, W, torch.empty_like(Q)))
    ws_bytes = _lib.nystrom_attn_workspace_bytes(wl.batch, wl.heads, wl.n, wl.d, wl.m)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    code = _lib.NYS_BF16 if wl.dtype == "bf16" else _lib.NYS_F32
    conv_k = wl.conv_k if wl.conv_k else 0
    lens_dev = None if lengths is None else torch.tensor(lengths, dtype=torch.int32, device=dev)

    def step(i):
        Q, K, V, W, O = bufs[i % sets]
        if lens_dev is None:
            rc = _lib.nystrom_attn_fwd(Q, K, V, W, wl.n, wl.d, wl.m, wl.heads, wl.iters, O, wl.batch, conv_k, code,
                                       ws, ws_bytes, stream)
        else:
            rc = _lib.nystrom_attn_fwd_masked(Q, K, V, W, wl.n, wl.d, wl.m, wl.heads, wl.iters, O, wl.batch, conv_k,
                                              code, lens_dev, ws, ws_bytes, stream)
        if rc != 0:
            raise RuntimeError(_lib.nystrom_strerror(rc))

    print(f"[bench] workload={wl.name} sets={sets} ({sets * io_bytes / 2**20:.0f} MiB) steps={args.steps} "
          f"warmup={args.warmup}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: exactly `steps` whole calls between two events on the
    # launch stream, synchronised on both sides.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_s = ev0.elapsed_time(ev1) / 1e3
    ms_per_step = 1e3 * gpu_s / args.steps
    tokens = sum(eff)
    value = tokens * args.steps / gpu_s

    # Per-call distribution: an event between consecutive calls.
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(args.steps):
        step(i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per_call_us = np.array([1e3 * evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])

    # Per-kernel durations: HIP events the library records around each launch
    # on the stream it launches on (the side-stream pseudoinverse included).
    _lib.nystrom_timing_enable(True)
    _lib.nystrom_timing_read()  # clear
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    kern = _lib.nystrom_timing_read()
    _lib.nystrom_timing_enable(False)

    per_kernel = {}
    for name, (ms, launches) in kern.items():
        per_kernel[name] = {"ms_per_step": ms / args.steps, "launches_per_step": launches / args.steps,
                            "avg_us_per_launch": 1e3 * ms / max(launches, 1)}
    dom = max(kern.items(), key=lambda kv: kv[1][0])[0] if kern else None
    roof = None
    if dom is not None:
        ms, launches = kern[dom]
        avg_s = ms / launches / 1e3
        ab = algorithmic_bytes(wl, dom, token_rows)
        if ab:
            from efficient_transformer_attention_mean_amd.profiling import read_traffic
            achieved = ab / avg_s / 1e9
            tr = read_traffic(os.path.join(ROOT, "profiles", f"hbm_traffic_{wl.name}.txt"), dom)
            roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None if tr is None else round(tr),
                    "kernel": dom, "algorithmic_bytes": ab, "avg_us": round(avg_s * 1e6, 3)}
        else:
            # The pseudoinverse's flops per call, spread over that call's
            # launches of the kernel (for m > 64 every launch but the first
            # runs one m x m product, so this is the average per launch).
            fl = pinv_flops(wl) / max(launches / args.steps, 1.0)
            achieved = fl / avg_s / 1e12
            roof = {"bound": "mfma", "achieved": round(achieved, 3), "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 6), "traffic": None,
                    "kernel": dom, "algorithmic_flops": fl, "avg_us": round(avg_s * 1e6, 3)}

    if args.copy_calibration:
        # A plain copy of known size for scaling the HBM byte counters:
        # reads and writes 256 MiB (fp32 elementwise add).
        src = torch.ones(64 * 2 ** 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.add(src, 1.0, out=dst)
        torch.cuda.synchronize()
    copy_gbs = measured_copy_gbs(torch, dev, stream)
    if roof is not None and roof["unit"] == "GB/s":
        roof["frac_of_measured_copy"] = round(roof["achieved"] / copy_gbs, 4)
    if roof is not None:
        # The committed kernel trace of this workload, when made from these
        # sources: its mean duration excludes the dispatch and completion
        # time that the events around each launch include.
        from efficient_transformer_attention_mean_amd.profiling import read_kernel_mean_us
        traced = read_kernel_mean_us(os.path.join(ROOT, "profiles", f"kernels_{wl.name}.txt"), roof["kernel"])
        if traced:
            roof["traced_avg_us"] = traced
            if roof["unit"] == "GB/s":
                roof["traced_frac"] = round(roof["algorithmic_bytes"] / (traced * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "heads": wl.heads, "n": wl.n, "d": wl.d, "m": wl.m,
                   "iters": wl.iters, "conv_k": wl.conv_k, "io": wl.dtype, "input_sets": sets,
                   **({} if lengths is None else {"lengths": lengths})},
        "hbm_roofline_frac_end_to_end": round(io_bytes / (ms_per_step / 1e3) / (HBM_PEAK_GBS * 1e9), 4),
        "compulsory_bytes": io_bytes,
        "measured_copy_gbs": round(copy_gbs, 1),
        "frac_of_measured_copy_end_to_end": round(io_bytes / (ms_per_step / 1e3) / (copy_gbs * 1e9), 4),
        "per_call_us": {"median": round(float(np.median(per_call_us)), 2),
                        "p10": round(float(np.percentile(per_call_us, 10)), 2),
                        "p90": round(float(np.percentile(per_call_us, 90)), 2)},
        "wall_s": round(wall, 4),
        "roofline": roof,
        "kernels": per_kernel,
    }

    if not args.no_cpu_baseline or not args.no_parity:
        # CPU oracle: whole calls on set 0, repeated within the time budget.
        from oracle import exact_attention, nystrom_attention
        threads = blas_threads()
        reps = 0
        c0 = time.perf_counter()
        O_ref = None
        while True:
            O_ref, inter = nystrom_attention(host0["Q"], host0["K"], host0["V"], wl.m, wl.iters, host0["conv_w"],
                                             with_intermediates=True, lengths=lengths)
            reps += 1
            if args.no_cpu_baseline or time.perf_counter() - c0 >= args.cpu_seconds:
                break
        cpu_s = time.perf_counter() - c0
        if not args.no_cpu_baseline:
            result["cpu_baseline"] = {
                "value": round(tokens * reps / cpu_s, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
                "sample": f"{reps} whole call(s) of the workload (batch {wl.batch} x {wl.heads} heads, n={wl.n}"
                          f"{'' if lengths is None else ', lengths ' + args.lengths}), "
                          f"fp64 NumPy, {cpu_s:.1f} s, host has {os.cpu_count()} logical CPUs"}
            # The same oracle with its BLAS held to one thread, on one
            # (batch, head) slice of set 0 repeated within a third of the budget.
            one = single_thread_oracle(wl, host0, lengths, args.cpu_seconds / 3)
            if one is not None:
                result["cpu_baseline"]["single_thread"] = one
        if not args.no_parity:
            Q, K, V, W, O = bufs[0]
            step(0)  # recompute set 0 into its own output
            torch.cuda.synchronize()
            if wl.dtype == "bf16":
                out = bf16_bits_to_f32(O.view(torch.int16).cpu().numpy().view(np.uint16))
            else:
                out = O.float().cpu().numpy()
            err = float(np.linalg.norm(out - O_ref) / np.linalg.norm(O_ref))
            # Context: distance of the method from exact softmax attention on
            # sampled query rows (attention part only, no skip).
            rng = np.random.default_rng(7)
            rows = np.sort(rng.choice(min(eff), size=min(256, min(eff)), replace=False))
            ex = np.stack([np.stack([exact_attention(host0["Q"][b, h][rows], host0["K"][b, h, :eff[b]],
                                                     host0["V"][b, h, :eff[b]])
                                     for h in range(wl.heads)]) for b in range(wl.batch)])
            att = inter["O_att"][:, :, rows]
            result["parity_rel_l2_vs_oracle"] = err
            result["nystrom_vs_exact_attention_rel_l2_sampled_rows"] = float(
                np.linalg.norm(att - ex) / np.linalg.norm(ex))
    result["pages_context"] = PAGES_CONTEXT
    print(json.dumps(result), flush=True)
    return 0


def error_bench(args, wl, dev) -> int:
    """One step = one nystrom_attn_error call: the method's attention output
    and exact softmax attention for every head, and their relative distance."""
    import torch
    from efficient_transformer_attention_mean_amd import _lib
    from efficient_transformer_attention_mean_amd.workloads import bf16_bits, make_inputs

    def to_dev(x):
        if wl.dtype == "bf16":
            return torch.from_numpy(bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev)

    inp = make_inputs(wl)
    Q, K, V = (to_dev(inp[k]) for k in ("Q", "K", "V"))
    code = _lib.NYS_BF16 if wl.dtype == "bf16" else _lib.NYS_F32
    ws_bytes = _lib.nystrom_attn_error_workspace_bytes(wl.batch, wl.heads, wl.n, wl.d, wl.m, code)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    err = torch.empty(wl.batch, wl.heads, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        rc = _lib.nystrom_attn_error(Q, K, V, wl.n, wl.d, wl.m, wl.heads, wl.iters, err, wl.batch, code, ws,
                                     ws_bytes, stream)
        if rc != 0:
            raise RuntimeError(_lib.nystrom_strerror(rc))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    _lib.nystrom_timing_enable(True)
    _lib.nystrom_timing_read()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kern = _lib.nystrom_timing_read()
    _lib.nystrom_timing_enable(False)
    per_kernel = {name: {"avg_us_per_launch": 1e3 * ms / max(n, 1)} for name, (ms, n) in kern.items()}
    roof = None
    if "exact_error" in kern:
        ms, launches = kern["exact_error"]
        avg_s = ms / launches / 1e3
        fl = 4.0 * wl.batch * wl.heads * wl.n * wl.n * wl.d  # Q K^T and P V
        peak = MFMA_BF16_PEAK_TFLOPS
        achieved = fl / avg_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": None, "kernel": "exact_error",
                "algorithmic_flops": fl, "avg_us": round(avg_s * 1e6, 3)}
    e = err.cpu().numpy()
    result = {
        "metric": "Nyström attention approximation-error diagnostic, heads/s (method vs exact attention, on device)",
        "value": round(wl.batch * wl.heads / (ms_per_step / 1e3), 1), "unit": "heads/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "pass": "error", "batch": wl.batch, "heads": wl.heads, "n": wl.n, "d": wl.d,
                   "m": wl.m, "iters": wl.iters, "io": wl.dtype},
        "roofline": roof, "kernels": per_kernel,
        "rel_error_per_head": {"mean": float(e.mean()), "min": float(e.min()), "max": float(e.max())},
    }
    if not args.no_parity:
        from oracle import approximation_error
        b0 = min(wl.batch, 1)
        ref = approximation_error(inp["Q"][:b0], inp["K"][:b0], inp["V"][:b0], wl.m, wl.iters)
        result["parity_max_abs_vs_oracle_first_batch_entry"] = float(np.abs(e[:b0] - ref).max())
    print(json.dumps(result), flush=True)
    return 0


def layer_bench(args, wl, dev) -> int:
    """One step = one nystrom_layer_fwd call: X [batch][n][E] -> Y, with
    random projections of the layer's shape (E = heads * d)."""
    import torch
    from efficient_transformer_attention_mean_amd import _lib
    from efficient_transformer_attention_mean_amd.workloads import bf16_bits, bf16_bits_to_f32, round_to_bf16

    E, rows = wl.heads * wl.d, wl.batch * wl.n
    e = wl.elem_bytes
    io_bytes = 2 * rows * E * e + 4 * E * E * e + (4 * wl.heads * wl.d * wl.conv_k if wl.conv_k else 0)
    sets = args.sets or max(2, int(np.ceil(512 * 2 ** 20 / io_bytes)) + 1)

    def draw(seed):
        rng = np.random.default_rng(seed)
        X = rng.standard_normal((wl.batch, wl.n, E)).astype(np.float32)
        Wqkv = (rng.standard_normal((E, 3 * E)) / np.sqrt(E)).astype(np.float32)
        Wo = (rng.standard_normal((E, E)) / np.sqrt(E)).astype(np.float32)
        w = rng.normal(0, 0.02, (wl.heads, wl.d, wl.conv_k)).astype(np.float32) if wl.conv_k else None
        if wl.dtype == "bf16":
            X, Wqkv, Wo = round_to_bf16(X), round_to_bf16(Wqkv), round_to_bf16(Wo)
        return X, Wqkv, Wo, w

    def to_dev(x):
        if wl.dtype == "bf16":
            return torch.from_numpy(bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev)

    host0 = None
    bufs = []
    for i in range(sets):
        X, Wqkv, Wo, w = draw(wl.seed + 1000 * i)
        if i == 0:
            host0 = (X, Wqkv, Wo, w)
        Xd = to_dev(X)
        bufs.append((Xd, to_dev(Wqkv), to_dev(Wo), None if w is None else torch.from_numpy(w).to(dev),
                     torch.empty_like(Xd)))
    conv_k = wl.conv_k if wl.conv_k else 0
    code = _lib.NYS_BF16 if wl.dtype == "bf16" else _lib.NYS_F32
    ws_bytes = _lib.nystrom_layer_workspace_bytes(wl.batch, wl.heads, wl.n, wl.d, wl.m, code)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        Xd, Wd, Wod, wd, Y = bufs[i % sets]
        rc = _lib.nystrom_layer_fwd(Xd, Wd, Wod, wd, wl.n, wl.d, wl.m, wl.heads, wl.iters, Y, wl.batch, conv_k, code,
                                    ws, ws_bytes, stream)
        if rc != 0:
            raise RuntimeError(_lib.nystrom_strerror(rc))

    print(f"[bench] layer workload={wl.name} sets={sets} steps={args.steps} warmup={args.warmup}", file=sys.stderr,
          flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_s = ev0.elapsed_time(ev1) / 1e3
    ms_per_step = 1e3 * gpu_s / args.steps
    tokens = rows
    value = tokens * args.steps / gpu_s

    _lib.nystrom_timing_enable(True)
    _lib.nystrom_timing_read()
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    kern = _lib.nystrom_timing_read()
    _lib.nystrom_timing_enable(False)
    per_kernel = {name: {"ms_per_step": ms / args.steps, "launches_per_step": n / args.steps,
                         "avg_us_per_launch": 1e3 * ms / max(n, 1)} for name, (ms, n) in kern.items()}
    dom = max(kern.items(), key=lambda kv: kv[1][0])[0] if kern else None
    roof = None
    if dom is not None:
        ms, launches = kern[dom]
        avg_s = ms / launches / 1e3
        gemm_flops = {"qkv_gemm": 2.0 * rows * E * 3 * E, "out_gemm": 2.0 * rows * E * E}
        if dom in gemm_flops:
            peak = MFMA_BF16_PEAK_TFLOPS if wl.dtype == "bf16" else FP32_VECTOR_PEAK_TFLOPS
            achieved = gemm_flops[dom] / avg_s / 1e12
            roof = {"bound": "mfma" if wl.dtype == "bf16" else "alu", "achieved": round(achieved, 2), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None, "kernel": dom,
                    "algorithmic_flops": gemm_flops[dom], "avg_us": round(avg_s * 1e6, 3)}
        else:
            ab = {"split_heads": 6 * rows * E * e}.get(dom) or algorithmic_bytes(wl, dom)
            if ab:
                achieved = ab / avg_s / 1e9
                roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "kernel": dom,
                        "algorithmic_bytes": ab, "avg_us": round(avg_s * 1e6, 3)}
    result = {
        "metric": "Nyström attention layer fwd tokens/s (QKV projection, heads, attention + skip, output projection)",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "pass": "layer", "batch": wl.batch, "heads": wl.heads, "n": wl.n, "d": wl.d,
                   "embed": E, "m": wl.m, "iters": wl.iters, "conv_k": wl.conv_k, "io": wl.dtype,
                   "input_sets": sets},
        "hbm_roofline_frac_end_to_end": round(io_bytes / (ms_per_step / 1e3) / (HBM_PEAK_GBS * 1e9), 4),
        "compulsory_bytes": io_bytes, "wall_s": round(wall, 4), "roofline": roof, "kernels": per_kernel,
    }
    if not args.no_cpu_baseline or not args.no_parity:
        from oracle import nystrom_layer
        threads = blas_threads()
        reps, c0 = 0, time.perf_counter()
        while True:
            ref = nystrom_layer(host0[0], host0[1], host0[2], wl.heads, wl.m, wl.iters, host0[3])
            reps += 1
            if args.no_cpu_baseline or time.perf_counter() - c0 >= args.cpu_seconds:
                break
        cpu_s = time.perf_counter() - c0
        if not args.no_cpu_baseline:
            result["cpu_baseline"] = {
                "value": round(tokens * reps / cpu_s, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
                "sample": f"{reps} whole layer call(s) (batch {wl.batch}, n={wl.n}, E={E}), fp64 NumPy, "
                          f"{cpu_s:.1f} s, host has {os.cpu_count()} logical CPUs"}
        if not args.no_parity:
            step(0)
            torch.cuda.synchronize()
            Y = bufs[0][4]
            got = (bf16_bits_to_f32(Y.view(torch.int16).cpu().numpy().view(np.uint16)) if wl.dtype == "bf16"
                   else Y.float().cpu().numpy())
            result["parity_rel_l2_vs_oracle"] = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    print(json.dumps(result), flush=True)
    return 0


def backward_bench(args, wl, dev) -> int:
    """One step = one nystrom_attn_bwd call over the workload (the landmark
    side of the forward is recomputed inside it)."""
    import torch
    from efficient_transformer_attention_mean_amd import _lib
    from efficient_transformer_attention_mean_amd.workloads import bf16_bits, bf16_bits_to_f32, make_inputs, \
        round_to_bf16

    e = wl.elem_bytes
    io_bytes = 7 * wl.batch * wl.heads * wl.n * wl.d * e + (8 * wl.heads * wl.d * wl.conv_k if wl.conv_k else 0)
    sets = args.sets or max(2, int(np.ceil(512 * 2 ** 20 / io_bytes)) + 1)

    def to_dev(x):
        if wl.dtype == "bf16":
            return torch.from_numpy(bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev)

    def upstream(seed):
        g = np.random.default_rng(seed).standard_normal((wl.batch, wl.heads, wl.n, wl.d)).astype(np.float32)
        return round_to_bf16(g) if wl.dtype == "bf16" else g

    host0, g0 = None, None
    bufs = []
    for i in range(sets):
        inp = make_inputs(wl, seed=wl.seed + 1000 * i)
        g = upstream(wl.seed + 1000 * i + 1)
        if i == 0:
            host0, g0 = inp, g
        Q, K, V, G = (to_dev(x) for x in (inp["Q"], inp["K"], inp["V"], g))
        W = None if inp["conv_w"] is None else torch.from_numpy(inp["conv_w"]).to(dev)
        dW = None if W is None else torch.empty_like(W)
        bufs.append((Q, K, V, G, W, torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V), dW))
    conv_k = wl.conv_k if wl.conv_k else 0
    ws_bytes = _lib.nystrom_attn_bwd_workspace_bytes(wl.batch, wl.heads, wl.n, wl.d, wl.m, wl.iters, conv_k)
    if ws_bytes == 0:
        print(f"workload {wl.name} is outside the backward kernels (m <= 64, conv_k <= 33)", file=sys.stderr)
        return 2
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    code = _lib.NYS_BF16 if wl.dtype == "bf16" else _lib.NYS_F32

    def step(i):
        Q, K, V, G, W, dQ, dK, dV, dW = bufs[i % sets]
        rc = _lib.nystrom_attn_bwd(Q, K, V, W, G, wl.n, wl.d, wl.m, wl.heads, wl.iters, dQ, dK, dV, dW, wl.batch,
                                   conv_k, code, ws, ws_bytes, stream)
        if rc != 0:
            raise RuntimeError(_lib.nystrom_strerror(rc))

    print(f"[bench] backward workload={wl.name} sets={sets} steps={args.steps} warmup={args.warmup}",
          file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_s = ev0.elapsed_time(ev1) / 1e3
    ms_per_step = 1e3 * gpu_s / args.steps
    tokens = wl.batch * wl.n
    value = tokens * args.steps / gpu_s

    _lib.nystrom_timing_enable(True)
    _lib.nystrom_timing_read()
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    kern = _lib.nystrom_timing_read()
    _lib.nystrom_timing_enable(False)
    per_kernel = {name: {"ms_per_step": ms / args.steps, "launches_per_step": n / args.steps,
                         "avg_us_per_launch": 1e3 * ms / max(n, 1)} for name, (ms, n) in kern.items()}
    dom = max(kern.items(), key=lambda kv: kv[1][0])[0] if kern else None
    roof = None
    if dom is not None:
        ms, launches = kern[dom]
        avg_s = ms / launches / 1e3
        fl = backward_flops(wl, dom)
        if fl:
            # bf16 I/O at d = 32, 64 runs the products on the matrix cores
            # (bf16 peak); otherwise they are fp32 vector work.  The
            # landmark-side block always uses the matrix cores; the skip's
            # filter gradient and the prep kernel are vector work.
            mm = ((wl.dtype == "bf16" and wl.d in (32, 64)) or dom == "bwd_landmarks") and \
                dom not in ("bwd_skip_grad", "bwd_land_prep")
            peak = MFMA_BF16_PEAK_TFLOPS if mm else FP32_VECTOR_PEAK_TFLOPS
            achieved = fl / avg_s / 1e12
            roof = {"bound": "mfma" if mm else "alu", "achieved": round(achieved, 2), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(achieved / peak, 5), "traffic": None,
                    "kernel": dom, "algorithmic_flops": fl, "avg_us": round(avg_s * 1e6, 3)}
        else:
            roof = {"bound": "latency", "achieved": None, "peak": None, "unit": None, "frac": None,
                    "traffic": None, "kernel": dom, "avg_us": round(avg_s * 1e6, 3)}

    result = {
        "metric": "Nyström attention bwd tokens/s (gradients of Q, K, V and the filters)",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "pass": "backward", "batch": wl.batch, "heads": wl.heads, "n": wl.n,
                   "d": wl.d, "m": wl.m, "iters": wl.iters, "conv_k": wl.conv_k, "io": wl.dtype,
                   "input_sets": sets},
        "hbm_roofline_frac_end_to_end": round(io_bytes / (ms_per_step / 1e3) / (HBM_PEAK_GBS * 1e9), 4),
        "compulsory_bytes": io_bytes, "wall_s": round(wall, 4), "roofline": roof, "kernels": per_kernel,
    }

    # The training pair: nystrom_attn_fwd_save once per input set (each set
    # keeps its own saved state), then nystrom_attn_bwd_saved timed over the
    # same rotation: the backward without recomputing the forward's landmark side.
    saved = [torch.empty(ws_bytes, dtype=torch.uint8, device=dev) for _ in range(sets)]
    for i in range(sets):
        Q, K, V, G, W, dQ, dK, dV, dW = bufs[i]
        rc = _lib.nystrom_attn_fwd_save(Q, K, V, W, wl.n, wl.d, wl.m, wl.heads, wl.iters, torch.empty_like(Q),
                                        wl.batch, conv_k, code, saved[i], ws_bytes, stream)
        if rc != 0:
            raise RuntimeError(_lib.nystrom_strerror(rc))

    def step_saved(i):
        Q, K, V, G, W, dQ, dK, dV, dW = bufs[i % sets]
        rc = _lib.nystrom_attn_bwd_saved(Q, K, V, W, G, wl.n, wl.d, wl.m, wl.heads, wl.iters, dQ, dK, dV, dW,
                                         wl.batch, conv_k, code, saved[i % sets], ws_bytes, stream)
        if rc != 0:
            raise RuntimeError(_lib.nystrom_strerror(rc))

    for i in range(args.warmup):
        step_saved(i)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.steps):
        step_saved(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    saved_s = ev0.elapsed_time(ev1) / 1e3
    result["backward_from_saved_forward"] = {
        "ms_per_step": round(1e3 * saved_s / args.steps, 5),
        "value": round(tokens * args.steps / saved_s, 1), "unit": "tokens/s",
        "note": "nystrom_attn_bwd_saved after nystrom_attn_fwd_save: the forward's landmark-side state is reused, "
                "not recomputed",
    }

    # A whole training step's attention work, both ways: the plain forward
    # then the backward that recomputes the landmark side, against the saving
    # forward (its pseudoinverse also stores every step) then the backward
    # from that state.
    outs = [torch.empty_like(b[0]) for b in bufs]
    fws_bytes = _lib.nystrom_attn_workspace_bytes(wl.batch, wl.heads, wl.n, wl.d, wl.m)
    fws = torch.empty(fws_bytes, dtype=torch.uint8, device=dev)

    def step_plain_pair(i):
        Q, K, V, G, W, dQ, dK, dV, dW = bufs[i % sets]
        rc = _lib.nystrom_attn_fwd(Q, K, V, W, wl.n, wl.d, wl.m, wl.heads, wl.iters, outs[i % sets], wl.batch,
                                   conv_k, code, fws, fws_bytes, stream)
        if rc != 0:
            raise RuntimeError(_lib.nystrom_strerror(rc))
        step(i)

    def step_saved_pair(i):
        Q, K, V, G, W, dQ, dK, dV, dW = bufs[i % sets]
        rc = _lib.nystrom_attn_fwd_save(Q, K, V, W, wl.n, wl.d, wl.m, wl.heads, wl.iters, outs[i % sets],
                                        wl.batch, conv_k, code, saved[i % sets], ws_bytes, stream)
        if rc != 0:
            raise RuntimeError(_lib.nystrom_strerror(rc))
        step_saved(i)

    def time_steps(fn):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(args.steps):
            fn(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / args.steps

    plain_ms = time_steps(step_plain_pair)
    saved_ms = time_steps(step_saved_pair)
    result["training_step"] = {
        "fwd_then_bwd_ms": round(plain_ms, 5),
        "fwd_save_then_bwd_saved_ms": round(saved_ms, 5),
        "note": "one forward and one backward per step over the same input rotation: nystrom_attn_fwd + "
                "nystrom_attn_bwd (landmark side recomputed) against nystrom_attn_fwd_save + "
                "nystrom_attn_bwd_saved (landmark side and pseudoinverse steps kept)",
    }
    del saved
    if not args.no_cpu_baseline or not args.no_parity:
        from oracle import nystrom_attention_backward
        threads = blas_threads()
        reps, c0 = 0, time.perf_counter()
        while True:
            ref = nystrom_attention_backward(host0["Q"], host0["K"], host0["V"], wl.m, wl.iters, g0,
                                             host0["conv_w"])
            reps += 1
            if args.no_cpu_baseline or time.perf_counter() - c0 >= args.cpu_seconds:
                break
        cpu_s = time.perf_counter() - c0
        if not args.no_cpu_baseline:
            result["cpu_baseline"] = {
                "value": round(tokens * reps / cpu_s, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
                "sample": f"{reps} whole backward call(s) of the workload (batch {wl.batch} x {wl.heads} heads, "
                          f"n={wl.n}), fp64 NumPy, {cpu_s:.1f} s, host has {os.cpu_count()} logical CPUs"}
        if not args.no_parity:
            step(0)
            torch.cuda.synchronize()
            Q, K, V, G, W, dQ, dK, dV, dW = bufs[0]

            def host(t):
                if t.dtype == torch.bfloat16:
                    return bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16))
                return t.float().cpu().numpy()
            got = (host(dQ), host(dK), host(dV), None if dW is None else dW.cpu().numpy())
            result["parity_rel_l2_vs_oracle"] = {
                nm: float(np.linalg.norm(g - r) / np.linalg.norm(r))
                for nm, g, r in zip(("dQ", "dK", "dV", "dconv_w"), got, ref) if r is not None}
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
