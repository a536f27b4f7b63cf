"""Benchmark of the KDA layer's hot path on one MI355X.

One step = one prompt pass of the whole layer over a T=4096, H=16, d=128 bf16
sequence (kda_prep -> kda_prefill_varlen -> gated_rmsnorm_out), carrying the
recurrent state and conv state from step to step.  Throughput `value` is
prompt tokens per second.  Batched decode (B=256 sequences, H=32, d=128, one
row per sequence per step, 512 MiB of fp32 state) is timed in the same run and
reported under "decode".  Inputs are synthetic (seeded), resident in HBM
before timing starts.  Prints one JSON line.

Timing: HIP events on torch's current stream (every library call is enqueued
on it), W warmup steps, then exactly K steps bracketed by synchronize().  Each
entry point is bracketed by its own events inside the timed region; the
roofline object uses those live durations and the algorithmic bytes / FLOPs
per launch documented in the design doc.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix cores
FP32_PEAK_TFLOPS = 157.3    # fp32 matrix / vector


def prefill_algorithmic(T, H, dk, dv, chunk=64, y_bytes=4, in_bytes=2):
    """Algorithmic work of one prompt pass (per token-head counts times T*H).

    FLOPs (multiply-add = 2): A (C-1)/2*dk, P/W/U~/PU (C+1)/2*(2dk+2dv), the three
    state products 3*dk*dv, triangular solve ~C^2/6 -- all per token-head.
    Bytes: raw q,k,g (dk each), v,z (dv each) in the input dtype, beta logit,
    y out; state and conv state read + written once per sequence."""
    C = chunk
    macs = (C - 1) / 2 * dk + (C + 1) / 2 * (2 * dk + 2 * dv) + 3 * dk * dv + C * C / 6
    flops = 2 * macs * T * H
    bytes_ = T * H * (in_bytes * (3 * dk + 2 * dv) + in_bytes + y_bytes * dv)
    bytes_ += 2 * (H * dk * dv * 4) + 2 * 3 * H * (2 * dk + dv) * in_bytes
    return flops, bytes_


def decode_algorithmic(B, H, dk, dv, in_bytes=2):
    """One decode row per sequence: fp32 state read + write, conv state read + write,
    raw rows in, o out (fp32)."""
    state = 2 * B * H * dk * dv * 4
    conv = 2 * B * 3 * H * (2 * dk + dv) * in_bytes
    rows = B * H * (in_bytes * (3 * dk + dv) + in_bytes)
    out = B * H * dv * 4
    flops = 2 * B * H * (4 * dk * dv)  # decay, two projections, rank-1 update (+ readout folded)
    return flops, state + conv + rows + out


def cpu_baseline(w):
    """The fp64 oracle, as it stands, on the host cores: the same prompt pass
    (conv preamble, token-serial recurrence, gated RMSNorm) over the whole workload."""
    from oracle import oracle as O
    threads = O.default_threads()
    t0 = time.perf_counter()
    O.layer(w.f64("q"), w.f64("k"), w.f64("v"), w.f64("conv_w"), w.f64("conv_state0"), w.f64("g"), w.f64("beta"),
            w.f64("z"), w.f64("norm_w"), w.f64("state0"), w.cu_seqlens.numpy(), gate_mode=w.gate_mode,
            lower_bound=w.lower_bound, threads=threads)
    dt = time.perf_counter() - t0
    return {"value": w.T / dt, "unit": "tokens/s", "cores": min(threads, w.N * w.H), "kind": "oracle",
            "sample": f"one full prompt pass of the benchmark workload (T={w.T}, H={w.H}), fp64 token-serial, "
                      f"threads over (sequence, head) units; {dt:.2f} s wall, {threads} host threads available"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--unfused", action="store_true", help="run kda_prep separately instead of inside the prompt pass")
    ap.add_argument("--precision", choices=("fp16", "bf16x3", "fp32"), default="bf16x3",
                    help="arithmetic of the prompt path's matrix products (see kda_precision)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import kimi_delta_attention_prep_amd as K
    from kimi_delta_attention_prep_amd import inputs as I

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    K.load_library()
    dev = "cuda"
    stream = torch.cuda.current_stream()

    # ---------------- prompt workload ----------------
    w = I.prefill()
    T, H, dk, dv = w.T, w.H, w.dk, w.dv
    prec = {"fp16": K.PREC_FP16, "bf16x3": K.PREC_BF16X3, "fp32": K.PREC_FP32}[args.precision]
    d = K.Dims(H, dk, dv, w.dtype, precision=prec)
    wd = w.to(dev)
    f = lambda *s: torch.empty(*s, device=dev, dtype=torch.float32)
    qh, kh, vv, gg, bb = f(T, H, dk), f(T, H, dk), f(T, H, dv), f(T, H, dk), f(T, H)
    state = wd.state0.clone()
    cs = wd.conv_state0.clone()
    o = f(T, H, dv)
    y = torch.empty(T, H, dv, device=dev, dtype=torch.bfloat16)
    ws = torch.empty(K.kda_prefill_workspace_bytes(d, w.N, T), dtype=torch.uint8, device=dev)
    raw = dict(q_raw=wd.q, k_raw=wd.k, v_raw=wd.v, g_raw=wd.g, beta_logit=wd.beta, conv_weight=wd.conv_w,
               conv_state_in=cs, conv_state_out=cs, gate_mode=w.gate_mode, lower_bound=w.lower_bound)
    if args.unfused:
        names = ("kda_prep", "kda_prefill_varlen", "gated_rmsnorm_out")
    else:
        names = ("kda_prefill_varlen", "gated_rmsnorm_out")

    def step(ev=None):
        i = 0
        if ev is not None:
            ev[i].record(stream)
        if args.unfused:
            K.kda_prep(d, wd.cu_seqlens, wd.q, wd.k, wd.v, wd.conv_w, cs, cs, wd.g, wd.beta, w.gate_mode,
                       w.lower_bound, qh, kh, vv, gg, bb)
            i += 1
            if ev is not None:
                ev[i].record(stream)
            K.kda_prefill_varlen(d, wd.cu_seqlens, qh, kh, vv, gg, bb, state, o, ws)
        else:
            K.kda_prefill_varlen(d, wd.cu_seqlens, None, None, None, None, None, state, o, ws, raw=raw)
        i += 1
        if ev is not None:
            ev[i].record(stream)
        K.gated_rmsnorm_out(o, wd.z, wd.norm_w, 1e-6, y)
        i += 1
        if ev is not None:
            ev[i].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for s in range(args.steps):
        step(evs[s])
    t_end.record(stream)
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_end) / args.steps
    per_entry = {n: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / args.steps for i, n in enumerate(names)}
    tokens_per_s = T / (ms * 1e-3)

    flops, bytes_ = prefill_algorithmic(T, H, dk, dv, y_bytes=2)
    dom = max(per_entry, key=per_entry.get)
    dom_ms = per_entry[dom]
    # prefill entry point: matrix-core work dominates its kernels' arithmetic; the
    # roofline object prices the whole pass's algorithmic FLOPs against it
    if dom == "kda_prefill_varlen":
        roof = {"kernel": "kda_prefill_varlen (chunk_intra + chunk_scan)", "bound": "hbm",
                "achieved": bytes_ / (dom_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"kernel": dom, "bound": "hbm", "achieved": bytes_ / (dom_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    out = {
        "metric": "KDA tokens/s: prefill (T=4096,H=16) and decode (B=256); % MFMA/HBM peak",
        "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill T=4096 H=16 d_k=d_v=128 bf16 rows, fp32 state, safe gate lb=-5, chunk 64",
                   "matrix_products": args.precision, "preamble": "separate" if args.unfused else "fused",
                   "global_batch": 1, "seq_len": T, "parallelism": "none"},
        "roofline": roof,
        "entry_points_ms": per_entry,
        "whole_pass": {"algorithmic_GB": bytes_ / 1e9, "algorithmic_GFLOP": flops / 1e9,
                       "GB_per_s": bytes_ / (ms * 1e-3) / 1e9, "hbm_frac": bytes_ / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                       "TFLOP_per_s": flops / (ms * 1e-3) / 1e12,
                       "bf16_mfma_frac": flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS},
    }

    # ---------------- decode workload ----------------
    if not args.no_decode:
        del qh, kh, vv, gg, bb, o, y, ws
        wdec = I.decode(steps=args.decode_steps)
        B, Hd = wdec.N, wdec.H
        dd = K.Dims(Hd, wdec.dk, wdec.dv, wdec.dtype)
        rows = {n: I.step_rows(wdec, n, args.decode_steps).to(dev) for n in ("q", "k", "v", "g", "beta")}
        st = wdec.state0.to(dev)
        cst = wdec.conv_state0.to(dev)
        cw = wdec.conv_w.to(dev)
        od = torch.empty(B, Hd, wdec.dv, device=dev)

        def dstep(s):
            K.kda_decode(dd, st, cst, cw, rows["q"][s], rows["k"][s], rows["v"][s], rows["g"][s], rows["beta"][s],
                         wdec.gate_mode, wdec.lower_bound, od)

        for s in range(min(args.warmup, args.decode_steps)):
            dstep(s)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s in range(args.decode_steps):
            dstep(s)
        e1.record(stream)
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / args.decode_steps
        dflops, dbytes = decode_algorithmic(B, Hd, wdec.dk, wdec.dv)
        out["decode"] = {"workload": "decode B=256 H=32 d=128 bf16 rows, fp32 state (512 MiB), safe gate lb=-5",
                         "value": B / (dms * 1e-3), "unit": "tokens/s", "ms_per_step": dms,
                         "roofline": {"kernel": "kda_rows_kernel (kda_decode)", "bound": "hbm",
                                      "achieved": dbytes / (dms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": dbytes / (dms * 1e-3) / 1e9 / HBM_PEAK_GBS, "traffic": None},
                         "algorithmic_bytes_per_step": dbytes}

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
