"""Benchmark of the KDA layer's hot path on one MI355X.

One step = one prompt pass of the whole layer over a T=4096, H=16, d=128 bf16
sequence: one kda_prefill_varlen call with the preamble fused (raw rows in)
and the gated output norm as its epilogue (bf16 y), carrying the recurrent
state and conv state from step to step.  `value` is prompt tokens per second.  Batched decode (B=256
sequences, H=32, d=128, one row per sequence per step, 512 MiB of fp32 state)
is timed in the same run and reported under "decode".  Inputs are synthetic
(seeded) and resident in HBM before timing starts.  Prints one JSON line.

Timing: HIP events on torch's current stream (every library call is enqueued
on it): W warmup steps, then exactly K steps bracketed by synchronize(), with
one event before and one after; `value` and `ms_per_step` come from these.  A
second pass of K steps records events around every entry point and, through
the library's timing hook (kda_set_timing_events), around every kernel of the
prompt call; the roofline object uses the dominant kernel's live average
duration from that pass.  Its `traffic` comes from the
rocprofv3 counter summary committed under profiles/, and is null when the
kernel sources have changed since those counters were taken.  `rw_reference`
is the rate this GPU sustains for a read-then-write pass (torch's in-place
scale of 512 MiB, timed in the same run); the decode roofline and the whole
pass also give their fraction of it.

Modes besides the default run:
  --copy-calibration   also time a plain 1 GiB device copy (for counter runs:
                       the copy's FETCH_SIZE / WRITE_SIZE scale the kernels')
  --verify-only        only the verify-window line (for profiler runs of its kernel)
  --pmc-summary F W    turn two rocprofv3 --pmc runs (FETCH_SIZE, then
                       WRITE_SIZE; their counter_collection.csv files) of the
                       --workload's prompt pass into its committed traffic summary
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


def kernel_algorithmic(name, T, H, dk, dv, N=1, chunk=64, in_bytes=2, y_bytes=2):
    """Algorithmic work of one launch of a kernel of the prompt pass: the HBM bytes
    the pass cannot avoid that this kernel moves, and the FLOPs it must do.
      chunk_intra  raw q, k, g, v rows + beta logit in; A, P, W, U~ and the solve
      chunk_scan   o out + the state read and written; the three state products
      gated_rmsnorm  o and z in, y out"""
    C = chunk
    th = T * H
    if name == "chunk_intra":
        macs = (C - 1) / 2 * dk + (C + 1) / 2 * (2 * dk + dv) + C * C / 6
        return 2 * macs * th, th * (in_bytes * (3 * dk + dv) + in_bytes)
    if name == "chunk_scan":
        return 2 * 3 * dk * dv * th, th * dv * 4 + 2 * N * H * dk * dv * 4
    if name == "gated_rmsnorm":
        return 4 * dv * th, th * dv * (4 + in_bytes + y_bytes)
    return 0.0, 0.0


def pass_bytes_per_token_head(dk, dv, in_bytes=2, y_bytes=2):
    """Algorithmic HBM bytes of one prompt pass per token-head: the raw q, k, g (d_k each) and v, z (d_v each)
    rows and the beta logit in, y out (1538 B at d = 128 with bf16 rows and bf16 y)."""
    return in_bytes * (3 * dk + 2 * dv) + in_bytes + y_bytes * dv


def prompt_roofline(per_kernel, T, H, dk, dv, N, precision, workload=None):
    """Roofline entry of a prompt pass for its dominant kernel: the pass's algorithmic bytes (per token-head
    figure x T*H) over that kernel's average launch duration, against the HBM peak (the pass is HBM-bound by
    its arithmetic intensity).  The kernel's own share of the bytes and FLOPs is reported beside it.  The
    counter traffic is that of the committed summary of the same workload (name and shape), if any."""
    dom = max(per_kernel, key=per_kernel.get)
    dom_ms = per_kernel[dom]
    per_unit = pass_bytes_per_token_head(dk, dv)
    units = T * H
    achieved = per_unit * units / (dom_ms * 1e-3) / 1e9
    kf, kb = kernel_algorithmic(dom, T, H, dk, dv, N=N)
    return {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": committed_traffic(dom, precision, workload, (N, T, H, dk, dv)),
            "basis": "whole-pass algorithmic bytes per token-head x token-heads / dominant kernel launch",
            "bytes_per_token_head": per_unit, "token_heads": units, "ms_per_launch": dom_ms,
            "kernel_share": {"algorithmic_bytes": kb, "algorithmic_flops": kf,
                             "GB_per_s": kb / (dom_ms * 1e-3) / 1e9,
                             "hbm_frac": kb / (dom_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}}


def source_digest():
    """Digest of the sources the prompt and decode kernels are built from."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kimi_delta_attention_prep_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp", ".cpp")):
            h.update(f.encode())
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


# committed counter summaries per prompt workload (the prefill one also holds decode's kernel)
TRAFFIC_FILES = {"prefill": os.path.join(ROOT, "profiles", "traffic_prefill_T4096_H16_decode_B256.json"),
                 "varlen": os.path.join(ROOT, "profiles", "traffic_prefill_varlen_8seq_H32.json")}


def committed_traffic(kernel, precision, workload="prefill", shape=None):
    """HBM bytes per launch of `kernel` from the workload's committed counter summary, or
    None if there is none, it was taken on another shape (sequences, rows, heads, d_k, d_v)
    or at another precision policy, or the kernel sources changed since it was taken."""
    try:
        t = json.load(open(TRAFFIC_FILES[workload]))
    except (KeyError, OSError, ValueError):
        return None
    if t.get("source_sha256") != source_digest() or t.get("precision") != precision:
        return None
    if shape is not None and t.get("shape") != list(shape):
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k["hbm_bytes_per_launch"]


def pmc_summary(fetch_csv, write_csv, command, precision, workload, shape):
    """Per-kernel FETCH_SIZE / WRITE_SIZE (KiB per dispatch) from two rocprofv3
    counter runs, scaled by what the same counters read for the 1 GiB copy."""
    import csv
    from collections import defaultdict

    def per_kernel(path, counter):
        # average per dispatch of each kernel; for the copy, only the 1 GiB calibration copies (the
        # dispatches within half of the largest count: the workloads' own tensor copies can share
        # their grid size but move far fewer bytes)
        acc = defaultdict(list)
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        out = {}
        for k, v in acc.items():
            if "copyBuffer" in k:
                top = max(v)
                v = [x for x in v if x >= 0.5 * top]
            out[k] = sum(v) / len(v)
        return out

    f, w = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")

    def find(d, key):
        m = [k for k in d if key in k]
        return max(m, key=lambda k: d[k]) if m else None

    copy = find(f, "copyBuffer")
    copy_kib = COPY_BYTES / 1024
    ff = copy_kib / f[copy] if copy else 1.0
    fw = copy_kib / w[find(w, "copyBuffer")] if copy else 1.0
    keys = {"chunk_intra": "chunk_intra_kernel", "chunk_scan": "chunk_scan_kernel",
            "gated_rmsnorm": "gated_rmsnorm_kernel", "kda_rows (decode)": "kda_rows_kernel"}
    out = {"command": command, "source_sha256": source_digest(), "precision": precision,
           "workload": workload, "shape": list(shape),
           "copy_calibration": {"kernel": copy, "bytes": COPY_BYTES, "fetch_kib": f.get(copy), "write_kib":
                                w.get(find(w, "copyBuffer")), "fetch_scale": ff, "write_scale": fw},
           "kernels": {}}
    for name, key in keys.items():
        kf, kw = find(f, key), find(w, key)
        if kf is None or kw is None:
            continue
        rd, wr = f[kf] * ff * 1024, w[kw] * fw * 1024
        out["kernels"][name] = {"kernel": kf, "fetch_kib_raw": f[kf], "write_kib_raw": w[kw],
                                "read_bytes": rd, "write_bytes": wr, "hbm_bytes_per_launch": rd + wr}
    return out


COPY_BYTES = 1 << 30


def decode_algorithmic(B, H, dk, dv, in_bytes=2):
    """One decode row per sequence: fp32 state read + write, conv state read + write,
    raw rows in, o out (fp32)."""
    state = 2 * B * H * dk * dv * 4
    conv = 2 * B * 3 * H * (2 * dk + dv) * in_bytes
    rows = B * H * (in_bytes * (3 * dk + dv) + in_bytes)
    out = B * H * dv * 4
    flops = 2 * B * H * (4 * dk * dv)  # decay, two projections, rank-1 update (+ readout folded)
    return flops, state + conv + rows + out


def cpu_baseline(w, min_seconds=10.0, max_passes=50):
    """The fp64 oracle, as it stands, on the host cores: full prompt passes of the
    benchmark workload (conv preamble, token-serial recurrence, gated RMSNorm),
    repeated until about `min_seconds` of wall time; the rate is the average."""
    from oracle import oracle as O
    threads = O.default_threads()
    args = (w.f64("q"), w.f64("k"), w.f64("v"), w.f64("conv_w"), w.f64("conv_state0"), w.f64("g"), w.f64("beta"),
            w.f64("z"), w.f64("norm_w"), w.f64("state0"), w.cu_seqlens.numpy())
    passes, t0 = 0, time.perf_counter()
    while True:
        O.layer(*args, gate_mode=w.gate_mode, lower_bound=w.lower_bound, threads=threads)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or passes >= max_passes:
            break
    return {"value": passes * w.T / dt, "unit": "tokens/s", "cores": min(threads, w.N * w.H), "kind": "oracle",
            "sample": f"{passes} full prompt passes of the benchmark workload (T={w.T}, H={w.H}), fp64 token-serial, "
                      f"threads over the {w.N * w.H} (sequence, head) units; {dt:.1f} s wall, "
                      f"{threads} host threads available"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the clocks settle over the first few ms of sustained work: the intra-chunk kernel's first calls run
    # up to 20 % slower than later ones, so the default warmup covers that ramp
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--decode-steps", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the prompt pass and B=256 decode (for profiler runs: the extra lines launch the same "
                         "kernels on other shapes)")
    ap.add_argument("--unfused", action="store_true", help="run kda_prep separately instead of inside the prompt pass")
    ap.add_argument("--precision", choices=("fp16", "bf16x2", "bf16x3", "fp32"), default="fp16",
                    help="arithmetic of the prompt path's matrix products (see kda_precision)")
    ap.add_argument("--workload", choices=("prefill", "varlen"), default="prefill",
                    help="the timed prompt workload: T=4096 H=16 (the metric's), or the 8 packed sequences at H=32 "
                         "(for profiler runs of that workload's kernels)")
    ap.add_argument("--verify-only", action="store_true",
                    help="only the verify-window line (B=64, window <= 4, H=32), for profiler runs of its kernel")
    ap.add_argument("--copy-calibration", action="store_true", help="also run a plain 1 GiB device copy")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--pmc-command", default="", help="the counter command, stored in the summary")
    args = ap.parse_args()
    if args.pmc_summary:
        from kimi_delta_attention_prep_amd import inputs as I
        w = I.prefill() if args.workload == "prefill" else I.varlen()
        out = pmc_summary(*args.pmc_summary, args.pmc_command, args.precision, args.workload,
                          (w.N, w.T, w.H, w.dk, w.dv))
        with open(TRAFFIC_FILES[args.workload], "w") as fh:
            json.dump(out, fh, indent=1)
        print(json.dumps(out, indent=1))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: there is no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import kimi_delta_attention_prep_amd as K
    from kimi_delta_attention_prep_amd import inputs as I

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    K.load_library()
    dev = "cuda"
    stream = torch.cuda.current_stream()

    if args.verify_only:
        print(json.dumps({"verify_window": verify_windows(stream, args.steps, args.warmup)}))
        return

    if args.copy_calibration:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---------------- prompt workload ----------------
    w = I.prefill() if args.workload == "prefill" else I.varlen()
    T, H, dk, dv = w.T, w.H, w.dk, w.dv
    prec = PRECISIONS[args.precision](K)
    pp = time_prompt_pass(stream, w, prec, args.steps, args.warmup, unfused=args.unfused)
    ms = pp["ms_per_step"]
    tokens_per_s = T / (ms * 1e-3)
    flops, bytes_ = prefill_algorithmic(T, H, dk, dv, y_bytes=2)
    roof = prompt_roofline(pp["kernels_ms"], T, H, dk, dv, w.N, args.precision, args.workload)
    out = {
        "metric": "KDA tokens/s: prefill (T=4096,H=16) and decode (B=256); % MFMA/HBM peak",
        "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": DTYPE_NAMES[args.precision],
        "data": "synthetic",
        "config": {"workload": ("prefill T=4096 H=16 d_k=d_v=128 bf16 rows, fp32 state, safe gate lb=-5, chunk 64"
                                if args.workload == "prefill" else
                                f"varlen {w.N} packed sequences, {T} rows, H={H} d_k=d_v=128 bf16 rows, fp32 state, "
                                "softplus gate, chunk 64"),
                   "matrix_products": args.precision, "preamble": "separate" if args.unfused else "fused",
                   "output_norm": "epilogue",
                   "global_batch": w.N, "seq_len": T, "parallelism": "none"},
        "roofline": roof,
        "entry_points_ms": pp["entry_points_ms"],
        "kernels_ms": pp["kernels_ms"],
        "whole_pass": {"algorithmic_GB": bytes_ / 1e9, "algorithmic_GFLOP": flops / 1e9,
                       "GB_per_s": bytes_ / (ms * 1e-3) / 1e9, "hbm_frac": bytes_ / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                       "TFLOP_per_s": flops / (ms * 1e-3) / 1e12,
                       "bf16_mfma_frac": flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS},
    }

    # ---------------- decode workload ----------------
    if not args.no_decode:
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
                         "roofline": {"kernel": "kda_rows (decode)", "bound": "hbm",
                                      "achieved": dbytes / (dms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": dbytes / (dms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                      "traffic": committed_traffic("kda_rows (decode)", args.precision)},
                         "algorithmic_bytes_per_step": dbytes}

    # ---------------- the same pass under the other bf16-row policy; the varlen workload ----------------
    if not args.no_extras:
        other = "bf16x3" if args.precision != "bf16x3" else "fp16"
        out[f"prefill_{other}"] = prompt_line(stream, w, other, args.steps, args.warmup, K)
        if args.workload == "prefill":
            wv = I.varlen()
            out["prefill_varlen"] = prompt_line(stream, wv, args.precision, max(5, args.steps // 2),
                                                max(8, args.warmup // 2), K)
            del wv

    # ---------------- the scalar-decay layer on the same prompt workload ----------------
    if not args.no_extras:
        out["prefill_scalar_decay"] = scalar_decay_prefill(stream, w, prec, args.steps, args.warmup)
        if not args.unfused:
            out["prefill_two_call"] = two_call_prefill(stream, w, prec, args.steps, args.warmup)

    # ---------------- small-batch decode: eager calls against one graph replay ----------------
    if not args.no_decode and not args.no_extras:
        out["decode_small_batch"] = small_batch_decode(stream, args.decode_steps)
        out["verify_window"] = verify_windows(stream, args.steps, args.warmup)

    # ---------------- measured read-write reference ----------------
    # the HBM rate this GPU sustains for the decode's access pattern (every byte read
    # once, then written once): torch's in-place scale of a 512 MiB fp32 buffer, the
    # size of the decode state pool
    if not args.no_extras:
        ref = measured_rw_reference(stream)
        out["rw_reference"] = ref
        out["whole_pass"]["rw_reference_frac"] = out["whole_pass"]["GB_per_s"] / ref["GB_per_s"]
        if "decode" in out:
            out["decode"]["roofline"]["rw_reference_frac"] = out["decode"]["roofline"]["achieved"] / ref["GB_per_s"]

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


PRECISIONS = {"fp16": lambda K: K.PREC_FP16, "bf16x2": lambda K: K.PREC_BF16X2, "bf16x3": lambda K: K.PREC_BF16X3,
              "fp32": lambda K: K.PREC_FP32}
DTYPE_NAMES = {"fp16": "fp16", "bf16x2": "bf16", "bf16x3": "bf16", "fp32": "f32"}


def time_prompt_pass(stream, w, prec, steps, warmup, unfused=False):
    """Times prompt passes over workload w (bf16 rows): each pass is one kda_prefill_varlen call with the
    preamble fused and the norm epilogue to bf16 y (or kda_prep, then that call, when unfused), carrying state
    and conv state from pass to pass.  W warmup passes, then exactly K passes between two events (the
    throughput), then K more with events around every entry point and, through the library's timing hook,
    around every kernel of the prompt call (recording events between kernels adds gaps, so the throughput
    comes from the first K)."""
    import torch
    import kimi_delta_attention_prep_amd as K
    T, H, dk, dv = w.T, w.H, w.dk, w.dv
    d = K.Dims(H, dk, dv, w.dtype, precision=prec)
    wd = w.to("cuda")
    f = lambda *s: torch.empty(*s, device="cuda", dtype=torch.float32)
    pre = (f(T, H, dk), f(T, H, dk), f(T, H, dv), f(T, H, dk), f(T, H)) if unfused else None
    state = wd.state0.clone()
    cs = wd.conv_state0.clone()
    o = f(T, H, dv)
    y = torch.empty(T, H, dv, device="cuda", dtype=torch.bfloat16)
    ws = torch.empty(K.kda_prefill_workspace_bytes(d, w.N, T), dtype=torch.uint8, device="cuda")
    raw = dict(q_raw=wd.q, k_raw=wd.k, v_raw=wd.v, g_raw=wd.g, beta_logit=wd.beta, conv_weight=wd.conv_w,
               conv_state_in=cs, conv_state_out=cs, gate_mode=w.gate_mode, lower_bound=w.lower_bound)
    norm = dict(z=wd.z, weight=wd.norm_w, eps=1e-6, y=y)
    names = ("kda_prep", "kda_prefill_varlen") if unfused else ("kda_prefill_varlen",)

    def step(ev=None):
        i = 0
        if ev is not None:
            ev[i].record(stream)
        if unfused:
            K.kda_prep(d, wd.cu_seqlens, wd.q, wd.k, wd.v, wd.conv_w, cs, cs, wd.g, wd.beta, w.gate_mode,
                       w.lower_bound, *pre)
            i += 1
            if ev is not None:
                ev[i].record(stream)
            K.kda_prefill_varlen(d, wd.cu_seqlens, *pre, state, o, ws, norm=norm)
        else:
            K.kda_prefill_varlen(d, wd.cu_seqlens, None, None, None, None, None, state, o, ws, raw=raw, norm=norm)
        i += 1
        if ev is not None:
            ev[i].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    mk = lambda: torch.cuda.Event(enable_timing=True)
    t_start, t_end = mk(), mk()
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_end) / steps
    evs = [[mk() for _ in range(len(names) + 1)] for _ in range(steps)]
    kev = [[mk() for _ in range(2 * len(K.PREFILL_KERNELS))] for _ in range(steps)]
    for e in (x for row in kev for x in row):
        e.record(stream)  # creates the HIP events the hook records into
    torch.cuda.synchronize()
    for i in range(steps):
        K.kda_set_timing_events(kev[i])
        step(evs[i])
    torch.cuda.synchronize()
    K.kda_set_timing_events(None)
    per_entry = {n: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / steps for i, n in enumerate(names)}
    per_kernel = {n: sum(e[2 * i].elapsed_time(e[2 * i + 1]) for e in kev) / steps
                  for i, n in enumerate(K.PREFILL_KERNELS)}
    return {"ms_per_step": ms, "entry_points_ms": per_entry, "kernels_ms": per_kernel}


def prompt_line(stream, w, precision, steps, warmup, K):
    """One extra line: the fused prompt pass over workload w under `precision`, with its kernel times and
    its roofline entry."""
    T, H = w.T, w.H
    pp = time_prompt_pass(stream, w, PRECISIONS[precision](K), steps, warmup)
    lens = (w.cu_seqlens[1:] - w.cu_seqlens[:-1]).tolist()
    return {"workload": f"{w.name}: {w.N} sequence(s), {T} rows (lengths {lens}), H={H}, d={w.dk}, bf16 rows, "
                        f"{'softplus' if w.gate_mode == 0 else 'safe'} gate",
            "matrix_products": precision, "value": T / (pp["ms_per_step"] * 1e-3), "unit": "tokens/s",
            "ms_per_step": pp["ms_per_step"], "steps": steps, "kernels_ms": pp["kernels_ms"],
            "roofline": prompt_roofline(pp["kernels_ms"], T, H, w.dk, w.dv, w.N, precision, w.name)}


def scalar_decay_prefill(stream, w, prec, steps, warmup):
    """The prompt pass of the benchmark workload with one decay per head and row
    (raw g rows [T, H], the scalar-decay layer), same call as the timed step."""
    import torch
    import kimi_delta_attention_prep_amd as K
    T, H, dk, dv = w.T, w.H, w.dk, w.dv
    d = K.Dims(H, dk, dv, w.dtype, precision=prec, decay_per_head=True)
    wd = w.to("cuda")
    gh = wd.g[:, :, 0].contiguous()
    state, cs = wd.state0.clone(), wd.conv_state0.clone()
    o = torch.empty(T, H, dv, device="cuda")
    y = torch.empty(T, H, dv, device="cuda", dtype=torch.bfloat16)
    ws = torch.empty(K.kda_prefill_workspace_bytes(d, w.N, T), dtype=torch.uint8, device="cuda")
    raw = dict(q_raw=wd.q, k_raw=wd.k, v_raw=wd.v, g_raw=gh, beta_logit=wd.beta, conv_weight=wd.conv_w,
               conv_state_in=cs, conv_state_out=cs, gate_mode=w.gate_mode, lower_bound=w.lower_bound)
    norm = dict(z=wd.z, weight=wd.norm_w, eps=1e-6, y=y)
    step = lambda: K.kda_prefill_varlen(d, wd.cu_seqlens, None, None, None, None, None, state, o, ws, raw=raw,
                                        norm=norm)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"workload": f"prefill T={T} H={H} d={dk}, one decay per head and row (g rows [T, H])",
            "value": T / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms}


def two_call_prefill(stream, w, prec, steps, warmup):
    """The same prompt pass as two calls: kda_prep writes q_hat, k_hat, v, g and
    beta in fp32, then kda_prefill_varlen (with the norm epilogue) reads them.
    Reports the step and the preamble call on its own (HIP events)."""
    import torch
    import kimi_delta_attention_prep_amd as K
    T, H, dk, dv = w.T, w.H, w.dk, w.dv
    d = K.Dims(H, dk, dv, w.dtype, precision=prec)
    wd = w.to("cuda")
    f = lambda *s: torch.empty(*s, device="cuda", dtype=torch.float32)
    qh, kh, vv, gg, bb = f(T, H, dk), f(T, H, dk), f(T, H, dv), f(T, H, dk), f(T, H)
    state, cs = wd.state0.clone(), wd.conv_state0.clone()
    o = f(T, H, dv)
    y = torch.empty(T, H, dv, device="cuda", dtype=torch.bfloat16)
    ws = torch.empty(K.kda_prefill_workspace_bytes(d, w.N, T), dtype=torch.uint8, device="cuda")
    norm = dict(z=wd.z, weight=wd.norm_w, eps=1e-6, y=y)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]

    def step(i=None):
        if i is not None:
            ev[2 * i].record(stream)
        K.kda_prep(d, wd.cu_seqlens, wd.q, wd.k, wd.v, wd.conv_w, cs, cs, wd.g, wd.beta, w.gate_mode,
                   w.lower_bound, qh, kh, vv, gg, bb)
        if i is not None:
            ev[2 * i + 1].record(stream)
        K.kda_prefill_varlen(d, wd.cu_seqlens, qh, kh, vv, gg, bb, state, o, ws, norm=norm)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    prep_ms = sorted(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps))[steps // 2]
    prep_bytes = T * H * (w.q.element_size() * (3 * dk + dv + 1) + 4 * (3 * dk + dv + 1))
    return {"workload": f"prefill T={T} H={H} d={dk} as kda_prep + kda_prefill_varlen (fp32 preamble outputs "
                        "through HBM)", "value": T / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms,
            "kda_prep_ms": prep_ms, "kda_prep_GB_per_s": prep_bytes / (prep_ms * 1e-3) / 1e9}


def verify_windows(stream, steps, warmup, B=64, W=4, H=32, d=128):
    """Speculative verify: each step commits the previous window's accepted rows
    (seeded, within the rows each sequence ran) and runs a new window whose
    length per sequence is seeded in 1..W, in one kda_verify_window call."""
    import torch
    import kimi_delta_attention_prep_amd as K
    from kimi_delta_attention_prep_amd import inputs as I
    w = I.generate("verify", lengths=[W] * B, H=H, dk=d, dv=d, dtype=torch.bfloat16, gate_mode=I.GATE_SAFE,
                   state_std=0.02, conv_state_std=1.0, seed=5)
    dd = K.Dims(H, d, d, w.dtype)
    rows = {n: getattr(w, n).view(B, W, *getattr(w, n).shape[1:]).cuda() for n in ("q", "k", "v", "g", "beta")}
    st, cs, cw = w.state0.cuda(), w.conv_state0.cuda(), w.conv_w.cuda()
    gen = torch.Generator().manual_seed(6)
    lens = torch.randint(1, W + 1, (B,), generator=gen, dtype=torch.int32)
    keep = (torch.rand(B, generator=gen) * (lens.float() + 1)).floor().clamp(max=lens.float()).to(torch.int32)
    lens, keep = lens.cuda(), keep.cuda()
    logs = [K.VerifyLog.empty(dd, B, W), K.VerifyLog.empty(dd, B, W)]
    o = torch.empty(B, W, H, d, device="cuda")
    K.kda_verify_window(dd, st, cs, cw, None, None, logs[0], rows["q"], rows["k"], rows["v"], rows["g"],
                        rows["beta"], w.gate_mode, w.lower_bound, o, window_lens=lens)

    def step(i):
        K.kda_verify_window(dd, st, cs, cw, keep, logs[i % 2], logs[(i + 1) % 2], rows["q"], rows["k"], rows["v"],
                            rows["g"], rows["beta"], w.gate_mode, w.lower_bound, o, window_lens=lens)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        step(warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nrows = int(lens.sum())
    return {"workload": f"verify B={B} window<={W} H={H} d={d}: commit + new window per call, lengths 1..{W} seeded",
            "ms_per_call": ms, "draft_rows_per_call": nrows, "draft_rows_per_s": nrows / (ms * 1e-3),
            "state_GB_per_s": 2 * B * H * d * d * 4 / (ms * 1e-3) / 1e9}


def small_batch_decode(stream, steps, B=1, H=32, d=128):
    """Per-step time of B=1 decode issued call by call, and of the same steps
    captured once in a HIP graph and replayed (launch overhead is what a small
    batch pays)."""
    import torch
    import kimi_delta_attention_prep_amd as K
    from kimi_delta_attention_prep_amd import inputs as I
    w = I.decode(B=B, steps=steps, H=H, d=d, seed=3)
    dd = K.Dims(H, d, d, w.dtype)
    rows = {n: I.step_rows(w, n, steps).cuda() for n in ("q", "k", "v", "g", "beta")}
    st, cs, cw = w.state0.cuda(), w.conv_state0.cuda(), w.conv_w.cuda()
    o = torch.empty(steps, B, H, d, device="cuda")

    def run():
        for t in range(steps):
            K.kda_decode(dd, st, cs, cw, rows["q"][t], rows["k"][t], rows["v"][t], rows["g"][t], rows["beta"][t],
                         w.gate_mode, w.lower_bound, o[t])

    run()
    torch.cuda.synchronize()
    mk = lambda: torch.cuda.Event(enable_timing=True)
    e0, e1 = mk(), mk()
    e0.record(stream)
    run()
    e1.record(stream)
    torch.cuda.synchronize()
    eager = e0.elapsed_time(e1) / steps
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = mk(), mk()
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    graph = e0.elapsed_time(e1) / steps
    return {"workload": f"decode B={B} H={H} d={d}, {steps} steps", "eager_us_per_step": eager * 1e3,
            "graph_us_per_step": graph * 1e3, "graph_tokens_per_s": B / (graph * 1e-3)}


def measured_rw_reference(stream, mib=512, reps=20):
    import torch
    x = torch.ones(mib * (1 << 20) // 4, device="cuda")
    for _ in range(3):
        x.mul_(0.999999)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        x.mul_(0.999999)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del x
    return {"kind": f"torch in-place scale of {mib} MiB fp32 (read then write every byte)",
            "GB_per_s": 2 * mib * (1 << 20) / (ms * 1e-3) / 1e9, "ms": ms}


if __name__ == "__main__":
    main()
