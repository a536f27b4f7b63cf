"""Shared plumbing of the GPU parity tests: run the HIP path through the C ABI
and the fp64 oracle on the same seeded workload, and compare."""
from __future__ import annotations

import numpy as np
import torch

import kimi_delta_attention_prep_amd as K
from kimi_delta_attention_prep_amd.inputs import Workload
from oracle import oracle as O

EPS = 1e-6
TOL_BF16 = 2e-3   # relative L2 for bf16 inputs with an fp32 state
TOL_FP32 = 1e-5   # relative L2 on the all-fp32 path


def rel(x, ref) -> float:
    x = np.asarray(x.detach().cpu().double() if isinstance(x, torch.Tensor) else x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    return float(np.linalg.norm((x - ref).ravel()) / (den if den > 0 else 1.0))


def tol_for(w: Workload) -> float:
    return TOL_FP32 if w.dtype == torch.float32 else TOL_BF16


def dims_for(w: Workload, precision=None) -> K.Dims:
    return K.Dims(w.H, w.dk, w.dv, w.dtype, K.ACT_SILU, precision)


def select_heads(w: Workload, heads) -> Workload:
    return w.select_heads(heads)


def oracle_layer(w: Workload, with_log=False):
    return O.layer(w.f64("q"), w.f64("k"), w.f64("v"), w.f64("conv_w"), w.f64("conv_state0"), w.f64("g"),
                   w.f64("beta"), w.f64("z"), w.f64("norm_w"), w.f64("state0"), w.cu_seqlens.numpy(),
                   gate_mode=w.gate_mode, lower_bound=w.lower_bound, with_log=with_log)


def gpu_prep(w: Workload, d: K.Dims, dev="cuda"):
    wd = w.to(dev)
    T, H, dk, dv = w.T, w.H, w.dk, w.dv
    f = lambda *s: torch.empty(*s, device=dev, dtype=torch.float32)
    out = dict(q_hat=f(T, H, dk), k_hat=f(T, H, dk), v=f(T, H, dv), g=f(T, H, dk), beta=f(T, H),
               conv_state=torch.empty_like(wd.conv_state0))
    K.kda_prep(d, wd.cu_seqlens, wd.q, wd.k, wd.v, wd.conv_w, wd.conv_state0, out["conv_state"], wd.g, wd.beta,
               w.gate_mode, w.lower_bound, out["q_hat"], out["k_hat"], out["v"], out["g"], out["beta"])
    return wd, out


def raw_rows(wd: Workload, conv_state_out):
    return dict(q_raw=wd.q, k_raw=wd.k, v_raw=wd.v, g_raw=wd.g, beta_logit=wd.beta, conv_weight=wd.conv_w,
                conv_state_in=wd.conv_state0, conv_state_out=conv_state_out, gate_mode=wd.gate_mode,
                lower_bound=wd.lower_bound)


def gpu_layer_prefill(w: Workload, precision=None, y_dtype=torch.float32, dev="cuda", fused=False):
    """prep -> chunked prefill -> gated RMSNorm, all through the C ABI (fused: the preamble runs inside
    kda_prefill_varlen from the raw rows)."""
    d = dims_for(w, precision)
    T, H, dv = w.T, w.H, w.dv
    if fused:
        wd = w.to(dev)
        p = {"conv_state": torch.empty_like(wd.conv_state0)}
    else:
        wd, p = gpu_prep(w, d, dev)
    state = wd.state0.clone()
    o = torch.empty(T, H, dv, device=dev, dtype=torch.float32)
    ws = torch.empty(max(K.kda_prefill_workspace_bytes(d, w.N, T), 1), dtype=torch.uint8, device=dev)
    if fused:
        K.kda_prefill_varlen(d, wd.cu_seqlens, None, None, None, None, None, state, o, ws,
                             raw=raw_rows(wd, p["conv_state"]))
    else:
        K.kda_prefill_varlen(d, wd.cu_seqlens, p["q_hat"], p["k_hat"], p["v"], p["g"], p["beta"], state, o, ws)
    y = torch.empty(T, H, dv, device=dev, dtype=y_dtype)
    K.gated_rmsnorm_out(o, wd.z, wd.norm_w, EPS, y)
    torch.cuda.synchronize()
    return dict(prep=p, o=o, y=y, state=state)


def gpu_decode_steps(w: Workload, steps: int, dev="cuda"):
    """Run `steps` decode rows per sequence (row s of every sequence at step s)."""
    from kimi_delta_attention_prep_amd.inputs import step_rows
    d = dims_for(w)
    wd = w.to(dev)
    B, H, dv = w.N, w.H, w.dv
    rows = {n: step_rows(w, n, steps).to(dev) for n in ("q", "k", "v", "g", "beta", "z")}
    state = wd.state0.clone()
    cs = wd.conv_state0.clone()
    o = torch.empty(steps, B, H, dv, device=dev, dtype=torch.float32)
    for s in range(steps):
        K.kda_decode(d, state, cs, wd.conv_w, rows["q"][s], rows["k"][s], rows["v"][s], rows["g"][s],
                     rows["beta"][s], w.gate_mode, w.lower_bound, o[s])
    y = torch.empty_like(o)
    K.gated_rmsnorm_out(o, rows["z"], wd.norm_w, EPS, y)
    torch.cuda.synchronize()
    return dict(o=o, y=y, state=state, conv_state=cs)


def oracle_pieces(w: Workload, pieces, seqs=None, heads=None, state0=None, conv_state0=None, with_log=False):
    """The oracle over sequences made of chosen packed rows of w: sequence b runs rows pieces[b] (indices into w's
    rows, in order) from the initial state and conv state of w's sequence seqs[b] (default b), or from the given
    state0 [len(pieces), H, dk, dv] / conv_state0 [len(pieces), 3, C] (float64).  heads restricts every tensor to
    those heads (conv channels picked per stream)."""
    ww = w.select_heads(heads) if heads is not None else w
    seqs = list(range(len(pieces))) if seqs is None else list(seqs)
    idx = np.concatenate([np.asarray(p, dtype=np.int64) for p in pieces]) if len(pieces) else np.zeros(0, np.int64)
    cu = np.zeros(len(pieces) + 1, dtype=np.int64)
    cu[1:] = np.cumsum([len(p) for p in pieces])
    take = lambda name: ww.f64(name)[idx]
    st0 = ww.f64("state0")[seqs] if state0 is None else state0
    cs0 = ww.f64("conv_state0")[seqs] if conv_state0 is None else conv_state0
    return O.layer(take("q"), take("k"), take("v"), ww.f64("conv_w"), cs0, take("g"), take("beta"), take("z"),
                   ww.f64("norm_w"), st0, cu, gate_mode=w.gate_mode, lower_bound=w.lower_bound, with_log=with_log)
