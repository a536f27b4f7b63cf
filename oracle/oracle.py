"""Python face of the fp64 CPU oracle (``kda_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package smoke check and
by the benchmark's CPU-baseline leg, never by the product path.  It shares no
code with the HIP library; inputs arrive as numpy arrays (already rounded the
way the GPU receives them, then widened exactly to float64).

The layer it evaluates (TensorFold issue #850, the comment that lists the shared
KDA module's parts; onnxruntime-genai PR #2843, the op list in its
description):
  1. causal short conv over the q, k, v projected rows with a carried conv
     state, then the conv activation (SiLU, or none);
  2. q/k L2 normalisation per head;
  3. per-key-dim log-decay gate (softplus, or lower-bounded "safe" sigmoid) and
     per-head beta = sigmoid(logit);
  4. the gated delta rule  S_t = (I - b k k^T) Diag(a) S_{t-1} + b k v^T,
     o_t = S_t^T q_t, on one d_k x d_v state per (sequence, head);
  5. the sigmoid-gated output RMSNorm  y = o / rms(o) * w * sigmoid(z).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")

GATE_SOFTPLUS = 0
GATE_SAFE = 1
ACT_NONE = 0
ACT_SILU = 1
EPS = 1e-6

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with the host C compiler (no GPU code involved)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-std=c99", "-D_POSIX_C_SOURCE=200809L", "-ffp-contract=off", "-fPIC",
             "-shared", "-o", tmp, _SRC, "-lm", "-lpthread"],
            check=True,
        )
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        # KDA_ORACLE_LIB lets the mutation tests load a deliberately broken copy of the oracle
        alt = os.environ.get("KDA_ORACLE_LIB")
        if not alt:
            build()
        _lib = ctypes.CDLL(alt or _LIB)
        D = ctypes.POINTER(ctypes.c_double)
        I64 = ctypes.POINTER(ctypes.c_int64)
        ci, cd = ctypes.c_int, ctypes.c_double
        _lib.kda_oracle_prep.argtypes = [ci, ci, ci, ci, ci, ci, I64, D, D, D, D, D, D, D, D, ci, cd, cd,
                                         D, D, D, D, D, ci]
        _lib.kda_oracle_recurrent.argtypes = [ci, ci, ci, ci, I64, D, D, D, D, D, D, D, D, D, D, ci]
        _lib.kda_oracle_chunked.argtypes = [ci, ci, ci, ci, ci, I64, D, D, D, D, D, D, D, ci]
        _lib.kda_oracle_gated_rmsnorm.argtypes = [ctypes.c_int64, ci, D, D, D, cd, D]
        for f in ("kda_oracle_prep", "kda_oracle_recurrent", "kda_oracle_chunked", "kda_oracle_gated_rmsnorm"):
            getattr(_lib, f).restype = ci
    return _lib


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _d(a):
    """Contiguous float64 view + ctypes pointer (keeps the array alive via the caller)."""
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _cu(cu_seqlens):
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    if cu.ndim != 1 or cu[0] != 0 or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0 and be non-decreasing")
    return cu


@dataclass
class PrepOut:
    q_hat: np.ndarray
    k_hat: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    conv_state: np.ndarray


def prep(q_raw, k_raw, v_raw, conv_w, conv_state, g_raw, beta_logit, cu_seqlens, *, gate_mode=GATE_SOFTPLUS,
         lower_bound=-5.0, act=ACT_SILU, eps=EPS, threads=None) -> PrepOut:
    """Preamble: conv + activation, q/k L2 norm, gates, beta.

    q_raw,k_raw,g_raw [T,H,dk]; v_raw [T,H,dv]; conv_w [C,W]; conv_state [N,W-1,C]; beta_logit [T,H]."""
    q_raw, k_raw, v_raw, g_raw = map(_f64, (q_raw, k_raw, v_raw, g_raw))
    conv_w, conv_state, beta_logit = map(_f64, (conv_w, conv_state, beta_logit))
    cu = _cu(cu_seqlens)
    T, H, dk = q_raw.shape
    dv = v_raw.shape[2]
    C, W = conv_w.shape
    N = len(cu) - 1
    assert C == H * (2 * dk + dv) and conv_state.shape == (N, W - 1, C) and cu[-1] == T
    out = PrepOut(np.empty((T, H, dk)), np.empty((T, H, dk)), np.empty((T, H, dv)), np.empty((T, H, dk)),
                  np.empty((T, H)), np.empty((N, W - 1, C)))
    rc = _load().kda_oracle_prep(
        H, dk, dv, W, act, N, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _d(q_raw), _d(k_raw), _d(v_raw),
        _d(conv_w), _d(conv_state), _d(out.conv_state), _d(g_raw), _d(beta_logit), gate_mode, float(lower_bound),
        float(eps), _d(out.q_hat), _d(out.k_hat), _d(out.v), _d(out.g), _d(out.beta), threads or default_threads())
    assert rc == 0
    return out


@dataclass
class CoreOut:
    o: np.ndarray
    state: np.ndarray
    log_a: np.ndarray | None = None
    log_k: np.ndarray | None = None
    log_u: np.ndarray | None = None


def recurrent(q_hat, k_hat, v, g, beta, state0, cu_seqlens, *, with_log=False, threads=None) -> CoreOut:
    """Token-serial gated delta rule.  state0 [N,H,dk,dv] is not modified."""
    q_hat, k_hat, v, g, beta = map(_f64, (q_hat, k_hat, v, g, beta))
    cu = _cu(cu_seqlens)
    T, H, dk = q_hat.shape
    dv = v.shape[2]
    N = len(cu) - 1
    state = _f64(state0).copy()
    assert state.shape == (N, H, dk, dv) and cu[-1] == T
    o = np.empty((T, H, dv))
    la = np.empty((T, H, dk)) if with_log else None
    lk = np.empty((T, H, dk)) if with_log else None
    lu = np.empty((T, H, dv)) if with_log else None
    nul = ctypes.POINTER(ctypes.c_double)()
    rc = _load().kda_oracle_recurrent(
        H, dk, dv, N, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _d(q_hat), _d(k_hat), _d(v), _d(g),
        _d(beta), _d(state), _d(o), _d(la) if with_log else nul, _d(lk) if with_log else nul,
        _d(lu) if with_log else nul, threads or default_threads())
    assert rc == 0
    return CoreOut(o, state, la, lk, lu)


def chunked(q_hat, k_hat, v, g, beta, state0, cu_seqlens, *, chunk=64, threads=None) -> CoreOut:
    """Chunked (WY/UT) evaluation of the same recurrence, chunks anchored at each sequence start."""
    q_hat, k_hat, v, g, beta = map(_f64, (q_hat, k_hat, v, g, beta))
    cu = _cu(cu_seqlens)
    T, H, dk = q_hat.shape
    dv = v.shape[2]
    N = len(cu) - 1
    state = _f64(state0).copy()
    o = np.empty((T, H, dv))
    rc = _load().kda_oracle_chunked(H, dk, dv, int(chunk), N, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                    _d(q_hat), _d(k_hat), _d(v), _d(g), _d(beta), _d(state), _d(o),
                                    threads or default_threads())
    assert rc == 0
    return CoreOut(o, state)


def gated_rmsnorm(o, z, w, eps=EPS):
    o, z, w = map(_f64, (o, z, w))
    dv = o.shape[-1]
    rows = o.size // dv
    y = np.empty_like(o)
    rc = _load().kda_oracle_gated_rmsnorm(rows, dv, _d(o), _d(z), _d(w), float(eps), _d(y))
    assert rc == 0
    return y


@dataclass
class LayerOut:
    prep: PrepOut
    o: np.ndarray
    y: np.ndarray
    state: np.ndarray
    log_a: np.ndarray | None = None
    log_k: np.ndarray | None = None
    log_u: np.ndarray | None = None


def layer(q_raw, k_raw, v_raw, conv_w, conv_state, g_raw, beta_logit, z, norm_w, state0, cu_seqlens, *,
          gate_mode=GATE_SOFTPLUS, lower_bound=-5.0, act=ACT_SILU, eps=EPS, with_log=False,
          threads=None) -> LayerOut:
    """The whole layer, token-serial: prep -> recurrence -> gated RMSNorm."""
    p = prep(q_raw, k_raw, v_raw, conv_w, conv_state, g_raw, beta_logit, cu_seqlens, gate_mode=gate_mode,
             lower_bound=lower_bound, act=act, eps=eps, threads=threads)
    c = recurrent(p.q_hat, p.k_hat, p.v, p.g, p.beta, state0, cu_seqlens, with_log=with_log, threads=threads)
    y = gated_rmsnorm(c.o, z, norm_w, eps)
    return LayerOut(p, c.o, y, c.state, c.log_a, c.log_k, c.log_u)
