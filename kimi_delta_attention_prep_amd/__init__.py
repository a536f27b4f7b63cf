"""kimi_delta_attention_prep_amd -- Python binding of the gfx950 KDA library (libkda.so).

Argument marshalling only: each function checks shapes and dtypes of torch
tensors, passes their device pointers and torch's current HIP stream to the
C entry point of the same name (include/kda.h), and raises KdaError on a
non-zero status.  Every step of the layer runs in the library's HIP kernels;
there is no fallback of any kind -- a missing library is an error.

The layer (TensorFold issue #850, the shared KDA module; onnxruntime-genai PR
#2843, the KDA ops): causal short conv with carried state + SiLU, q/k L2
norms, softplus or lower-bounded sigmoid ("safe") log-decay gate, sigmoid
beta, the gated delta rule S_t = (I - b k k^T) Diag(a) S_{t-1} + b k v^T with
o_t = S_t^T q_t, and the sigmoid-gated output RMSNorm.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")

KDA_OK, KDA_E_ARG, KDA_E_GEOMETRY, KDA_E_ALIGN, KDA_E_GATE, KDA_E_DTYPE, KDA_E_WORKSPACE, KDA_E_HIP = range(8)
DTYPE_F32, DTYPE_BF16 = 0, 1
GATE_SOFTPLUS, GATE_SAFE = 0, 1
ACT_NONE, ACT_SILU = 0, 1
PREC_FP32, PREC_BF16X3, PREC_FP16, PREC_BF16X2 = 0, 1, 2, 3
DECAY_PER_DIM, DECAY_PER_HEAD = 0, 1
EXPORTS = ("kda_prep", "kda_prefill_workspace_bytes", "kda_prefill_varlen", "kda_prefill_varlen_noalloc",
           "kda_decode", "kda_verify_window", "gated_rmsnorm_out", "kda_last_error", "kda_set_timing_events")
NOALLOC_SCRATCH_BYTES = 160 << 20  # KDA_NOALLOC_SCRATCH_BYTES


class KdaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"KDA error {code}: {msg}")
        self.code = code


class KdaDims(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("head_dim_k", ctypes.c_int32), ("head_dim_v", ctypes.c_int32),
                ("conv_width", ctypes.c_int32), ("in_dtype", ctypes.c_int32), ("conv_act", ctypes.c_int32),
                ("precision", ctypes.c_int32), ("decay_shape", ctypes.c_int32)]


class KdaRawRows(ctypes.Structure):
    _fields_ = [("q_raw", ctypes.c_void_p), ("k_raw", ctypes.c_void_p), ("v_raw", ctypes.c_void_p),
                ("g_raw", ctypes.c_void_p), ("beta_logit", ctypes.c_void_p), ("conv_weight", ctypes.c_void_p),
                ("conv_state_in", ctypes.c_void_p), ("conv_state_out", ctypes.c_void_p),
                ("gate_mode", ctypes.c_int32), ("lower_bound", ctypes.c_float)]


class KdaNormArgs(ctypes.Structure):
    _fields_ = [("z", ctypes.c_void_p), ("z_dtype", ctypes.c_int32), ("weight", ctypes.c_void_p),
                ("eps", ctypes.c_float), ("y", ctypes.c_void_p), ("y_dtype", ctypes.c_int32)]


class KdaLog(ctypes.Structure):
    _fields_ = [("a", ctypes.c_void_p), ("k_hat", ctypes.c_void_p), ("u", ctypes.c_void_p),
                ("conv_rows", ctypes.c_void_p), ("window", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libkda.so (built by build.py); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m kimi_delta_attention_prep_amd.build`")
        lib = ctypes.CDLL(path)
        vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        D = ctypes.POINTER(KdaDims)
        Lg = ctypes.POINTER(KdaLog)
        lib.kda_prep.argtypes = [D, i32, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, f32, vp, vp, vp, vp, vp, vp]
        lib.kda_prefill_workspace_bytes.argtypes = [D, i32, i64]
        lib.kda_prefill_workspace_bytes.restype = ctypes.c_size_t
        lib.kda_prefill_varlen.argtypes = [D, i32, i64, vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(KdaRawRows),
                                           ctypes.POINTER(KdaNormArgs), vp, vp, vp, ctypes.c_size_t, vp]
        lib.kda_prefill_varlen_noalloc.argtypes = [D, i32, i64, vp, vp, vp, vp, vp, vp, vp,
                                                   ctypes.POINTER(KdaRawRows), ctypes.POINTER(KdaNormArgs), vp, vp,
                                                   vp]
        lib.kda_decode.argtypes = [D, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, f32, vp, vp]
        lib.kda_verify_window.argtypes = [D, i32, i32, vp, vp, vp, vp, vp, vp, Lg, Lg, vp, vp, vp, vp, vp, i32, f32, vp,
                                          vp]
        lib.gated_rmsnorm_out.argtypes = [i64, i32, vp, vp, i32, vp, f32, vp, i32, vp]
        lib.kda_last_error.restype = ctypes.c_char_p
        lib.kda_set_timing_events.argtypes = [vp, i32]
        for f in ("kda_prep", "kda_prefill_varlen", "kda_prefill_varlen_noalloc", "kda_decode", "kda_verify_window",
                  "gated_rmsnorm_out", "kda_set_timing_events"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


def _check(rc: int):
    if rc != KDA_OK:
        raise KdaError(rc, load_library().kda_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return DTYPE_F32
    if dt == torch.bfloat16:
        return DTYPE_BF16
    raise TypeError(f"unsupported dtype {dt}")


def _shape_ok(t, shape) -> bool:
    """`shape` entries are sizes, or None for any size (a pool's slot count)."""
    return t.dim() == len(shape) and all(want is None or have == want for have, want in zip(t.shape, shape))


def _validate(specs, device=True):
    """Check every (name, tensor, dtype or None, shape or None) entry: first the type, dtype and shape of all of
    them, then (unless device is False) that each is a contiguous device tensor.  The library receives bare
    pointers and cannot check a buffer's size, so this is the guard against reads and writes past an allocation;
    it runs before any launch."""
    for name, t, dtype, shape in specs:
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a tensor")
        if dtype is not None and t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if shape is not None and not _shape_ok(t, shape):
            want = tuple("*" if x is None else x for x in shape)
            raise ValueError(f"{name} must have shape {want}, got {tuple(t.shape)}")
    for name, t, _, _ in specs if device else ():
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")


def _need(t, name, dtype=None, shape=None):
    _validate([(name, t, dtype, shape)])
    return t


# Debug mode: the device-side contents the library takes as preconditions
# (cu_seqlens, slot maps, commit counts, window lengths) are copied to the host
# and checked before the call.  Each check synchronises with the device, so it
# is off by default; KDA_DEBUG=1 in the environment or set_debug(True) turns it on.
_debug = os.environ.get("KDA_DEBUG", "0") not in ("", "0")


def set_debug(on: bool) -> None:
    global _debug
    _debug = bool(on)


def _host_ints(t) -> list:
    return [int(x) for x in t.detach().to("cpu", torch.int64).tolist()]


def _debug_cu(cu_seqlens, t_tot: int) -> None:
    """cu_seqlens[0] = 0, non-decreasing, cu_seqlens[N] = t_tot."""
    cu = _host_ints(cu_seqlens)
    if not cu or cu[0] != 0 or cu[-1] != t_tot:
        raise ValueError(f"cu_seqlens must start at 0 and end at {t_tot} (the row count), got {cu[:1]}..{cu[-1:]}")
    bad = next((n for n in range(len(cu) - 1) if cu[n + 1] < cu[n]), None)
    if bad is not None:
        raise ValueError(f"cu_seqlens decreases at sequence {bad}: {cu[bad]} -> {cu[bad + 1]}")


def _debug_slots(slots, pools) -> None:
    """Every slot below each pool size (negative = skipped); no two sequences share a slot."""
    sl = _host_ints(slots)
    for name, size in pools:
        over = [x for x in sl if x >= size]
        if over:
            raise ValueError(f"slot {over[0]} is outside the {name} pool of {size} slots")
    live = [x for x in sl if x >= 0]
    if len(set(live)) != len(live):
        raise ValueError("two sequences map to the same slot (their state updates would race)")


def _debug_range(t, name: str, lo: int, hi: int) -> None:
    v = _host_ints(t)
    bad = next((x for x in v if x < lo or x > hi), None)
    if bad is not None:
        raise ValueError(f"{name} holds {bad}, outside [{lo}, {hi}]")


def _need_pool(n: int, slots, pools) -> None:
    """Without a slot map, sequence i uses slot i: every pool needs n slots (shapes only, always checked)."""
    if slots is None:
        for name, size in pools:
            if size < n:
                raise ValueError(f"{name} has {size} slots for {n} sequences and no slot map")


@dataclass(frozen=True)
class Dims:
    num_heads: int
    head_dim_k: int
    head_dim_v: int
    in_dtype: torch.dtype = torch.bfloat16
    conv_act: int = ACT_SILU
    precision: int | None = None  # default: FP32 for fp32 rows, BF16X3 for bf16 rows
    decay_per_head: bool = False  # raw g rows [.., H]: one decay per head (scalar-decay layer)

    def c(self) -> KdaDims:
        prec = self.precision
        if prec is None:
            prec = PREC_FP32 if self.in_dtype == torch.float32 else PREC_BF16X3
        return KdaDims(self.num_heads, self.head_dim_k, self.head_dim_v, 4, _dtype_code(self.in_dtype), self.conv_act,
                       prec, DECAY_PER_HEAD if self.decay_per_head else DECAY_PER_DIM)

    def g_shape(self, *lead) -> tuple:
        """Shape of raw g rows with leading dims `lead` (then H, and d_k unless the decay is per head)."""
        return (*lead, self.num_heads) if self.decay_per_head else (*lead, self.num_heads, self.head_dim_k)

    @property
    def conv_channels(self) -> int:
        return self.num_heads * (2 * self.head_dim_k + self.head_dim_v)


def kda_prep(d: Dims, cu_seqlens, q_raw, k_raw, v_raw, conv_weight, conv_state_in, conv_state_out, g_raw,
             beta_logit, gate_mode, lower_bound, q_hat, k_hat, v_out, g_out, beta_out, slots=None):
    lib = load_library()
    H, dk, dv, dt = d.num_heads, d.head_dim_k, d.head_dim_v, d.in_dtype
    _validate([("cu_seqlens", cu_seqlens, torch.int32, (None,)), ("q_raw", q_raw, dt, (None, H, dk))], device=False)
    T = q_raw.shape[0]
    N = cu_seqlens.numel() - 1
    C = d.conv_channels
    specs = [("cu_seqlens", cu_seqlens, None, None), ("q_raw", q_raw, None, None), ("k_raw", k_raw, dt, (T, H, dk)), ("v_raw", v_raw, dt, (T, H, dv)), ("g_raw", g_raw, dt, d.g_shape(T)),
             ("beta_logit", beta_logit, dt, (T, H)), ("conv_weight", conv_weight, torch.float32, (C, 4)),
             ("conv_state_in", conv_state_in, dt, (None, 3, C)),
             ("conv_state_out", conv_state_out, dt, tuple(conv_state_in.shape)),
             ("q_hat", q_hat, torch.float32, (T, H, dk)), ("k_hat", k_hat, torch.float32, (T, H, dk)),
             ("v_out", v_out, torch.float32, (T, H, dv)), ("g_out", g_out, torch.float32, (T, H, dk)),
             ("beta_out", beta_out, torch.float32, (T, H))]
    if slots is not None:
        specs.append(("slots", slots, torch.int32, (N,)))
    _validate(specs)
    pools = (("conv_state", conv_state_in.shape[0]),)
    _need_pool(N, slots, pools)
    if _debug:
        _debug_cu(cu_seqlens, T)
        if slots is not None:
            _debug_slots(slots, pools)
    dims = d.c()
    _check(lib.kda_prep(ctypes.byref(dims), N, T, _ptr(cu_seqlens), _ptr(slots), _ptr(q_raw), _ptr(k_raw),
                        _ptr(v_raw), _ptr(conv_weight), _ptr(conv_state_in), _ptr(conv_state_out), _ptr(g_raw),
                        _ptr(beta_logit), int(gate_mode), float(lower_bound), _ptr(q_hat), _ptr(k_hat), _ptr(v_out),
                        _ptr(g_out), _ptr(beta_out), _stream()))


def kda_prefill_workspace_bytes(d: Dims, num_seqs: int, t_tot: int) -> int:
    dims = d.c()
    return int(load_library().kda_prefill_workspace_bytes(ctypes.byref(dims), int(num_seqs), int(t_tot)))


def kda_prefill_varlen_noalloc(d: Dims, cu_seqlens, q_hat, k_hat, v, g, beta, state, o, slots=None, raw=None,
                               norm=None):
    """kda_prefill_varlen without a workspace: the chunk records go to the library's per-device scratch
    (NOALLOC_SCRATCH_BYTES), for callers that cannot allocate device memory.  Calls that overlap on one device
    race on that scratch."""
    kda_prefill_varlen(d, cu_seqlens, q_hat, k_hat, v, g, beta, state, o, None, slots=slots, raw=raw, norm=norm)


def kda_prefill_varlen(d: Dims, cu_seqlens, q_hat, k_hat, v, g, beta, state, o, workspace, slots=None, raw=None,
                       norm=None):
    """Chunked prompt pass.  With raw=dict(q_raw, k_raw, v_raw, g_raw, beta_logit, conv_weight, conv_state_in,
    conv_state_out, gate_mode, lower_bound) the preamble runs inside the prompt kernels and q_hat..beta may be None.
    With norm=dict(z, weight, eps, y) the gated output norm runs as the call's epilogue (y as gated_rmsnorm_out).
    workspace=None calls kda_prefill_varlen_noalloc instead."""
    lib = load_library()
    H, dk, dv = d.num_heads, d.head_dim_k, d.head_dim_v
    _validate([("cu_seqlens", cu_seqlens, torch.int32, (None,))], device=False)
    N = cu_seqlens.numel() - 1
    rr = None
    if raw is None:
        _validate([("q_hat", q_hat, torch.float32, (None, H, dk))], device=False)
        T = q_hat.shape[0]
        specs = [("q_hat", q_hat, None, None), ("k_hat", k_hat, torch.float32, (T, H, dk)), ("v", v, torch.float32, (T, H, dv)),
                 ("g", g, torch.float32, (T, H, dk)), ("beta", beta, torch.float32, (T, H))]
    else:
        dt = d.in_dtype
        _validate([("q_raw", raw["q_raw"], dt, (None, H, dk))], device=False)
        T = raw["q_raw"].shape[0]
        specs = [("q_raw", raw["q_raw"], None, None)]
        specs += [(name, raw[name], dt, shp) for name, shp in
                 (("k_raw", (T, H, dk)), ("v_raw", (T, H, dv)), ("g_raw", d.g_shape(T)), ("beta_logit", (T, H)))]
        specs += [("conv_weight", raw["conv_weight"], torch.float32, (d.conv_channels, 4)),
                  ("conv_state_in", raw["conv_state_in"], dt, (None, 3, d.conv_channels))]
        specs.append(("conv_state_out", raw["conv_state_out"], dt, tuple(raw["conv_state_in"].shape)))
    specs += [("cu_seqlens", cu_seqlens, None, None), ("o", o, torch.float32, (T, H, dv)),
              ("state", state, torch.float32, (None, H, dk, dv))]
    if workspace is not None:
        specs.append(("workspace", workspace, None, None))
    if norm is not None:
        specs += [("z", norm["z"], None, (T, H, dv)), ("weight", norm["weight"], torch.float32, (dv,)),
                  ("y", norm["y"], None, (T, H, dv))]
    if slots is not None:
        specs.append(("slots", slots, torch.int32, (N,)))
    _validate(specs)
    if raw is not None:
        rr = KdaRawRows(*(raw[n].data_ptr() for n in ("q_raw", "k_raw", "v_raw", "g_raw", "beta_logit", "conv_weight",
                                                      "conv_state_in", "conv_state_out")),
                        int(raw["gate_mode"]), float(raw["lower_bound"]))
    nn = None
    if norm is not None:
        nn = KdaNormArgs(norm["z"].data_ptr(), _dtype_code(norm["z"].dtype), norm["weight"].data_ptr(),
                         float(norm["eps"]), norm["y"].data_ptr(), _dtype_code(norm["y"].dtype))
    pools = (("state", state.shape[0]),) + ((("conv_state", raw["conv_state_in"].shape[0]),) if raw else ())
    _need_pool(N, slots, pools)
    if _debug:
        _debug_cu(cu_seqlens, T)
        if slots is not None:
            _debug_slots(slots, pools)
    dims = d.c()
    common = (ctypes.byref(dims), N, T, _ptr(cu_seqlens), _ptr(slots), _ptr(q_hat), _ptr(k_hat), _ptr(v), _ptr(g),
              _ptr(beta), ctypes.byref(rr) if rr is not None else None, ctypes.byref(nn) if nn is not None else None,
              _ptr(state), _ptr(o))
    if workspace is None:
        _check(lib.kda_prefill_varlen_noalloc(*common, _stream()))
    else:
        _check(lib.kda_prefill_varlen(*common, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream()))


def kda_decode(d: Dims, state, conv_state, conv_weight, q_raw, k_raw, v_raw, g_raw, beta_logit, gate_mode,
               lower_bound, o, slots=None):
    lib = load_library()
    H, dk, dv, dt = d.num_heads, d.head_dim_k, d.head_dim_v, d.in_dtype
    _validate([("q_raw", q_raw, dt, (None, H, dk))], device=False)
    B = q_raw.shape[0]
    specs = [("q_raw", q_raw, None, None), ("k_raw", k_raw, dt, (B, H, dk)), ("v_raw", v_raw, dt, (B, H, dv)), ("g_raw", g_raw, dt, d.g_shape(B)),
             ("beta_logit", beta_logit, dt, (B, H)), ("state", state, torch.float32, (None, H, dk, dv)),
             ("conv_state", conv_state, dt, (None, 3, d.conv_channels)),
             ("conv_weight", conv_weight, torch.float32, (d.conv_channels, 4)), ("o", o, torch.float32, (B, H, dv))]
    if slots is not None:
        specs.append(("slots", slots, torch.int32, (B,)))
    _validate(specs)
    pools = (("state", state.shape[0]), ("conv_state", conv_state.shape[0]))
    _need_pool(B, slots, pools)
    if _debug and slots is not None:
        _debug_slots(slots, pools)
    dims = d.c()
    _check(lib.kda_decode(ctypes.byref(dims), B, _ptr(slots), _ptr(state), _ptr(conv_state), _ptr(conv_weight),
                          _ptr(q_raw), _ptr(k_raw), _ptr(v_raw), _ptr(g_raw), _ptr(beta_logit), int(gate_mode),
                          float(lower_bound), _ptr(o), _stream()))


@dataclass
class VerifyLog:
    """Device buffers of one verify window's log (see kda_log in include/kda.h)."""
    a: torch.Tensor  # [B, W, H, dk] fp32
    k_hat: torch.Tensor  # [B, W, H, dk] fp32
    u: torch.Tensor  # [B, W, H, dv] fp32
    conv_rows: torch.Tensor  # [B, W, C] raw dtype

    @property
    def window(self) -> int:
        return self.a.shape[1]

    @staticmethod
    def empty(d: Dims, batch: int, window: int, device="cuda") -> "VerifyLog":
        H, dk, dv = d.num_heads, d.head_dim_k, d.head_dim_v
        f = dict(device=device, dtype=torch.float32)
        return VerifyLog(torch.empty(batch, window, H, dk, **f), torch.empty(batch, window, H, dk, **f),
                         torch.empty(batch, window, H, dv, **f),
                         torch.empty(batch, window, d.conv_channels, device=device, dtype=d.in_dtype))

    def c(self) -> KdaLog:
        return KdaLog(self.a.data_ptr(), self.k_hat.data_ptr(), self.u.data_ptr(), self.conv_rows.data_ptr(),
                      self.window)

    def specs(self, d: Dims, batch: int, window: int, tag: str) -> list:
        """Validation entries of every field for a log of `batch` sequences and `window` rows."""
        H, dk, dv = d.num_heads, d.head_dim_k, d.head_dim_v
        return [(f"{tag}.a", self.a, torch.float32, (batch, window, H, dk)),
                (f"{tag}.k_hat", self.k_hat, torch.float32, (batch, window, H, dk)),
                (f"{tag}.u", self.u, torch.float32, (batch, window, H, dv)),
                (f"{tag}.conv_rows", self.conv_rows, d.in_dtype, (batch, window, d.conv_channels))]


def kda_verify_window(d: Dims, state, conv_state, conv_weight, n_commit, log_in, log_out, q_raw, k_raw, v_raw,
                      g_raw, beta_logit, gate_mode, lower_bound, o, slots=None, batch=None, window_lens=None):
    lib = load_library()
    H, dk, dv, dt = d.num_heads, d.head_dim_k, d.head_dim_v, d.in_dtype
    if q_raw is not None:
        _validate([("q_raw", q_raw, dt, (None, None, H, dk))], device=False)
    W = 0 if q_raw is None else q_raw.shape[1]
    B = batch if batch is not None else (q_raw.shape[0] if q_raw is not None else n_commit.numel())
    specs = [("state", state, torch.float32, (None, H, dk, dv)),
             ("conv_state", conv_state, dt, (None, 3, d.conv_channels)),
             ("conv_weight", conv_weight, torch.float32, (d.conv_channels, 4))]
    if W > 0:
        specs += [("q_raw", q_raw, dt, (B, W, H, dk)), ("k_raw", k_raw, dt, (B, W, H, dk)),
                  ("v_raw", v_raw, dt, (B, W, H, dv)), ("g_raw", g_raw, dt, d.g_shape(B, W)),
                  ("beta_logit", beta_logit, dt, (B, W, H)), ("o", o, torch.float32, (B, W, H, dv))]
        if log_out is None:
            raise ValueError("a window with rows needs log_out")
        specs += log_out.specs(d, B, W, "log_out")
    if n_commit is not None:
        if log_in is None:
            raise ValueError("n_commit needs the log it commits from (log_in)")
        specs.append(("n_commit", n_commit, torch.int32, (B,)))
        specs += log_in.specs(d, B, log_in.window, "log_in")
    if slots is not None:
        specs.append(("slots", slots, torch.int32, (B,)))
    if window_lens is not None:
        specs.append(("window_lens", window_lens, torch.int32, (B,)))
    _validate(specs)
    dims = d.c()
    lin = log_in.c() if log_in is not None else None
    lout = log_out.c() if log_out is not None else None
    pools = (("state", state.shape[0]), ("conv_state", conv_state.shape[0]))
    _need_pool(B, slots, pools)
    if _debug:
        if slots is not None:
            _debug_slots(slots, pools)
        if n_commit is not None:
            _debug_range(n_commit, "n_commit", 0, log_in.window if log_in is not None else 0)
        if window_lens is not None:
            _debug_range(window_lens, "window_lens", 0, W)
    _check(lib.kda_verify_window(ctypes.byref(dims), B, W, _ptr(window_lens), _ptr(slots), _ptr(state),
                                 _ptr(conv_state),
                                 _ptr(conv_weight), _ptr(n_commit), ctypes.byref(lin) if lin else None,
                                 ctypes.byref(lout) if lout else None, _ptr(q_raw), _ptr(k_raw), _ptr(v_raw),
                                 _ptr(g_raw), _ptr(beta_logit), int(gate_mode), float(lower_bound), _ptr(o),
                                 _stream()))


def gated_rmsnorm_out(o, z, w, eps, y):
    lib = load_library()
    _validate([("o", o, torch.float32, None)], device=False)
    if o.dim() < 1:
        raise ValueError("o must have at least one dimension (the d_v values of a row)")
    dv = o.shape[-1]
    rows = o.numel() // dv if dv else 0
    _validate([("o", o, torch.float32, None), ("z", z, None, tuple(o.shape)), ("w", w, torch.float32, (dv,)),
               ("y", y, None, tuple(o.shape))])
    _check(lib.gated_rmsnorm_out(rows, dv, _ptr(o), _ptr(z), _dtype_code(z.dtype), _ptr(w), float(eps), _ptr(y),
                                 _dtype_code(y.dtype), _stream()))


# kernels of one kda_prefill_varlen call, in the order the timing hook numbers them
# (the third only when the call has the norm epilogue)
PREFILL_KERNELS = ("chunk_intra", "chunk_scan", "gated_rmsnorm")


def kda_set_timing_events(events):
    """Record events around each kernel of later kda_prefill_varlen calls on this
    thread: events[2i] / events[2i+1] bracket kernel i (PREFILL_KERNELS order).
    `events` is a sequence of torch.cuda.Event(enable_timing=True) that have
    been recorded once (so that the HIP events exist), or None to stop.  The
    handle array is kept alive here until the next call."""
    global _timing_handles
    lib = load_library()
    if not events:
        _check(lib.kda_set_timing_events(None, 0))
        _timing_handles = None
        return
    handles = [int(e.cuda_event) for e in events]
    if any(h == 0 for h in handles):
        raise ValueError("record every event once before passing it (HIP events are created lazily)")
    arr = (ctypes.c_void_p * len(handles))(*handles)
    _check(lib.kda_set_timing_events(arr, len(handles)))
    _timing_handles = arr


_timing_handles = None
