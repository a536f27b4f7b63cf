"""The C-ABI library loads on the host, exports every entry point its header
declares, and rejects bad arguments before any launch (CPU only: every call
here fails validation or has nothing to do, so no HIP work is issued)."""
import ctypes
import math
import os
import re
import subprocess

import pytest

import kimi_delta_attention_prep_amd as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(K.LIB_PATH):
        from kimi_delta_attention_prep_amd import build
        build.build(verbose=False)
    return K.load_library()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^(?:int|size_t|const char\*)\s+(\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_entry_points():
    assert set(_declared()) == set(K.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", K.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in _declared():
        assert name in exported, name
        assert hasattr(lib, name)


A = ctypes.c_void_p(0x10000)   # aligned, never dereferenced (validation fails first)
MIS = ctypes.c_void_p(0x10001)  # misaligned for every element type
MIS4 = ctypes.c_void_p(0x10004)  # element-aligned, not 16-byte aligned


def dims(H=2, dk=128, dv=128, W=4, dt=K.DTYPE_BF16, act=K.ACT_SILU, prec=K.PREC_BF16X3, decay=K.DECAY_PER_DIM):
    return K.KdaDims(H, dk, dv, W, dt, act, prec, decay)


def decode(lib, d, *, q=A, gate=K.GATE_SAFE, lb=-5.0, batch=4, slots=None, state=A):
    return lib.kda_decode(ctypes.byref(d), batch, slots, state, A, A, q, A, A, A, A, gate, lb, A, None)


@pytest.mark.parametrize("d,code", [
    (dims(dk=96), K.KDA_E_GEOMETRY), (dims(dv=32), K.KDA_E_GEOMETRY), (dims(W=3), K.KDA_E_GEOMETRY),
    (dims(dt=7), K.KDA_E_DTYPE), (dims(act=3), K.KDA_E_DTYPE), (dims(prec=5), K.KDA_E_DTYPE),
    (dims(H=0), K.KDA_E_ARG), (dims(decay=2), K.KDA_E_GEOMETRY), (dims(decay=-1), K.KDA_E_GEOMETRY),
])
def test_geometry_and_dtype_rejected_before_launch(lib, d, code):
    assert decode(lib, d) == code
    assert lib.kda_last_error()  # a message is left


def test_every_precision_policy_accepted(lib):
    """The four policies pass the argument checks; 4 is refused. FP16 and BF16X2 keep one 16-byte
    fragment per A operand, BF16X3 and FP32 two, so their workspaces are the larger."""
    ws = {p: lib.kda_prefill_workspace_bytes(ctypes.byref(dims(prec=p)), 2, 1000)
          for p in (K.PREC_FP32, K.PREC_BF16X3, K.PREC_FP16, K.PREC_BF16X2)}
    assert all(v > 0 for v in ws.values())
    assert ws[K.PREC_FP16] == ws[K.PREC_BF16X2] < ws[K.PREC_BF16X3] == ws[K.PREC_FP32]
    assert lib.kda_prefill_workspace_bytes(ctypes.byref(dims(prec=4)), 2, 1000) == 0
    assert decode(lib, dims(prec=4)) == K.KDA_E_DTYPE


@pytest.mark.parametrize("gate,lb,code", [
    (9, -5.0, K.KDA_E_GATE), (K.GATE_SAFE, 0.0, K.KDA_E_GATE), (K.GATE_SAFE, 1.0, K.KDA_E_GATE),
    (K.GATE_SAFE, float("nan"), K.KDA_E_GATE), (K.GATE_SAFE, -math.inf, K.KDA_E_GATE),
])
def test_gate_checks(lib, gate, lb, code):
    assert decode(lib, dims(), gate=gate, lb=lb) == code


def test_lower_bound_ignored_in_softplus_mode(lib):
    # a nonsense bound passes the gate check in softplus mode; the misaligned row pointer then stops the call
    assert decode(lib, dims(), gate=K.GATE_SOFTPLUS, lb=float("nan"), q=MIS) == K.KDA_E_ALIGN


def test_pointer_checks(lib):
    assert decode(lib, dims(), q=MIS) == K.KDA_E_ALIGN
    assert decode(lib, dims(), state=MIS4) == K.KDA_E_ALIGN  # the state moves with 128-bit accesses
    assert decode(lib, dims(), q=None) == K.KDA_E_ARG
    assert decode(lib, dims(), slots=MIS) == K.KDA_E_ALIGN
    assert decode(lib, dims(), batch=-1) == K.KDA_E_ARG
    assert decode(lib, dims(), batch=0, q=None) == K.KDA_OK  # nothing to do, nothing launched


def test_verify_window_checks(lib):
    d = dims()
    log = K.KdaLog(A.value, A.value, A.value, A.value, 4)
    bad = K.KdaLog(A.value, A.value, A.value, A.value, 3)
    call = lambda W, nc, lin, lout, wl=None: lib.kda_verify_window(ctypes.byref(d), 4, W, wl, None, A, A, A, nc, lin,
                                                                    lout, MIS, A, A, A, A, K.GATE_SAFE, -5.0, A, None)
    assert call(9, None, None, ctypes.byref(log)) == K.KDA_E_GEOMETRY
    assert call(-1, None, None, ctypes.byref(log)) == K.KDA_E_GEOMETRY
    assert call(4, None, None, None) == K.KDA_E_ARG              # rows without a log to write
    assert call(4, None, None, ctypes.byref(bad)) == K.KDA_E_GEOMETRY  # log sized for another window
    assert call(4, A, None, ctypes.byref(log)) == K.KDA_E_ARG    # commit counts without a log
    assert call(4, A, ctypes.byref(log), ctypes.byref(log)) == K.KDA_E_ALIGN  # misaligned q row first
    assert call(0, None, None, None) == K.KDA_OK                 # nothing to commit, no rows
    assert call(4, None, None, ctypes.byref(log), MIS) == K.KDA_E_ALIGN  # window lengths are int32


def test_prep_and_prefill_checks(lib):
    d = dims()
    prep = lambda N, T, q: lib.kda_prep(ctypes.byref(d), N, T, A, None, q, A, A, A, A, A, A, A, K.GATE_SAFE, -5.0,
                                        A, A, A, A, A, None)
    assert prep(-1, 10, A) == K.KDA_E_ARG
    assert prep(0, 10, A) == K.KDA_E_ARG
    assert prep(2, 10, MIS) == K.KDA_E_ALIGN
    assert prep(2, 10, MIS4) == K.KDA_E_ALIGN  # raw rows are read 16 bytes at a time
    need = lib.kda_prefill_workspace_bytes(ctypes.byref(d), 2, 1000)
    assert need > 0
    pf = lambda ws, nb: lib.kda_prefill_varlen(ctypes.byref(d), 2, 1000, A, None, A, A, A, A, A, None, None, A, A,
                                               ws, nb, None)
    assert pf(A, need - 1) == K.KDA_E_WORKSPACE
    assert pf(None, need) == K.KDA_E_WORKSPACE
    assert pf(ctypes.c_void_p(0x10010), need) == K.KDA_E_ALIGN
    # o is written with 16-byte stores: an element-aligned o is refused
    assert lib.kda_prefill_varlen(ctypes.byref(d), 2, 1000, A, None, A, A, A, A, A, None, None, A, MIS4, A, need,
                                  None) == K.KDA_E_ALIGN
    assert lib.kda_prefill_workspace_bytes(ctypes.byref(dims(dk=96)), 2, 1000) == 0
    # the norm epilogue's arguments are checked with the rest, before any launch
    def pn(z, zt, eps, y, yt):
        nrm = K.KdaNormArgs(z, zt, 0x10000, eps, y, yt)
        return lib.kda_prefill_varlen(ctypes.byref(d), 2, 1000, A, None, A, A, A, A, A, None, ctypes.byref(nrm), A,
                                      A, A, need, None)
    assert pn(0x10000, 7, 1e-6, 0x10000, K.DTYPE_F32) == K.KDA_E_DTYPE
    assert pn(0x10000, K.DTYPE_BF16, 1e-6, 0x10000, 7) == K.KDA_E_DTYPE
    assert pn(0x10000, K.DTYPE_F32, -1.0, 0x10000, K.DTYPE_F32) == K.KDA_E_ARG
    assert pn(0x10000, K.DTYPE_F32, float("nan"), 0x10000, K.DTYPE_F32) == K.KDA_E_ARG
    assert pn(0x10000, K.DTYPE_F32, 1e-6, 0x10008, K.DTYPE_BF16) == K.KDA_E_ALIGN  # y written 16 bytes at a time
    assert pn(0x10004, K.DTYPE_F32, 1e-6, 0x10000, K.DTYPE_F32) == K.KDA_E_ALIGN
    assert pn(None, K.DTYPE_F32, 1e-6, 0x10000, K.DTYPE_F32) == K.KDA_E_ARG


def test_norm_checks(lib):
    nf = lambda dv, zt, eps, o: lib.gated_rmsnorm_out(10, dv, o, A, zt, A, eps, A, K.DTYPE_F32, None)
    assert nf(96, K.DTYPE_F32, 1e-6, A) == K.KDA_E_GEOMETRY
    assert nf(128, 4, 1e-6, A) == K.KDA_E_DTYPE
    assert nf(128, K.DTYPE_F32, -1.0, A) == K.KDA_E_ARG
    assert nf(128, K.DTYPE_F32, 1e-6, MIS) == K.KDA_E_ALIGN


def test_binding_has_no_fallback(tmp_path, monkeypatch):
    """A missing library is an error, never a silent substitute."""
    monkeypatch.setattr(K, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        K.load_library(str(tmp_path / "nope.so"))


def test_timing_hook_checks(lib):
    arr = (ctypes.c_void_p * 2)(0x10000, 0x10000)  # never used: no prompt call follows while set
    assert lib.kda_set_timing_events(arr, -2) == K.KDA_E_ARG
    assert lib.kda_set_timing_events(arr, 3) == K.KDA_E_ARG
    assert lib.kda_set_timing_events(None, 2) == K.KDA_E_ARG
    assert lib.kda_set_timing_events(arr, 2) == K.KDA_OK
    assert lib.kda_set_timing_events(None, 0) == K.KDA_OK


def test_debug_checks_of_device_contents():
    """The debug-mode checks of what the library takes as preconditions, on host copies."""
    import torch
    i32 = lambda v: torch.tensor(v, dtype=torch.int32)
    K._debug_cu(i32([0, 5, 5, 9]), 9)
    for bad, t in (([1, 5, 9], 9), ([0, 5, 8], 9), ([0, 6, 5, 9], 9)):
        with pytest.raises(ValueError):
            K._debug_cu(i32(bad), t)
    K._debug_slots(i32([3, -1, 0, 2]), (("state", 4),))
    with pytest.raises(ValueError, match="outside"):
        K._debug_slots(i32([3, 4]), (("state", 8), ("conv_state", 4)))
    with pytest.raises(ValueError, match="same slot"):
        K._debug_slots(i32([1, -1, 1]), (("state", 4),))
    K._debug_range(i32([0, 4, 2]), "n_commit", 0, 4)
    with pytest.raises(ValueError):
        K._debug_range(i32([0, 5]), "n_commit", 0, 4)
    with pytest.raises(ValueError):
        K._debug_range(i32([-1]), "window_lens", 0, 4)


def test_pool_size_without_slot_map():
    """Without a slot map sequence i uses slot i: a pool smaller than the batch is refused (shapes only)."""
    K._need_pool(3, None, (("state", 3), ("conv_state", 5)))
    K._need_pool(3, object(), (("state", 1),))  # with a slot map only the device contents can tell
    with pytest.raises(ValueError, match="no slot map"):
        K._need_pool(4, None, (("state", 8), ("conv_state", 3)))


def test_head_count_and_grid_limits(lib):
    """Heads go on a grid axis of at most 65535, and the prompt path's workgroup counts must fit a grid."""
    assert decode(lib, dims(H=65536)) == K.KDA_E_GEOMETRY
    d = dims()
    big = 1 << 31  # more rows than cu_seqlens (int32) can address
    assert lib.kda_prep(ctypes.byref(d), 2, big, A, None, A, A, A, A, A, A, A, A, K.GATE_SAFE, -5.0, A, A, A, A, A,
                        None) == K.KDA_E_ARG
    wide = dims(H=65535)
    rows = (1 << 31) - 1  # (rows / 64) record slots x 65535 heads overflow the grid
    assert lib.kda_prefill_varlen(ctypes.byref(wide), 1, rows, A, None, A, A, A, A, A, None, None, A, A, A, 1 << 40,
                                  None) == K.KDA_E_ARG


def _cpu_call_args(H=2, dk=128, dv=128, T=70, B=3, W=4):
    """Host tensors of the right dtypes and shapes for every binding call (the binding validates shapes before it
    requires device tensors, so a wrong shape is reported on the host with no launch)."""
    import torch
    d = K.Dims(H, dk, dv, torch.bfloat16)
    C = d.conv_channels
    bf = lambda *s: torch.zeros(*s, dtype=torch.bfloat16)
    f = lambda *s: torch.zeros(*s, dtype=torch.float32)
    return d, C, bf, f


def test_binding_rejects_wrong_shapes_before_any_launch(lib):
    import torch
    d, C, bf, f = _cpu_call_args()
    H, dk, dv, B, W = 2, 128, 128, 3, 4
    cw = f(C, 4)
    rows = lambda lead: (bf(*lead, H, dk), bf(*lead, H, dk), bf(*lead, H, dv), bf(*lead, H, dk), bf(*lead, H))

    def decode_call(state=None, conv_state=None, o=None):
        q, k, v, g, b = rows((B,))
        K.kda_decode(d, f(B, H, dk, dv) if state is None else state, bf(B, 3, C) if conv_state is None else conv_state,
                     cw, q, k, v, g, b, K.GATE_SAFE, -5.0, f(B, H, dv) if o is None else o)

    with pytest.raises(ValueError, match="state must have shape"):
        decode_call(state=f(B, H, 64, 64))  # a pool for d = 64 under d = 128 dims
    with pytest.raises(ValueError, match="conv_state must have shape"):
        decode_call(conv_state=bf(B, 3, C - 8))
    with pytest.raises(TypeError, match="conv_state must be"):
        decode_call(conv_state=f(B, 3, C))  # the conv state holds raw-row dtype
    with pytest.raises(ValueError, match="o must have shape"):
        decode_call(o=f(B + 1, H, dv))
    with pytest.raises(ValueError, match="contiguous device tensor"):
        decode_call()  # right shapes: the call still needs device tensors

    def verify_call(log_in=None, log_out=None, n_commit=None):
        q, k, v, g, b = (x.view(B, 1, *x.shape[1:]).expand(B, W, *x.shape[1:]).contiguous() for x in rows((B,)))
        lo = K.VerifyLog(f(B, W, H, dk), f(B, W, H, dk), f(B, W, H, dv), bf(B, W, C)) if log_out is None else log_out
        K.kda_verify_window(d, f(B, H, dk, dv), bf(B, 3, C), cw, n_commit, log_in, lo, q, k, v, g, b, K.GATE_SAFE,
                            -5.0, f(B, W, H, dv))

    with pytest.raises(ValueError, match="log_out.u must have shape"):
        verify_call(log_out=K.VerifyLog(f(B, W, H, dk), f(B, W, H, dk), f(B, W, H, dv - 1), bf(B, W, C)))
    with pytest.raises(ValueError, match="log_out.a must have shape"):
        verify_call(log_out=K.VerifyLog(f(B + 1, W, H, dk), f(B, W, H, dk), f(B, W, H, dv), bf(B, W, C)))
    with pytest.raises(TypeError, match="log_out.conv_rows must be"):
        verify_call(log_out=K.VerifyLog(f(B, W, H, dk), f(B, W, H, dk), f(B, W, H, dv), f(B, W, C)))
    short = K.VerifyLog(f(B, 2, H, dk), f(B, 2, H, dk), f(B, 2, H, dv), bf(B, 3, C))  # conv rows of another window
    with pytest.raises(ValueError, match="log_in.conv_rows must have shape"):
        verify_call(log_in=short, n_commit=torch.zeros(B, dtype=torch.int32))
    with pytest.raises(ValueError, match="log_in"):
        verify_call(n_commit=torch.zeros(B, dtype=torch.int32))  # commit counts without their log

    T, N = 70, 2
    q, k, v, g, b = rows((T,))
    cu = torch.tensor([0, 30, T], dtype=torch.int32)
    with pytest.raises(ValueError, match="conv_state_in must have shape"):
        K.kda_prep(d, cu, q, k, v, cw, bf(N, 2, C), bf(N, 2, C), g, b, K.GATE_SAFE, -5.0, f(T, H, dk), f(T, H, dk),
                   f(T, H, dv), f(T, H, dk), f(T, H))
    with pytest.raises(ValueError, match="g_out must have shape"):
        K.kda_prep(d, cu, q, k, v, cw, bf(N, 3, C), bf(N, 3, C), g, b, K.GATE_SAFE, -5.0, f(T, H, dk), f(T, H, dk),
                   f(T, H, dv), f(T, H), f(T, H))
    with pytest.raises(ValueError, match="state must have shape"):
        K.kda_prefill_varlen(d, cu, f(T, H, dk), f(T, H, dk), f(T, H, dv), f(T, H, dk), f(T, H), f(N, H, dk),
                             f(T, H, dv), torch.zeros(16, dtype=torch.uint8))
    raw = dict(q_raw=q, k_raw=k, v_raw=v, g_raw=g, beta_logit=b, conv_weight=cw, conv_state_in=bf(N, 3, C),
               conv_state_out=bf(N + 1, 3, C), gate_mode=K.GATE_SAFE, lower_bound=-5.0)
    with pytest.raises(ValueError, match="conv_state_out must have shape"):
        K.kda_prefill_varlen(d, cu, None, None, None, None, None, f(N, H, dk, dv), f(T, H, dv),
                             torch.zeros(16, dtype=torch.uint8), raw=raw)
    with pytest.raises(ValueError, match="y must have shape"):
        K.gated_rmsnorm_out(f(T, dv), bf(T, dv), f(dv), 1e-6, f(T, dv + 1))


def test_noalloc_prompt_call_checks(lib):
    """The allocation-free prompt call validates like kda_prefill_varlen, and refuses a geometry whose records
    exceed the library's scratch before resolving or touching it."""
    d = dims()
    call = lambda N, T, o=A: lib.kda_prefill_varlen_noalloc(ctypes.byref(d), N, T, A, None, A, A, A, A, A, None, None,
                                                            A, o, None)
    assert lib.kda_prefill_workspace_bytes(ctypes.byref(d), 8, 40000) > K.NOALLOC_SCRATCH_BYTES
    assert call(8, 40000) == K.KDA_E_WORKSPACE
    assert b"scratch" in lib.kda_last_error()
    assert call(2, 1000, MIS4) == K.KDA_E_ALIGN  # o is written with 16-byte stores
    assert call(-1, 10) == K.KDA_E_ARG
    assert call(0, 0) == K.KDA_OK  # nothing to do, nothing launched


def test_header_and_library_from_plain_c(lib, tmp_path):
    """include/kda.h compiles as C99 with every warning an error, and a C program linked against libkda.so
    gets the workspace sizes and the pre-launch argument checks (tests/abi_from_c.c; no GPU needed)."""
    import shutil
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    exe = tmp_path / "abi_from_c"
    libdir = os.path.dirname(K.LIB_PATH)
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "abi_from_c.c"), "-o", str(exe), "-L", libdir, "-lkda",
                        f"-Wl,-rpath,{libdir}"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
