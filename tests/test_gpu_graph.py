"""HIP-graph capture of the C-ABI calls.  Every entry point only enqueues kernels
on the caller's stream (no allocation, no host synchronisation, no memset), so a
captured decode step, verify window or prompt pass replays with the bits of the
eager call.  Each graph is replayed several times, with eager work of the
library on other buffers between the replays, and every replay is checked bit
for bit against the eager call and against the fp64 oracle."""
import numpy as np
import pytest
import torch

import kimi_delta_attention_prep_amd as K
from kimi_delta_attention_prep_amd import inputs as I

from helpers import EPS, TOL_BF16, dims_for, oracle_layer, oracle_pieces, raw_rows, rel

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _rows(w, B, W):
    return {n: getattr(w, n).view(B, W, *getattr(w, n).shape[1:]).cuda() for n in ("q", "k", "v", "g", "beta")}


def _capture(fn):
    """Capture fn() into a graph after one eager warm-up run on a side stream."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def _busy(w, d):
    """Eager library work between replays, on buffers of its own."""
    st, cs = w.state0.cuda().clone(), w.conv_state0.cuda().clone()
    B, H = w.N, w.H
    x = torch.randn(B, H, w.dk, device="cuda").to(torch.bfloat16)
    o = torch.empty(B, H, w.dv, device="cuda")
    K.kda_decode(d, st, cs, w.conv_w.cuda(), x, x, torch.randn(B, H, w.dv, device="cuda").to(torch.bfloat16), x,
                 torch.zeros(B, H, device="cuda").to(torch.bfloat16), w.gate_mode, w.lower_bound, o)


@pytest.mark.parametrize("B", [1, 8])
def test_decode_steps_replay_from_a_graph(B):
    steps, H = 6, 4
    w = I.generate("graph", lengths=[steps] * B, H=H, dk=128, dv=128, dtype=torch.bfloat16, gate_mode=I.GATE_SAFE,
                   state_std=0.02, conv_state_std=1.0, seed=101 + B)
    d = dims_for(w)
    rows = _rows(w, B, steps)
    per = [{n: rows[n][:, s].contiguous() for n in rows} for s in range(steps)]
    cw = w.conv_w.cuda()
    st0, cs0 = w.state0.cuda(), w.conv_state0.cuda()
    print(f"graph decode B={B} H={H} steps={steps}", flush=True)

    def run(st, cs, o):
        for s in range(steps):
            K.kda_decode(d, st, cs, cw, per[s]["q"], per[s]["k"], per[s]["v"], per[s]["g"], per[s]["beta"],
                         w.gate_mode, w.lower_bound, o[s])

    st_e, cs_e = st0.clone(), cs0.clone()
    o_e = torch.empty(steps, B, H, w.dv, device="cuda")
    run(st_e, cs_e, o_e)
    st_g, cs_g = st0.clone(), cs0.clone()
    o_g = torch.empty_like(o_e)
    g = _capture(lambda: run(st_g, cs_g, o_g))
    ref = oracle_layer(w)  # row s of every sequence at step s
    for r in range(REPLAYS):
        st_g.copy_(st0)
        cs_g.copy_(cs0)
        o_g.fill_(float("nan"))
        g.replay()
        _busy(w, d)
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), f"replay {r}: o"
        assert torch.equal(st_g, st_e), f"replay {r}: state"
        assert torch.equal(cs_g, cs_e), f"replay {r}: conv state"
        assert rel(o_g.transpose(0, 1).reshape(w.T, H, w.dv), ref.o) < TOL_BF16, f"replay {r}: o vs oracle"
        assert rel(st_g, ref.state) < TOL_BF16, f"replay {r}: state vs oracle"
        assert np.array_equal(cs_g.cpu().double().numpy(), ref.prep.conv_state), f"replay {r}: conv state vs oracle"


def test_verify_window_and_commit_replay_from_a_graph():
    B, W, H = 5, 4, 2
    w = I.generate("graphver", lengths=[W] * B, H=H, dk=128, dv=128, dtype=torch.bfloat16, gate_mode=I.GATE_SAFE,
                   state_std=0.02, conv_state_std=1.0, seed=111)
    d = dims_for(w)
    rows = _rows(w, B, W)
    cw = w.conv_w.cuda()
    st0, cs0 = w.state0.cuda(), w.conv_state0.cuda()
    n_commit = torch.tensor([1, 4, 2, 3, 4], dtype=torch.int32, device="cuda")

    def run(st, cs, log, o):
        K.kda_verify_window(d, st, cs, cw, None, None, log, rows["q"], rows["k"], rows["v"], rows["g"], rows["beta"],
                            w.gate_mode, w.lower_bound, o)
        K.kda_verify_window(d, st, cs, cw, n_commit, log, None, None, None, None, None, None, w.gate_mode,
                            w.lower_bound, None, batch=B)

    st_e, cs_e, log_e = st0.clone(), cs0.clone(), K.VerifyLog.empty(d, B, W)
    o_e = torch.empty(B, W, H, w.dv, device="cuda")
    run(st_e, cs_e, log_e, o_e)
    st_g, cs_g, log_g = st0.clone(), cs0.clone(), K.VerifyLog.empty(d, B, W)
    o_g = torch.empty_like(o_e)
    g = _capture(lambda: run(st_g, cs_g, log_g, o_g))
    ref = oracle_layer(w, with_log=True)  # the whole window of every sequence from S0
    kept = oracle_pieces(w, [range(b * W, b * W + int(n_commit[b])) for b in range(B)])
    for r in range(REPLAYS):
        st_g.copy_(st0)
        cs_g.copy_(cs0)
        o_g.fill_(float("nan"))
        g.replay()
        _busy(w, d)
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), f"replay {r}: o"
        assert torch.equal(st_g, st_e) and torch.equal(cs_g, cs_e), f"replay {r}: committed state"
        for n in ("a", "k_hat", "u", "conv_rows"):
            assert torch.equal(getattr(log_g, n), getattr(log_e, n)), f"replay {r}: log {n}"
        assert rel(o_g.reshape(w.T, H, w.dv), ref.o) < TOL_BF16, f"replay {r}: o vs oracle"
        assert rel(log_g.u.reshape(w.T, H, w.dv), ref.log_u) < TOL_BF16, f"replay {r}: logged update vs oracle"
        assert rel(log_g.a.reshape(w.T, H, w.dk), ref.log_a) < 1e-6, f"replay {r}: logged decay vs oracle"
        assert rel(st_g, kept.state) < TOL_BF16, f"replay {r}: committed state vs oracle"
        assert np.array_equal(cs_g.cpu().double().numpy(), kept.prep.conv_state), f"replay {r}: conv state vs oracle"


def test_prompt_pass_replays_from_a_graph():
    w = I.generate("graphpf", lengths=[150, 3, 0, 64, 70], H=2, dk=128, dv=128, dtype=torch.bfloat16,
                   gate_mode=I.GATE_SOFTPLUS, state_std=0.02, conv_state_std=1.0, seed=121)
    d = dims_for(w, K.PREC_FP16)
    wd = w.to("cuda")
    ws = torch.empty(K.kda_prefill_workspace_bytes(d, w.N, w.T), dtype=torch.uint8, device="cuda")

    def run(st, cs, o, y):
        K.kda_prefill_varlen(d, wd.cu_seqlens, None, None, None, None, None, st, o, ws, raw=raw_rows(wd, cs),
                             norm=dict(z=wd.z, weight=wd.norm_w, eps=EPS, y=y))

    mk = lambda: (wd.state0.clone(), torch.empty_like(wd.conv_state0), torch.empty(w.T, w.H, w.dv, device="cuda"),
                  torch.empty(w.T, w.H, w.dv, device="cuda", dtype=torch.bfloat16))
    e = mk()
    run(*e)
    gbuf = mk()
    g = _capture(lambda: run(*gbuf))
    ref = oracle_layer(w)
    for r in range(REPLAYS):
        gbuf[0].copy_(wd.state0)
        gbuf[2].fill_(float("nan"))
        g.replay()
        _busy(w, dims_for(w))
        torch.cuda.synchronize()
        for a, b, n in zip(gbuf, e, ("state", "conv state", "o", "y")):
            assert torch.equal(a, b), f"replay {r}: {n}"
        errs = {"state": rel(gbuf[0], ref.state), "o": rel(gbuf[2], ref.o), "y": rel(gbuf[3].float(), ref.y)}
        assert all(x < TOL_BF16 for x in errs.values()), f"replay {r}: {errs}"
        assert np.array_equal(gbuf[1].cpu().double().numpy(), ref.prep.conv_state), f"replay {r}: conv state"
