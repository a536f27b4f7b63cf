"""Parity at the full sizes of the benchmark workloads, in the launch
configuration bench.py times.  Heads are independent, so where the oracle
would take minutes it runs on a subset of heads and the GPU result of those
heads is compared element by element."""
import numpy as np
import pytest
import torch

import kimi_delta_attention_prep_amd as K
from kimi_delta_attention_prep_amd import inputs as I

from helpers import TOL_BF16, dims_for, gpu_decode_steps, gpu_layer_prefill, oracle_layer, oracle_pieces, rel

pytestmark = pytest.mark.gpu


def _heads(r, hs):
    hs = torch.tensor(hs)
    return {k: (v[:, hs] if k in ("o", "y") else v) for k, v in r.items()}


@pytest.fixture(scope="module")
def prefill_ref():
    w = I.prefill()
    return w, oracle_layer(w)


@pytest.mark.parametrize("precision,fused", [(K.PREC_BF16X3, False), (K.PREC_FP16, True), (K.PREC_FP32, False),
                                             (K.PREC_BF16X2, True)])
def test_prefill_T4096_H16_full_oracle(prefill_ref, precision, fused):
    w, ref = prefill_ref
    print(f"prefill workload T={w.T} H={w.H} precision={precision} fused={fused}", flush=True)
    r = gpu_layer_prefill(w, precision=precision, y_dtype=torch.float32, fused=fused)
    errs = {"o": rel(r["o"], ref.o), "y": rel(r["y"], ref.y), "state": rel(r["state"], ref.state)}
    print(errs, flush=True)
    assert all(e < TOL_BF16 for e in errs.values()), errs


@pytest.mark.parametrize("precision,fused", [(K.PREC_BF16X3, False), (K.PREC_FP16, True), (K.PREC_BF16X2, True)])
def test_varlen_8_sequences_H32_head_subset(precision, fused):
    w = I.varlen()
    print(f"varlen workload T={w.T} lengths={torch.diff(w.cu_seqlens).tolist()}", flush=True)
    r = gpu_layer_prefill(w, precision=precision, fused=fused)
    hs = [0, 13, 31]
    sub = w.select_heads(hs)
    ref = oracle_layer(sub)
    hsi = torch.tensor(hs)
    errs = {"o": rel(r["o"][:, hsi], ref.o), "y": rel(r["y"][:, hsi], ref.y),
            "state": rel(r["state"][:, hsi], ref.state)}
    print(errs, flush=True)
    assert all(e < TOL_BF16 for e in errs.values()), errs
    # every head finite; per-sequence worst case also within tolerance
    assert torch.isfinite(r["o"]).all()
    cu = w.cu_seqlens.tolist()
    for n in range(w.N):
        assert rel(r["o"][cu[n]:cu[n + 1]][:, hsi], ref.o[cu[n]:cu[n + 1]]) < TOL_BF16


def test_decode_B256_64_steps_equals_prompt_and_oracle():
    steps = 64
    w = I.decode(steps=steps)
    dec = gpu_decode_steps(w, steps)
    # the same 64 rows as one prompt per sequence from the same initial state
    pf = gpu_layer_prefill(w)
    o_dec = dec["o"].transpose(0, 1).reshape(w.T, w.H, w.dv)
    errs = {"o": rel(o_dec, pf["o"].double().cpu().numpy()), "state": rel(dec["state"], pf["state"].double().cpu().numpy())}
    print("decode vs prompt", errs, flush=True)
    assert all(e < TOL_BF16 for e in errs.values()), errs
    assert torch.equal(dec["conv_state"], pf["prep"]["conv_state"])  # carried conv state bytes agree
    hs = [0, 31]
    ref = oracle_layer(w.select_heads(hs))
    hsi = torch.tensor(hs)
    errs = {"o": rel(o_dec[:, hsi], ref.o), "state": rel(dec["state"][:, hsi], ref.state)}
    print("decode vs oracle", errs, flush=True)
    assert all(e < TOL_BF16 for e in errs.values()), errs


def _verify_and_commit(w, rows, accept, state, cs):
    d = dims_for(w)
    B, W = rows["q"].shape[:2]
    log = K.VerifyLog.empty(d, B, W)
    o = torch.empty(B, W, w.H, w.dv, device="cuda")
    cw = w.conv_w.cuda()
    K.kda_verify_window(d, state, cs, cw, None, None, log, rows["q"], rows["k"], rows["v"], rows["g"], rows["beta"],
                        w.gate_mode, w.lower_bound, o)
    K.kda_verify_window(d, state, cs, cw, (accept + 1).cuda(), log, None, None, None, None, None, None, w.gate_mode,
                        w.lower_bound, None, batch=B)
    return o, log


def _serial(w, rows, accept, state, cs):
    d = dims_for(w)
    B, W = rows["q"].shape[:2]
    cw = w.conv_w.cuda()
    outs = []
    for s in range(W):
        slots = torch.tensor([b if s <= int(accept[b]) else -1 for b in range(B)], dtype=torch.int32, device="cuda")
        o = torch.zeros(B, w.H, w.dv, device="cuda")
        K.kda_decode(d, state, cs, cw, *(rows[n][:, s].contiguous() for n in ("q", "k", "v", "g", "beta")),
                     w.gate_mode, w.lower_bound, o, slots=slots)
        outs.append(o)
    return torch.stack(outs, 1)


def test_verify_B64_window4_bitwise_and_oracle():
    w = I.verify()
    B, W = w.N, w.meta["window"]
    accept = w.meta["accept"]
    rows = {n: getattr(w, n).view(B, W, *getattr(w, n).shape[1:]).cuda() for n in ("q", "k", "v", "g", "beta")}
    st_v, cs_v = w.state0.cuda().clone(), w.conv_state0.cuda().clone()
    o_v, _ = _verify_and_commit(w, rows, accept, st_v, cs_v)
    st_s, cs_s = w.state0.cuda().clone(), w.conv_state0.cuda().clone()
    o_s = _serial(w, rows, accept, st_s, cs_s)
    torch.cuda.synchronize()
    assert torch.equal(st_v, st_s) and torch.equal(cs_v, cs_s)
    for b in range(B):
        j = int(accept[b])
        assert torch.equal(o_v[b, :j + 1], o_s[b, :j + 1])
    hs = [0, 17]
    ref = oracle_layer(w.select_heads(hs))
    hsi = torch.tensor(hs)
    assert rel(o_v.reshape(w.T, w.H, w.dv)[:, hsi], ref.o) < TOL_BF16


def test_verify_B64_H32_window4_on_a_2048_row_prefilled_state():
    """The speculative-verify workload at its stated shape: 64 sequences x 32 heads, each prefilled with a
    2048-row prompt through kda_prefill_varlen, then a 4-row verify window with seeded accept lengths on the
    carried state and conv state, and the commit of the kept rows.  Bit for bit equal to serial decode on every
    head; against the oracle on two heads of all 64 sequences (the prompt's outputs, the window's outputs,
    the committed state and conv state)."""
    w = I.verify_prefilled()
    B, P, W, H = w.N, w.meta["prompt"], w.meta["window"], w.H
    L = P + W
    accept = w.meta["accept"]
    print(f"prefilled verify B={B} H={H} prompt={P} window={W}", flush=True)
    idx = torch.cat([torch.arange(b * L, b * L + P) for b in range(B)])
    widx = torch.cat([torch.arange(b * L + P, (b + 1) * L) for b in range(B)])
    pre = I.Workload("pre", H, w.dk, w.dv, torch.arange(0, B * P + 1, P, dtype=torch.int32), w.q[idx], w.k[idx],
                     w.v[idx], w.g[idx], w.beta[idx], w.z[idx], w.conv_w, w.norm_w, w.state0, w.conv_state0,
                     w.gate_mode, w.lower_bound)
    r = gpu_layer_prefill(pre, fused=True)
    del pre
    rows = {n: getattr(w, n)[widx].view(B, W, *getattr(w, n).shape[1:]).cuda() for n in ("q", "k", "v", "g", "beta")}
    st_v, cs_v = r["state"].clone(), r["prep"]["conv_state"].clone()
    o_v, _ = _verify_and_commit(w, rows, accept, st_v, cs_v)
    st_s, cs_s = r["state"].clone(), r["prep"]["conv_state"].clone()
    o_s = _serial(w, rows, accept, st_s, cs_s)
    torch.cuda.synchronize()
    assert torch.equal(st_v, st_s) and torch.equal(cs_v, cs_s)
    for b in range(B):
        j = int(accept[b])
        assert torch.equal(o_v[b, :j + 1], o_s[b, :j + 1])
    hs = [0, 31]
    hsi = torch.tensor(hs)
    ref = oracle_pieces(w, [range(b * L, (b + 1) * L) for b in range(B)], heads=hs)
    ref_o = ref.o.reshape(B, L, len(hs), w.dv)
    errs = {"window o": rel(o_v[:, :, hsi], ref_o[:, P:]),
            "prompt o": rel(r["o"].reshape(B, P, H, w.dv)[:, :, hsi], ref_o[:, :P])}
    kept = oracle_pieces(w, [range(b * L, b * L + P + int(accept[b]) + 1) for b in range(B)], heads=hs)
    errs["committed state"] = rel(st_v[:, hsi], kept.state)
    print(errs, flush=True)
    assert all(e < TOL_BF16 for e in errs.values()), errs
    ch = w.head_channels(hs)
    assert np.array_equal(cs_v[:, :, ch.cuda()].cpu().double().numpy(), kept.prep.conv_state)


def test_prefill_T4096_H16_fused_is_bitwise_the_two_call_path():
    """At the benchmark's own size and policy, the fused prompt call (preamble inside the prompt
    kernels) gives the bits of kda_prep followed by kda_prefill_varlen: o, final state, conv state."""
    w = I.prefill()
    a = gpu_layer_prefill(w, precision=K.PREC_FP16)
    b = gpu_layer_prefill(w, precision=K.PREC_FP16, fused=True)
    assert torch.equal(a["o"], b["o"])
    assert torch.equal(a["state"], b["state"])
    assert torch.equal(a["prep"]["conv_state"], b["prep"]["conv_state"])
