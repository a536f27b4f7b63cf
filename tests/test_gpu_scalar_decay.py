"""The scalar-decay layer (one decay per head and row, raw g rows [.., H]) through
the same kernels: every entry point must give, bit for bit, what it gives for the
per-dim rows that repeat that decay over d_k, and the prompt pass must match the
fp64 oracle run on those broadcast rows."""
import dataclasses

import pytest
import torch

import kimi_delta_attention_prep_amd as K
from kimi_delta_attention_prep_amd import inputs as I

from helpers import EPS, TOL_BF16, oracle_layer, rel

pytestmark = pytest.mark.gpu


def _pair(lens, H=2, d=128, gate=I.GATE_SOFTPLUS, seed=131):
    """(workload with per-head g [T, H], the same workload with g repeated over d_k)."""
    w = I.generate("scalar", lengths=list(lens), H=H, dk=d, dv=d, dtype=torch.bfloat16, gate_mode=gate,
                   state_std=0.02, conv_state_std=1.0, seed=seed)
    gen = torch.Generator().manual_seed(seed + 1)
    gh = torch.randn(w.T, H, generator=gen).to(torch.bfloat16)
    wh = dataclasses.replace(w, g=gh)
    wb = dataclasses.replace(w, g=gh[:, :, None].expand(w.T, H, d).contiguous())
    return wh, wb


def _dims(w, per_head, precision=None):
    return K.Dims(w.H, w.dk, w.dv, w.dtype, K.ACT_SILU, precision, decay_per_head=per_head)


def test_prep_scalar_decay_is_the_broadcast_decay():
    wh, wb = _pair([150, 3, 0, 64])
    outs = []
    for w, ph in ((wh, True), (wb, False)):
        wd = w.to("cuda")
        T, H = w.T, w.H
        f = lambda *s: torch.empty(*s, device="cuda")
        o = dict(q=f(T, H, w.dk), k=f(T, H, w.dk), v=f(T, H, w.dv), g=f(T, H, w.dk), b=f(T, H),
                 cs=torch.empty_like(wd.conv_state0))
        K.kda_prep(_dims(w, ph), wd.cu_seqlens, wd.q, wd.k, wd.v, wd.conv_w, wd.conv_state0, o["cs"], wd.g, wd.beta,
                   w.gate_mode, w.lower_bound, o["q"], o["k"], o["v"], o["g"], o["b"])
        outs.append(o)
    torch.cuda.synchronize()
    for n in outs[0]:
        assert torch.equal(outs[0][n], outs[1][n]), n


@pytest.mark.parametrize("precision", [K.PREC_FP16, K.PREC_BF16X3])
def test_prompt_pass_scalar_decay_is_the_broadcast_decay(precision):
    wh, wb = _pair([150, 3, 0, 64, 70], seed=141)
    print(f"scalar decay prompt precision={precision} T={wh.T}", flush=True)
    res = []
    for w, ph in ((wh, True), (wb, False)):
        wd = w.to("cuda")
        d = _dims(w, ph, precision)
        st, cs = wd.state0.clone(), torch.empty_like(wd.conv_state0)
        o = torch.empty(w.T, w.H, w.dv, device="cuda")
        y = torch.empty(w.T, w.H, w.dv, device="cuda")
        ws = torch.empty(K.kda_prefill_workspace_bytes(d, w.N, w.T), dtype=torch.uint8, device="cuda")
        raw = dict(q_raw=wd.q, k_raw=wd.k, v_raw=wd.v, g_raw=wd.g, beta_logit=wd.beta, conv_weight=wd.conv_w,
                   conv_state_in=wd.conv_state0, conv_state_out=cs, gate_mode=w.gate_mode, lower_bound=w.lower_bound)
        K.kda_prefill_varlen(d, wd.cu_seqlens, None, None, None, None, None, st, o, ws, raw=raw,
                             norm=dict(z=wd.z, weight=wd.norm_w, eps=EPS, y=y))
        res.append((o, st, cs, y))
    torch.cuda.synchronize()
    for a, b, n in zip(res[0], res[1], ("o", "state", "conv state", "y")):
        assert torch.equal(a, b), n
    ref = oracle_layer(wb)
    assert rel(res[0][0], ref.o) < TOL_BF16
    assert rel(res[0][3], ref.y) < TOL_BF16
    assert rel(res[0][1], ref.state) < TOL_BF16


def test_decode_and_verify_scalar_decay_are_the_broadcast_decay():
    B, W = 4, 3
    wh, wb = _pair([W] * B, seed=151)
    res = []
    for w, ph in ((wh, True), (wb, False)):
        d = _dims(w, ph)
        rows = {n: getattr(w, n).view(B, W, *getattr(w, n).shape[1:]).cuda() for n in ("q", "k", "v", "g", "beta")}
        cw = w.conv_w.cuda()
        # decode the first row of every sequence, then a verify window over all W rows from the start state
        st, cs = w.state0.cuda().clone(), w.conv_state0.cuda().clone()
        od = torch.empty(B, w.H, w.dv, device="cuda")
        K.kda_decode(d, st, cs, cw, *(rows[n][:, 0].contiguous() for n in ("q", "k", "v", "g", "beta")), w.gate_mode,
                     w.lower_bound, od)
        sv, cv = w.state0.cuda().clone(), w.conv_state0.cuda().clone()
        log = K.VerifyLog.empty(d, B, W)
        ov = torch.empty(B, W, w.H, w.dv, device="cuda")
        K.kda_verify_window(d, sv, cv, cw, None, None, log, rows["q"], rows["k"], rows["v"], rows["g"], rows["beta"],
                            w.gate_mode, w.lower_bound, ov)
        res.append((od, st, cs, ov, log.a, log.k_hat, log.u, log.conv_rows))
    torch.cuda.synchronize()
    for a, b, n in zip(res[0], res[1], ("decode o", "decode state", "decode conv state", "window o", "log a",
                                        "log k", "log u", "log rows")):
        assert torch.equal(a, b), n
    assert torch.equal(res[0][3][:, 0], res[0][0])  # the window's first row is the decoded row
