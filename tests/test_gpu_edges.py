"""Edge and degenerate cases of the GPU path against the fp64 oracle: empty
inputs, a gate that freezes the state, and one long sequence next to a short
one at the full head size."""
import numpy as np
import pytest
import torch

import kimi_delta_attention_prep_amd as K
from kimi_delta_attention_prep_amd import inputs as I

from helpers import TOL_BF16, dims_for, gpu_decode_steps, gpu_layer_prefill, oracle_layer, rel

pytestmark = pytest.mark.gpu


def _small(lens, dtype=torch.bfloat16, H=2, d=128, gate=I.GATE_SOFTPLUS, seed=5):
    return I.generate("edge", lengths=list(lens), H=H, dk=d, dv=d, dtype=dtype, gate_mode=gate, state_std=0.02,
                      conv_state_std=1.0, seed=seed)


@pytest.mark.parametrize("fused", [False, True])
def test_prefill_every_sequence_empty(fused):
    """Sequences of length 0 only: the call succeeds and state and conv state keep their bits."""
    w = _small((0, 0, 0))
    print(f"empty prompt fused={fused}", flush=True)
    r = gpu_layer_prefill(w, fused=fused)
    assert torch.equal(r["state"].cpu(), w.state0)
    if fused:
        assert torch.equal(r["prep"]["conv_state"].cpu(), w.conv_state0)


def test_prefill_no_sequences_is_a_no_op():
    w = _small((5,))
    d = dims_for(w)
    state = torch.zeros(1, w.H, w.dk, w.dv, device="cuda")
    o = torch.empty(0, w.H, w.dv, device="cuda")
    ws = torch.empty(1, dtype=torch.uint8, device="cuda")
    cu = torch.zeros(1, dtype=torch.int32, device="cuda")
    empty = torch.empty(0, w.H, w.dk, device="cuda")
    K.kda_prefill_varlen(d, cu, empty, empty, torch.empty(0, w.H, w.dv, device="cuda"), empty,
                         torch.empty(0, w.H, device="cuda"), state, o, ws)
    torch.cuda.synchronize()
    assert torch.count_nonzero(state) == 0


@pytest.mark.parametrize("precision", [K.PREC_BF16X3, K.PREC_FP16])
@pytest.mark.parametrize("fused", [False, True])
def test_prefill_beta_zero_and_unit_decay_freezes_the_state(precision, fused):
    """beta logits of -100 (beta = 0) and softplus raw gates of -100 (a = 1 to fp32): the state stays S0
    and o_t = S0^T q_t; the A and P products see nothing but zero keys' weights."""
    w = _small((150, 64, 9), seed=7)
    w.beta.fill_(-100.0)
    w.g.fill_(-100.0)
    print(f"frozen state precision={precision} fused={fused}", flush=True)
    r = gpu_layer_prefill(w, precision=precision, fused=fused)
    ref = oracle_layer(w)
    assert np.allclose(ref.state, w.state0.double().numpy(), rtol=0, atol=1e-12)  # the oracle agrees it froze
    assert rel(r["state"], ref.state) < 1e-6
    assert rel(r["o"], ref.o) < TOL_BF16


def test_decode_beta_zero_only_decays():
    w = I.generate("edge_decode", lengths=[4] * 8, H=4, dk=128, dv=128, dtype=torch.bfloat16,
                   gate_mode=I.GATE_SAFE, state_std=0.02, conv_state_std=1.0, seed=8)
    w.beta.fill_(-100.0)
    dec = gpu_decode_steps(w, 4)
    ref = oracle_layer(w)
    assert rel(dec["state"], ref.state) < 1e-6
    o = dec["o"].transpose(0, 1).reshape(w.T, w.H, w.dv)
    assert rel(o, ref.o) < TOL_BF16


def test_long_sequence_next_to_a_short_one():
    """512 chunks of one sequence packed with a 3-row one (H=2, d=128): oracle parity, and the long one
    cut at row 16384 with the state and conv state carried gives the same bits."""
    n_long = 32768
    w = _small((n_long, 3), H=2, seed=9, gate=I.GATE_SAFE)
    print(f"long prompt T={w.T}", flush=True)
    r = gpu_layer_prefill(w, precision=K.PREC_FP16, fused=True)
    ref = oracle_layer(w)
    assert rel(r["o"], ref.o) < TOL_BF16 and rel(r["state"], ref.state) < TOL_BF16
    cut = 16384
    sl = slice(0, cut)
    a = I.Workload("a", w.H, w.dk, w.dv, torch.tensor([0, cut], dtype=torch.int32), w.q[sl], w.k[sl], w.v[sl],
                   w.g[sl], w.beta[sl], w.z[sl], w.conv_w, w.norm_w, w.state0[:1], w.conv_state0[:1], w.gate_mode,
                   w.lower_bound)
    ra = gpu_layer_prefill(a, precision=K.PREC_FP16, fused=True)
    sl = slice(cut, n_long)
    b = I.Workload("b", w.H, w.dk, w.dv, torch.tensor([0, n_long - cut], dtype=torch.int32), w.q[sl], w.k[sl],
                   w.v[sl], w.g[sl], w.beta[sl], w.z[sl], w.conv_w, w.norm_w, ra["state"].cpu(),
                   ra["prep"]["conv_state"].cpu(), w.gate_mode, w.lower_bound)
    rb = gpu_layer_prefill(b, precision=K.PREC_FP16, fused=True)
    assert torch.equal(torch.cat([ra["o"], rb["o"]]), r["o"][:n_long])
    assert torch.equal(rb["state"][0], r["state"][0])


def test_decode_batch_beyond_one_grid_row():
    """A decode batch larger than a grid's y extent (65535): sampled sequences on both sides of the
    boundary, decoded again alone through a slot map, give the same bits (o, state, conv state)."""
    B, H, d = 65540, 1, 64
    dm = K.Dims(H, d, d, torch.bfloat16)
    g = torch.Generator(device="cuda").manual_seed(9)
    rn = lambda *s: torch.randn(*s, generator=g, device="cuda")
    state0 = rn(B, H, d, d) * 0.02
    cs0 = rn(B, 3, dm.conv_channels).to(torch.bfloat16)
    cw = rn(dm.conv_channels, 4) * 0.5
    rows = [rn(B, H, d).to(torch.bfloat16) for _ in range(4)]
    beta = rn(B, H).to(torch.bfloat16)
    st, cs = state0.clone(), cs0.clone()
    o = torch.empty(B, H, d, device="cuda")
    K.kda_decode(dm, st, cs, cw, *rows, beta, I.GATE_SAFE, -5.0, o)
    idx = torch.tensor([0, 65534, 65535, 65539], device="cuda")
    st2, cs2 = state0.clone(), cs0.clone()
    o2 = torch.empty(4, H, d, device="cuda")
    K.kda_decode(dm, st2, cs2, cw, *[r[idx].contiguous() for r in rows], beta[idx].contiguous(), I.GATE_SAFE,
                 -5.0, o2, slots=idx.to(torch.int32))
    torch.cuda.synchronize()
    assert torch.equal(o[idx], o2)
    assert torch.equal(st[idx], st2[idx])
    assert torch.equal(cs[idx], cs2[idx])
    assert not torch.equal(st[65539], state0[65539])  # the last sequence was decoded


def test_prep_sequences_beyond_one_grid_row():
    """kda_prep over more sequences than a grid's y extent (65535): the conv-state carry of the last
    sequences (past the boundary) is the bit copy of their raw rows the oracle gives, and every
    preamble output matches the oracle."""
    from oracle import oracle as O
    N, H, d = 65540, 1, 64
    lens = [2 if n % 3 else 5 for n in range(N)]  # sequences shorter and longer than the 3 carried rows
    w = I.generate("many_seqs", lengths=lens, H=H, dk=d, dv=d, dtype=torch.bfloat16, gate_mode=I.GATE_SAFE,
                   conv_state_std=1.0, seed=13)
    print(f"prep over N={w.N} sequences, T={w.T}", flush=True)
    dm = K.Dims(H, d, d, torch.bfloat16)
    wd = w.to("cuda")
    T = w.T
    f = lambda *s: torch.empty(*s, device="cuda")
    out = dict(q_hat=f(T, H, d), k_hat=f(T, H, d), v=f(T, H, d), g=f(T, H, d), beta=f(T, H))
    cs = torch.empty_like(wd.conv_state0)
    K.kda_prep(dm, wd.cu_seqlens, wd.q, wd.k, wd.v, wd.conv_w, wd.conv_state0, cs, wd.g, wd.beta, w.gate_mode,
               w.lower_bound, out["q_hat"], out["k_hat"], out["v"], out["g"], out["beta"])
    torch.cuda.synchronize()
    ref = O.prep(w.f64("q"), w.f64("k"), w.f64("v"), w.f64("conv_w"), w.f64("conv_state0"), w.f64("g"),
                 w.f64("beta"), w.cu_seqlens.numpy(), gate_mode=w.gate_mode, lower_bound=w.lower_bound)
    assert np.array_equal(cs.cpu().double().numpy(), ref.conv_state)
    for name, r in (("q_hat", ref.q_hat), ("k_hat", ref.k_hat), ("v", ref.v), ("g", ref.g), ("beta", ref.beta)):
        assert rel(out[name], r) < 2e-6, name
