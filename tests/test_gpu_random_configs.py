"""Seeded random configurations against the oracle: key and value head dims, head count, sequence count and
lengths (empty sequences included), input dtype, gate mode and lower bound, initial state and conv state,
precision policy and fused or separate preamble for the prompt call; batch, heads and steps for decode.
Each draw is small enough for the fp64 oracle to finish in about a second, and the draws are fixed by their
seeds, so a failure names a reproducible configuration."""
import numpy as np
import pytest
import torch

import kimi_delta_attention_prep_amd as K
from kimi_delta_attention_prep_amd import inputs as I

from helpers import TOL_BF16, TOL_FP32, gpu_decode_steps, gpu_layer_prefill, oracle_layer, rel

pytestmark = pytest.mark.gpu

POLICIES = (None, K.PREC_FP32, K.PREC_BF16X3, K.PREC_FP16, K.PREC_BF16X2)


def _draw(case):
    rng = np.random.default_rng(7000 + case)
    dk, dv = (int(x) for x in rng.choice([64, 128], 2))
    H = int(rng.integers(1, 7))
    N = int(rng.integers(1, 13))
    lens = rng.integers(0, 260, N)
    lens[rng.random(N) < 0.15] = 0
    dtype = torch.float32 if rng.random() < 0.3 else torch.bfloat16
    gate = I.GATE_SAFE if rng.random() < 0.5 else I.GATE_SOFTPLUS
    lb = float(rng.choice([-5.0, -1.0, -0.25]))
    precision = POLICIES[int(rng.integers(0, len(POLICIES)))]
    fused = bool(rng.random() < 0.5)
    state_std = float(rng.choice([0.0, 0.02]))
    conv_std = float(rng.choice([0.0, 1.0]))
    w = I.generate(f"random{case}", lengths=lens.tolist(), H=H, dk=dk, dv=dv, dtype=dtype, gate_mode=gate,
                   lower_bound=lb, state_std=state_std, conv_state_std=conv_std, seed=case)
    return w, precision, fused


@pytest.mark.parametrize("case", range(24))
def test_random_prompt_config(case):
    w, precision, fused = _draw(case)
    lens = (w.cu_seqlens[1:] - w.cu_seqlens[:-1]).tolist()
    print(f"case {case}: N={w.N} lengths={lens} H={w.H} dk={w.dk} dv={w.dv} dtype={w.dtype} gate={w.gate_mode} "
          f"lb={w.lower_bound} precision={precision} fused={fused}", flush=True)
    r = gpu_layer_prefill(w, precision=precision, fused=fused)
    ref = oracle_layer(w)
    all_fp32 = w.dtype == torch.float32 and precision in (None, K.PREC_FP32)
    tol = TOL_FP32 if all_fp32 else TOL_BF16
    errs = {"o": rel(r["o"], ref.o), "y": rel(r["y"], ref.y)}
    st = r["state"].cpu().double().numpy()
    errs["state"] = max(rel(st[n], ref.state[n]) for n in range(w.N))
    print(f"case {case}: {errs} (tolerance {tol})", flush=True)
    assert all(e < tol for e in errs.values()), errs
    assert np.array_equal(r["prep"]["conv_state"].cpu().double().numpy(), ref.prep.conv_state)


@pytest.mark.parametrize("case", range(8))
def test_random_decode_config(case):
    rng = np.random.default_rng(9000 + case)
    d = int(rng.choice([64, 128]))
    B, H, steps = int(rng.integers(1, 40)), int(rng.integers(1, 9)), int(rng.integers(1, 12))
    dtype = torch.float32 if rng.random() < 0.3 else torch.bfloat16
    gate = I.GATE_SAFE if rng.random() < 0.5 else I.GATE_SOFTPLUS
    lb = float(rng.choice([-5.0, -1.0, -0.25]))
    w = I.generate(f"rdec{case}", lengths=[steps] * B, H=H, dk=d, dv=d, dtype=dtype, gate_mode=gate, lower_bound=lb,
                   state_std=0.02, conv_state_std=1.0, seed=100 + case)
    print(f"decode case {case}: B={B} H={H} d={d} steps={steps} dtype={dtype} gate={gate} lb={lb}", flush=True)
    r = gpu_decode_steps(w, steps)
    ref = oracle_layer(w)
    tol = TOL_FP32 if dtype == torch.float32 else TOL_BF16
    o = r["o"].transpose(0, 1).reshape(w.T, w.H, w.dv)  # [steps, B, ...] -> packed rows
    y = r["y"].transpose(0, 1).reshape(w.T, w.H, w.dv)
    errs = {"o": rel(o, ref.o), "y": rel(y, ref.y), "state": rel(r["state"], ref.state)}
    print(f"decode case {case}: {errs} (tolerance {tol})", flush=True)
    assert all(e < tol for e in errs.values()), errs
    assert np.array_equal(r["conv_state"].cpu().double().numpy(), ref.prep.conv_state)
