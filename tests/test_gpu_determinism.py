"""Repeat runs of the prompt pass give the same bits.

Every reduction on the HIP path has a fixed order, so a difference between two
runs on the same inputs can only come from a race: a workgroup reading LDS or a
record that another wavefront or kernel has not finished writing.  Such a race
shows up rarely and only as a small perturbation (often within the parity
tolerance), so it is hunted here at the full prompt size, where one run holds
about a thousand chunk workgroups, with device memory refilled between runs."""
import pytest
import torch

import kimi_delta_attention_prep_amd as K
from kimi_delta_attention_prep_amd import inputs as I

from helpers import dims_for, gpu_prep, raw_rows

pytestmark = pytest.mark.gpu

REPS = 12


def _poison(kind):
    x = torch.empty(64 << 20, dtype=torch.float32, device="cuda")
    x.fill_(float("nan") if kind == 0 else 1e30)
    del x


@pytest.mark.parametrize("precision", [K.PREC_FP16, K.PREC_BF16X2, K.PREC_BF16X3])
@pytest.mark.parametrize("fused", [False, True])
def test_prompt_pass_repeats_bitwise(precision, fused):
    lens = [1500, 64, 1, 2531]  # 4096 rows, ragged chunk tails
    w = I.generate("repeat", lengths=lens, H=16, dk=128, dv=128, dtype=torch.bfloat16, gate_mode=I.GATE_SAFE,
                   state_std=0.02, conv_state_std=1.0, seed=31)
    d = dims_for(w, precision)
    print(f"repeat runs precision={precision} fused={fused} T={w.T} H={w.H}", flush=True)
    if fused:
        wd, p = w.to("cuda"), None
    else:
        wd, p = gpu_prep(w, d)
    ws = torch.empty(K.kda_prefill_workspace_bytes(d, w.N, w.T), dtype=torch.uint8, device="cuda")
    first = None
    for rep in range(REPS):
        _poison(rep % 2)
        state = wd.state0.clone()
        o = torch.empty(w.T, w.H, w.dv, device="cuda")
        ws.fill_(0xA5)
        if fused:
            cs = torch.empty_like(wd.conv_state0)
            K.kda_prefill_varlen(d, wd.cu_seqlens, None, None, None, None, None, state, o, ws,
                                 raw=raw_rows(wd, cs))
        else:
            cs = None
            K.kda_prefill_varlen(d, wd.cu_seqlens, p["q_hat"], p["k_hat"], p["v"], p["g"], p["beta"], state, o, ws)
        torch.cuda.synchronize()
        if first is None:
            first = (o, state, cs)
            continue
        assert torch.equal(o, first[0]), f"o differs on repeat {rep}"
        assert torch.equal(state, first[1]), f"state differs on repeat {rep}"
        if fused:
            assert torch.equal(cs, first[2]), f"conv state differs on repeat {rep}"
