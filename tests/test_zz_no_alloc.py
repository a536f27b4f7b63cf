"""The allocation-free prompt call (kda_prefill_varlen_noalloc): the same kernels as kda_prefill_varlen with
the chunk records in the library's per-device scratch instead of a caller workspace.  Two calls in a row, the
second on a smaller input, each checked bit for bit against kda_prefill_varlen with a workspace on the same
inputs (o, final state, carried conv state, y), and against the fp64 oracle; a geometry beyond the scratch is
refused before any launch, with nothing written."""
import numpy as np
import pytest
import torch

import kimi_delta_attention_prep_amd as K
from kimi_delta_attention_prep_amd import inputs as I

from helpers import EPS, TOL_BF16, dims_for, oracle_layer, raw_rows, rel

pytestmark = pytest.mark.gpu


def _pass(w, precision, noalloc):
    d = dims_for(w, precision)
    wd = w.to("cuda")
    state, cs = wd.state0.clone(), torch.empty_like(wd.conv_state0)
    o = torch.full((w.T, w.H, w.dv), float("nan"), device="cuda")
    y = torch.full((w.T, w.H, w.dv), float("nan"), device="cuda", dtype=torch.bfloat16)
    args = (d, wd.cu_seqlens, None, None, None, None, None, state, o)
    kw = dict(raw=raw_rows(wd, cs), norm=dict(z=wd.z, weight=wd.norm_w, eps=EPS, y=y))
    if noalloc:
        K.kda_prefill_varlen_noalloc(*args, **kw)
    else:
        ws = torch.empty(K.kda_prefill_workspace_bytes(d, w.N, w.T), dtype=torch.uint8, device="cuda")
        K.kda_prefill_varlen(*args, ws, **kw)
    torch.cuda.synchronize()
    return {"o": o, "state": state, "conv_state": cs, "y": y}


@pytest.mark.parametrize("precision", [K.PREC_FP16, K.PREC_BF16X2, K.PREC_BF16X3])
def test_noalloc_prompt_call_twice_then_smaller(precision):
    assert torch.cuda.is_available()
    K.load_library()
    big = I.prefill()  # T=4096, H=16: the largest records the scratch holds at this policy
    small = I.generate("noalloc_small", lengths=[150, 3, 0, 64, 70], H=2, dk=128, dv=128, dtype=torch.bfloat16,
                       gate_mode=I.GATE_SOFTPLUS, state_std=0.02, conv_state_std=1.0, seed=131)
    for w in (big, small):
        print(f"no-alloc prompt call T={w.T} H={w.H} precision={precision}", flush=True)
        a = _pass(w, precision, noalloc=True)
        b = _pass(w, precision, noalloc=False)
        for n in a:
            assert torch.equal(a[n], b[n]), n
    ref = oracle_layer(small)
    assert rel(a["o"], ref.o) < TOL_BF16 and rel(a["state"], ref.state) < TOL_BF16
    assert np.array_equal(a["conv_state"].cpu().double().numpy(), ref.prep.conv_state)


def test_noalloc_refuses_records_beyond_its_scratch():
    K.load_library()
    w = I.generate("noalloc_big", lengths=[40000], H=8, dk=128, dv=128, dtype=torch.bfloat16,
                   gate_mode=I.GATE_SAFE, seed=132, device="cuda")
    d = dims_for(w, K.PREC_FP16)
    assert K.kda_prefill_workspace_bytes(d, w.N, w.T) > K.NOALLOC_SCRATCH_BYTES
    state = w.state0.clone()
    o = torch.full((w.T, w.H, w.dv), 3.0, device="cuda")
    with pytest.raises(K.KdaError) as e:
        K.kda_prefill_varlen_noalloc(d, w.cu_seqlens.cuda(), None, None, None, None, None, state, o,
                                     raw=raw_rows(w, torch.empty_like(w.conv_state0)))
    assert e.value.code == K.KDA_E_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(o == 3.0) and torch.equal(state, w.state0)
