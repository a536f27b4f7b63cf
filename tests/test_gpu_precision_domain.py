"""Numeric range of the prompt path's precision policies.

FP16 rounds the per-chunk operands (every entry bounded by 1) once to fp16 and splits each state and
update entry x into fp16 hi + lo.  While |x| < 65504 (the largest finite fp16 value) the pair keeps x to
within max(2^-22 |x|, 2^-25); beyond it the split overflows, and the call's outputs are then not finite
(the failure is loud, never a finite wrong value).  BF16X2, BF16X3 and FP32 keep the fp32 range.  The layer is
linear in (S0, v) only up to the conv activation, so the tests scale S0 directly and scale v's raw rows
by powers of two (exact in bf16)."""
import pytest
import torch

import kimi_delta_attention_prep_amd as K
from kimi_delta_attention_prep_amd import inputs as I

from helpers import TOL_BF16, gpu_layer_prefill, oracle_layer, rel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    K.load_library()


def _workload(state_std, v_scale=1.0):
    w = I.generate("domain", lengths=[200, 70], H=2, dk=128, dv=128, dtype=torch.bfloat16, gate_mode=I.GATE_SAFE,
                   state_std=state_std, conv_state_std=1.0, seed=123)
    if v_scale != 1.0:
        w.v.mul_(v_scale)
    return w


def _errs(w, precision):
    r = gpu_layer_prefill(w, precision=precision)
    ref = oracle_layer(w)
    return r, {"o": rel(r["o"], ref.o), "state": rel(r["state"], ref.state)}


@pytest.mark.parametrize("precision", [K.PREC_FP16, K.PREC_BF16X2, K.PREC_BF16X3, K.PREC_FP32])
@pytest.mark.parametrize("state_std,v_scale", [(300.0, 1.0), (0.0, 2.0 ** -8)])
def test_state_magnitudes_inside_the_fp16_range(precision, state_std, v_scale):
    """Entries far from unit magnitude but inside FP16's range: S0 ~ N(0, 300^2) (state and update
    entries up to about 10^4), and v rows scaled by 2^-8 from a zero state (entries about 10^-3)."""
    r, errs = _errs(_workload(state_std, v_scale), precision)
    print(f"precision {precision} S0 std {state_std} v scale {v_scale}: {errs}", flush=True)
    assert all(e < TOL_BF16 for e in errs.values()), errs


@pytest.mark.parametrize("precision", [K.PREC_BF16X2, K.PREC_BF16X3, K.PREC_FP32])
def test_state_beyond_the_fp16_range_under_fp32_range_policies(precision):
    r, errs = _errs(_workload(1e6), precision)
    print(f"precision {precision} S0 std 1e6: {errs}", flush=True)
    assert all(e < TOL_BF16 for e in errs.values()), errs


def test_fp16_beyond_its_range_gives_non_finite_outputs():
    """S0 ~ N(0, 10^12): state entries past 65504 overflow FP16's split, and the outputs show it."""
    r, _ = _errs(_workload(1e6), K.PREC_FP16)
    assert not torch.isfinite(r["o"]).all()
    assert not torch.isfinite(r["state"]).all()
