"""Host-side guards of the binding on the GPU: the pool-size check that always
runs, and debug mode, which reads cu_seqlens, slot maps and commit counts back
and refuses bad contents before anything is launched."""
import pytest
import torch

import kimi_delta_attention_prep_amd as K
from kimi_delta_attention_prep_amd import inputs as I

from helpers import dims_for, raw_rows

pytestmark = pytest.mark.gpu


@pytest.fixture()
def debug_on():
    K.set_debug(True)
    yield
    K.set_debug(False)


def _prompt(w, cu=None, slots=None, state=None):
    d = dims_for(w)
    wd = w.to("cuda")
    st = wd.state0.clone() if state is None else state
    o = torch.empty(w.T, w.H, w.dv, device="cuda")
    ws = torch.empty(K.kda_prefill_workspace_bytes(d, w.N, w.T), dtype=torch.uint8, device="cuda")
    cs = torch.empty_like(wd.conv_state0)
    K.kda_prefill_varlen(d, wd.cu_seqlens if cu is None else cu, None, None, None, None, None, st, o, ws,
                         slots=slots, raw=raw_rows(wd, cs))
    return o


def test_debug_mode_refuses_bad_contents_and_passes_good_ones(debug_on):
    w = I.generate("dbg", lengths=[70, 5, 130], H=2, dk=64, dv=64, dtype=torch.bfloat16, gate_mode=I.GATE_SAFE,
                   state_std=0.02, conv_state_std=1.0, seed=5)
    o = _prompt(w)  # valid contents pass
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    bad_cu = torch.tensor([0, 80, 75, w.T], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="decreases"):
        _prompt(w, cu=bad_cu)
    with pytest.raises(ValueError, match="same slot"):
        _prompt(w, slots=torch.tensor([0, 2, 0], dtype=torch.int32, device="cuda"))
    with pytest.raises(ValueError, match="outside"):
        _prompt(w, slots=torch.tensor([0, 1, 3], dtype=torch.int32, device="cuda"))


def test_pool_smaller_than_batch_is_refused_without_slot_map():
    w = I.generate("dbg2", lengths=[10, 10, 10], H=2, dk=64, dv=64, dtype=torch.bfloat16, gate_mode=I.GATE_SAFE,
                   state_std=0.02, conv_state_std=1.0, seed=6)
    small = torch.zeros(2, w.H, w.dk, w.dv, device="cuda")
    with pytest.raises(ValueError, match="no slot map"):
        _prompt(w, state=small)
