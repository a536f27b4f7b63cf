"""Verify windows case by case over batch, head count, negative slot and gate (sglang PR #33561,
"实现拆解" key-file list: the fused conv + recurrent verify test compares the fused path with an
unfused reference over batch, heads, negative slots and the gate's lower bound).

Each case runs three kda_verify_window calls on a permuted state / conv-state pool in which some
sequences have a negative slot: a first window; the commit of its accepted rows together with the
next window, in one call; and a commit-only call for the second window.  The results are checked

  - bit for bit against serial kda_decode of the same rows on a copy of the pools (outputs of every
    window row, the committed state and conv state), with skipped sequences' outputs and every pool
    row no sequence maps to left untouched;
  - against the fp64 oracle: window outputs, the logged decay, normalised key and update, the
    committed state, and the carried conv state (bit for bit).
"""
import numpy as np
import pytest
import torch

import kimi_delta_attention_prep_amd as K
from kimi_delta_attention_prep_amd import inputs as I

from helpers import TOL_BF16, dims_for, oracle_pieces, rel

pytestmark = pytest.mark.gpu

W = 4  # draft rows per window
GATES = [(I.GATE_SAFE, -5.0), (I.GATE_SAFE, -1.0), (I.GATE_SAFE, -0.25), (I.GATE_SOFTPLUS, -5.0)]
SHAPES = [(1, 2), (5, 2), (64, 2), (1, 32), (5, 32), (64, 32)]  # (batch, heads)
ROWS = ("q", "k", "v", "g", "beta")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    K.load_library()


def _decode(d, w, rows, pool, cpool, slots, active):
    """Serial kda_decode of the W rows of a window; sequence b takes row s only if it has a slot and
    active(b, s).  Returns o [B, W, H, dv] (NaN where a sequence did not take the row)."""
    B = len(slots)
    outs = []
    for s in range(W):
        sl = torch.tensor([slots[b] if slots[b] >= 0 and active(b, s) else -1 for b in range(B)], dtype=torch.int32,
                          device="cuda")
        o = torch.full((B, w.H, w.dv), float("nan"), device="cuda")
        K.kda_decode(d, pool, cpool, w.conv_w.cuda(), *(rows[n][:, s].contiguous() for n in ROWS), w.gate_mode,
                     w.lower_bound, o, slots=sl)
        outs.append(o)
    return torch.stack(outs, 1)


def _last_rows(x, lens, n):
    """The last n rows of every piece of a packed [sum(lens), ...] array."""
    ends = np.cumsum(lens)
    return np.concatenate([x[e - n:e] for e in ends])


@pytest.mark.parametrize("gate,lb", GATES)
@pytest.mark.parametrize("B,H", SHAPES)
def test_verify_windows_on_a_slot_pool(B, H, gate, lb):
    seed = 1000 + 7 * B + H + int(-4 * lb) + 50 * gate
    print(f"verify case B={B} H={H} gate={gate} lb={lb} seed={seed}", flush=True)
    w = I.generate("verify_case", lengths=[2 * W] * B, H=H, dk=128, dv=128, dtype=torch.bfloat16, gate_mode=gate,
                   lower_bound=lb, state_std=0.02, conv_state_std=1.0, seed=seed)
    d = dims_for(w)
    C = w.C
    gen = torch.Generator().manual_seed(seed + 1)
    S = B + 3  # pool slots; three of them belong to no sequence
    perm = torch.randperm(S, generator=gen)[:B].tolist()
    skip = (torch.rand(B, generator=gen) < 0.2).tolist()
    if B > 1 and not any(skip):
        skip[B // 2] = True
    if B == 1:
        skip = [False]
    slots = [-1 if skip[b] else perm[b] for b in range(B)]
    live = [b for b in range(B) if slots[b] >= 0]
    j1 = torch.randint(0, W, (B,), generator=gen, dtype=torch.int32)  # rows 0..j kept
    j2 = torch.randint(0, W, (B,), generator=gen, dtype=torch.int32)
    pool0 = torch.randn(S, H, 128, 128, generator=gen) * 0.02
    cpool0 = torch.randn(S, 3, C, generator=gen).to(torch.bfloat16)
    for b in live:
        pool0[slots[b]] = w.state0[b]
        cpool0[slots[b]] = w.conv_state0[b]
    rows = {n: getattr(w, n).view(B, 2 * W, *getattr(w, n).shape[1:]).cuda() for n in ROWS}
    first = {n: r[:, :W].contiguous() for n, r in rows.items()}
    second = {n: r[:, W:].contiguous() for n, r in rows.items()}
    cw = w.conv_w.cuda()
    slots_t = torch.tensor(slots, dtype=torch.int32, device="cuda")

    pool, cpool = pool0.cuda(), cpool0.cuda()
    log1, log2 = K.VerifyLog.empty(d, B, W), K.VerifyLog.empty(d, B, W)
    o1 = torch.full((B, W, H, 128), float("nan"), device="cuda")
    o2 = torch.full_like(o1, float("nan"))
    K.kda_verify_window(d, pool, cpool, cw, None, None, log1, *(first[n] for n in ROWS), gate, lb, o1, slots=slots_t)
    K.kda_verify_window(d, pool, cpool, cw, (j1 + 1).cuda(), log1, log2, *(second[n] for n in ROWS), gate, lb, o2,
                        slots=slots_t)
    K.kda_verify_window(d, pool, cpool, cw, (j2 + 1).cuda(), log2, None, None, None, None, None, None, gate, lb, None,
                        slots=slots_t, batch=B)

    # serial decode: every window row on a copy (its outputs), then the kept rows on the pools
    ps, cs = pool0.cuda(), cpool0.cuda()
    o1s = _decode(d, w, first, ps.clone(), cs.clone(), slots, lambda b, s: True)
    _decode(d, w, first, ps, cs, slots, lambda b, s: s <= int(j1[b]))
    o2s = _decode(d, w, second, ps.clone(), cs.clone(), slots, lambda b, s: True)
    _decode(d, w, second, ps, cs, slots, lambda b, s: s <= int(j2[b]))
    torch.cuda.synchronize()
    assert torch.equal(pool, ps), "committed state differs from serial decode"
    assert torch.equal(cpool, cs), "committed conv state differs from serial decode"
    for b in range(B):
        if slots[b] >= 0:
            assert torch.equal(o1[b], o1s[b]) and torch.equal(o2[b], o2s[b]), f"sequence {b}: window outputs"
        else:
            assert torch.isnan(o1[b]).all() and torch.isnan(o2[b]).all(), f"skipped sequence {b} was written"
    for s_ in set(range(S)) - {slots[b] for b in live}:
        assert torch.equal(pool[s_].cpu(), pool0[s_]) and torch.equal(cpool[s_].cpu(), cpool0[s_]), f"slot {s_}"

    # the fp64 oracle over the live sequences
    base = [b * 2 * W for b in live]
    lv = torch.tensor(live)
    r1 = oracle_pieces(w, [range(s0, s0 + W) for s0 in base], seqs=live, with_log=True)
    assert rel(o1[lv].reshape(-1, H, 128), r1.o) < TOL_BF16
    assert rel(log1.a[lv].reshape(-1, H, 128), r1.log_a) < 1e-6
    assert rel(log1.k_hat[lv].reshape(-1, H, 128), r1.log_k) < 1e-5
    assert rel(log1.u[lv].reshape(-1, H, 128), r1.log_u) < TOL_BF16
    p2 = [list(range(s0, s0 + int(j1[b]) + 1)) + list(range(s0 + W, s0 + 2 * W)) for b, s0 in zip(live, base)]
    r2 = oracle_pieces(w, p2, seqs=live, with_log=True)
    lens2 = [len(p) for p in p2]
    assert rel(o2[lv].reshape(-1, H, 128), _last_rows(r2.o, lens2, W)) < TOL_BF16
    assert rel(log2.a[lv].reshape(-1, H, 128), _last_rows(r2.log_a, lens2, W)) < 1e-6
    assert rel(log2.k_hat[lv].reshape(-1, H, 128), _last_rows(r2.log_k, lens2, W)) < 1e-5
    assert rel(log2.u[lv].reshape(-1, H, 128), _last_rows(r2.log_u, lens2, W)) < TOL_BF16
    p3 = [list(range(s0, s0 + int(j1[b]) + 1)) + list(range(s0 + W, s0 + W + int(j2[b]) + 1))
          for b, s0 in zip(live, base)]
    r3 = oracle_pieces(w, p3, seqs=live)
    sl = torch.tensor([slots[b] for b in live])
    err = rel(pool[sl.cuda()], r3.state)
    print(f"committed state rel-L2 {err:.2e}", flush=True)
    assert err < TOL_BF16
    assert np.array_equal(cpool[sl.cuda()].cpu().double().numpy(), r3.prep.conv_state)
