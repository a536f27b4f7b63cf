"""GPU parity of every entry point against the fp64 oracle (small and ragged
shapes), plus the bit-exact invariants: carried conv state bytes, packed vs
alone, prompt cut at a chunk multiple, and verify-window replay vs serial
decode.  Everything goes through the C ABI."""
import numpy as np
import pytest
import torch

import kimi_delta_attention_prep_amd as K
from kimi_delta_attention_prep_amd import inputs as I
from oracle import oracle as O

from helpers import (EPS, TOL_BF16, TOL_FP32, dims_for, gpu_decode_steps, gpu_layer_prefill, gpu_prep, raw_rows,
                     oracle_layer, oracle_pieces, rel, tol_for)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    K.load_library()  # must exist: no fallback


def small(dtype=torch.bfloat16, lens=(70, 5, 0, 130), H=2, d=128, gate=I.GATE_SAFE, seed=3, dv=None):
    return I.generate("small", lengths=list(lens), H=H, dk=d, dv=dv or d, dtype=dtype, gate_mode=gate,
                      state_std=0.02, conv_state_std=1.0, seed=seed)


# ---------------------------------------------------------------------------
# output norm and preamble
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dv", [64, 128])
@pytest.mark.parametrize("zdt,ydt", [(torch.float32, torch.float32), (torch.bfloat16, torch.float32),
                                     (torch.bfloat16, torch.bfloat16)])
def test_gated_rmsnorm(dv, zdt, ydt):
    g = torch.Generator().manual_seed(1)
    rows = 1037
    o = torch.randn(rows, dv, generator=g)
    z = torch.randn(rows, dv, generator=g).to(zdt)
    w = torch.rand(dv, generator=g) + 0.5
    y = torch.empty(rows, dv, dtype=ydt, device="cuda")
    K.gated_rmsnorm_out(o.cuda(), z.cuda(), w.cuda(), EPS, y)
    ref = O.gated_rmsnorm(o.double().numpy(), z.double().numpy(), w.double().numpy(), EPS)
    # a bf16 y carries its own rounding, at most 2^-9 of each value (round to nearest even with 8
    # significant bits), so its relative L2 error is at most 2^-9 plus that of the fp32 arithmetic
    assert rel(y, ref) < (2.0 ** -9 + 2e-6 if ydt == torch.bfloat16 else 2e-6)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (64, 128)])
@pytest.mark.parametrize("gate", [I.GATE_SAFE, I.GATE_SOFTPLUS])
def test_prep_parity_and_conv_state_bytes(dtype, dk, dv, gate):
    w = small(dtype, d=dk, dv=dv, gate=gate)
    _, p = gpu_prep(w, dims_for(w))
    ref = O.prep(w.f64("q"), w.f64("k"), w.f64("v"), w.f64("conv_w"), w.f64("conv_state0"), w.f64("g"),
                 w.f64("beta"), w.cu_seqlens.numpy(), gate_mode=w.gate_mode, lower_bound=w.lower_bound)
    for name, r in (("q_hat", ref.q_hat), ("k_hat", ref.k_hat), ("v", ref.v), ("g", ref.g), ("beta", ref.beta)):
        assert rel(p[name], r) < 2e-6, name
    # the carried conv state is a bit copy of raw rows
    assert np.array_equal(p["conv_state"].cpu().double().numpy(), ref.conv_state)


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_prep_tile_edges_with_slots(dtype, d):
    """The preamble's 64-row tiles at their edges: sequences shorter than the
    three conv rows, tiles ending one row before, at and after 64, an empty
    sequence, and a slot map that permutes the conv-state pool and skips one
    sequence (whose rows and pool row stay untouched)."""
    lens = [1, 2, 3, 63, 64, 65, 0, 67, 129, 4]
    w = I.generate("prep_edges", lengths=lens, H=3, dk=d, dv=d, dtype=dtype, gate_mode=I.GATE_SAFE,
                   state_std=0.02, conv_state_std=1.0, seed=11)
    N, T, H = w.N, w.T, w.H
    slots = [5, 0, 9, 2, 7, 1, 3, -1, 8, 4]  # sequence 7 (67 rows) is skipped
    S = 10
    dm = dims_for(w)
    wd = w.to("cuda")
    pool = torch.randn(S, 3, dm.conv_channels, generator=torch.Generator().manual_seed(2)).to(dtype).cuda()
    for n, s_ in enumerate(slots):
        if s_ >= 0:
            pool[s_] = wd.conv_state0[n]
    pool_in = pool.clone()
    nan = lambda *sh: torch.full(sh, float("nan"), device="cuda")
    out = dict(q_hat=nan(T, H, d), k_hat=nan(T, H, d), v=nan(T, H, d), g=nan(T, H, d), beta=nan(T, H))
    K.kda_prep(dm, wd.cu_seqlens, wd.q, wd.k, wd.v, wd.conv_w, pool, pool, wd.g, wd.beta, w.gate_mode, w.lower_bound,
               out["q_hat"], out["k_hat"], out["v"], out["g"], out["beta"],
               slots=torch.tensor(slots, dtype=torch.int32, device="cuda"))
    ref = O.prep(w.f64("q"), w.f64("k"), w.f64("v"), w.f64("conv_w"), w.f64("conv_state0"), w.f64("g"),
                 w.f64("beta"), w.cu_seqlens.numpy(), gate_mode=w.gate_mode, lower_bound=w.lower_bound)
    cu = w.cu_seqlens.tolist()
    live = np.ones(T, dtype=bool)
    live[cu[7]:cu[8]] = False
    for name, r in (("q_hat", ref.q_hat), ("k_hat", ref.k_hat), ("v", ref.v), ("g", ref.g), ("beta", ref.beta)):
        got = out[name].cpu()
        assert torch.isnan(got[~torch.from_numpy(live)]).all(), name  # the skipped sequence's rows untouched
        assert rel(got[torch.from_numpy(live)], r[live]) < 2e-6, name
    for n, s_ in enumerate(slots):
        if s_ >= 0:  # the carried conv state is a bit copy of raw rows, in the sequence's pool row
            assert np.array_equal(pool[s_].cpu().double().numpy(), ref.conv_state[n]), n
    assert torch.equal(pool[6], pool_in[6])  # a pool row no sequence maps to


# ---------------------------------------------------------------------------
# decode and verify windows
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64), (torch.bfloat16, 64)])
def test_decode_parity(dtype, d):
    steps = 9
    w = I.generate("dec", lengths=[steps] * 6, H=3, dk=d, dv=d, dtype=dtype, gate_mode=I.GATE_SAFE,
                   state_std=0.02, conv_state_std=1.0, seed=5)
    r = gpu_decode_steps(w, steps)
    ref = oracle_layer(w)
    o = r["o"].transpose(0, 1).reshape(w.T, w.H, w.dv)  # [steps,B,..] -> packed rows
    y = r["y"].transpose(0, 1).reshape(w.T, w.H, w.dv)
    tol = tol_for(w)
    assert rel(o, ref.o) < tol
    assert rel(y, ref.y) < tol
    assert rel(r["state"], ref.state) < tol
    assert np.array_equal(r["conv_state"].cpu().double().numpy(), ref.prep.conv_state)


def _verify_setup(B=5, W=4, H=2, d=128, seed=7):
    w = I.generate("ver", lengths=[W] * B, H=H, dk=d, dv=d, dtype=torch.bfloat16, gate_mode=I.GATE_SAFE,
                   state_std=0.02, conv_state_std=1.0, seed=seed)
    rows = {n: getattr(w, n).view(B, W, *getattr(w, n).shape[1:]).cuda() for n in ("q", "k", "v", "g", "beta")}
    return w, rows


def _decode_rows(w, rows, d, state, cs, row_ids, active):
    """Serial decode of rows row_ids; a sequence takes part at step s only if active(b, s)."""
    B = w.N
    outs = []
    for s in row_ids:
        slots = torch.tensor([b if active(b, s) else -1 for b in range(B)], dtype=torch.int32, device="cuda")
        o = torch.full((B, w.H, w.dv), float("nan"), device="cuda")
        K.kda_decode(d, state, cs, w.conv_w.cuda(), rows["q"][:, s].contiguous(), rows["k"][:, s].contiguous(),
                     rows["v"][:, s].contiguous(), rows["g"][:, s].contiguous(), rows["beta"][:, s].contiguous(),
                     w.gate_mode, w.lower_bound, o, slots=slots)
        outs.append(o)
    return torch.stack(outs, 1)  # [B, steps, H, dv]


@pytest.mark.parametrize("W,accepted,dk", [(4, [0, 3, 1, 2, 3], 128), (8, [0, 7, 3, 5, 2], 128), (8, [7, 0, 6, 1, 4], 64),
                                            (1, [0, 0, 0, 0, 0], 128)])
def test_verify_window_replay_is_bitwise_serial_decode(W, accepted, dk):
    """Windows of 1, 4 and 8 rows (8 is the longest the library takes)."""
    B = 5
    w, rows = _verify_setup(B, W, d=dk)
    d = dims_for(w)
    accept = torch.tensor(accepted, dtype=torch.int32)  # rows 0..j kept
    n_commit = (accept + 1).cuda()
    # verify path: window, then commit-only
    st_v, cs_v = w.state0.cuda().clone(), w.conv_state0.cuda().clone()
    log = K.VerifyLog.empty(d, B, W)
    o_v = torch.empty(B, W, w.H, w.dv, device="cuda")
    K.kda_verify_window(d, st_v, cs_v, w.conv_w.cuda(), None, None, log, rows["q"], rows["k"], rows["v"], rows["g"],
                        rows["beta"], w.gate_mode, w.lower_bound, o_v)
    st_after_window = st_v.clone()
    assert torch.equal(st_after_window, w.state0.cuda())  # uncommitted rows leave the state alone
    K.kda_verify_window(d, st_v, cs_v, w.conv_w.cuda(), n_commit, log, None, None, None, None, None, None,
                        w.gate_mode, w.lower_bound, None, batch=B)
    # serial decode of the kept rows only (negative slots skip the others)
    st_d, cs_d = w.state0.cuda().clone(), w.conv_state0.cuda().clone()
    o_d = _decode_rows(w, rows, d, st_d, cs_d, range(W), lambda b, s: s <= int(accept[b]))
    torch.cuda.synchronize()
    assert torch.equal(st_v, st_d)
    assert torch.equal(cs_v, cs_d)
    for b in range(B):
        j = int(accept[b])
        assert torch.equal(o_v[b, :j + 1], o_d[b, :j + 1])
    # every window row equals decode of all W rows
    st_a, cs_a = w.state0.cuda().clone(), w.conv_state0.cuda().clone()
    o_all = _decode_rows(w, rows, d, st_a, cs_a, range(W), lambda b, s: True)
    assert torch.equal(o_v, o_all)
    # log contents equal the oracle's per-row decay, key and update within tolerance
    ref = oracle_layer(w, with_log=True)
    assert rel(log.a.reshape(-1, w.H, w.dk), ref.log_a) < 1e-6
    assert rel(log.k_hat.reshape(-1, w.H, w.dk), ref.log_k) < 1e-5
    assert rel(log.u.reshape(-1, w.H, w.dv), ref.log_u) < TOL_BF16
    assert rel(o_v.reshape(-1, w.H, w.dv), ref.o) < TOL_BF16


def test_verify_window_with_per_sequence_lengths():
    """Sequence b runs only its first lens[b] rows: those rows and their log equal the full window's, the rest of
    o and the log keep their contents, and committing the kept rows gives the state of serial decode."""
    B, W = 5, 4
    w, rows = _verify_setup(B, W, seed=17)
    d = dims_for(w)
    lens = torch.tensor([0, 4, 1, 3, 2], dtype=torch.int32)
    cw = w.conv_w.cuda()
    full_log, full_o = K.VerifyLog.empty(d, B, W), torch.empty(B, W, w.H, w.dv, device="cuda")
    st, cs = w.state0.cuda().clone(), w.conv_state0.cuda().clone()
    K.kda_verify_window(d, st, cs, cw, None, None, full_log, rows["q"], rows["k"], rows["v"], rows["g"], rows["beta"],
                        w.gate_mode, w.lower_bound, full_o)
    log = K.VerifyLog.empty(d, B, W)
    for t in (log.a, log.k_hat, log.u):
        t.fill_(3.0)
    log.conv_rows.fill_(0)
    o = torch.full((B, W, w.H, w.dv), 7.0, device="cuda")
    K.kda_verify_window(d, st, cs, cw, None, None, log, rows["q"], rows["k"], rows["v"], rows["g"], rows["beta"],
                        w.gate_mode, w.lower_bound, o, window_lens=lens.cuda())
    torch.cuda.synchronize()
    for b in range(B):
        n = int(lens[b])
        assert torch.equal(o[b, :n], full_o[b, :n])
        assert torch.all(o[b, n:] == 7.0)
        for got, ref in ((log.a, full_log.a), (log.k_hat, full_log.k_hat), (log.u, full_log.u),
                         (log.conv_rows, full_log.conv_rows)):
            assert torch.equal(got[b, :n], ref[b, :n])
        assert torch.all(log.a[b, n:] == 3.0) and torch.all(log.conv_rows[b, n:] == 0)
    keep = torch.tensor([0, 3, 1, 2, 2], dtype=torch.int32)  # rows kept, at most the rows run
    K.kda_verify_window(d, st, cs, cw, keep.cuda(), log, None, None, None, None, None, None, w.gate_mode,
                        w.lower_bound, None, batch=B)
    st_d, cs_d = w.state0.cuda().clone(), w.conv_state0.cuda().clone()
    _decode_rows(w, rows, d, st_d, cs_d, range(W), lambda b, s: s < int(keep[b]))
    torch.cuda.synchronize()
    assert torch.equal(st, st_d)
    assert torch.equal(cs, cs_d)
    # the fp64 oracle: sequence b's rows are the first lens[b] rows of its window run from S0, and the
    # committed state is the oracle's after the first keep[b] rows
    ref = oracle_layer(w, with_log=True)
    ran = [b * W + r for b in range(B) for r in range(int(lens[b]))]
    got = lambda t: torch.cat([t[b, :int(lens[b])] for b in range(B)])
    assert rel(got(o), ref.o[ran]) < TOL_BF16
    assert rel(got(log.a), ref.log_a[ran]) < 1e-6
    assert rel(got(log.k_hat), ref.log_k[ran]) < 1e-5
    assert rel(got(log.u), ref.log_u[ran]) < TOL_BF16
    kept = oracle_pieces(w, [range(b * W, b * W + int(keep[b])) for b in range(B)])
    assert rel(st, kept.state) < TOL_BF16
    assert np.array_equal(cs.cpu().double().numpy(), kept.prep.conv_state)


def test_verify_commit_and_next_window_in_one_call():
    """Commit the previous window and run the next one in the same call; equals serial decode bitwise."""
    B, W = 4, 3
    w, rows = _verify_setup(B, 2 * W, seed=11)
    d = dims_for(w)
    first = {k: v[:, :W].contiguous() for k, v in rows.items()}
    second = {k: v[:, W:].contiguous() for k, v in rows.items()}
    acc1 = torch.tensor([3, 1, 2, 3], dtype=torch.int32)  # rows committed from window 1 (count)
    st, cs = w.state0.cuda().clone(), w.conv_state0.cuda().clone()
    log1, log2 = K.VerifyLog.empty(d, B, W), K.VerifyLog.empty(d, B, W)
    o1 = torch.empty(B, W, w.H, w.dv, device="cuda")
    o2 = torch.empty_like(o1)
    K.kda_verify_window(d, st, cs, w.conv_w.cuda(), None, None, log1, first["q"], first["k"], first["v"],
                        first["g"], first["beta"], w.gate_mode, w.lower_bound, o1)
    K.kda_verify_window(d, st, cs, w.conv_w.cuda(), acc1.cuda(), log1, log2, second["q"], second["k"], second["v"],
                        second["g"], second["beta"], w.gate_mode, w.lower_bound, o2)
    # serial: rows 0..acc1-1 of window 1, then all rows of window 2 on top
    for b in range(B):
        n1 = int(acc1[b])
        seq_rows = {k: torch.cat([first[k][b:b + 1, :n1], second[k][b:b + 1]], 1) for k in first}
        sd = K.Dims(w.H, w.dk, w.dv, w.dtype)
        stb = w.state0[b:b + 1].cuda().clone()
        csb = w.conv_state0[b:b + 1].cuda().clone()
        outs = []
        committed = stb.clone()
        for s in range(n1 + W):
            if s == n1:
                committed = stb.clone()
            o = torch.empty(1, w.H, w.dv, device="cuda")
            K.kda_decode(sd, stb, csb, w.conv_w.cuda(), *(seq_rows[k][:, s].contiguous() for k in
                                                        ("q", "k", "v", "g", "beta")), w.gate_mode, w.lower_bound, o)
            outs.append(o)
        torch.cuda.synchronize()
        assert torch.equal(torch.cat(outs[n1:], 0), o2[b])
        assert torch.equal(committed[0], st[b])  # state committed through window 1 only
        del csb


# ---------------------------------------------------------------------------
# chunked prefill
# ---------------------------------------------------------------------------

def test_prefill_tiny_fp32_config():
    """The tiny all-fp32 workload (1 x 1 head, T=256, d=64, softplus gate): <= 1e-5."""
    w = I.tiny()
    r = gpu_layer_prefill(w)
    ref = oracle_layer(w)
    assert rel(r["o"], ref.o) < TOL_FP32
    assert rel(r["y"], ref.y) < TOL_FP32
    assert rel(r["state"], ref.state) < TOL_FP32


@pytest.mark.parametrize("dtype,precision", [(torch.bfloat16, None), (torch.bfloat16, K.PREC_FP16),
                                             (torch.float32, None)])
@pytest.mark.parametrize("gate", [I.GATE_SAFE, I.GATE_SOFTPLUS])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
def test_prefill_varlen_parity(dtype, precision, gate, dk, dv):
    w = small(dtype, lens=(200, 1, 0, 64, 127, 65), H=2, d=dk, dv=dv, gate=gate, seed=dk + dv)
    r = gpu_layer_prefill(w, precision=precision)
    ref = oracle_layer(w)
    tol = tol_for(w)
    assert rel(r["o"], ref.o) < tol
    assert rel(r["y"], ref.y) < tol
    assert rel(r["state"], ref.state) < tol


@pytest.mark.parametrize("dk,dv,precision,fused", [(64, 64, None, False), (128, 128, K.PREC_FP16, False),
                                                    (128, 128, K.PREC_FP16, True), (128, 64, K.PREC_BF16X3, True)])
def test_prefill_many_ragged_sequences(dk, dv, precision, fused):
    """400 sequences, many empty, single-row or one row either side of a chunk boundary: the chunk-record
    slot of every sequence and thousands of scan workgroups over eight XCD groups."""
    rng = np.random.default_rng(dk + dv)
    lens = rng.choice([0, 1, 2, 63, 64, 65, 127, 128, 129], size=300).tolist() + rng.integers(0, 200, 100).tolist()
    w = small(torch.bfloat16, lens=lens, H=2, d=dk, dv=dv, gate=I.GATE_SOFTPLUS, seed=81)
    print(f"many sequences N={w.N} T={w.T} dk={dk} dv={dv} precision={precision} fused={fused}", flush=True)
    r = gpu_layer_prefill(w, precision=precision, fused=fused)
    ref = oracle_layer(w)
    assert rel(r["o"], ref.o) < TOL_BF16
    assert rel(r["y"], ref.y) < TOL_BF16
    assert rel(r["state"], ref.state) < TOL_BF16
    assert np.array_equal(r["prep"]["conv_state"].cpu().double().numpy(), ref.prep.conv_state)
    # every sequence on its own, including the ones that start with an empty prompt
    st = r["state"].cpu().double().numpy()
    per_seq = [rel(st[n], ref.state[n]) for n in range(w.N)]
    worst = int(np.argmax(per_seq))
    print(f"worst per-sequence state rel-L2 {per_seq[worst]:.2e} (sequence {worst}, length {lens[worst]})", flush=True)
    for n in range(w.N):
        assert per_seq[n] < TOL_BF16, f"sequence {n} (length {lens[n]})"


@pytest.mark.parametrize("precision", [K.PREC_FP32, K.PREC_BF16X3, K.PREC_FP16, K.PREC_BF16X2])
def test_prefill_precision_policies_on_bf16_rows(precision):
    w = small(torch.bfloat16, lens=(300, 77), H=2, d=128, gate=I.GATE_SAFE, seed=21)
    r = gpu_layer_prefill(w, precision=precision)
    ref = oracle_layer(w)
    assert rel(r["y"], ref.y) < TOL_BF16
    assert rel(r["state"], ref.state) < TOL_BF16


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("precision", [None, K.PREC_FP16])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64)])
def test_fused_preamble_is_bitwise_the_unfused_path(dtype, precision, dk, dv):
    """kda_prefill_varlen with raw rows == kda_prep then kda_prefill_varlen, bit for bit (o, state, conv state)."""
    w = small(dtype, lens=(150, 3, 0, 64, 70), H=2, d=dk, dv=dv, gate=I.GATE_SOFTPLUS, seed=71)
    a = gpu_layer_prefill(w, precision=precision)
    b = gpu_layer_prefill(w, precision=precision, fused=True)
    assert torch.equal(a["o"], b["o"])
    assert torch.equal(a["state"], b["state"])
    assert torch.equal(a["prep"]["conv_state"], b["prep"]["conv_state"])


def test_fused_preamble_with_slots_and_in_place_conv_state():
    w = small(torch.bfloat16, lens=(90, 2, 70), H=2, d=128, seed=81)
    d = dims_for(w, K.PREC_FP16)
    wd = w.to("cuda")
    slots = torch.tensor([2, -1, 0], dtype=torch.int32, device="cuda")
    pool = torch.zeros(3, w.H, w.dk, w.dv, device="cuda")
    pool[2], pool[0] = wd.state0[0], wd.state0[2]
    cpool = torch.zeros(3, 3, w.C, device="cuda", dtype=w.dtype)
    cpool[2], cpool[0] = wd.conv_state0[0], wd.conv_state0[2]
    cpool_before = cpool.clone()
    o = torch.full((w.T, w.H, w.dv), 5.0, device="cuda")
    ws = torch.empty(K.kda_prefill_workspace_bytes(d, w.N, w.T), dtype=torch.uint8, device="cuda")
    raw = dict(q_raw=wd.q, k_raw=wd.k, v_raw=wd.v, g_raw=wd.g, beta_logit=wd.beta, conv_weight=wd.conv_w,
               conv_state_in=cpool, conv_state_out=cpool, gate_mode=w.gate_mode, lower_bound=w.lower_bound)
    K.kda_prefill_varlen(d, wd.cu_seqlens, None, None, None, None, None, pool, o, ws, slots=slots, raw=raw)
    torch.cuda.synchronize()
    ref = oracle_layer(w)
    cu = w.cu_seqlens.tolist()
    assert rel(pool[2], ref.state[0]) < TOL_BF16 and rel(pool[0], ref.state[2]) < TOL_BF16
    assert torch.all(o[cu[1]:cu[2]] == 5.0)
    assert torch.equal(cpool[1], cpool_before[1])
    assert np.array_equal(cpool[2].cpu().double().numpy(), ref.prep.conv_state[0])
    assert np.array_equal(cpool[0].cpu().double().numpy(), ref.prep.conv_state[2])
    assert rel(o[:cu[1]], ref.o[:cu[1]]) < TOL_BF16


def test_prefill_steep_decay_takes_exact_path():
    """Softplus gate fed with very large raw gates: decay spans far beyond e^40 within half a block."""
    w = small(torch.float32, lens=(150, 40), H=2, d=64, gate=I.GATE_SOFTPLUS, seed=31)
    w.g.mul_(30.0)
    r = gpu_layer_prefill(w)
    ref = oracle_layer(w)
    assert np.all(np.isfinite(r["o"].cpu().numpy()))
    errs = {"o": rel(r["o"], ref.o), "state": rel(r["state"], ref.state)}
    print("steep decay, exact path:", errs, flush=True)
    assert all(e < TOL_FP32 for e in errs.values()), errs


@pytest.mark.parametrize("boundary", [20.0, 10.0])
def test_prefill_steep_gate_on_block_first_rows(boundary):
    """Softplus gate of about 5 on every row inside each 16-row block (a within-block span of 75, under
    the guard of 80) and a steeper one on each block's first row.  With 20 a block's full decay is about
    95 and the chunk takes the exact path; with 10 it is about 85 and the pivoted path keeps e^{T}
    a normal fp32 number."""
    w = small(torch.float32, lens=(150, 40), H=2, d=64, gate=I.GATE_SOFTPLUS, seed=33)
    cu = w.cu_seqlens.tolist()
    for n in range(w.N):
        for t in range(cu[n], cu[n + 1]):
            w.g[t] = boundary if (t - cu[n]) % 16 == 0 else 5.0
    print(f"block-boundary gate {boundary}", flush=True)
    r = gpu_layer_prefill(w)
    ref = oracle_layer(w)
    assert np.all(np.isfinite(r["o"].cpu().numpy()))
    errs = {"o": rel(r["o"], ref.o), "state": rel(r["state"], ref.state)}
    print(errs, flush=True)
    assert all(e < TOL_FP32 for e in errs.values()), errs


@pytest.mark.parametrize("precision", [K.PREC_BF16X3, K.PREC_FP16])
def test_prefill_packed_equals_alone_bitwise(precision):
    w = small(torch.bfloat16, lens=(100, 64, 3, 129), H=2, d=128, seed=41)
    full = gpu_layer_prefill(w, precision=precision)
    cu = w.cu_seqlens.tolist()
    for n in range(w.N):
        sl = slice(cu[n], cu[n + 1])
        one = I.Workload("one", w.H, w.dk, w.dv, torch.tensor([0, cu[n + 1] - cu[n]], dtype=torch.int32),
                         w.q[sl], w.k[sl], w.v[sl], w.g[sl], w.beta[sl], w.z[sl], w.conv_w, w.norm_w,
                         w.state0[n:n + 1], w.conv_state0[n:n + 1], w.gate_mode, w.lower_bound)
        alone = gpu_layer_prefill(one, precision=precision)
        assert torch.equal(alone["o"], full["o"][sl])
        assert torch.equal(alone["state"][0], full["state"][n])


@pytest.mark.parametrize("dk,dv,precision,blocks", [
    (128, 128, K.PREC_FP16, 2), (128, 128, K.PREC_FP16, 4), (128, 128, K.PREC_BF16X2, 4),
    (128, 128, K.PREC_BF16X3, 2), (64, 128, K.PREC_FP32, 2), (128, 64, K.PREC_FP16, 4), (128, 64, K.PREC_BF16X3, 2)])
def test_prefill_wide_scan_equals_narrow_bitwise(dk, dv, precision, blocks):
    """The scan gives each workgroup 1, 2 or 4 blocks of 16 state columns: 4 (FP16 and BF16X2 only) where
    groups = sequences x heads reach half the CU count, 2 where they reach a quarter, else 1.  Enough
    sequences x 2 heads packed in one call take the `blocks` shape, each sequence alone (2 groups) the one-block
    shape; every column's arithmetic is the same in all shapes, so o, the state and the conv state agree bit for
    bit (fused preamble, so the conv-state carry runs in both)."""
    H = 2
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    N = cus // (4 * H) + 4 if blocks == 2 else cus // (2 * H) + 2
    assert 4 * N * H >= cus and (blocks == 4) == (2 * N * H >= cus) and 4 * H < cus
    rng = np.random.default_rng(dk * 3 + dv + blocks)
    lens = rng.integers(1, 200, N).tolist()
    lens[5], lens[17] = 64, 128  # chunk multiples
    w = small(torch.bfloat16, lens=lens, H=H, d=dk, dv=dv, gate=I.GATE_SOFTPLUS, seed=dk + dv + precision)
    print(f"scan shapes: {blocks} blocks (N={w.N}, {cus} CUs) vs 1, T={w.T} dk={dk} dv={dv} precision={precision}",
          flush=True)
    full = gpu_layer_prefill(w, precision=precision, fused=True)
    cu = w.cu_seqlens.tolist()
    for n in range(w.N):
        sl = slice(cu[n], cu[n + 1])
        one = I.Workload("one", w.H, w.dk, w.dv, torch.tensor([0, cu[n + 1] - cu[n]], dtype=torch.int32),
                         w.q[sl], w.k[sl], w.v[sl], w.g[sl], w.beta[sl], w.z[sl], w.conv_w, w.norm_w,
                         w.state0[n:n + 1], w.conv_state0[n:n + 1], w.gate_mode, w.lower_bound)
        alone = gpu_layer_prefill(one, precision=precision, fused=True)
        assert torch.equal(alone["o"], full["o"][sl]), f"sequence {n} (length {lens[n]})"
        assert torch.equal(alone["state"][0], full["state"][n]), f"sequence {n} (length {lens[n]})"
        assert torch.equal(alone["prep"]["conv_state"][0], full["prep"]["conv_state"][n])


@pytest.mark.parametrize("H,d,precision", [(5, 128, K.PREC_FP16), (3, 64, K.PREC_BF16X3), (5, 64, K.PREC_BF16X2)])
def test_prefill_odd_heads_against_oracle(H, d, precision):
    """Head counts that are not powers of two and (sequences x heads) groups that are not a multiple of the
    eight XCD groups, with enough groups that the scan takes a several-column-block shape (four blocks for
    the one-part policies at 5 heads, two for BF16X3), ragged lengths: o, y and the state of every sequence
    against the oracle."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    N = cus // (2 * H) + 3
    rng = np.random.default_rng(H * 100 + d)
    lens = rng.integers(1, 150, N).tolist()
    lens[1], lens[2] = 0, 64
    w = small(torch.bfloat16, lens=lens, H=H, d=d, gate=I.GATE_SOFTPLUS, seed=H + d)
    print(f"odd heads N={w.N} H={H} groups={w.N * H} T={w.T} d={d} precision={precision}", flush=True)
    r = gpu_layer_prefill(w, precision=precision, fused=True)
    ref = oracle_layer(w)
    assert rel(r["o"], ref.o) < TOL_BF16
    assert rel(r["y"], ref.y) < TOL_BF16
    st = r["state"].cpu().double().numpy()
    for n in range(w.N):
        assert rel(st[n], ref.state[n]) < TOL_BF16, f"sequence {n} (length {lens[n]})"
    assert np.array_equal(r["prep"]["conv_state"].cpu().double().numpy(), ref.prep.conv_state)


@pytest.mark.parametrize("cut,precision", [(64, K.PREC_BF16X3), (128, K.PREC_BF16X3), (128, K.PREC_FP16)])
def test_prefill_cut_at_chunk_multiple_is_bitwise(cut, precision):
    w = small(torch.bfloat16, lens=(300,), H=2, d=128, seed=51)
    full = gpu_layer_prefill(w, precision=precision)
    a = I.Workload("a", w.H, w.dk, w.dv, torch.tensor([0, cut], dtype=torch.int32), w.q[:cut], w.k[:cut], w.v[:cut],
                   w.g[:cut], w.beta[:cut], w.z[:cut], w.conv_w, w.norm_w, w.state0, w.conv_state0, w.gate_mode,
                   w.lower_bound)
    ra = gpu_layer_prefill(a, precision=precision)
    b = I.Workload("b", w.H, w.dk, w.dv, torch.tensor([0, 300 - cut], dtype=torch.int32), w.q[cut:], w.k[cut:],
                   w.v[cut:], w.g[cut:], w.beta[cut:], w.z[cut:], w.conv_w, w.norm_w, ra["state"].cpu(),
                   ra["prep"]["conv_state"].cpu(), w.gate_mode, w.lower_bound)
    rb = gpu_layer_prefill(b, precision=precision)
    assert torch.equal(torch.cat([ra["o"], rb["o"]]), full["o"])
    assert torch.equal(rb["state"], full["state"])


@pytest.mark.parametrize("fused,ydt", [(False, torch.float32), (True, torch.bfloat16), (True, torch.float32)])
def test_prefill_norm_epilogue_is_bitwise_the_separate_norm(fused, ydt):
    """kda_prefill_varlen with `norm`: o as without it, and y bit for bit what gated_rmsnorm_out gives on that o."""
    w = small(torch.bfloat16, lens=(150, 3, 0, 64, 70), H=2, d=128, gate=I.GATE_SOFTPLUS, seed=91)
    d = dims_for(w, K.PREC_FP16)
    ref = gpu_layer_prefill(w, precision=K.PREC_FP16, y_dtype=ydt, fused=fused)
    wd = w.to("cuda")
    state = wd.state0.clone()
    o = torch.empty(w.T, w.H, w.dv, device="cuda")
    y = torch.empty(w.T, w.H, w.dv, device="cuda", dtype=ydt)
    ws = torch.empty(K.kda_prefill_workspace_bytes(d, w.N, w.T), dtype=torch.uint8, device="cuda")
    norm = dict(z=wd.z, weight=wd.norm_w, eps=EPS, y=y)
    if fused:
        K.kda_prefill_varlen(d, wd.cu_seqlens, None, None, None, None, None, state, o, ws,
                             raw=raw_rows(wd, torch.empty_like(wd.conv_state0)), norm=norm)
    else:
        _, p = gpu_prep(w, d)
        K.kda_prefill_varlen(d, wd.cu_seqlens, p["q_hat"], p["k_hat"], p["v"], p["g"], p["beta"], state, o, ws,
                             norm=norm)
    torch.cuda.synchronize()
    assert torch.equal(o, ref["o"])
    assert torch.equal(state, ref["state"])
    assert torch.equal(y, ref["y"])


def test_prefill_norm_epilogue_skips_negative_slots():
    w = small(torch.bfloat16, lens=(90, 70, 40), H=2, d=64, seed=93)
    d = dims_for(w)
    wd, p = gpu_prep(w, d)
    pool = torch.randn(4, w.H, w.dk, w.dv, device="cuda") * 0.02
    pool[2] = wd.state0[0]
    pool[0] = wd.state0[2]
    slots = torch.tensor([2, -1, 0], dtype=torch.int32, device="cuda")
    o = torch.full((w.T, w.H, w.dv), 7.0, device="cuda")
    y = torch.full((w.T, w.H, w.dv), 5.0, device="cuda")
    ws = torch.empty(K.kda_prefill_workspace_bytes(d, w.N, w.T), dtype=torch.uint8, device="cuda")
    K.kda_prefill_varlen(d, wd.cu_seqlens, p["q_hat"], p["k_hat"], p["v"], p["g"], p["beta"], pool, o, ws,
                         slots=slots, norm=dict(z=wd.z, weight=wd.norm_w, eps=EPS, y=y))
    torch.cuda.synchronize()
    cu = w.cu_seqlens.tolist()
    assert torch.all(y[cu[1]:cu[2]] == 5.0)  # the skipped sequence: y untouched
    y_sep = torch.empty_like(y)
    K.gated_rmsnorm_out(o, wd.z, wd.norm_w, EPS, y_sep)
    torch.cuda.synchronize()
    for a, b in ((0, cu[1]), (cu[2], cu[3])):
        assert torch.equal(y[a:b], y_sep[a:b])
    ref = oracle_layer(w)
    assert rel(y[:cu[1]], ref.y[:cu[1]]) < TOL_BF16
    assert rel(y[cu[2]:], ref.y[cu[2]:]) < TOL_BF16


def test_prefill_slots_and_negative_slot():
    w = small(torch.bfloat16, lens=(90, 70, 40), H=2, d=64, seed=61)
    d = dims_for(w)
    wd, p = gpu_prep(w, d)
    pool = torch.randn(5, w.H, w.dk, w.dv, device="cuda") * 0.02
    slots = torch.tensor([3, -1, 0], dtype=torch.int32, device="cuda")
    pool_before = pool.clone()
    # the state pool is indexed by slot: put each sequence's initial state there
    pool[3] = wd.state0[0]
    pool[0] = wd.state0[2]
    expect_untouched = pool.clone()
    o = torch.full((w.T, w.H, w.dv), 7.0, device="cuda")
    ws = torch.empty(K.kda_prefill_workspace_bytes(d, w.N, w.T), dtype=torch.uint8, device="cuda")
    K.kda_prefill_varlen(d, wd.cu_seqlens, p["q_hat"], p["k_hat"], p["v"], p["g"], p["beta"], pool, o, ws,
                         slots=slots)
    torch.cuda.synchronize()
    ref = oracle_layer(w)
    cu = w.cu_seqlens.tolist()
    assert rel(pool[3], ref.state[0]) < TOL_BF16
    assert rel(pool[0], ref.state[2]) < TOL_BF16
    for s in (1, 2, 4):
        assert torch.equal(pool[s], expect_untouched[s])
    assert torch.all(o[cu[1]:cu[2]] == 7.0)  # skipped sequence: outputs untouched
    assert rel(o[:cu[1]], ref.o[:cu[1]]) < TOL_BF16
    del pool_before


def test_errors_write_nothing():
    w = small(torch.bfloat16, lens=(10,), H=2, d=128)
    d = dims_for(w)
    wd = w.to("cuda")
    o = torch.full((1, w.H, w.dv), 3.0, device="cuda")
    st = wd.state0.clone()
    with pytest.raises(K.KdaError) as e:
        K.kda_decode(d, st, wd.conv_state0, wd.conv_w, wd.q[:1], wd.k[:1], wd.v[:1], wd.g[:1], wd.beta[:1],
                     I.GATE_SAFE, 0.5, o)  # bad lower bound
    assert e.value.code == K.KDA_E_GATE
    torch.cuda.synchronize()
    assert torch.all(o == 3.0) and torch.equal(st, wd.state0)
