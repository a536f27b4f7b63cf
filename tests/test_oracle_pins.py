"""Pins of the fp64 CPU oracle against facts fixed by the mathematics.

Each test checks the oracle against something other than itself: a hand-worked
example, a closed form, an invariant, an independent brute-force evaluation or
a library routine.  All run on the CPU (no GPU marker).
"""
import os

import numpy as np
import pytest
from scipy.special import expit

from oracle import brute
from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng_seed = 1234


def _golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            out[key.strip()] = np.array([float(x) for x in val.split()])
    return out


def _rand_core(rng, lens, H, dk, dv, *, unit_keys=True, gscale=1.0):
    T = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    g = -gscale * np.log1p(np.exp(rng.standard_normal((T, H, dk))))
    b = expit(rng.standard_normal((T, H)))
    S0 = 0.1 * rng.standard_normal((len(lens), H, dk, dv))
    return cu, q, k, v, g, b, S0


def _rel(x, ref):
    return np.linalg.norm((x - ref).ravel()) / np.linalg.norm(ref.ravel())


# ----------------------------------------------------------------------------
# hand-worked example and special values
# ----------------------------------------------------------------------------

def test_hand_worked_recurrence(oracle_mod):
    gd = _golden("hand_recurrence.txt")
    q = gd["q"].reshape(2, 1, 2)
    k = gd["k"].reshape(2, 1, 2)
    g = np.log(gd["a"]).reshape(2, 1, 2)
    v = gd["v"].reshape(2, 1, 1)
    b = gd["b"].reshape(2, 1)
    S0 = gd["S0"].reshape(1, 1, 2, 1)
    for fn in (O.recurrent, lambda *a: O.chunked(*a, chunk=2), lambda *a: O.chunked(*a, chunk=1)):
        r = fn(q, k, v, g, b, S0, [0, 2])
        np.testing.assert_allclose(r.o.ravel(), gd["o"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(r.state.ravel(), gd["S_T"], rtol=0, atol=1e-14)


def test_scalar_special_values(oracle_mod):
    """Gate and activation values at points where the definition gives them in closed form.
    Driven through prep with a single identity conv tap so the activation sees the raw value."""
    gd = _golden("scalar_functions.txt")
    H, dk, dv = 1, 1, 1
    C = H * (2 * dk + dv)
    w = np.zeros((C, 4)); w[:, 3] = 1.0
    cs = np.zeros((1, 3, C))
    xs = np.array([1.0, -2.0])
    q = xs.reshape(2, 1, 1); k = q.copy(); v = q.copy()
    graw = np.array([0.0, 20.0]).reshape(2, 1, 1)
    bl = np.zeros((2, 1))
    p = O.prep(q, k, v, w, cs, graw, bl, [0, 2], gate_mode=O.GATE_SOFTPLUS, act=O.ACT_SILU)
    assert p.v[0, 0, 0] == pytest.approx(gd["silu_1"][0], abs=1e-15)
    assert p.v[1, 0, 0] == pytest.approx(gd["silu_-2"][0], abs=1e-15)
    assert p.g[0, 0, 0] == pytest.approx(gd["softplus_gate_at_0"][0], abs=1e-15)
    assert p.g[1, 0, 0] == pytest.approx(gd["softplus_gate_at_20"][0], abs=1e-13)
    assert p.beta[0, 0] == 0.5
    p2 = O.prep(q, k, v, w, cs, graw, bl, [0, 2], gate_mode=O.GATE_SAFE, lower_bound=-5.0)
    assert p2.g[0, 0, 0] == pytest.approx(gd["safe_gate_at_0_lb_-5"][0], abs=1e-15)


def test_gates_match_library_routines(oracle_mod):
    """softplus gate = -logaddexp(0,x) and safe gate = lb*expit(x), against numpy/scipy, over a wide range."""
    rng = np.random.default_rng(rng_seed)
    T, H, dk, dv = 50, 2, 3, 2
    C = H * (2 * dk + dv)
    x = np.concatenate([rng.standard_normal(T * H * dk - 4) * 8, [0.0, 40.0, -40.0, 700.0]]).reshape(T, H, dk)
    bl = rng.standard_normal((T, H)) * 5
    z3 = np.zeros((T, H, dk)); zv = np.zeros((T, H, dv))
    w = rng.standard_normal((C, 4)); cs = np.zeros((1, 3, C))
    p = O.prep(z3, z3, zv, w, cs, x, bl, [0, T], gate_mode=O.GATE_SOFTPLUS)
    np.testing.assert_allclose(p.g, -np.logaddexp(0.0, x), rtol=1e-15, atol=1e-300)
    np.testing.assert_allclose(p.beta, expit(bl), rtol=1e-15)
    for lb in (-5.0, -0.25):
        p = O.prep(z3, z3, zv, w, cs, x, bl, [0, T], gate_mode=O.GATE_SAFE, lower_bound=lb)
        np.testing.assert_allclose(p.g, lb * expit(x), rtol=1e-15)
        assert np.all(p.g >= lb) and np.all(p.g <= 0)


# ----------------------------------------------------------------------------
# recurrence pins (P1-P4, P7, P8, P11)
# ----------------------------------------------------------------------------

def test_p1_unit_decay_zero_beta_freezes_state(oracle_mod):
    rng = np.random.default_rng(1)
    cu, q, k, v, g, b, S0 = _rand_core(rng, [7, 0, 12], 3, 5, 4)
    g[:] = 0.0
    b[:] = 0.0
    r = O.recurrent(q, k, v, g, b, S0, cu)
    assert np.array_equal(r.state, S0)
    seq = np.repeat(np.arange(3), np.diff(cu))
    ref = np.einsum("thd,thde->the", q, S0[seq])
    np.testing.assert_allclose(r.o, ref, rtol=0, atol=1e-14)


def test_p2_linear_attention_with_orthonormal_keys(oracle_mod):
    """a=1, b=1, S0=0, mutually orthonormal keys: o_t = sum_{i<=t} (q_t . k_i) v_i."""
    rng = np.random.default_rng(2)
    dk, dv, T, H = 8, 3, 8, 2
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = np.stack([Qm[:, :T].T] * H, axis=1)  # [T,H,dk], orthonormal rows
    q = rng.standard_normal((T, H, dk))
    v = rng.standard_normal((T, H, dv))
    g = np.zeros((T, H, dk)); b = np.ones((T, H)); S0 = np.zeros((1, H, dk, dv))
    r = O.recurrent(q, k, v, g, b, S0, [0, T])
    ref = np.zeros((T, H, dv))
    for t in range(T):
        for i in range(t + 1):
            ref[t] += np.sum(q[t] * k[i], axis=-1)[:, None] * v[i]
    np.testing.assert_allclose(r.o, ref, rtol=0, atol=1e-14)


def test_p3_beta_one_overwrites_and_general_update(oracle_mod):
    """With |k|=1: S_t^T k_t = (1-b)(Diag(a) S_{t-1})^T k_t + b v_t; b=1 gives v_t exactly (to rounding)."""
    rng = np.random.default_rng(3)
    cu, q, k, v, g, b, S0 = _rand_core(rng, [10], 2, 6, 5)
    for force_one in (True, False):
        bb = np.ones_like(b) if force_one else b
        S = S0.copy()
        for t in range(10):
            r = O.recurrent(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], bb[t:t + 1], S, [0, 1])
            Sp = np.exp(g[t])[:, :, None] * S[0]  # Diag(a) S_{t-1}, per head
            lhs = np.einsum("hde,hd->he", r.state[0], k[t])
            rhs = (1 - bb[t])[:, None] * np.einsum("hde,hd->he", Sp, k[t]) + bb[t][:, None] * v[t]
            np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-13)
            if force_one:
                np.testing.assert_allclose(lhs, v[t], rtol=0, atol=1e-13)
            S = r.state


def test_p4_zero_beta_closed_form_through_layer(oracle_mod):
    """beta = sigmoid(-inf) = 0: S_T = Diag(prod a) S0 with a from the gate; checked per gate mode."""
    rng = np.random.default_rng(4)
    T, H, dk, dv = 33, 2, 4, 3
    C = H * (2 * dk + dv)
    raw = lambda *s: rng.standard_normal(s)
    graw = raw(T, H, dk) * 2
    S0 = raw(1, H, dk, dv)
    for mode, gfun in ((O.GATE_SOFTPLUS, lambda x: -np.logaddexp(0, x)), (O.GATE_SAFE, lambda x: -5 * expit(x))):
        L = O.layer(raw(T, H, dk), raw(T, H, dk), raw(T, H, dv), raw(C, 4), raw(1, 3, C), graw,
                    np.full((T, H), -np.inf), raw(T, H, dv), raw(dv), S0, [0, T], gate_mode=mode)
        decay = np.exp(gfun(graw).sum(axis=0))  # [H,dk]
        np.testing.assert_allclose(L.state[0], decay[:, :, None] * S0[0], rtol=1e-12, atol=0)


@pytest.mark.parametrize("dk,dv,T", [(5, 3, 8), (3, 4, 6), (1, 1, 8), (4, 4, 1)])
def test_p7_brute_force_products(oracle_mod, dk, dv, T):
    """Oracle vs explicit products of transition matrices (numpy), several sequences and heads."""
    rng = np.random.default_rng(70 + dk * 10 + T)
    lens = [T, max(T - 3, 0), T]
    H = 2
    cu, q, k, v, g, b, S0 = _rand_core(rng, lens, H, dk, dv)
    r = O.recurrent(q, k, v, g, b, S0, cu)
    for n in range(len(lens)):
        for h in range(H):
            sl = slice(cu[n], cu[n + 1])
            if cu[n + 1] == cu[n]:
                assert np.array_equal(r.state[n, h], S0[n, h])
                continue
            o_ref, S_ref = brute.states_by_products(q[sl, h], k[sl, h], v[sl, h], np.exp(g[sl, h]), b[sl, h],
                                                    S0[n, h])
            np.testing.assert_allclose(r.o[sl, h], o_ref, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(r.state[n, h], S_ref, rtol=1e-12, atol=1e-13)


def test_p13_verify_log_against_products(oracle_mod):
    """The per-row log a verify window keeps (decay a_t = e^{g_t}, key k_t, update u_t)
    against the brute-force products: the state after each prefix of rows, S_t, is
    built from the transition matrices, and since the step is S_t = Diag(a_t) S_{t-1}
    + k_t u_t^T, the update is recovered as (S_t - Diag(a_t) S_{t-1})^T k_t / |k_t|^2.
    Replaying the logged rows from the initial state then gives the final state."""
    rng = np.random.default_rng(13)
    lens = [5, 0, 6]
    H, dk, dv = 2, 3, 2
    cu, q, k, v, g, b, S0 = _rand_core(rng, lens, H, dk, dv, unit_keys=False)
    r = O.recurrent(q, k, v, g, b, S0, cu, with_log=True)
    np.testing.assert_allclose(r.log_a, np.exp(g), rtol=1e-15, atol=0)
    assert np.array_equal(r.log_k, k)
    for n in range(len(lens)):
        for h in range(H):
            S_prev, S_rep = S0[n, h], S0[n, h].copy()
            for t in range(cu[n], cu[n + 1]):
                sl = slice(cu[n], t + 1)
                _, S_t = brute.states_by_products(q[sl, h], k[sl, h], v[sl, h], np.exp(g[sl, h]), b[sl, h],
                                                  S0[n, h])
                a_t, k_t = np.exp(g[t, h]), k[t, h]
                u_ref = (S_t - a_t[:, None] * S_prev).T @ k_t / (k_t @ k_t)
                np.testing.assert_allclose(r.log_u[t, h], u_ref, rtol=1e-10, atol=1e-12)
                S_rep = r.log_a[t, h][:, None] * S_rep + np.outer(r.log_k[t, h], r.log_u[t, h])
                S_prev = S_t
            np.testing.assert_allclose(S_rep, r.state[n, h], rtol=1e-12, atol=1e-13)


def test_p8_scalar_state_closed_form(oracle_mod):
    """d_k = d_v = 1: S_t = (1 - b k^2) a S_{t-1} + b k v, o_t = S_t q (keys not unit)."""
    rng = np.random.default_rng(8)
    cu, q, k, v, g, b, S0 = _rand_core(rng, [40], 1, 1, 1, unit_keys=False)
    r = O.recurrent(q, k, v, g, b, S0, cu)
    S = S0[0, 0, 0, 0]
    for t in range(40):
        kk, a = k[t, 0, 0], np.exp(g[t, 0, 0])
        S = (1 - b[t, 0] * kk * kk) * a * S + b[t, 0] * kk * v[t, 0, 0]
        assert r.o[t, 0, 0] == pytest.approx(S * q[t, 0, 0], rel=1e-12, abs=1e-14)
    assert r.state[0, 0, 0, 0] == pytest.approx(S, rel=1e-12)


def test_p11_state_norm_bound(oracle_mod):
    """||S_t||_F <= ||S_{t-1}||_F + b_t ||v_t|| when |k|<=1, a in (0,1], b in [0,1]."""
    rng = np.random.default_rng(11)
    cu, q, k, v, g, b, S0 = _rand_core(rng, [30], 3, 8, 8)
    S = S0
    for t in range(30):
        r = O.recurrent(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], b[t:t + 1], S, [0, 1])
        for h in range(3):
            assert np.linalg.norm(r.state[0, h]) <= np.linalg.norm(S[0, h]) + b[t, h] * np.linalg.norm(v[t, h]) + 1e-12
        S = r.state


# ----------------------------------------------------------------------------
# chunked form (P5) and carries (P6, zero-length)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("chunk", [1, 3, 16, 64])
@pytest.mark.parametrize("gate", ["softplus", "safe", "softplus_large"])
def test_p5_chunked_equals_serial(oracle_mod, chunk, gate):
    rng = np.random.default_rng(5)
    H, dk, dv = 2, 16, 8
    lens = [150, 1, 0, 64, 77]
    cu, q, k, v, g, b, S0 = _rand_core(rng, lens, H, dk, dv)
    if gate == "safe":
        g = -5.0 * expit(rng.standard_normal(g.shape))
    elif gate == "softplus_large":
        g = -np.logaddexp(0, 30.0 * rng.standard_normal(g.shape))  # log-decays down to ~ -100 per row
    s = O.recurrent(q, k, v, g, b, S0, cu)
    c = O.chunked(q, k, v, g, b, S0, cu, chunk=chunk)
    assert np.all(np.isfinite(c.o)) and np.all(np.isfinite(c.state))
    assert _rel(c.o, s.o) < 1e-12
    assert _rel(c.state, s.state) < 1e-12


def _layer_inputs(rng, lens, H, dk, dv):
    T = int(sum(lens))
    C = H * (2 * dk + dv)
    f = lambda *s: rng.standard_normal(s)
    return dict(q_raw=f(T, H, dk), k_raw=f(T, H, dk), v_raw=f(T, H, dv), conv_w=rng.uniform(-.5, .5, (C, 4)),
                conv_state=f(len(lens), 3, C), g_raw=f(T, H, dk), beta_logit=f(T, H), z=f(T, H, dv),
                norm_w=rng.uniform(.5, 1.5, dv), state0=0.02 * f(len(lens), H, dk, dv),
                cu_seqlens=np.concatenate([[0], np.cumsum(lens)]))


@pytest.mark.parametrize("cut", [1, 2, 3, 17, 64, 99])
def test_p6_split_prompt_with_carry_is_bitwise(oracle_mod, cut):
    rng = np.random.default_rng(6)
    H, dk, dv, T = 2, 8, 4, 100
    x = _layer_inputs(rng, [T], H, dk, dv)
    full = O.layer(**x, gate_mode=O.GATE_SAFE)
    rows = ("q_raw", "k_raw", "v_raw", "g_raw", "beta_logit", "z")
    a = dict(x, **{r: x[r][:cut] for r in rows}, cu_seqlens=[0, cut])
    A = O.layer(**a, gate_mode=O.GATE_SAFE)
    bpart = dict(x, **{r: x[r][cut:] for r in rows}, cu_seqlens=[0, T - cut], conv_state=A.prep.conv_state,
                 state0=A.state)
    B = O.layer(**bpart, gate_mode=O.GATE_SAFE)
    assert np.array_equal(np.concatenate([A.y, B.y]), full.y)
    assert np.array_equal(np.concatenate([A.o, B.o]), full.o)
    assert np.array_equal(B.state, full.state)
    assert np.array_equal(B.prep.conv_state, full.prep.conv_state)


def test_zero_length_sequence_passes_carries_through(oracle_mod):
    rng = np.random.default_rng(13)
    x = _layer_inputs(rng, [5, 0, 3], 2, 4, 4)
    L = O.layer(**x)
    assert np.array_equal(L.state[1], x["state0"][1])
    assert np.array_equal(L.prep.conv_state[1], x["conv_state"][1])


def test_packed_equals_alone(oracle_mod):
    """A sequence packed with others gives the same bits as the same sequence alone (layout/indexing)."""
    rng = np.random.default_rng(14)
    lens = [9, 4, 0, 13]
    x = _layer_inputs(rng, lens, 2, 4, 3)
    L = O.layer(**x)
    cu = x["cu_seqlens"]
    rows = ("q_raw", "k_raw", "v_raw", "g_raw", "beta_logit", "z")
    for n in range(len(lens)):
        sl = slice(cu[n], cu[n + 1])
        one = dict(x, **{r: x[r][sl] for r in rows}, cu_seqlens=[0, lens[n]], conv_state=x["conv_state"][n:n + 1],
                   state0=x["state0"][n:n + 1])
        A = O.layer(**one)
        assert np.array_equal(A.y, L.y[sl])
        assert np.array_equal(A.state[0], L.state[n])
        assert np.array_equal(A.prep.conv_state[0], L.prep.conv_state[n])


# ----------------------------------------------------------------------------
# conv (P9), norms (P10)
# ----------------------------------------------------------------------------

def test_p9_conv_delta_taps_identity_and_shift(oracle_mod):
    rng = np.random.default_rng(9)
    lens = [7, 2]
    H, dk, dv = 2, 3, 2
    x = _layer_inputs(rng, lens, H, dk, dv)
    C = H * (2 * dk + dv)
    T = sum(lens)
    args = {k: x[k] for k in ("q_raw", "k_raw", "v_raw", "conv_state", "g_raw", "beta_logit", "cu_seqlens")}
    # identity tap (current row), no activation: v passes through, q_hat = q / |q|
    w = np.zeros((C, 4)); w[:, 3] = 1.0
    p = O.prep(conv_w=w, act=O.ACT_NONE, **args)
    assert np.array_equal(p.v, x["v_raw"])
    qn = x["q_raw"] / np.sqrt((x["q_raw"] ** 2).sum(-1, keepdims=True) + O.EPS)
    np.testing.assert_allclose(p.q_hat, qn, rtol=1e-15)
    # oldest tap: row t sees x_{t-3}, reaching into the carried conv state (channel order q|k|v)
    w = np.zeros((C, 4)); w[:, 0] = 1.0
    p = O.prep(conv_w=w, act=O.ACT_NONE, **args)
    cu = x["cu_seqlens"]
    for n in range(2):
        sl = slice(cu[n], cu[n + 1])
        rows = np.concatenate([x["q_raw"][sl].reshape(-1, H * dk), x["k_raw"][sl].reshape(-1, H * dk),
                               x["v_raw"][sl].reshape(-1, H * dv)], axis=1)
        src = np.concatenate([x["conv_state"][n], rows], axis=0)  # [3 + len, C], oldest first
        for t in range(lens[n]):
            assert np.array_equal(p.v[cu[n] + t].ravel(), src[t, 2 * H * dk:])
            qs = src[t, :H * dk].reshape(H, dk)
            np.testing.assert_allclose(p.q_hat[cu[n] + t], qs / np.sqrt((qs ** 2).sum(-1, keepdims=True) + O.EPS),
                                       rtol=1e-15)
        # carried state = last 3 source rows, bit copies (reaching back into the old state for short rows)
        assert np.array_equal(p.conv_state[n], src[-3:])


def test_p9_silu_against_library(oracle_mod):
    rng = np.random.default_rng(19)
    x = _layer_inputs(rng, [20], 1, 2, 3)
    C = 1 * (2 * 2 + 3)
    w = np.zeros((C, 4)); w[:, 3] = 1.0
    p = O.prep(x["q_raw"], x["k_raw"], x["v_raw"], w, x["conv_state"], x["g_raw"], x["beta_logit"], [0, 20],
               act=O.ACT_SILU)
    np.testing.assert_allclose(p.v, x["v_raw"] * expit(x["v_raw"]), rtol=1e-15)


def test_p10_norms(oracle_mod):
    rng = np.random.default_rng(10)
    x = _layer_inputs(rng, [31], 3, 16, 8)
    L = O.layer(**x)
    kn = np.linalg.norm(L.prep.k_hat, axis=-1)
    qn = np.linalg.norm(L.prep.q_hat, axis=-1)
    assert np.all(np.abs(kn - 1) < 1e-4) and np.all(np.abs(qn - 1) < 1e-4)
    # output norm: y / (w sigmoid(z)) is o scaled to RMS sqrt(m/(m+eps)), m = mean(o^2), and parallel to o
    r = L.y / (x["norm_w"] * expit(x["z"]))
    m = np.mean(L.o ** 2, axis=-1)
    np.testing.assert_allclose(np.sqrt(np.mean(r ** 2, axis=-1)), np.sqrt(m / (m + O.EPS)), rtol=1e-12)
    cos = np.sum(r * L.o, -1) / (np.linalg.norm(r, axis=-1) * np.linalg.norm(L.o, axis=-1))
    np.testing.assert_allclose(cos, 1.0, rtol=1e-12)


# ----------------------------------------------------------------------------
# the 2e-3 tolerance is discriminative (P12)
# ----------------------------------------------------------------------------

def test_p12_negative_controls_exceed_tolerance(oracle_mod):
    rng = np.random.default_rng(12)
    x = _layer_inputs(rng, [96], 2, 32, 32)
    base = O.layer(**x, gate_mode=O.GATE_SAFE)
    swapped = O.layer(**dict(x, g_raw=x["z"], z=x["g_raw"]), gate_mode=O.GATE_SAFE)
    soft = O.layer(**x, gate_mode=O.GATE_SOFTPLUS)
    assert _rel(swapped.y, base.y) > 0.05
    assert _rel(soft.y, base.y) > 0.05
