"""Brute-force matrix-product evaluation of the gated delta rule for short rows.

TEST INFRASTRUCTURE ONLY (a second, independent statement of the recurrence
used to pin the C oracle; never called by the product path).

The recurrence (gated delta rule with per-key-dim decay, the form the KDA layer
uses; TensorFold issue #850 names it "the delta rule" inside the shared KDA
module) is written as a product of d_k x d_k transition matrices
    M_t = (I - b_t k_t k_t^T) Diag(a_t),
so that
    S_t = M_t S_{t-1} + b_t k_t v_t^T
        = (M_t ... M_1) S_0 + sum_{i<=t} (M_t ... M_{i+1}) b_i k_i v_i^T,
    o_t = S_t^T q_t.
Every S_t is formed from that closed sum with explicit matrix products, not by
stepping the recurrence, so a mistake in either statement shows as a mismatch.
"""
from __future__ import annotations

import numpy as np


def transition(k, a, b):
    """M = (I - b k k^T) Diag(a), a d_k x d_k matrix."""
    k = np.asarray(k, dtype=np.float64)
    dk = k.shape[0]
    return (np.eye(dk) - b * np.outer(k, k)) @ np.diag(np.asarray(a, dtype=np.float64))


def states_by_products(q, k, v, a, b, S0):
    """One (sequence, head): q,k,a [T,dk], v [T,dv], b [T], S0 [dk,dv].

    Returns (o [T,dv], S_T [dk,dv]) built from the closed-form sum of products."""
    q, k, v, a, b, S0 = (np.asarray(x, dtype=np.float64) for x in (q, k, v, a, b, S0))
    T, dk = k.shape
    if T > 8:
        raise ValueError("brute force is meant for T <= 8")
    M = [transition(k[t], a[t], b[t]) for t in range(T)]
    o = np.zeros((T, v.shape[1]))
    S_t = S0
    for t in range(T):
        # (M_t ... M_1) S_0
        prod = np.eye(dk)
        for j in range(t, -1, -1):
            prod = prod @ M[j]
        S_t = prod @ S0
        # + sum_i (M_t ... M_{i+1}) b_i k_i v_i^T
        for i in range(t + 1):
            tail = np.eye(dk)
            for j in range(t, i, -1):
                tail = tail @ M[j]
            S_t = S_t + tail @ (b[i] * np.outer(k[i], v[i]))
        o[t] = S_t.T @ q[t]
    return o, S_t
