"""Brute-force forms of the KDA recurrence -- TEST INFRASTRUCTURE ONLY.

These are deliberately different computations of the same definition, used
to pin the token-by-token oracle in ``kda_oracle.c``:

* ``product_form``: the state after T tokens written as one product of
  per-token transition matrices plus the written terms,
      S_T = M_T ... M_1 S_0 + sum_t M_T ... M_{t+1} beta_t k_t v_t^T,
      M_t = (I - beta_t k_t k_t^T) Diag(alpha_t),
  with dense numpy matrices (the update in this unexpanded form is the gated
  delta rule used for the state of the page "Ling-3.0-flash: a 124B open MoE
  that runs like a 5B and reaches for 1M tokens", section "KDA:
  constant-size memory over a very long context");
* ``product_form_exact``: the same product in exact rational arithmetic
  (``fractions.Fraction``), for tiny inputs whose decays are given directly as
  rationals;
* ``conv_reference``: the short conv as ``numpy.convolve`` per channel;
* ``scalar_recurrence``: the dk = dv = 1 special case, where the update is the
  textbook scalar recursion s_t = (1 - beta_t k_t^2) alpha_t s_{t-1} + beta_t k_t v_t.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np


def product_form(q, k, v, log_alpha, beta, S0=None):
    """Single sequence, single head: returns (o [T, dv], S_T [dk, dv]).

    o_t = S_t^T q_t, with S_t built from the full matrix product up to t.
    """
    q, k, v, la, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, log_alpha, beta))
    T, dk = k.shape
    dv = v.shape[1]
    S0 = np.zeros((dk, dv)) if S0 is None else np.asarray(S0, dtype=np.float64)
    Ms = [(np.eye(dk) - beta[t] * np.outer(k[t], k[t])) @ np.diag(np.exp(la[t])) for t in range(T)]
    o = np.zeros((T, dv))
    S_t = None
    for t in range(T):
        # S_t from scratch: prod_{i<=t} M_i S0 + sum_{s<=t} prod_{s<i<=t} M_i beta_s k_s v_s^T
        P = np.eye(dk)
        for i in range(t, -1, -1):
            P = P @ Ms[i]
        S_t = P @ S0
        for s in range(t + 1):
            Q = np.eye(dk)
            for i in range(t, s, -1):
                Q = Q @ Ms[i]
            S_t = S_t + Q @ (beta[s] * np.outer(k[s], v[s]))
        o[t] = S_t.T @ q[t]
    return o, S_t


def _fmat_mul(A, B):
    n, m, p = len(A), len(B), len(B[0])
    return [[sum((A[i][j] * B[j][c] for j in range(m)), Fraction(0)) for c in range(p)]
            for i in range(n)]


def product_form_exact(q, k, v, alpha, beta, S0=None):
    """Exact rational version of ``product_form``; alpha given directly (not log).

    All inputs are nested lists (or arrays) of numbers convertible to Fraction.
    Returns (o as list of lists of Fraction, S_T likewise).
    """
    F = Fraction
    T, dk = len(k), len(k[0])
    dv = len(v[0])
    q = [[F(x) for x in r] for r in q]
    k = [[F(x) for x in r] for r in k]
    v = [[F(x) for x in r] for r in v]
    alpha = [[F(x) for x in r] for r in alpha]
    beta = [F(x) for x in beta]
    S = [[F(0)] * dv for _ in range(dk)] if S0 is None else [[F(x) for x in r] for r in S0]
    o = []
    for t in range(T):
        M = [[((1 if i == j else 0) - beta[t] * k[t][i] * k[t][j]) * alpha[t][j] for j in range(dk)]
             for i in range(dk)]
        S = _fmat_mul(M, S)
        S = [[S[i][c] + beta[t] * k[t][i] * v[t][c] for c in range(dv)] for i in range(dk)]
        o.append([sum((S[i][c] * q[t][i] for i in range(dk)), F(0)) for c in range(dv)])
    return o, S


def conv_reference(x, w, history=None):
    """Causal 4-tap conv of one channel over one sequence with numpy.convolve.

    x: [L]; w: [4] with w[3] the current-token tap; history: None or [3]
    (oldest first).  Returns [L].
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    h = np.zeros(3) if history is None else np.asarray(history, dtype=np.float64)
    if x.shape[0] == 0:
        return np.zeros(0)
    full = np.concatenate([h, x])
    # out[tau] = sum_j w[j] full[tau + j]  ==  correlation with w
    return np.convolve(full, w[::-1], mode="valid")


def scalar_recurrence(k, v, q, alpha, beta, s0=0.0):
    """dk = dv = 1: s_t = (1 - beta_t k_t^2) alpha_t s_{t-1} + beta_t k_t v_t, o_t = s_t q_t."""
    s = float(s0)
    o = []
    for kt, vt, qt, at, bt in zip(k, v, q, alpha, beta):
        s = (1.0 - bt * kt * kt) * at * s + bt * kt * vt
        o.append(s * qt)
    return np.array(o), s
