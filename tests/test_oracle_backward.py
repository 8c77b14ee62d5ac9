"""Pins of the oracle's backward (CPU): every gradient it returns must match
central finite differences of the forward oracle, a different code path
(the forward is pinned on its own in test_oracle_pins.py).  The loss is
L = sum(dy * y) + sum(dS_final * S_final) with fixed random dy, dS_final,
so dL/dx is exactly what the backward is asked for."""

import numpy as np
import pytest

pytestmark = pytest.mark.parametrize("with_gate", [False, True])


def _case(seed, lengths, H, dk, dv):
    rng = np.random.default_rng(seed)
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    N = len(lengths)
    k = rng.standard_normal((T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)  # unit keys, as after the L2 norm
    x = {"q": rng.standard_normal((T, H, dk)) / np.sqrt(dk), "k": k,
         "v": rng.standard_normal((T, H, dv)), "log_alpha": -rng.exponential(0.5, (T, H, dk)),
         "beta": rng.uniform(0.1, 0.9, (T, H)), "z": rng.standard_normal((T, H, dv)),
         "S0": rng.standard_normal((N, H, dk, dv)) * 0.5}
    dy = rng.standard_normal((T, H, dv))
    dSf = rng.standard_normal((N, H, dk, dv))
    return x, dy, dSf, cu


def _loss(oracle_mod, x, dy, dSf, cu, with_gate):
    y, S = oracle_mod.recurrence(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"],
                                 z=x["z"] if with_gate else None, S0=x["S0"], cu_seqlens=cu, nthreads=1)
    return float(np.sum(dy * y) + np.sum(dSf * S))


def test_backward_matches_finite_differences(oracle_mod, with_gate):
    x, dy, dSf, cu = _case(3, [4, 1, 3], 2, 3, 2)
    g = oracle_mod.recurrence_backward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], dy,
                                       z=x["z"] if with_gate else None, S0=x["S0"], dS_final=dSf,
                                       cu_seqlens=cu, nthreads=1)
    names = {"q": "dq", "k": "dk", "v": "dv", "log_alpha": "dlog_alpha", "beta": "dbeta", "S0": "dS0"}
    if with_gate:
        names["z"] = "dz"
    eps = 1e-6
    for name, gname in names.items():
        fd = np.empty_like(x[name])
        flat = x[name].reshape(-1)
        for i in range(flat.size):
            keep = flat[i]
            flat[i] = keep + eps
            lp = _loss(oracle_mod, x, dy, dSf, cu, with_gate)
            flat[i] = keep - eps
            lm = _loss(oracle_mod, x, dy, dSf, cu, with_gate)
            flat[i] = keep
            fd.reshape(-1)[i] = (lp - lm) / (2 * eps)
        err = np.max(np.abs(g[gname] - fd)) / max(np.max(np.abs(fd)), 1e-12)
        assert err < 1e-7, (gname, err)


def test_backward_without_final_state_gradient(oracle_mod, with_gate):
    """dS_final omitted means zero: equal to passing zeros explicitly."""
    x, dy, dSf, cu = _case(4, [5], 1, 4, 3)
    z = x["z"] if with_gate else None
    a = oracle_mod.recurrence_backward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], dy, z=z, S0=x["S0"],
                                       cu_seqlens=cu)
    b = oracle_mod.recurrence_backward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], dy, z=z, S0=x["S0"],
                                       dS_final=np.zeros_like(dSf), cu_seqlens=cu)
    for key in ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dS0"):
        assert np.array_equal(a[key], b[key])
