"""Planted mistakes in the oracle must be caught by its pins.

Each case copies ``oracle/kda_oracle.c`` to a temporary directory, plants one
plausible mistake (a dropped term, a wrong sign, a swapped operand, a wrong
index), compiles it with gcc and runs the brute-force and library pins on
it.  The mutant must fail at least one of them, while the real oracle passes
all of them.  Everything runs on the CPU.
"""

import ctypes
import os
import subprocess

import numpy as np
import pytest
from scipy.special import expit

from oracle import brute

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kda_oracle.c")

MUTANTS = {
    "decay_squared": ("row[j] *= a;", "row[j] *= a * a;"),
    "decay_sign": ("double a = exp(lat[i]);", "double a = exp(-0.5 * lat[i]);"),
    "u_reads_query": ("u[j] += row[j] * kt[i];", "u[j] += row[j] * qt[i];"),
    "write_sign": ("row[j] += bk * (vt[j] - u[j]);", "row[j] += bk * (vt[j] + u[j]);"),
    "write_drops_erase": ("row[j] += bk * (vt[j] - u[j]);", "row[j] += bk * vt[j];"),
    "beta_dropped": ("double bk = bt * kt[i];", "double bk = kt[i];"),
    "read_uses_key": ("yt[j] += row[j] * qt[i];", "yt[j] += row[j] * kt[i];"),
    "gate_not_sigmoid": ("yt[j] *= sigmoid(zt[j]);", "yt[j] *= zt[j];"),
    "conv_taps_reversed": ("acc += wc[j] * raw_at(", "acc += wc[3 - j] * raw_at("),
    "history_reversed": ("[((int64_t)n * 3 + (3 + tau)) * cs_width", "[((int64_t)n * 3 + (-1 - tau)) * cs_width"),
    "l2_eps_large": ("#define L2_EPS 1e-6", "#define L2_EPS 1e-1"),
    "decay_not_negated": ("P->la_out[idx] = -softplus(", "P->la_out[idx] = softplus("),
    "beta_is_identity": ("P->beta_out[t * H + h] = sigmoid(P->b[t * H + h]);",
                         "P->beta_out[t * H + h] = P->b[t * H + h];"),
    "state_transposed": ("const double* s0 = R->S0 ? R->S0 + ((int64_t)n * H + h) * (int64_t)sdim : NULL;\n"
                         "    for (size_t i = 0; i < sdim; ++i) S[i] = s0 ? s0[i] : 0.0;",
                         "const double* s0 = R->S0 ? R->S0 + ((int64_t)n * H + h) * (int64_t)sdim : NULL;\n"
                         "    for (size_t i = 0; i < sdim; ++i) S[i] = s0 ? s0[(i % dv) * dk + i / dv] : 0.0;"),
}


def build(tmp_path, name, src_text):
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"{name}.so"
    c.write_text(src_text)
    subprocess.check_call(["gcc", "-O1", "-shared", "-fPIC", "-pthread", "-o", str(so), str(c), "-lm"])
    lib = ctypes.CDLL(str(so))
    dp = ctypes.POINTER(ctypes.c_double)
    lp = ctypes.POINTER(ctypes.c_int64)
    i64, i32 = ctypes.c_int64, ctypes.c_int
    lib.kdao_preprocess.argtypes = [i64, i32, i32, i32, lp, i32] + [dp] * 15 + [i32]
    lib.kdao_recurrence.argtypes = [i64, i32, i32, i32, lp, i32] + [dp] * 9 + [i32]
    return lib


def P(x):
    return None if x is None else x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def pins_hold(lib):
    """Runs the brute-force / library pins against a compiled oracle; True if all hold."""
    r = np.random.default_rng(5)
    ok = True
    # recurrence vs product expansion (dk != dv, non-symmetric S0, output gate)
    T, H, dk, dv = 6, 2, 5, 3
    q = r.standard_normal((T, H, dk))
    k = r.standard_normal((T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((T, H, dv))
    la = -r.exponential(0.5, (T, H, dk))
    b = r.uniform(0, 1, (T, H))
    S0 = r.standard_normal((1, H, dk, dv))
    z = r.standard_normal((T, H, dv))
    y = np.empty((T, H, dv))
    S = np.empty((1, H, dk, dv))
    cu = np.array([0, T], dtype=np.int64)
    lib.kdao_recurrence(T, H, dk, dv, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), 1,
                        P(q), P(k), P(v), P(la), P(b), P(z), P(S0), P(y), P(S), 1)
    for h in range(H):
        o, ST = brute.product_form(q[:, h], k[:, h], v[:, h], la[:, h], b[:, h], S0=S0[0, h])
        ok &= np.allclose(S[0, h], ST, rtol=1e-10, atol=1e-12)
        ok &= np.allclose(y[:, h], o * expit(z[:, h]), rtol=1e-10, atol=1e-12)
    # preprocess vs numpy.convolve / linalg.norm / logaddexp / expit, with history
    T, H, dk, dv = 7, 2, 4, 3
    lengths = [5, 2]
    cu = np.array([0, 5, 7], dtype=np.int64)
    N = 2
    raw = {nm: r.standard_normal((T, H * d)) for nm, d in (("q", dk), ("k", dk), ("v", dv), ("g", dk))}
    raw["b"] = r.standard_normal((T, H))
    w = {nm: r.standard_normal((H * d, 4)) for nm, d in (("q", dk), ("k", dk), ("v", dv))}
    cs = r.standard_normal((N, 3, H * (2 * dk + dv)))
    outs = {nm: np.empty((T, H, d)) for nm, d in (("q", dk), ("k", dk), ("v", dv), ("la", dk))}
    beta = np.empty((T, H))
    cs_out = np.empty_like(cs)
    lib.kdao_preprocess(T, H, dk, dv, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), N,
                        P(raw["q"]), P(raw["k"]), P(raw["v"]), P(w["q"]), P(w["k"]), P(w["v"]),
                        P(raw["g"]), P(raw["b"]), P(cs), P(cs_out), P(outs["q"]), P(outs["k"]),
                        P(outs["v"]), P(outs["la"]), P(beta), 1)
    offs = {"q": 0, "k": H * dk, "v": 2 * H * dk}
    for nm, d in (("q", dk), ("k", dk), ("v", dv)):
        for n in range(N):
            s, e = cu[n], cu[n + 1]
            pre = np.stack([brute.conv_reference(raw[nm][s:e, c], w[nm][c], cs[n, :, offs[nm] + c])
                            for c in range(H * d)], axis=1).reshape(e - s, H, d)
            if nm != "v":
                pre = pre / np.sqrt(np.sum(pre * pre, axis=-1, keepdims=True) + 1e-6)
            ok &= np.allclose(outs[nm][s:e], pre, rtol=1e-12, atol=1e-13)
    ok &= np.allclose(outs["la"].reshape(T, H * dk), -np.logaddexp(0.0, raw["g"]), rtol=1e-13)
    ok &= np.allclose(beta, expit(raw["b"]), rtol=1e-13)
    return bool(ok)


def test_real_oracle_passes(tmp_path):
    assert pins_hold(build(tmp_path, "real", open(SRC).read()))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not found exactly once"
    lib = build(tmp_path, name, text.replace(old, new))
    with np.errstate(all="ignore"):
        assert not pins_hold(lib), f"planted mistake {name} was not caught"
