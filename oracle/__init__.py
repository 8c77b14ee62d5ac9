"""CPU oracle for the KDA token mixer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the bench's CPU-baseline leg
may import this package.  The GPU library and its Python binding never do,
and this package imports nothing from them.

``kda_oracle.c`` is a plain fp64, token-by-token implementation (see its
header for what it follows and the readings it takes); this module compiles
it with gcc, loads it with ctypes and converts numpy inputs to fp64.
``brute.py`` holds independent brute-force forms used to pin it.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle library (plain gcc, IEEE semantics, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
                               "-pthread", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        lp = ctypes.POINTER(ctypes.c_int64)
        i64, i32 = ctypes.c_int64, ctypes.c_int
        lib.kdao_preprocess.argtypes = [i64, i32, i32, i32, lp, i32] + [dp] * 8 + [dp, dp] + \
            [dp] * 5 + [i32]
        lib.kdao_preprocess.restype = i32
        lib.kdao_recurrence.argtypes = [i64, i32, i32, i32, lp, i32] + [dp] * 7 + [dp, dp, i32]
        lib.kdao_recurrence.restype = i32
        lib.kdao_recurrence_backward.argtypes = [i64, i32, i32, i32, lp, i32] + [dp] * 9 + [dp] * 7 + [i32]
        lib.kdao_recurrence_backward.restype = i32
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    if x is None:
        return None
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _cu(cu_seqlens, T):
    if cu_seqlens is None:
        return np.array([0, T], dtype=np.int64)
    return np.ascontiguousarray(cu_seqlens, dtype=np.int64)


def preprocess(q_in, k_in, v_in, w_q, w_k, w_v, g, b, H, dk, dv, cu_seqlens=None,
               conv_state=None, want_conv_state=False, nthreads=None):
    """Short conv, L2 norm and gates of a packed batch, in fp64.

    q_in, k_in, g: [T, H*dk]; v_in: [T, H*dv]; w_*: [H*d, 4]; b: [T, H];
    conv_state: None or [N, 3, H*(2dk+dv)].
    Returns dict q, k [T, H, dk], v [T, H, dv], log_alpha [T, H, dk], beta [T, H]
    and conv_state [N, 3, H*(2dk+dv)] when asked for.
    """
    q_in, k_in, v_in, w_q, w_k, w_v, g, b = (_f64(x) for x in (q_in, k_in, v_in, w_q, w_k, w_v, g, b))
    T = q_in.shape[0]
    cu = _cu(cu_seqlens, T)
    N = cu.shape[0] - 1
    assert q_in.shape == (T, H * dk) and k_in.shape == (T, H * dk) and v_in.shape == (T, H * dv)
    assert g.shape == (T, H * dk) and b.shape == (T, H)
    cs_in = _f64(conv_state)
    cs_width = H * (2 * dk + dv)
    if cs_in is not None:
        assert cs_in.shape == (N, 3, cs_width)
    out = {
        "q": np.empty((T, H, dk)), "k": np.empty((T, H, dk)), "v": np.empty((T, H, dv)),
        "log_alpha": np.empty((T, H, dk)), "beta": np.empty((T, H)),
    }
    cs_out = np.empty((N, 3, cs_width)) if want_conv_state else None
    rc = _load().kdao_preprocess(
        T, H, dk, dv, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), N,
        _ptr(q_in), _ptr(k_in), _ptr(v_in), _ptr(w_q), _ptr(w_k), _ptr(w_v), _ptr(g), _ptr(b),
        _ptr(cs_in), _ptr(cs_out),
        _ptr(out["q"]), _ptr(out["k"]), _ptr(out["v"]), _ptr(out["log_alpha"]), _ptr(out["beta"]),
        nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle preprocess rejected its arguments")
    if want_conv_state:
        out["conv_state"] = cs_out
    return out


def recurrence(q, k, v, log_alpha, beta, z=None, S0=None, cu_seqlens=None, nthreads=None):
    """Token-by-token gated delta rule over a packed batch, in fp64.

    q, k, log_alpha: [T, H, dk]; v: [T, H, dv]; beta: [T, H];
    z: None or [T, H, dv] output-gate logits; S0: None or [N, H, dk, dv].
    Returns (y [T, H, dv], S_final [N, H, dk, dv]).
    """
    q, k, v, log_alpha, beta, z, S0 = (_f64(x) for x in (q, k, v, log_alpha, beta, z, S0))
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = _cu(cu_seqlens, T)
    N = cu.shape[0] - 1
    assert k.shape == (T, H, dk) and log_alpha.shape == (T, H, dk)
    assert v.shape == (T, H, dv) and beta.shape == (T, H)
    if z is not None:
        assert z.shape == (T, H, dv)
    if S0 is not None:
        assert S0.shape == (N, H, dk, dv)
    y = np.empty((T, H, dv))
    S = np.empty((N, H, dk, dv))
    rc = _load().kdao_recurrence(
        T, H, dk, dv, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), N,
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(z), _ptr(S0),
        _ptr(y), _ptr(S), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle recurrence rejected its arguments")
    return y, S


def recurrence_backward(q, k, v, log_alpha, beta, dy, z=None, S0=None, dS_final=None, cu_seqlens=None,
                        nthreads=None):
    """Gradients of the recurrence (reverse mode, fp64) for a loss with
    gradients dy [T, H, dv] on the outputs and dS_final (None: zero) on the
    final states.  Returns a dict with dq, dk, dlog_alpha [T, H, dk], dv
    [T, H, dv], dbeta [T, H], dz [T, H, dv] (None without z) and dS0
    [N, H, dk, dv] (the gradient with respect to the initial states)."""
    q, k, v, log_alpha, beta, dy, z, S0, dS_final = (
        _f64(x) for x in (q, k, v, log_alpha, beta, dy, z, S0, dS_final))
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = _cu(cu_seqlens, T)
    N = cu.shape[0] - 1
    assert dy.shape == (T, H, dv)
    out = {"dq": np.empty((T, H, dk)), "dk": np.empty((T, H, dk)), "dv": np.empty((T, H, dv)),
           "dlog_alpha": np.empty((T, H, dk)), "dbeta": np.empty((T, H)),
           "dz": np.empty((T, H, dv)) if z is not None else None, "dS0": np.empty((N, H, dk, dv))}
    rc = _load().kdao_recurrence_backward(
        T, H, dk, dv, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), N,
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(z), _ptr(S0), _ptr(dy), _ptr(dS_final),
        _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dlog_alpha"]), _ptr(out["dbeta"]),
        _ptr(out["dz"]), _ptr(out["dS0"]), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle backward rejected its arguments")
    return out


def layer(inputs: dict, nthreads=None, want_conv_state=False):
    """Preprocess then recurrence, from a dict of fp64-convertible raw inputs.

    ``inputs`` holds q_in, k_in, v_in, w_q, w_k, w_v, g, b, z (or None),
    S0 (or None), conv_state (or None), cu_seqlens, H, dk, dv -- every array
    already widened to a float dtype by the caller.
    Returns dict with y, S, and the preprocessed tensors.
    """
    p = preprocess(inputs["q_in"], inputs["k_in"], inputs["v_in"], inputs["w_q"], inputs["w_k"],
                   inputs["w_v"], inputs["g"], inputs["b"], inputs["H"], inputs["dk"], inputs["dv"],
                   cu_seqlens=inputs["cu_seqlens"], conv_state=inputs.get("conv_state"),
                   want_conv_state=want_conv_state, nthreads=nthreads)
    z = inputs.get("z")
    if z is not None:
        z = _f64(z).reshape(p["v"].shape)
    y, S = recurrence(p["q"], p["k"], p["v"], p["log_alpha"], p["beta"], z=z, S0=inputs.get("S0"),
                      cu_seqlens=inputs["cu_seqlens"], nthreads=nthreads)
    p["y"] = y
    p["S"] = S
    return p
