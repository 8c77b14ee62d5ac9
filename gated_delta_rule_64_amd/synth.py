"""Seeded synthetic inputs for the KDA token mixer.

This module draws random numbers and stores them in the formats the library
consumes (bf16 bit patterns in ``uint16`` arrays, or ``float32``).  It holds
none of the mixer's arithmetic: no convolution, normalisation, gate or state
update.  The GPU tests, the bench and the CPU oracle all read what it
produces, so both sides start from bit-identical values.

Recipe (the same for every workload):

* every tensor is drawn in fp64 from ``numpy.random.PCG64`` seeded with
  ``SeedSequence([20261203, workload_id, tensor_id, block])``, where token
  tensors are drawn in blocks of 4096 token rows (so any slice can be
  regenerated and blocks are drawn in parallel threads);
* draws are rounded to fp32 and then, for bf16 workloads, to bf16, both
  round-to-nearest-even;
* ``N(mu, s)`` means mean ``mu`` and standard deviation ``s``.

Workloads (named by what they are; sizes are the defaults, every size can be
overridden for reduced parity cases):

* ``core_tiny``    1 sequence of 64 tokens, 2 heads, dk = dv = 16, fp32.  Raw
  q, k, v, gate logits ~ N(0, 1); the conv weights are the identity (only the
  current-token tap is 1), so the preprocess reduces to the L2 norm and the
  gates.  No output gate.  Zero initial state.
* ``layer_t4k``    1 sequence of 4096 tokens, 32 heads, dk = dv = 128, bf16.
  q, k, v, decay logits g, write logits b and output-gate logits z ~ N(0, 1);
  conv weights ~ N(0, 0.5).  Zero initial state.
* ``long_t256k``   as ``layer_t4k`` with 262,144 tokens; initial state fp32
  ~ N(0, 0.02).
* ``decode_b256``  256 sequences of one token each, 32 heads, d = 128, bf16
  raw inputs as ``layer_t4k``; the conv history (three earlier raw tokens per
  sequence) is drawn ~ N(0, 1) and rounded to bf16 values; fp32 state
  ~ N(0, 0.02).
* ``varlen_64``    64 sequences, lengths uniform in [1024, 32768] (inclusive)
  packed in order; bf16 inputs as ``layer_t4k``; even-indexed sequences start
  from a zero state, odd-indexed ones from fp32 ~ N(0, 0.02).
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

SEED_ROOT = 20261203
BLOCK = 4096

TENSOR_IDS = {
    "q": 0, "k": 1, "v": 2, "g": 3, "b": 4, "z": 5,
    "w_q": 6, "w_k": 7, "w_v": 8, "S0": 9, "conv_state": 10, "lengths": 11,
    # direct core inputs (already preprocessed form)
    "core_q": 20, "core_k": 21, "core_v": 22, "core_la": 23, "core_beta": 24,
    "core_z": 25, "core_S0": 26,
}


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return the bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    nan = np.isnan(x)
    if nan.any():
        r = np.where(nan, (u >> np.uint64(16)) | np.uint64(0x40), r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(u) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    u = np.ascontiguousarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(x) -> np.ndarray:
    """Exact fp64 copy of an input array (bf16 bit patterns or a float array)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return x.astype(np.float64)


def _rng(workload_id: int, tensor: str, block: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence([SEED_ROOT, workload_id, TENSOR_IDS[tensor], block])
    return np.random.Generator(np.random.PCG64(ss))


def _store(x64: np.ndarray, fmt: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return f32_to_bf16_bits(x32) if fmt == "bf16" else x32


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _token_tensor(workload_id, tensor, T, width, fmt, mean=0.0, std=1.0):
    """[T, width] tensor drawn N(mean, std) in blocks of BLOCK rows."""
    out = np.empty((T, width), dtype=np.uint16 if fmt == "bf16" else np.float32)
    nblk = (T + BLOCK - 1) // BLOCK

    def fill(blk):
        r0 = blk * BLOCK
        r1 = min(T, r0 + BLOCK)
        x = _rng(workload_id, tensor, blk).standard_normal((r1 - r0, width))
        if std != 1.0:
            x *= std
        if mean != 0.0:
            x += mean
        out[r0:r1] = _store(x, fmt)

    if nblk <= 1:
        for blk in range(nblk):
            fill(blk)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nblk)))
    return out


# --------------------------------------------------------------------------
# raw-input workloads (inputs of the preprocess)
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    name: str
    workload_id: int
    H: int
    dk: int
    dv: int
    lengths: tuple
    x_dtype: str                 # "bf16" | "f32"
    identity_conv: bool = False  # conv weights = current-token tap only
    out_gate: bool = True
    s0: str = "zero"             # "zero" | "random" | "alternate"
    s0_std: float = 0.02
    conv_w_std: float = 0.5
    conv_history: bool = False   # draw a conv history per sequence
    g_mean: float = 0.0          # mean of the decay logits (stress cases move it)
    b_mean: float = 0.0          # mean of the write logits

    @property
    def N(self) -> int:
        return len(self.lengths)

    @property
    def T_tot(self) -> int:
        return int(sum(self.lengths))


def _varlen_lengths() -> tuple:
    rng = _rng(4, "lengths")
    return tuple(int(x) for x in rng.integers(1024, 32768, endpoint=True, size=64))


WORKLOADS = {
    "core_tiny": Workload("core_tiny", 0, H=2, dk=16, dv=16, lengths=(64,), x_dtype="f32",
                          identity_conv=True, out_gate=False, s0="zero"),
    "layer_t4k": Workload("layer_t4k", 1, H=32, dk=128, dv=128, lengths=(4096,), x_dtype="bf16"),
    "long_t256k": Workload("long_t256k", 2, H=32, dk=128, dv=128, lengths=(262144,),
                           x_dtype="bf16", s0="random"),
    "decode_b256": Workload("decode_b256", 3, H=32, dk=128, dv=128, lengths=(1,) * 256,
                            x_dtype="bf16", s0="random", conv_history=True),
    "varlen_64": Workload("varlen_64", 4, H=32, dk=128, dv=128, lengths=_varlen_lengths(),
                          x_dtype="bf16", s0="alternate"),
}


def workload(name: str, **overrides) -> Workload:
    """A named workload, optionally resized (``lengths``, ``H``, ``dk``, ``dv`` ...)."""
    w = WORKLOADS[name]
    if "lengths" in overrides:
        overrides["lengths"] = tuple(int(x) for x in overrides["lengths"])
    return replace(w, **overrides) if overrides else w


def make(w: Workload | str, **overrides) -> dict:
    """Draw the raw inputs of one workload.

    Returns a dict of numpy arrays (row-major):
      cu_seqlens int32 [N+1]; q_in, k_in [T_tot, H*dk]; v_in [T_tot, H*dv];
      w_q, w_k [H*dk, 4]; w_v [H*dv, 4]; g [T_tot, H*dk]; b [T_tot, H];
      z [T_tot, H*dv] or None; S0 fp32 [N, H, dk, dv] or None;
      conv_state fp32 [N, 3, H*(2*dk+dv)] or None.
    Token tensors and weights are bf16 bit patterns (uint16) or fp32.
    """
    if isinstance(w, str):
        w = workload(w, **overrides)
    elif overrides:
        w = replace(w, **overrides)
    fmt = w.x_dtype
    H, dk, dv, T = w.H, w.dk, w.dv, w.T_tot
    wid = w.workload_id
    cu = np.zeros(w.N + 1, dtype=np.int64)
    cu[1:] = np.cumsum(np.asarray(w.lengths, dtype=np.int64))
    if cu[-1] >= 2**31:
        raise ValueError("packed token count must stay below 2^31")
    out = {"workload": w, "x_dtype": fmt, "H": H, "dk": dk, "dv": dv, "N": w.N, "T_tot": T,
           "cu_seqlens": cu.astype(np.int32)}
    out["q_in"] = _token_tensor(wid, "q", T, H * dk, fmt)
    out["k_in"] = _token_tensor(wid, "k", T, H * dk, fmt)
    out["v_in"] = _token_tensor(wid, "v", T, H * dv, fmt)
    out["g"] = _token_tensor(wid, "g", T, H * dk, fmt, mean=w.g_mean)
    out["b"] = _token_tensor(wid, "b", T, H, fmt, mean=w.b_mean)
    out["z"] = _token_tensor(wid, "z", T, H * dv, fmt) if w.out_gate else None
    for name, width in (("w_q", H * dk), ("w_k", H * dk), ("w_v", H * dv)):
        if w.identity_conv:
            x = np.zeros((width, 4))
            x[:, 3] = 1.0
        else:
            x = _rng(wid, name).standard_normal((width, 4)) * w.conv_w_std
        out[name] = _store(x, fmt)
    out["S0"] = _initial_state(w)
    if w.conv_history:
        x = _rng(wid, "conv_state").standard_normal((w.N, 3, H * (2 * dk + dv)))
        x32 = x.astype(np.float32)
        if fmt == "bf16":
            x32 = bf16_bits_to_f32(f32_to_bf16_bits(x32))
        out["conv_state"] = x32
    else:
        out["conv_state"] = None
    return out


def _initial_state(w: Workload):
    if w.s0 == "zero":
        return None
    S0 = np.zeros((w.N, w.H, w.dk, w.dv), dtype=np.float32)
    for n in range(w.N):
        if w.s0 == "alternate" and n % 2 == 0:
            continue
        S0[n] = (_rng(w.workload_id, "S0", n).standard_normal((w.H, w.dk, w.dv)) * w.s0_std)
    return S0


# --------------------------------------------------------------------------
# direct core inputs (already in the form the recurrence consumes)
# --------------------------------------------------------------------------

def core(seed: int, lengths, H: int, dk: int, dv: int, x_dtype: str = "f32",
         gate_dtype: str = "f32", decay_scale: float = 0.8, beta: str = "uniform",
         s0_std: float | None = None, out_gate: bool = False) -> dict:
    """Inputs for the chunked core alone, without the preprocess.

    q, k ~ N(0, 1/dk) (so |k|^2 is near 1 and every write is a contraction),
    v ~ N(0, 1); log decay = -Exponential(decay_scale) per channel; write
    strength ~ U(0, 1) (or all ones / all zeros); optional output-gate logits
    ~ N(0, 1); optional fp32 initial state ~ N(0, s0_std).
    Returns q, k [T, H, dk]; v [T, H, dv]; log_alpha [T, H, dk]; beta [T, H];
    z [T, H, dv] or None; S0 [N, H, dk, dv] fp32 or None; cu_seqlens int32.
    """
    lengths = [int(x) for x in lengths]
    T = int(sum(lengths))
    N = len(lengths)
    cu = np.zeros(N + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    wid = 1000 + seed

    def draw(name, shape):
        return _rng(wid, name).standard_normal(shape)

    out = {"x_dtype": x_dtype, "gate_dtype": gate_dtype, "H": H, "dk": dk, "dv": dv,
           "N": N, "T_tot": T, "cu_seqlens": cu.astype(np.int32)}
    out["q"] = _store(draw("core_q", (T, H, dk)) / np.sqrt(dk), x_dtype)
    out["k"] = _store(draw("core_k", (T, H, dk)) / np.sqrt(dk), x_dtype)
    out["v"] = _store(draw("core_v", (T, H, dv)), x_dtype)
    la = -_rng(wid, "core_la").exponential(decay_scale, (T, H, dk)) if decay_scale > 0 \
        else np.zeros((T, H, dk))
    out["log_alpha"] = _store(la, gate_dtype)
    if beta == "uniform":
        bt = _rng(wid, "core_beta").uniform(0.0, 1.0, (T, H))
    elif beta == "one":
        bt = np.ones((T, H))
    elif beta == "zero":
        bt = np.zeros((T, H))
    else:
        raise ValueError(beta)
    out["beta"] = _store(bt, gate_dtype)
    out["z"] = _store(draw("core_z", (T, H, dv)), x_dtype) if out_gate else None
    if s0_std:
        out["S0"] = (_rng(wid, "core_S0").standard_normal((N, H, dk, dv)) * s0_std).astype(np.float32)
    else:
        out["S0"] = None
    return out
