"""Gradients of the chunked recurrence on the GPU against the oracle's fp64
reverse-mode gradients (themselves pinned to finite differences of the
forward oracle), on the same seeded inputs and output gradients."""

import numpy as np
import pytest
import torch

from gated_delta_rule_64_amd import synth
from kda_helpers import TOL, assert_close, f64, to_dev, to_host64

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dz", "dS0")


@pytest.fixture(scope="module")
def K():
    from gated_delta_rule_64_amd import kda
    return kda


def _grads(seed, c, with_dsf):
    """Output gradients: dy ~ N(0, 1), optional dS_final ~ N(0, 0.1)."""
    rng = np.random.default_rng(seed)
    T, H, dv = c["v"].shape
    N = len(c["cu_seqlens"]) - 1
    dk = c["q"].shape[2]
    dy = rng.standard_normal((T, H, dv)).astype(np.float32)
    if c["q"].dtype == np.uint16:  # bf16 run: dy in bf16 too
        dy = synth.f32_to_bf16_bits(dy)
    dSf = (rng.standard_normal((N, H, dk, dv)) * 0.1).astype(np.float32) if with_dsf else None
    return dy, dSf


def _check(K, oracle_mod, c, dy, dSf, tol, heads=None):
    g = K.kda_prefill_backward(*(to_dev(c[n]) for n in ("q", "k", "v", "log_alpha", "beta")), to_dev(dy),
                               out_gate=to_dev(c["z"]), initial_state=to_dev(c["S0"]), dS_final=to_dev(dSf),
                               cu_seqlens=to_dev(c["cu_seqlens"]))
    torch.cuda.synchronize()
    hs = slice(None) if heads is None else slice(0, heads)
    sub = lambda x: None if x is None else f64(x)[:, hs]  # token-major tensors: [T, H, ...]
    subn = lambda x: None if x is None else f64(x)[:, hs]  # state tensors: [N, H, ...]
    ref = oracle_mod.recurrence_backward(sub(c["q"]), sub(c["k"]), sub(c["v"]), sub(c["log_alpha"]),
                                         sub(c["beta"]), sub(dy), z=sub(c["z"]), S0=subn(c["S0"]),
                                         dS_final=subn(dSf), cu_seqlens=c["cu_seqlens"])
    for name in NAMES:
        if ref[name] is None:
            assert g[name] is None
            continue
        got = to_host64(g[name])[:, hs]
        assert_close(name, got, ref[name], tol)


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 128)])
def test_backward_f32_matches_oracle(K, oracle_mod, dk, dv):
    lengths = [70, 1, 130, 64, 0, 5]
    c = synth.core(31, lengths, 2, dk, dv, x_dtype="f32", s0_std=0.3, out_gate=True)
    dy, dSf = _grads(32, c, True)
    print(f"backward f32 dk={dk} dv={dv}", flush=True)
    _check(K, oracle_mod, c, dy, dSf, 1e-4)


def test_backward_without_gate_state_or_final_gradient(K, oracle_mod):
    c = synth.core(33, [100, 28], 3, 64, 64, x_dtype="f32")
    dy, _ = _grads(34, c, False)
    _check(K, oracle_mod, c, dy, None, 1e-4)


@pytest.mark.parametrize("gate_dtype", ["f32", "bf16"])
def test_backward_bf16_inputs(K, oracle_mod, gate_dtype):
    c = synth.core(35, [200, 57], 2, 128, 128, x_dtype="bf16", gate_dtype=gate_dtype, s0_std=0.3, out_gate=True)
    dy, dSf = _grads(36, c, True)
    print(f"backward bf16 gate={gate_dtype}", flush=True)
    _check(K, oracle_mod, c, dy, dSf, TOL["bf16"])


def test_backward_strong_decay(K, oracle_mod):
    """Decays strong enough that e^{G} underflows inside a chunk: the
    pairwise factors are formed from differences, so nothing overflows."""
    c = synth.core(37, [192], 2, 32, 32, x_dtype="f32", decay_scale=6.0, s0_std=0.3, out_gate=True)
    dy, dSf = _grads(38, c, True)
    _check(K, oracle_mod, c, dy, dSf, 1e-4)


def test_backward_layer_shape_t4k(K, oracle_mod):
    """The 4096-token, 32-head, d = 128 bf16 layer in the launch configuration
    the bench times; heads are independent, so the oracle checks heads 0-3."""
    c = synth.core(39, [4096], 32, 128, 128, x_dtype="bf16", s0_std=0.02, out_gate=True)
    dy, dSf = _grads(40, c, True)
    print("backward t4k full size, heads 0-3 checked", flush=True)
    _check(K, oracle_mod, c, dy, dSf, TOL["bf16"], heads=4)
