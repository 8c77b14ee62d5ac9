"""Decode step on the GPU against the fp64 oracle (same seeded inputs)."""

import numpy as np
import pytest
import torch

from gated_delta_rule_64_amd import synth
from kda_helpers import TOL, assert_close, f64, oracle_layer_inputs, to_dev, to_host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    from gated_delta_rule_64_amd import kda
    return kda


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 16), (16, 128), (128, 128)])
@pytest.mark.parametrize("x_dtype,gate_dtype", [("f32", "f32"), ("bf16", "f32"), ("bf16", "bf16"), ("f32", "bf16")])
def test_decode_matches_oracle(K, oracle_mod, dk, dv, x_dtype, gate_dtype):
    B, H = 5, 3
    inp = synth.core(11, [1] * B, H, dk, dv, x_dtype=x_dtype, gate_dtype=gate_dtype, s0_std=0.5, out_gate=True)
    print(f"decode dk={dk} dv={dv} x={x_dtype} gate={gate_dtype}", flush=True)
    state = to_dev(inp["S0"]).clone()
    out = K.kda_decode_step(to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"]), to_dev(inp["log_alpha"]),
                            to_dev(inp["beta"]), state, out_gate=to_dev(inp["z"]))
    torch.cuda.synchronize()
    y, S = oracle_mod.recurrence(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["log_alpha"]),
                                 f64(inp["beta"]), z=f64(inp["z"]), S0=f64(inp["S0"]),
                                 cu_seqlens=inp["cu_seqlens"])
    tol = TOL[x_dtype] if gate_dtype == x_dtype or x_dtype == "bf16" else TOL["f32"]
    assert_close("y", to_host64(out), y, tol)
    assert_close("state", to_host64(state), S, tol)


def test_decode_without_gate_and_zero_batch(K, oracle_mod):
    inp = synth.core(12, [1] * 4, 2, 128, 128, x_dtype="f32", s0_std=0.3)
    state = to_dev(inp["S0"]).clone()
    out = K.kda_decode_step(to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"]), to_dev(inp["log_alpha"]),
                            to_dev(inp["beta"]), state)
    torch.cuda.synchronize()
    y, S = oracle_mod.recurrence(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["log_alpha"]),
                                 f64(inp["beta"]), S0=f64(inp["S0"]), cu_seqlens=inp["cu_seqlens"])
    assert_close("y", to_host64(out), y, TOL["f32"])
    assert_close("state", to_host64(state), S, TOL["f32"])
    empty = torch.empty((0, 2, 128), device="cuda")
    K.kda_decode_step(empty, empty, empty, empty, torch.empty((0, 2), device="cuda"),
                      torch.empty((0, 2, 128, 128), device="cuda"))


def test_decode_workload_b256_through_preprocess(K, oracle_mod):
    """256 sequences x 32 heads x 128^2 fp32 state: raw bf16 tokens with a conv
    history go through the preprocess (T = 1 per sequence), then one decode
    step updates the state in place.  Same launch configuration as the bench."""
    inp = synth.make("decode_b256")
    H, dk, dv, B = inp["H"], inp["dk"], inp["dv"], inp["N"]
    print("decode_b256 full size", flush=True)
    cu = to_dev(inp["cu_seqlens"])
    cs = to_dev(inp["conv_state"]).clone()
    q, k, v, la, beta = K.kda_preprocess(to_dev(inp["q_in"]), to_dev(inp["k_in"]), to_dev(inp["v_in"]),
                                         to_dev(inp["w_q"]), to_dev(inp["w_k"]), to_dev(inp["w_v"]),
                                         to_dev(inp["g"]), to_dev(inp["b"]), H, dk, dv, cu_seqlens=cu,
                                         conv_state=cs)
    state = to_dev(inp["S0"]).clone()
    z = to_dev(inp["z"]).view(B, H, dv)
    out = K.kda_decode_step(q, k, v, la, beta, state, out_gate=z)
    torch.cuda.synchronize()
    ref = oracle_mod.layer(oracle_layer_inputs(inp), want_conv_state=True)
    assert_close("y", to_host64(out), ref["y"], TOL["bf16"])
    assert_close("state", to_host64(state), ref["S"], TOL["bf16"])
    assert np.array_equal(cs.cpu().numpy().astype(np.float64), ref["conv_state"])
