"""The fused decode layer (preprocess of one raw token + decode step in one
call, states in a pool) on the GPU, against the fp64 oracle run on the same
seeded inputs: the oracle's layer with one-token sequences is the same
computation (conv over the stored history, norm, gates, one recurrence step).
"""

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


def _decode_inputs(B, H, dk, dv, x_dtype, **kw):
    """One raw token per sequence, a drawn conv history and initial state."""
    return synth.make("decode_b256", lengths=(1,) * B, H=H, dk=dk, dv=dv, x_dtype=x_dtype, **kw)


def _call(K, inp, cs, state, idx=None):
    H, dk, dv = inp["H"], inp["dk"], inp["dv"]
    z = inp["z"]
    return K.kda_decode_layer(to_dev(inp["q_in"]), to_dev(inp["k_in"]), to_dev(inp["v_in"]),
                              to_dev(inp["w_q"]), to_dev(inp["w_k"]), to_dev(inp["w_v"]),
                              to_dev(inp["g"]), to_dev(inp["b"]), H, dk, dv, cs, state,
                              out_gate=None if z is None else to_dev(z), state_indices=idx)


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 16), (16, 128), (128, 128)])
@pytest.mark.parametrize("x_dtype", ["f32", "bf16"])
def test_decode_layer_matches_oracle(K, oracle_mod, dk, dv, x_dtype):
    B, H = 5, 3
    inp = _decode_inputs(B, H, dk, dv, x_dtype)
    print(f"decode_layer dk={dk} dv={dv} x={x_dtype}", flush=True)
    cs = to_dev(inp["conv_state"]).clone()
    state = to_dev(inp["S0"]).clone()
    out = _call(K, inp, cs, state)
    torch.cuda.synchronize()
    ref = oracle_mod.layer(oracle_layer_inputs(inp), want_conv_state=True)
    tol = TOL[x_dtype]
    assert_close("y", to_host64(out), ref["y"].reshape(B, H, dv), tol)
    assert_close("state", to_host64(state), ref["S"], tol)
    # the history is rolled by plain copies of raw values: exact
    assert np.array_equal(cs.cpu().numpy().astype(np.float64), ref["conv_state"])


def test_decode_layer_without_gate_and_empty_batch(K, oracle_mod):
    B, H, dk, dv = 4, 2, 64, 128
    inp = _decode_inputs(B, H, dk, dv, "f32", out_gate=False)
    cs = to_dev(inp["conv_state"]).clone()
    state = to_dev(inp["S0"]).clone()
    out = _call(K, inp, cs, state)
    torch.cuda.synchronize()
    ref = oracle_mod.layer(oracle_layer_inputs(inp), want_conv_state=True)
    assert_close("y", to_host64(out), ref["y"].reshape(B, H, dv), TOL["f32"])
    assert_close("state", to_host64(state), ref["S"], TOL["f32"])
    e = torch.empty((0, H * dk), device="cuda")
    w = torch.zeros((H * dk, 4), device="cuda")
    out0 = K.kda_decode_layer(e, e, torch.empty((0, H * dv), device="cuda"), w, w,
                              torch.zeros((H * dv, 4), device="cuda"), e, torch.empty((0, H), device="cuda"),
                              H, dk, dv, torch.empty((0, 3, H * (2 * dk + dv)), device="cuda"),
                              torch.empty((0, H, dk, dv), device="cuda"))
    torch.cuda.synchronize()
    assert out0.shape == (0, H, dv)


def test_decode_layer_state_pool(K, oracle_mod):
    """Rows reach their state through state_indices into a larger pool; an
    index outside the pool marks a padding row (zero output, nothing read or
    written); pool slots no row names stay bit-identical."""
    B, H, dk, dv, slots = 7, 4, 128, 64, 13
    idx = np.array([9, -1, 2, 12, 13, 0, 5], dtype=np.int32)
    valid = (idx >= 0) & (idx < slots)
    inp = _decode_inputs(B, H, dk, dv, "bf16")
    rng = np.random.default_rng(2024)
    pool = (rng.standard_normal((slots, H, dk, dv)) * 0.05).astype(np.float32)
    cpool = inp["conv_state"][0][None].repeat(slots, 0) + rng.standard_normal((slots, 3, H * (2 * dk + dv)))
    cpool = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(cpool.astype(np.float32)))  # raw bf16 tokens
    print("decode_layer pool", idx.tolist(), flush=True)
    st = to_dev(pool).clone()
    cs = to_dev(cpool).clone()
    out = _call(K, inp, cs, st, idx=to_dev(idx))
    torch.cuda.synchronize()
    # the oracle on the rows that have a state, each starting from its slot
    sel = np.where(valid)[0]
    ref_in = oracle_layer_inputs(inp)
    for key in ("q_in", "k_in", "v_in", "g", "b", "z"):
        ref_in[key] = ref_in[key][sel]
    ref_in["cu_seqlens"] = np.arange(len(sel) + 1, dtype=np.int64)
    ref_in["S0"] = f64(pool[idx[sel]])
    ref_in["conv_state"] = f64(cpool[idx[sel]])
    ref = oracle_mod.layer(ref_in, want_conv_state=True)
    out_h = to_host64(out)
    assert_close("y", out_h[sel], ref["y"].reshape(len(sel), H, dv), TOL["bf16"])
    assert np.all(out_h[~valid] == 0.0)
    st_h = st.cpu().numpy()
    cs_h = cs.cpu().numpy()
    assert_close("state", st_h[idx[sel]].astype(np.float64), ref["S"], TOL["bf16"])
    assert np.array_equal(cs_h[idx[sel]].astype(np.float64), ref["conv_state"])
    untouched = np.setdiff1d(np.arange(slots), idx[sel])
    assert np.array_equal(st_h[untouched], pool[untouched])
    assert np.array_equal(cs_h[untouched], cpool[untouched])


def test_decode_layer_steps_roll_the_history(K, oracle_mod):
    """Six calls in a row, one token each, equal the oracle's layer over the
    six-token sequences: the conv history and the state carry across calls."""
    B, H, dk, dv, steps = 4, 2, 32, 32, 6
    inp = synth.make("decode_b256", lengths=(steps,) * B, H=H, dk=dk, dv=dv, x_dtype="f32")
    cs = to_dev(inp["conv_state"]).clone()
    state = to_dev(inp["S0"]).clone()
    starts = inp["cu_seqlens"][:-1]
    outs = []
    for t in range(steps):
        rows = {key: inp[key][starts + t] for key in ("q_in", "k_in", "v_in", "g", "b", "z")}
        step_inp = dict(inp, **rows)
        outs.append(to_host64(_call(K, step_inp, cs, state)))
    torch.cuda.synchronize()
    ref = oracle_mod.layer(oracle_layer_inputs(inp), want_conv_state=True)
    y_ref = ref["y"].reshape(B, steps, H, dv)
    assert_close("y", np.stack(outs, axis=1), y_ref, TOL["f32"])
    assert_close("state", to_host64(state), ref["S"], TOL["f32"])
    assert np.array_equal(cs.cpu().numpy().astype(np.float64), ref["conv_state"])


def test_decode_layer_b256_agrees_with_two_calls(K, oracle_mod):
    """The serving shape (256 sequences x 32 heads x 128^2 fp32 state, bf16
    tokens), in the launch configuration the bench times: the fused call
    against the oracle and against kda_preprocess + kda_decode_step."""
    inp = synth.make("decode_b256")
    H, dk, dv, B = inp["H"], inp["dk"], inp["dv"], inp["N"]
    print("decode_layer b256 full size", flush=True)
    cs1 = to_dev(inp["conv_state"]).clone()
    st1 = to_dev(inp["S0"]).clone()
    out1 = _call(K, inp, cs1, st1)
    cs2 = to_dev(inp["conv_state"]).clone()
    st2 = to_dev(inp["S0"]).clone()
    q, k, v, la, beta = K.kda_preprocess(to_dev(inp["q_in"]), to_dev(inp["k_in"]), to_dev(inp["v_in"]),
                                         to_dev(inp["w_q"]), to_dev(inp["w_k"]), to_dev(inp["w_v"]),
                                         to_dev(inp["g"]), to_dev(inp["b"]), H, dk, dv,
                                         cu_seqlens=to_dev(inp["cu_seqlens"]), conv_state=cs2)
    out2 = K.kda_decode_step(q, k, v, la, beta, st2, out_gate=to_dev(inp["z"]).view(B, H, dv))
    torch.cuda.synchronize()
    ref = oracle_mod.layer(oracle_layer_inputs(inp), want_conv_state=True)
    assert_close("y", to_host64(out1), ref["y"].reshape(B, H, dv), TOL["bf16"])
    assert_close("state", to_host64(st1), ref["S"], TOL["bf16"])
    assert np.array_equal(cs1.cpu().numpy().astype(np.float64), ref["conv_state"])
    # same arithmetic as the two calls up to the order of the norm's sum
    # (which can move a bf16 rounding of q^ or k^ by one unit)
    assert_close("y vs two calls", to_host64(out1), to_host64(out2), 2e-3)
    assert_close("state vs two calls", to_host64(st1), to_host64(st2), 2e-3)
    assert torch.equal(cs1, cs2)


def test_debug_check_rejects_duplicate_state_indices(K, monkeypatch):
    """With KDA_DEBUG_CHECK=1 the call copies state_indices to the host and
    rejects two rows on one slot before launching anything."""
    from gated_delta_rule_64_amd import _lib
    B, H, dk, dv = 3, 2, 16, 16
    inp = _decode_inputs(B, H, dk, dv, "f32")
    st = torch.zeros((5, H, dk, dv), device="cuda")
    cs = torch.zeros((5, 3, H * (2 * dk + dv)), device="cuda")
    monkeypatch.setenv("KDA_DEBUG_CHECK", "1")
    with pytest.raises(_lib.KdaError) as e:
        _call(K, inp, cs, st, idx=to_dev(np.array([4, 1, 4], dtype=np.int32)))
    assert "state_indices" in str(e.value)
    out = _call(K, inp, cs, st, idx=to_dev(np.array([4, 1, -1], dtype=np.int32)))  # distinct: accepted
    torch.cuda.synchronize()
    assert torch.all(out[2] == 0)
