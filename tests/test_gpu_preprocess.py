"""Fused preprocess (conv4 + L2 norm + gates) on the GPU against the oracle."""

import numpy as np
import pytest
import torch

from gated_delta_rule_64_amd import synth
from kda_helpers import TOL, assert_close, f64, to_dev, to_host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    from gated_delta_rule_64_amd import kda
    return kda


def run_both(K, oracle_mod, inp, with_state):
    H, dk, dv = inp["H"], inp["dk"], inp["dv"]
    cu = to_dev(inp["cu_seqlens"])
    N = inp["N"]
    cs_np = None
    if with_state:
        cs_np = np.random.default_rng(3).standard_normal((N, 3, H * (2 * dk + dv))).astype(np.float32)
    cs = to_dev(cs_np).clone() if with_state else None
    outs = K.kda_preprocess(to_dev(inp["q_in"]), to_dev(inp["k_in"]), to_dev(inp["v_in"]),
                            to_dev(inp["w_q"]), to_dev(inp["w_k"]), to_dev(inp["w_v"]),
                            to_dev(inp["g"]), to_dev(inp["b"]), H, dk, dv, cu_seqlens=cu, conv_state=cs)
    torch.cuda.synchronize()
    ref = oracle_mod.preprocess(f64(inp["q_in"]), f64(inp["k_in"]), f64(inp["v_in"]), f64(inp["w_q"]),
                                f64(inp["w_k"]), f64(inp["w_v"]), f64(inp["g"]), f64(inp["b"]), H, dk, dv,
                                cu_seqlens=inp["cu_seqlens"], conv_state=cs_np, want_conv_state=with_state)
    return outs, cs, ref


@pytest.mark.parametrize("x_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("with_state", [False, True])
def test_preprocess_matches_oracle(K, oracle_mod, x_dtype, dk, dv, with_state):
    lengths = [1, 0, 2, 300, 17, 0, 5, 512, 3]
    inp = synth.make("layer_t4k", lengths=lengths, H=3, dk=dk, dv=dv, x_dtype=x_dtype)
    print(f"preprocess x={x_dtype} dk={dk} dv={dv} state={with_state}", flush=True)
    (q, k, v, la, beta), cs, ref = run_both(K, oracle_mod, inp, with_state)
    tol = TOL[x_dtype]
    for name, g, r in (("q", q, ref["q"]), ("k", k, ref["k"]), ("v", v, ref["v"])):
        assert_close(name, to_host64(g), r, tol)
    assert_close("log_alpha", to_host64(la), ref["log_alpha"], 1e-5)
    assert_close("beta", to_host64(beta), ref["beta"], 1e-6)
    if with_state:
        # the new history holds raw input values: exact
        assert np.array_equal(cs.cpu().numpy().astype(np.float64), ref["conv_state"])


def test_preprocess_layer_t4k_full(K, oracle_mod):
    """The 4096-token, 32-head bf16 layer at full size, every output checked."""
    inp = synth.make("layer_t4k")
    print("preprocess layer_t4k full size", flush=True)
    (q, k, v, la, beta), _, ref = run_both(K, oracle_mod, inp, False)
    for name, g, r in (("q", q, ref["q"]), ("k", k, ref["k"]), ("v", v, ref["v"])):
        assert_close(name, to_host64(g), r, TOL["bf16"])
    assert_close("log_alpha", to_host64(la), ref["log_alpha"], 1e-5)
    assert_close("beta", to_host64(beta), ref["beta"], 1e-6)
    qn = np.linalg.norm(to_host64(q), axis=-1)
    assert np.all(np.abs(qn - 1) < 1e-2)
