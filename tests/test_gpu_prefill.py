"""Chunked prefill on the GPU against the fp64 token-by-token oracle."""

import numpy as np
import pytest
import torch

from gated_delta_rule_64_amd import synth
from kda_helpers import TOL, assert_close, f64, oracle_layer_inputs, to_dev, to_host64

pytestmark = pytest.mark.gpu


def chunk_decay_split(inp, limit=200.0):
    """How many (chunk, head) units have a decay range over their tokens of
    at most ``limit`` (log2 units, largest over the key channels), and how
    many more: the decay logs come from the oracle's own definition,
    log alpha = -softplus(g), on the host.  Chunks start at each sequence's
    first token; the range of a chunk is G(first row) - G(last row)."""
    H, dk = inp["H"], inp["dk"]
    g = synth.to_f64(inp["g"]).reshape(-1, H, dk)
    la2 = -np.logaddexp(0.0, g) / np.log(2.0)
    cu = inp["cu_seqlens"]
    fast = steep = 0
    for n in range(len(cu) - 1):
        for t0 in range(int(cu[n]), int(cu[n + 1]), 64):
            t1 = min(t0 + 64, int(cu[n + 1]))
            rng = -la2[t0 + 1:t1].sum(axis=0).max(axis=1)  # per head
            steep += int((rng > limit).sum())
            fast += int((rng <= limit).sum())
    return fast, steep


@pytest.fixture(scope="module")
def K():
    from gated_delta_rule_64_amd import kda
    return kda


def gpu_layer(K, inp, initial_state=None, final_state=None):
    """preprocess + chunked prefill (with the output gate when present)."""
    H, dk, dv, T = inp["H"], inp["dk"], inp["dv"], inp["T_tot"]
    cu = to_dev(inp["cu_seqlens"])
    q, k, v, la, beta = K.kda_preprocess(to_dev(inp["q_in"]), to_dev(inp["k_in"]), to_dev(inp["v_in"]),
                                         to_dev(inp["w_q"]), to_dev(inp["w_k"]), to_dev(inp["w_v"]),
                                         to_dev(inp["g"]), to_dev(inp["b"]), H, dk, dv, cu_seqlens=cu)
    z = to_dev(inp["z"]).view(T, H, dv) if inp["z"] is not None else None
    if initial_state is None and inp["S0"] is not None:
        initial_state = to_dev(inp["S0"])
    out, S = K.kda_prefill_chunked(q, k, v, la, beta, out_gate=z, initial_state=initial_state,
                                   final_state=final_state, cu_seqlens=cu)
    torch.cuda.synchronize()
    return out, S


def test_core_tiny_workload(K, oracle_mod):
    """1 x 64 tokens, 2 heads, d = 16, fp32, zero state (identity conv)."""
    inp = synth.make("core_tiny")
    out, S = gpu_layer(K, inp)
    ref = oracle_mod.layer(oracle_layer_inputs(inp))
    assert_close("o", to_host64(out), ref["y"], TOL["f32"])
    assert_close("state", to_host64(S), ref["S"], TOL["f32"])


@pytest.mark.parametrize("x_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 128), (128, 32)])
def test_core_parity_ragged(K, oracle_mod, x_dtype, dk, dv):
    lengths = [1, 63, 64, 0, 65, 200]
    inp = synth.core(21, lengths, 3, dk, dv, x_dtype=x_dtype, s0_std=0.3, out_gate=True)
    print(f"core x={x_dtype} dk={dk} dv={dv}", flush=True)
    cu = to_dev(inp["cu_seqlens"])
    out, S = K.kda_prefill_chunked(to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"]),
                                   to_dev(inp["log_alpha"]), to_dev(inp["beta"]), out_gate=to_dev(inp["z"]),
                                   initial_state=to_dev(inp["S0"]), cu_seqlens=cu)
    torch.cuda.synchronize()
    y, Sr = oracle_mod.recurrence(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["log_alpha"]),
                                  f64(inp["beta"]), z=f64(inp["z"]), S0=f64(inp["S0"]),
                                  cu_seqlens=inp["cu_seqlens"])
    assert_close("o", to_host64(out), y, TOL[x_dtype])
    assert_close("state", to_host64(S), Sr, TOL[x_dtype])


@pytest.mark.parametrize("lengths", [(1000,), (130, 0, 64, 1, 700)])
def test_layer_bf16_d128_reduced(K, oracle_mod, lengths):
    """Ling-shaped heads (d = 128, bf16) through preprocess and prefill."""
    inp = synth.make("varlen_64", lengths=lengths, H=4)
    print(f"layer bf16 d128 lengths={lengths}", flush=True)
    out, S = gpu_layer(K, inp)
    ref = oracle_mod.layer(oracle_layer_inputs(inp))
    assert_close("y", to_host64(out), ref["y"], TOL["bf16"])
    assert_close("state", to_host64(S), ref["S"], TOL["bf16"])


def test_state_in_place_and_repeat_bit_identical(K, oracle_mod):
    inp = synth.core(22, [150, 77], 2, 128, 128, x_dtype="bf16", s0_std=0.3, out_gate=True)
    args = [to_dev(inp[n]) for n in ("q", "k", "v", "log_alpha", "beta")]
    cu = to_dev(inp["cu_seqlens"])
    S_sep = to_dev(inp["S0"]).clone()
    o1, S1 = K.kda_prefill_chunked(*args, out_gate=to_dev(inp["z"]), initial_state=S_sep, cu_seqlens=cu)
    S_in = to_dev(inp["S0"]).clone()
    o2, S2 = K.kda_prefill_chunked(*args, out_gate=to_dev(inp["z"]), initial_state=S_in, final_state=S_in,
                                   cu_seqlens=cu)
    torch.cuda.synchronize()
    assert S2.data_ptr() == S_in.data_ptr()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_zero_length_sequences_keep_state(K):
    inp = synth.core(23, [0, 5, 0], 2, 64, 64, x_dtype="f32", s0_std=0.3)
    cu = to_dev(inp["cu_seqlens"])
    S0 = to_dev(inp["S0"])
    out, S = K.kda_prefill_chunked(*[to_dev(inp[n]) for n in ("q", "k", "v", "log_alpha", "beta")],
                                   initial_state=S0, cu_seqlens=cu)
    torch.cuda.synchronize()
    assert torch.equal(S[0], S0[0]) and torch.equal(S[2], S0[2])
    assert not torch.equal(S[1], S0[1])


def test_layer_t4k_full(K, oracle_mod):
    """The 4096-token, 32-head bf16 layer in the bench's launch configuration:
    every output and every state entry against the oracle."""
    inp = synth.make("layer_t4k")
    print("layer_t4k full size", flush=True)
    out, S = gpu_layer(K, inp)
    ref = oracle_mod.layer(oracle_layer_inputs(inp))
    assert_close("y", to_host64(out), ref["y"], TOL["bf16"])
    assert_close("state", to_host64(S), ref["S"], TOL["bf16"])


@pytest.mark.parametrize("case", ["fast_decay", "slow_decay", "beta_one", "zero_rows", "strong_decay",
                                  "decay_near_threshold"])
def test_stress_cases(K, oracle_mod, case):
    """Decay rates at both extremes (the fast one takes the exact diagonal-tile
    path), saturated writes, and all-zero q/k rows (must give 0, not NaN)."""
    kw = {"fast_decay": dict(g_mean=4.0), "slow_decay": dict(g_mean=-6.0),
          "beta_one": dict(b_mean=12.0), "zero_rows": {},
          # decay over a chunk near 2^-100 (one reference per channel), and
          # around 2^-200, beyond which the exact tile path takes over: chunks
          # fall on both sides
          "strong_decay": dict(g_mean=0.5), "decay_near_threshold": dict(g_mean=2.4)}[case]
    inp = synth.make("long_t256k", lengths=(700, 1300), H=3, **kw)
    if case == "decay_near_threshold":
        fast, steep = chunk_decay_split(inp)
        print(f"  chunk-heads with decay range <= 200 (log2): {fast}, above: {steep}", flush=True)
        assert fast > 0 and steep > 0
    if case == "zero_rows":
        inp["q_in"][100:180] = 0
        inp["k_in"][100:180] = 0
    print(f"stress {case}", flush=True)
    out, S = gpu_layer(K, inp)
    ref = oracle_mod.layer(oracle_layer_inputs(inp))
    assert_close("y", to_host64(out), ref["y"], TOL["bf16"])
    assert_close("state", to_host64(S), ref["S"], TOL["bf16"])


@pytest.mark.parametrize("gate", [True, False])
def test_state_workgroup_shapes_agree(K, oracle_mod, gate):
    """The state pass runs one or two 16-column slices (a chain wave and an
    output wave each) per workgroup, chosen by problem size alone: one while
    8 * N * H fits the CUs, two beyond.  The same five sequences run once on
    their own (3 heads: one slice per workgroup) and once followed by seven
    more sequences (12 x 3 groups: two slices per workgroup).  Each slice does
    the same arithmetic in the same order, and a sequence's outputs depend
    only on its own tokens, so the five sequences' outputs and states are
    bit-identical between the two runs, and each matches the oracle."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    small = (130, 0, 64, 1, 700)
    extra = (90, 65, 3, 128, 40, 200, 77)
    H = 3
    assert 8 * len(small) * H <= cus < 8 * (len(small) + len(extra)) * H
    res = {}
    for name, lengths in (("one slice", small), ("two slices", small + extra)):
        inp = synth.make("varlen_64", lengths=lengths, H=H)
        if not gate:
            inp["z"] = None
        print(f"state pass, {name} per workgroup, gate {gate}", flush=True)
        out, S = gpu_layer(K, inp)
        ref = oracle_mod.layer(oracle_layer_inputs(inp))
        assert_close(f"y ({name})", to_host64(out), ref["y"], TOL["bf16"])
        assert_close(f"state ({name})", to_host64(S), ref["S"], TOL["bf16"])
        res[name] = (out, S)
    t_small = sum(small)
    out1, S1 = res["one slice"]
    out2, S2 = res["two slices"]
    assert torch.equal(out2[:t_small], out1) and torch.equal(S2[:len(small)], S1)


def test_debug_check_rejects_bad_cu_seqlens(monkeypatch):
    """With KDA_DEBUG_CHECK=1 the prefill copies cu_seqlens to the host and
    rejects a map that does not end at T_tot, or that decreases, before any
    launch.  (Both maps stay inside the 64 tokens, so even a launch would
    read nothing out of range.)"""
    from gated_delta_rule_64_amd import _lib, kda
    c = synth.core(41, [30, 34], 2, 16, 16, x_dtype="f32")
    args = [to_dev(c[n]) for n in ("q", "k", "v", "log_alpha", "beta")]
    monkeypatch.setenv("KDA_DEBUG_CHECK", "1")
    for bad, what in (([0, 30, 63], "expected T_tot"), ([0, 34, 30], "decreases")):
        with pytest.raises(_lib.KdaError) as e:
            kda.kda_prefill_chunked(*args, cu_seqlens=torch.tensor(bad, dtype=torch.int32, device="cuda"))
        assert what in str(e.value)
    out, _ = kda.kda_prefill_chunked(*args, cu_seqlens=to_dev(c["cu_seqlens"]))  # the right map passes
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
