"""kda_prefill_layer (preprocess fused into the chunk kernel) against the fp64
oracle's preprocess + token-by-token recurrence, on the same seeded raw
inputs: ragged packed batches, conv history in and out, initial states,
decay/write extremes, the full 4096-token layer, and bad arguments."""

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


def fused(K, inp, conv_state=None):
    H, dk, dv, T = inp["H"], inp["dk"], inp["dv"], inp["T_tot"]
    z = to_dev(inp["z"]).view(T, H, dv) if inp["z"] is not None else None
    S0 = to_dev(inp["S0"]) if inp["S0"] is not None else None
    out, S = K.kda_prefill_layer(*(to_dev(inp[n]) for n in ("q_in", "k_in", "v_in", "w_q", "w_k", "w_v", "g", "b")),
                                 H, dk, dv, out_gate=z, initial_state=S0, cu_seqlens=to_dev(inp["cu_seqlens"]),
                                 conv_state=conv_state)
    torch.cuda.synchronize()
    return out, S


@pytest.mark.parametrize("lengths", [(1000,), (130, 0, 64, 1, 700), (63, 65, 3, 2, 1)])
def test_layer_matches_oracle(K, oracle_mod, lengths):
    inp = synth.make("varlen_64", lengths=lengths, H=4)
    print(f"fused layer lengths={lengths}", flush=True)
    out, S = fused(K, inp)
    ref = oracle_mod.layer(oracle_layer_inputs(inp))
    assert_close("y", to_host64(out), ref["y"], TOL["bf16"])
    assert_close("state", to_host64(S), ref["S"], TOL["bf16"])


def test_layer_many_sequences_use_the_chunk_map(K, oracle_mod):
    """Past 64 sequences the chunk kernels read a chunk map built on the device
    before them (up to 64 they derive each chunk from cu_seqlens themselves):
    70 short sequences, some empty, against the oracle."""
    rng = np.random.default_rng(70)
    lengths = tuple(int(x) for x in rng.integers(0, 150, size=70))
    inp = synth.make("varlen_64", lengths=lengths, H=2)
    print(f"fused layer, {len(lengths)} sequences", flush=True)
    out, S = fused(K, inp)
    ref = oracle_mod.layer(oracle_layer_inputs(inp))
    assert_close("y", to_host64(out), ref["y"], TOL["bf16"])
    assert_close("state", to_host64(S), ref["S"], TOL["bf16"])


@pytest.mark.parametrize("lengths", [(1000,), (130, 0, 64, 1, 700), (63, 65, 3, 2, 1)])
def test_layer_inline_chunk_lookup_equals_chunk_map(K, lengths):
    """Without snapshots and with at most 64 sequences the kernels find each
    chunk's sequence, first token and length themselves; asking for snapshots
    at an interval no sequence reaches builds the chunk map instead.  The
    arithmetic is the same, so the results are bit-identical."""
    inp = synth.make("varlen_64", lengths=lengths, H=3)
    H, dk, dv, T = inp["H"], inp["dk"], inp["dv"], inp["T_tot"]
    print(f"fused layer inline lookup vs chunk map, lengths={lengths}", flush=True)
    out1, S1 = fused(K, inp)
    args = [to_dev(inp[n]) for n in ("q_in", "k_in", "v_in", "w_q", "w_k", "w_v", "g", "b")]
    out2, S2, _, off = K.kda_prefill_layer(*args, H, dk, dv, out_gate=to_dev(inp["z"]).view(T, H, dv),
                                           initial_state=to_dev(inp["S0"]) if inp["S0"] is not None else None,
                                           cu_seqlens=to_dev(inp["cu_seqlens"]), snap_interval=64 * 1024)
    torch.cuda.synchronize()
    assert torch.all(off == 0)
    assert torch.equal(out1, out2)
    assert torch.equal(S1, S2)


def test_layer_conv_history_in_and_out(K, oracle_mod):
    """Sequences shorter and longer than the conv width, each starting from
    a caller-given history; the history is rewritten with the last three raw
    tokens (reaching back into the old one for short sequences)."""
    inp = synth.make("decode_b256", lengths=(5, 70, 2, 130, 1), H=2)
    assert inp["conv_state"] is not None
    cs = to_dev(inp["conv_state"]).clone()
    out, S = fused(K, inp, conv_state=cs)
    ref = oracle_mod.layer(oracle_layer_inputs(inp), want_conv_state=True)
    assert_close("y", to_host64(out), ref["y"], TOL["bf16"])
    assert_close("state", to_host64(S), ref["S"], TOL["bf16"])
    # the new history holds raw input values: exact
    np.testing.assert_array_equal(cs.cpu().numpy().astype(np.float64), ref["conv_state"])


def test_layer_agrees_with_two_calls(K, oracle_mod):
    """Same inputs through kda_preprocess + kda_prefill_chunked: equal up to
    rounding order (both inside the bf16 bar of each other)."""
    inp = synth.make("varlen_64", lengths=(300, 77), H=3)
    out_f, S_f = fused(K, inp)
    H, dk, dv, T = inp["H"], inp["dk"], inp["dv"], inp["T_tot"]
    cu = to_dev(inp["cu_seqlens"])
    q, k, v, la, beta = K.kda_preprocess(*(to_dev(inp[n]) for n in ("q_in", "k_in", "v_in", "w_q", "w_k", "w_v",
                                                                  "g", "b")), H, dk, dv, cu_seqlens=cu)
    out_2, S_2 = K.kda_prefill_chunked(q, k, v, la, beta, out_gate=to_dev(inp["z"]).view(T, H, dv),
                                       initial_state=to_dev(inp["S0"]), cu_seqlens=cu)
    torch.cuda.synchronize()
    assert_close("y fused vs two calls", to_host64(out_f), to_host64(out_2), 1e-2)
    assert_close("state fused vs two calls", to_host64(S_f), to_host64(S_2), 1e-2)


@pytest.mark.parametrize("history", [False, True])
def test_layer_sequence_starts_in_later_units(K, oracle_mod, history):
    """Forty sequences over 8 heads: the persistent chunk kernel walks several
    (head, chunk) units per workgroup, so most first chunks are staged after
    some other unit.  The first three rows of every sequence (the rows whose
    short conv reads the history: zeros, or the caller's) are checked row by
    row, so a wrong history on a single row cannot hide under the tensor-wide
    bar.  A row's error is taken relative to its own largest value, floored
    at the median of those over the checked rows: a row whose q.k nearly
    cancels (a first token from a zero state has y = beta (q.k) v sigma(z))
    carries the bf16 rounding of q and k at full size, while a wrong history
    changes q, k and v themselves.  The bar, 0.1 on that scale, is four times
    tighter than the tensor-wide 2e-2 of the largest output (about twenty
    median row scales here); a wrong history moves these rows by O(1)."""
    rng = np.random.default_rng(7)
    lengths = tuple(int(x) for x in rng.integers(1, 400, size=40))
    H = 8
    inp = synth.make("decode_b256" if history else "varlen_64", lengths=lengths, H=H)
    assert (inp["conv_state"] is not None) == history
    T = inp["T_tot"]
    assert H * ((T + 63) // 64 + len(lengths)) > 4 * 256  # several units per workgroup on any MI355X
    cs = to_dev(inp["conv_state"]).clone() if history else None
    print(f"fused layer, sequence starts, history={history}", flush=True)
    out, S = fused(K, inp, conv_state=cs)
    ref = oracle_mod.layer(oracle_layer_inputs(inp), want_conv_state=history)
    y = to_host64(out).reshape(T, H, -1)
    yr = np.asarray(ref["y"], dtype=np.float64).reshape(T, H, -1)
    assert_close("y", y, yr, TOL["bf16"])
    assert_close("state", to_host64(S), ref["S"], TOL["bf16"])
    cu = inp["cu_seqlens"].astype(np.int64)
    rows = [(n, t) for n in range(len(lengths)) for t in range(cu[n], min(cu[n] + 3, cu[n + 1]))]
    scale = np.abs(yr[[t for _, t in rows]]).max(axis=-1)  # [rows, H]
    floor = np.median(scale)
    worst = 0.0
    for i, (n, t) in enumerate(rows):
        for h in range(H):
            e = np.abs(y[t, h] - yr[t, h]).max() / max(scale[i, h], floor)
            worst = max(worst, e)
            assert e <= 0.1, f"sequence {n} token {t - cu[n]} head {h}: row rel err {e:.3e}"
    print(f"  first rows: worst row rel err {worst:.3e} (floor {floor:.3e})", flush=True)
    if history:
        np.testing.assert_array_equal(cs.cpu().numpy().astype(np.float64), ref["conv_state"])


@pytest.mark.parametrize("case", ["fast_decay", "slow_decay", "beta_one", "zero_rows", "strong_decay",
                                  "decay_near_threshold"])
def test_layer_stress(K, oracle_mod, case):
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
    print(f"fused stress {case}", flush=True)
    out, S = fused(K, inp)
    ref = oracle_mod.layer(oracle_layer_inputs(inp))
    assert_close("y", to_host64(out), ref["y"], TOL["bf16"])
    assert_close("state", to_host64(S), ref["S"], TOL["bf16"])


def test_layer_t4k_full(K, oracle_mod):
    """The 4096-token, 32-head layer the bench times, every output checked."""
    inp = synth.make("layer_t4k")
    out, S = fused(K, inp)
    ref = oracle_mod.layer(oracle_layer_inputs(inp))
    assert_close("y", to_host64(out), ref["y"], TOL["bf16"])
    assert_close("state", to_host64(S), ref["S"], TOL["bf16"])


def test_layer_rejects_unsupported_shapes(K):
    inp = synth.make("varlen_64", lengths=(10,), H=2, dk=64, dv=64)
    from gated_delta_rule_64_amd._lib import KdaError
    with pytest.raises(KdaError) as e:
        fused(K, inp)
    assert "KDA_ERR_UNSUPPORTED" in str(e.value)
