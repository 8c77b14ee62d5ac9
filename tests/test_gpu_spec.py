"""Speculative verify with a deferred commit on the GPU, against the fp64
oracle on the same seeded inputs.

A session is simulated: each call brings T fresh raw tokens per sequence and
afterwards a seeded draw decides how many of them are accepted.  The tokens
a sequence has accepted so far form its committed stream.  The oracle's layer
fixes every expected value: a call's outputs are the last T outputs of the
layer over (committed stream + that call's tokens), from the initial state and
conv history; after the final commit, the pool row holds the layer's final
state and conv history over the whole committed stream.
"""

import numpy as np
import pytest
import torch

from gated_delta_rule_64_amd import synth
from kda_helpers import TOL, assert_close, f64, to_dev, to_host64

pytestmark = pytest.mark.gpu

TOKEN_KEYS = ("q_in", "k_in", "v_in", "g", "b", "z")


@pytest.fixture(scope="module")
def K():
    from gated_delta_rule_64_amd import kda
    return kda


def _oracle_runs(oracle_mod, inp, streams, S0, cs0):
    """The oracle's layer over one packed batch, sequence b = rows streams[b]
    of the drawn tokens, from S0[b] and conv history cs0[b]."""
    lengths = [len(r) for r in streams]
    rows = np.concatenate(streams).astype(np.int64)
    cu = np.zeros(len(streams) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    d = {key: f64(inp[key][rows]) for key in TOKEN_KEYS}
    d.update({"w_q": f64(inp["w_q"]), "w_k": f64(inp["w_k"]), "w_v": f64(inp["w_v"]),
              "S0": S0, "conv_state": cs0, "cu_seqlens": cu, "H": inp["H"], "dk": inp["dk"], "dv": inp["dv"]})
    ref = oracle_mod.layer(d, want_conv_state=True)
    return ref, cu


def _session(K, oracle_mod, B, H, dk, dv, x_dtype, T, ncalls, seed, lazy=True, pool_extra=0, padding=False):
    inp = synth.make("decode_b256", lengths=(ncalls * T,) * B, H=H, dk=dk, dv=dv, x_dtype=x_dtype)
    rng = np.random.default_rng(seed)
    accepted = rng.integers(0, T + 1, size=(ncalls, B)).astype(np.int32)
    accepted[0, 0] = T  # every count and its extremes show up
    accepted[min(1, ncalls - 1), 0] = 0
    slots = B + pool_extra
    use_idx = bool(pool_extra or padding)
    idx = (rng.permutation(slots)[:B] if use_idx else np.arange(B)).astype(np.int32)
    if padding:
        idx[-1] = -1  # the last row is padding: no state, zero outputs
    live = idx >= 0
    pool = (rng.standard_normal((slots, H, dk, dv)) * 0.05).astype(np.float32)
    pool[idx[live]] = inp["S0"][live]
    cpool = rng.standard_normal((slots, 3, H * (2 * dk + dv))).astype(np.float32)
    if x_dtype == "bf16":
        cpool = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(cpool))
    cpool[idx[live]] = inp["conv_state"][live]
    S0 = f64(inp["S0"])
    cs0 = f64(inp["conv_state"])
    starts = inp["cu_seqlens"][:-1].astype(np.int64)

    st = to_dev(pool).clone()
    cs = to_dev(cpool).clone()
    drafts = torch.zeros(slots * K.kda_spec_draft_bytes(H, dk, dv, torch.bfloat16 if x_dtype == "bf16" else
                                                     torch.float32), dtype=torch.uint8, device="cuda")
    idx_d = to_dev(idx) if use_idx else None
    committed = [np.zeros(0, dtype=np.int64) for _ in range(B)]
    print(f"spec session B={B} H={H} dk={dk} dv={dv} {x_dtype} T={T} calls={ncalls} lazy={lazy}", flush=True)

    def verify(i, acc_prev):
        rows = starts[:, None] + i * T + np.arange(T)[None, :]
        toks = {key: to_dev(np.ascontiguousarray(inp[key][rows])) for key in TOKEN_KEYS}
        return K.kda_spec_verify(toks["q_in"], toks["k_in"], toks["v_in"], to_dev(inp["w_q"]), to_dev(inp["w_k"]),
                                 to_dev(inp["w_v"]), toks["g"], toks["b"], H, dk, dv, cs, st, drafts,
                                 accepted=None if acc_prev is None else to_dev(acc_prev), out_gate=toks["z"],
                                 state_indices=idx_d), rows

    xdt = torch.bfloat16 if x_dtype == "bf16" else torch.float32

    def commit(acc):
        # (a commit-only call: the draft buffer is read in the input type, so
        # the empty token tensors carry that type)
        e = torch.empty((B, 0, H * dk), dtype=xdt, device="cuda")
        K.kda_spec_verify(e, e, torch.empty((B, 0, H * dv), dtype=xdt, device="cuda"), to_dev(inp["w_q"]),
                          to_dev(inp["w_k"]), to_dev(inp["w_v"]), e, torch.empty((B, 0, H), dtype=xdt, device="cuda"),
                          H, dk, dv, cs, st, drafts, accepted=to_dev(acc), state_indices=idx_d)

    worst = 0.0
    for i in range(ncalls):
        acc_prev = accepted[i - 1] if (lazy and i > 0) else None
        out, rows = verify(i, acc_prev)
        torch.cuda.synchronize()
        ref, cu = _oracle_runs(oracle_mod, inp, [np.concatenate([committed[b], rows[b]]) for b in range(B)],
                               S0, cs0)
        y = ref["y"].reshape(-1, H, dv)
        want = np.stack([y[cu[b + 1] - T:cu[b + 1]] for b in range(B)])
        got = to_host64(out).reshape(B, T, H, dv)
        worst = max(worst, assert_close(f"call {i} y", got[live], want[live], TOL[x_dtype]))
        assert np.all(got[~live] == 0.0)
        for b in range(B):
            committed[b] = np.concatenate([committed[b], rows[b][:accepted[i, b]]])
        if not lazy:
            commit(accepted[i])
    if lazy:
        commit(accepted[ncalls - 1])
    torch.cuda.synchronize()
    ref, _ = _oracle_runs(oracle_mod, inp, committed, S0, cs0)
    st_h = st.cpu().numpy()
    cs_h = cs.cpu().numpy()
    assert_close("final state", st_h[idx[live]].astype(np.float64), ref["S"][live], TOL[x_dtype])
    assert np.array_equal(cs_h[idx[live]].astype(np.float64), ref["conv_state"][live])
    untouched = np.setdiff1d(np.arange(slots), idx[live])
    assert np.array_equal(st_h[untouched], pool[untouched])
    assert np.array_equal(cs_h[untouched], cpool[untouched])
    return worst


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 128)])
def test_spec_session_f32(K, oracle_mod, dk, dv):
    _session(K, oracle_mod, B=3, H=2, dk=dk, dv=dv, x_dtype="f32", T=4, ncalls=4, seed=dk + dv)


def test_spec_session_bf16_pool_with_padding(K, oracle_mod):
    _session(K, oracle_mod, B=5, H=4, dk=128, dv=128, x_dtype="bf16", T=4, ncalls=4, seed=1, pool_extra=3,
             padding=True)


@pytest.mark.parametrize("T", [1, 2, 8])
def test_spec_session_token_counts(K, oracle_mod, T):
    """T = 8 with up to 8 committed tokens runs 16 tokens in one call (both
    batches of the preprocess); T = 1 is the plain decode step, lagging by one."""
    _session(K, oracle_mod, B=3, H=2, dk=64, dv=64, x_dtype="f32", T=T, ncalls=3, seed=10 + T, pool_extra=1)


def test_spec_session_largest_call(K, oracle_mod):
    """The largest call the kernel takes: 8 new and up to 8 committed tokens
    at d = 128 with fp32 inputs, whose LDS (raw rows staged as fp32, two
    16-row product passes) is above the 64 KB a launch gets by default, and
    a non-square head (dk = 16, dv = 128) with the same token counts."""
    _session(K, oracle_mod, B=3, H=2, dk=128, dv=128, x_dtype="f32", T=8, ncalls=3, seed=88, pool_extra=1)
    _session(K, oracle_mod, B=3, H=2, dk=16, dv=128, x_dtype="f32", T=8, ncalls=3, seed=89)


def test_spec_session_commit_each_call(K, oracle_mod):
    """Verify, then a commit-only call (T = 0), every step."""
    _session(K, oracle_mod, B=4, H=2, dk=128, dv=64, x_dtype="bf16", T=4, ncalls=3, seed=5, lazy=False)


def test_spec_one_token_steps_equal_decode_layer(K):
    """T = 1 with every token accepted is the decode layer, one call behind:
    same outputs, and after a final commit the same state and history."""
    B, H, dk, dv, steps = 4, 2, 64, 64, 5
    inp = synth.make("decode_b256", lengths=(steps,) * B, H=H, dk=dk, dv=dv, x_dtype="f32")
    starts = inp["cu_seqlens"][:-1].astype(np.int64)
    cs1, st1 = to_dev(inp["conv_state"]).clone(), to_dev(inp["S0"]).clone()
    cs2, st2 = to_dev(inp["conv_state"]).clone(), to_dev(inp["S0"]).clone()
    drafts = torch.zeros(B * K.kda_spec_draft_bytes(H, dk, dv, torch.float32), dtype=torch.uint8, device="cuda")
    ones = torch.ones(B, dtype=torch.int32, device="cuda")
    w = [to_dev(inp[n]) for n in ("w_q", "w_k", "w_v")]
    for t in range(steps):
        tok = {key: to_dev(np.ascontiguousarray(inp[key][starts + t])) for key in TOKEN_KEYS}
        y1 = K.kda_decode_layer(tok["q_in"], tok["k_in"], tok["v_in"], *w, tok["g"], tok["b"], H, dk, dv, cs1, st1,
                                out_gate=tok["z"])
        y2 = K.kda_spec_verify(tok["q_in"].view(B, 1, -1), tok["k_in"].view(B, 1, -1), tok["v_in"].view(B, 1, -1),
                               *w, tok["g"].view(B, 1, -1), tok["b"].view(B, 1, -1), H, dk, dv, cs2, st2, drafts,
                               accepted=ones if t > 0 else None, out_gate=tok["z"].view(B, 1, -1))
        torch.cuda.synchronize()
        assert_close(f"step {t} y", to_host64(y2).reshape(B, H, dv), to_host64(y1), 1e-5)
    e = torch.empty((B, 0, H * dk), device="cuda")
    K.kda_spec_verify(e, e, e, *w, e, torch.empty((B, 0, H), device="cuda"), H, dk, dv, cs2, st2, drafts,
                      accepted=ones)
    torch.cuda.synchronize()
    assert_close("state", to_host64(st2), to_host64(st1), 1e-5)
    assert torch.equal(cs1, cs2)


def test_spec_serving_shape_b256(K, oracle_mod):
    """256 sequences x 32 heads x 128^2 fp32 states, bf16 tokens, one token
    plus three drafts per call (the launch configuration the bench times):
    two verify calls and the final commit against the oracle."""
    _session(K, oracle_mod, B=256, H=32, dk=128, dv=128, x_dtype="bf16", T=4, ncalls=2, seed=256)
