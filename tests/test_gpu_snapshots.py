"""State snapshots from the prefill (for prefix reuse) on the GPU: snapshot m
of sequence n must equal the oracle's state after the first m * interval
tokens of that sequence; the offsets are the exclusive prefix sums of
floor(len / interval); every other output equals the plain call's."""

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


def _expected_offsets(lengths, interval):
    counts = [L // interval for L in lengths]
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32), counts


def _prefix_rows(cu, lengths, interval):
    """(sequence, m, token rows) for every snapshot, in snapshot order."""
    out = []
    for n, L in enumerate(lengths):
        for m in range(1, L // interval + 1):
            out.append((n, m, np.arange(cu[n], cu[n] + m * interval)))
    return out


@pytest.mark.parametrize("interval", [64, 192, 512])
def test_layer_snapshots(K, oracle_mod, interval):
    lengths = (300, 64, 1000, 40, 0, 513)
    inp = synth.make("varlen_64", lengths=lengths, H=2)
    H, dk, dv, T = inp["H"], inp["dk"], inp["dv"], inp["T_tot"]
    cu = inp["cu_seqlens"]
    print(f"layer snapshots interval={interval}", flush=True)
    raw = [to_dev(inp[n]) for n in ("q_in", "k_in", "v_in", "w_q", "w_k", "w_v", "g", "b")]
    z = to_dev(inp["z"]).view(T, H, dv)
    S0 = to_dev(inp["S0"])
    y1, S1 = K.kda_prefill_layer(*raw, H, dk, dv, out_gate=z, initial_state=S0, cu_seqlens=to_dev(cu))
    y2, S2, snaps, off = K.kda_prefill_layer(*raw, H, dk, dv, out_gate=z, initial_state=S0,
                                              cu_seqlens=to_dev(cu), snap_interval=interval)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(S1, S2)  # the snapshots change nothing else
    want_off, _ = _expected_offsets(lengths, interval)
    assert np.array_equal(off.cpu().numpy(), want_off)
    pref = _prefix_rows(cu, lengths, interval)
    if not pref:
        return
    ref_in = oracle_layer_inputs(inp)
    rows = np.concatenate([r for _, _, r in pref])
    for key in ("q_in", "k_in", "v_in", "g", "b", "z"):
        ref_in[key] = ref_in[key][rows]
    ref_in["cu_seqlens"] = np.concatenate([[0], np.cumsum([len(r) for _, _, r in pref])]).astype(np.int64)
    ref_in["S0"] = f64(inp["S0"])[[n for n, _, _ in pref]]
    ref = oracle_mod.layer(ref_in)
    got = to_host64(snaps)[[want_off[n] + m - 1 for n, m, _ in pref]]
    assert_close("snapshots", got, ref["S"], TOL["bf16"])


@pytest.mark.parametrize("x_dtype,dk,dv", [("f32", 32, 64), ("bf16", 128, 128)])
def test_chunked_snapshots(K, oracle_mod, x_dtype, dk, dv):
    """Both state passes: the fp32 vector one and the matrix-core one."""
    lengths = [200, 128, 700, 5]
    interval = 128
    c = synth.core(21, lengths, 2, dk, dv, x_dtype=x_dtype, s0_std=0.3, out_gate=True)
    cu = c["cu_seqlens"]
    T, H = int(cu[-1]), 2
    print(f"chunked snapshots {x_dtype} dk={dk} dv={dv}", flush=True)
    args = [to_dev(c[n]) for n in ("q", "k", "v", "log_alpha", "beta")]
    y, S, snaps, off = K.kda_prefill_chunked(*args, out_gate=to_dev(c["z"]), initial_state=to_dev(c["S0"]),
                                            cu_seqlens=to_dev(cu), snap_interval=interval)
    torch.cuda.synchronize()
    want_off, _ = _expected_offsets(lengths, interval)
    assert np.array_equal(off.cpu().numpy(), want_off)
    pref = _prefix_rows(cu, lengths, interval)
    rows = np.concatenate([r for _, _, r in pref])
    pcu = np.concatenate([[0], np.cumsum([len(r) for _, _, r in pref])]).astype(np.int64)
    _, Sref = oracle_mod.recurrence(f64(c["q"])[rows], f64(c["k"])[rows], f64(c["v"])[rows],
                                    f64(c["log_alpha"])[rows], f64(c["beta"])[rows],
                                    S0=f64(c["S0"])[[n for n, _, _ in pref]], cu_seqlens=pcu)
    got = to_host64(snaps)[[want_off[n] + m - 1 for n, m, _ in pref]]
    assert_close("snapshots", got, Sref, TOL[x_dtype])


def test_snapshots_none_due(K):
    """Every sequence shorter than the interval: no snapshot, offsets all zero."""
    c = synth.core(22, [100, 30], 2, 16, 16, x_dtype="f32", s0_std=0.3)
    args = [to_dev(c[n]) for n in ("q", "k", "v", "log_alpha", "beta")]
    _, _, snaps, off = K.kda_prefill_chunked(*args, initial_state=to_dev(c["S0"]),
                                             cu_seqlens=to_dev(c["cu_seqlens"]), snap_interval=128)
    torch.cuda.synchronize()
    assert off.cpu().numpy().tolist() == [0, 0, 0]
