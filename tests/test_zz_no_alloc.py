"""kda_prefill_layer_noalloc: the layer prefill with its workspace in the
library's fixed scratch array instead of caller memory.

Through the C ABI, two calls in a row on the same GPU (the second with a
smaller input, so the array still holds the first call's larger contents),
each checked against kda_prefill_layer on the same inputs: the same kernels
run on the same data, so outputs, final states and conv histories must be
bit-identical, and both are also checked against the oracle at the bf16 bar.
A size beyond the array is rejected before any device work.
"""

import ctypes

import numpy as np
import pytest
import torch

from gated_delta_rule_64_amd import _lib, kda, synth
from kda_helpers import TOL, assert_close, oracle_layer_inputs, to_dev, to_host64

pytestmark = pytest.mark.gpu


def _inputs(lengths, H, seed_lengths=None):
    inp = synth.make("varlen_64", lengths=lengths, H=H, conv_history=True)
    d = {n: to_dev(inp[n]) for n in ("q_in", "k_in", "v_in", "w_q", "w_k", "w_v", "g", "b")}
    T = inp["T_tot"]
    d["z"] = to_dev(inp["z"]).view(T, H, 128)
    d["cu"] = to_dev(inp["cu_seqlens"])
    d["S0"] = to_dev(inp["S0"])
    return inp, d


def _noalloc_abi(inp, d, cs, out, S):
    """kda_prefill_layer_noalloc called through the C ABI (ctypes)."""
    P = ctypes.c_void_p
    H, T, N = inp["H"], inp["T_tot"], inp["N"]
    stream = P(torch.cuda.current_stream().cuda_stream)
    return _lib.lib().kda_prefill_layer_noalloc(
        T, H, 128, 128, P(d["cu"].data_ptr()), N, _lib.KDA_BF16,
        P(d["q_in"].data_ptr()), P(d["k_in"].data_ptr()), P(d["v_in"].data_ptr()),
        P(d["w_q"].data_ptr()), P(d["w_k"].data_ptr()), P(d["w_v"].data_ptr()),
        P(d["g"].data_ptr()), P(d["b"].data_ptr()), P(cs.data_ptr()), P(d["z"].data_ptr()),
        P(d["S0"].data_ptr()), P(S.data_ptr()), P(out.data_ptr()), stream)


@pytest.mark.parametrize("H", [32])
def test_noalloc_matches_workspace_call(oracle_mod, H):
    cases = [("larger", (700, 64, 1, 300)), ("smaller", (130, 5))]
    for label, lengths in cases:
        inp, d = _inputs(lengths, H)
        T, N = inp["T_tot"], inp["N"]
        need = kda.kda_prefill_workspace_bytes(T, N, H, 128, 128, _lib.KDA_BF16)
        assert need <= _lib.KDA_NOALLOC_SCRATCH_BYTES, (label, need)
        print(f"{label}: T_tot {T}, N {N}, H {H}, scratch {need} of {_lib.KDA_NOALLOC_SCRATCH_BYTES} bytes",
              flush=True)
        cs0 = to_dev(inp["conv_state"])
        # the existing entry point, with a caller workspace
        cs_ref = cs0.clone()
        out_ref, S_ref = kda.kda_prefill_layer(d["q_in"], d["k_in"], d["v_in"], d["w_q"], d["w_k"], d["w_v"],
                                               d["g"], d["b"], H, 128, 128, out_gate=d["z"],
                                               initial_state=d["S0"], cu_seqlens=d["cu"], conv_state=cs_ref)
        # the no-allocation entry point, through the C ABI
        cs = cs0.clone()
        out = torch.full((T, H, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        S = torch.full((N, H, 128, 128), float("nan"), dtype=torch.float32, device="cuda")
        _lib.check(_noalloc_abi(inp, d, cs, out, S))
        torch.cuda.synchronize()
        assert torch.equal(out, out_ref), f"{label}: outputs differ from kda_prefill_layer"
        assert torch.equal(S, S_ref), f"{label}: final states differ from kda_prefill_layer"
        assert torch.equal(cs, cs_ref), f"{label}: conv histories differ from kda_prefill_layer"
        ref = oracle_mod.layer(oracle_layer_inputs(inp), want_conv_state=True)
        assert_close(f"{label} y", to_host64(out), ref["y"], TOL["bf16"])
        assert_close(f"{label} state", to_host64(S), ref["S"], TOL["bf16"])
        assert_close(f"{label} conv history", to_host64(cs), ref["conv_state"], 1e-6)


def test_noalloc_rejects_sizes_beyond_its_scratch():
    """A size whose workspace exceeds the fixed array fails on the host with
    KDA_ERR_WORKSPACE_TOO_SMALL, before any pointer is used."""
    P = ctypes.c_void_p
    fake = 1 << 40  # never dereferenced: the size check comes first
    T, N, H = 1 << 16, 1, 32
    assert kda.kda_prefill_workspace_bytes(T, N, H, 128, 128, _lib.KDA_BF16) > _lib.KDA_NOALLOC_SCRATCH_BYTES
    st = _lib.lib().kda_prefill_layer_noalloc(T, H, 128, 128, None, N, _lib.KDA_BF16,
                                              *([P(fake)] * 8), None, None, None, None, P(fake), None)
    assert st == _lib.KDA_ERR_WORKSPACE_TOO_SMALL
    assert "kda_prefill_layer_noalloc" in _lib.lib().kda_last_error_detail().decode()
