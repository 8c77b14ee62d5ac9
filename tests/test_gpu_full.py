"""Full-size prefill parity: the 262,144-token single sequence (fp32 random
initial state, 4096 chunks carried in sequence) and the 64-sequence varlen
batch (lengths 1024..32768, about 1.03 M tokens, half of the sequences
starting from a random state).  Each runs whole on the GPU on both prefill
paths: the fused ``kda_prefill_layer`` (the call the bench times) and the two
calls ``kda_preprocess`` + ``kda_prefill_chunked``, both with the output gate.

Every output of both runs is checked against the fp64 oracle: every head of
the long sequence and every (sequence, head) pair of the varlen batch.  Heads
are independent and a sequence's outputs depend only on its own tokens, so
the oracle computes each pair on its own (one thread per pair, all pairs
spread over the host threads) and each result is compared as it arrives and
then dropped, so the host never holds the whole fp64 reference.  The error
metric is the usual one over each whole output tensor:
max |gpu - ref| / max |ref|, accumulated over the pairs.
"""

import os
import time
from concurrent.futures import ThreadPoolExecutor, as_completed

import numpy as np
import pytest
import torch

from gated_delta_rule_64_amd import synth
from kda_helpers import TOL, f64, to_dev

pytestmark = pytest.mark.gpu


def head_inputs(inp, n, h):
    """The raw inputs of sequence n, head h, as a one-head oracle problem."""
    dk, dv = inp["dk"], inp["dv"]
    cu = inp["cu_seqlens"]
    t0, t1 = int(cu[n]), int(cu[n + 1])
    kc, vc = slice(h * dk, (h + 1) * dk), slice(h * dv, (h + 1) * dv)
    S0 = inp["S0"]
    return {"q_in": f64(inp["q_in"][t0:t1, kc]), "k_in": f64(inp["k_in"][t0:t1, kc]),
            "v_in": f64(inp["v_in"][t0:t1, vc]), "w_q": f64(inp["w_q"][kc]), "w_k": f64(inp["w_k"][kc]),
            "w_v": f64(inp["w_v"][vc]), "g": f64(inp["g"][t0:t1, kc]), "b": f64(inp["b"][t0:t1, h:h + 1]),
            "z": f64(inp["z"][t0:t1, vc]), "S0": None if S0 is None else f64(S0[n:n + 1, h:h + 1]),
            "conv_state": None, "cu_seqlens": np.array([0, t1 - t0], dtype=np.int64),
            "H": 1, "dk": dk, "dv": dv}


def run_two_calls(K, inp, dinp):
    H, dk, dv, T = inp["H"], inp["dk"], inp["dv"], inp["T_tot"]
    q, k, v, la, beta = K.kda_preprocess(dinp["q_in"], dinp["k_in"], dinp["v_in"], dinp["w_q"], dinp["w_k"],
                                         dinp["w_v"], dinp["g"], dinp["b"], H, dk, dv, cu_seqlens=dinp["cu"])
    out, S = K.kda_prefill_chunked(q, k, v, la, beta, out_gate=dinp["z"].view(T, H, dv),
                                   initial_state=dinp["S0"], cu_seqlens=dinp["cu"])
    torch.cuda.synchronize()
    del q, k, v, la, beta
    return out, S


def run_layer(K, inp, dinp):
    H, dk, dv, T = inp["H"], inp["dk"], inp["dv"], inp["T_tot"]
    out, S = K.kda_prefill_layer(dinp["q_in"], dinp["k_in"], dinp["v_in"], dinp["w_q"], dinp["w_k"], dinp["w_v"],
                                 dinp["g"], dinp["b"], H, dk, dv, out_gate=dinp["z"].view(T, H, dv),
                                 initial_state=dinp["S0"], cu_seqlens=dinp["cu"])
    torch.cuda.synchronize()
    return out, S


def host_bits(t):
    """device bf16 tensor -> host uint16 bit patterns (exact), fp32 -> fp32."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class Err:
    """max |gpu - ref| and max |ref| accumulated over pieces of one tensor."""

    def __init__(self):
        self.diff = 0.0
        self.ref = 0.0

    def add(self, gpu, ref):
        assert np.all(np.isfinite(gpu)), "non-finite values in GPU output"
        self.diff = max(self.diff, float(np.max(np.abs(gpu - ref))) if gpu.size else 0.0)
        self.ref = max(self.ref, float(np.max(np.abs(ref))) if ref.size else 0.0)

    def rel(self):
        return self.diff / self.ref if self.ref > 0 else self.diff


def check_all_pairs(oracle_mod, inp, results, label):
    """Every (sequence, head) pair of inp against the oracle, for every GPU
    result in ``results`` ({path: (y bits [T, H, dv], S [N, H, dk, dv])})."""
    cu = inp["cu_seqlens"]
    N, H = inp["N"], inp["H"]
    pairs = [(n, h) for n in range(N) for h in range(H) if cu[n + 1] > cu[n]]
    # longest first, so the pool ends evenly
    pairs.sort(key=lambda p: -(int(cu[p[0] + 1]) - int(cu[p[0]])))
    errs = {path: {"y": Err(), "state": Err()} for path in results}
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    t_start = time.time()
    done = 0

    def ref(pair):
        n, h = pair
        return pair, oracle_mod.layer(head_inputs(inp, n, h), nthreads=1)

    with ThreadPoolExecutor(workers) as ex:
        futs = [ex.submit(ref, p) for p in pairs]
        for fut in as_completed(futs):
            (n, h), r = fut.result()
            t0, t1 = int(cu[n]), int(cu[n + 1])
            for path, (y, S) in results.items():
                errs[path]["y"].add(synth.to_f64(y[t0:t1, h, :]), r["y"][:, 0, :])
                errs[path]["state"].add(S[n, h].astype(np.float64), r["S"][0, 0])
            done += 1
            if done % max(1, len(pairs) // 16) == 0 or done == len(pairs):
                print(f"  {label}: oracle {done}/{len(pairs)} pairs ({time.time() - t_start:.0f} s)", flush=True)
    bad = []
    for path, e in errs.items():
        for name, acc in e.items():
            rel = acc.rel()
            print(f"  {label} [{path}] {name}: max rel err {rel:.3e} over all {len(pairs)} pairs "
                  f"(bar {TOL['bf16']:.0e})", flush=True)
            if not rel <= TOL["bf16"]:
                bad.append((path, name, rel))
    assert not bad, bad


def run_both(K, inp):
    dinp = {n: to_dev(inp[n]) for n in ("q_in", "k_in", "v_in", "w_q", "w_k", "w_v", "g", "b", "z")}
    dinp["cu"] = to_dev(inp["cu_seqlens"])
    dinp["S0"] = to_dev(inp["S0"]) if inp["S0"] is not None else None
    res = {}
    for path, fn in (("kda_prefill_layer", run_layer), ("preprocess + prefill_chunked", run_two_calls)):
        print(f"  GPU run: {path}", flush=True)
        out, S = fn(K, inp, dinp)
        assert torch.isfinite(out).all().item() and torch.isfinite(S).all().item()
        res[path] = (host_bits(out), host_bits(S))
        del out, S
        torch.cuda.empty_cache()
    del dinp
    torch.cuda.empty_cache()
    return res


@pytest.fixture(scope="module")
def K():
    from gated_delta_rule_64_amd import kda
    return kda


@pytest.mark.timeout(900)
def test_long_t256k_full(K, oracle_mod):
    """One 262,144-token sequence, 32 heads, random fp32 initial state: every
    head of both paths against the oracle."""
    print("long_t256k: drawing inputs", flush=True)
    inp = synth.make("long_t256k")
    res = run_both(K, inp)
    check_all_pairs(oracle_mod, inp, res, "long_t256k")


@pytest.mark.timeout(900)
def test_varlen_64_full(K, oracle_mod):
    """64 packed sequences (about 1.03 M tokens), 32 heads; even sequences start
    from zero, odd ones from a random fp32 state: every (sequence, head) pair
    of both paths against the oracle."""
    print("varlen_64: drawing inputs", flush=True)
    inp = synth.make("varlen_64")
    print(f"varlen_64: T_tot {inp['T_tot']}", flush=True)
    res = run_both(K, inp)
    check_all_pairs(oracle_mod, inp, res, "varlen_64")
