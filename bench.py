#!/usr/bin/env python3
"""Benchmark of libkda on one MI355X.

One step = one pass of the whole prefill path over one batch: short conv,
L2 norm and gates, the chunked prefill and the output gate, as one
``kda_prefill_layer`` call (the preprocess runs inside the chunk kernel), on
the 4096-token, 32-head, d = 128 bf16 layer (``layer_t4k``), inputs already
resident in HBM.  The same work as two calls (``kda_preprocess`` then
``kda_prefill_chunked``) is timed beside it for reference.  ``value`` is prefill tokens/s over the K timed steps.

The decode step (256 sequences x 32 heads x 128^2 fp32 state, in place) is
timed in its own loop and reported under ``decode`` in GB/s of algorithmic
traffic; the fused serving call (raw token in, preprocess and step in one
kernel, conv history and state rolled in place) likewise under
``decode_layer``, and the speculative verify (one token plus three drafts per
sequence, the previous call's four tokens committed first) under
``spec_verify``; the gradients of the chunked recurrence on the 4096-token
layer under ``backward``.  ``roofline`` covers the kernel with the largest share of the step:
algorithmic bytes per launch / average launch time from HIP events recorded
around each kernel during a second pass of the same K steps.  ``cpu_baseline``
times the fp64 CPU oracle on the same workload (rank 0, one GPU only).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16, published
FP32_PEAK_TFLOPS = 157.3  # dense fp32 MFMA (and fp32 vector), published
METRIC = "KDA prefill tokens/s @H32 d128 T4K; decode-step achieved HBM GB/s"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    # (the GPU's clock is still rising over the first few steps after the idle
    # time spent making the inputs: 5 warmup steps give 0.225 ms per step on
    # the 4096-token layer, 50 or more give 0.213)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--decode-steps", type=int, default=50)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--workload", default="layer_t4k")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a 1 GiB device copy (reference for HBM byte counters)")
    return p.parse_args()


def dev(arr):
    import torch
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(arr).cuda()


def threads_for_cpu():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ---------------------------------------------------------------------------
# algorithmic bytes per launch (what each kernel must move at least once)
# ---------------------------------------------------------------------------

def chunk_count(lengths):
    return int(sum((L + 63) // 64 for L in lengths))


def record_bytes(K, T, N, H, dk, dv, x_code):
    ws = K.kda_prefill_workspace_bytes(T, N, H, dk, dv, x_code)
    slots = (T + 63) // 64 + N
    # the chunk map (base[N+1], then the sequence of each slot) precedes the records
    cmap = ((N + 1) * 4 + 255) // 256 * 256 + (slots * 16 + 255) // 256 * 256
    return (ws - cmap) // (slots * H)


def prefill_kernel_bytes(name, w, x, g, rec, has_s0, has_gate):
    """x, g: bytes per input / gate element; rec: workspace bytes per (chunk, head)."""
    T, H, dk, dv, N = w.T_tot, w.H, w.dk, w.dv, w.N
    th = T * H
    chunks = chunk_count(w.lengths) * H
    state = N * H * dk * dv * 4
    if name == "preprocess":
        reads = th * (x * (2 * dk + dv) + x * dk + x) + H * (2 * dk + dv) * 4 * x
        writes = th * (x * (2 * dk + dv) + 4 * dk + 4)
        return reads + writes
    if name == "mfma_prep_intra":  # raw q, k, v, decay and write logits in; records out
        return th * (x * (2 * dk + dv) + x * dk + x) + chunks * rec
    if name.endswith("intra"):
        return th * (x * (2 * dk + dv) + g * dk + g) + chunks * rec
    if name.endswith("state"):
        return chunks * rec + th * x * dv * (2 if has_gate else 1) + state * (2 if has_s0 else 1)
    if name == "chunk_map":
        return (N + 1) * 8
    raise KeyError(name)


def decode_bytes(B, H, dk, dv, x, g, has_gate):
    per = 2 * dk * dv * 4 + x * (2 * dk + dv) + g * (dk + 1) + x * dv * (2 if has_gate else 1)
    return B * H * per


def decode_layer_bytes(B, H, dk, dv, x, has_gate):
    """Algorithmic bytes of one fused decode-layer call: per (sequence, head)
    the state read and written, the raw token (q, k, v, decay and write
    logits), the three-token conv history read and rewritten, the output (and
    gate); per call the conv taps once."""
    w = 2 * dk + dv
    per = 2 * dk * dv * 4 + x * (w + dk + 1) + 2 * 3 * w * 4 + x * dv * (2 if has_gate else 1)
    return B * H * per + H * w * 4 * x


def spec_bytes(B, H, dk, dv, T, na, x, has_gate):
    """Algorithmic bytes of one speculative-verify call that commits na
    tokens and verifies T: per (sequence, head) the state read and written
    once, the conv history read and written, na raw tokens read back from the
    draft buffer, T raw tokens read and written to it, T outputs (and gates);
    per call the conv taps once."""
    w = 2 * dk + dv
    raw = x * (w + dk + 1)
    per = 2 * dk * dv * 4 + 2 * 3 * w * 4 + (na + 2 * T) * raw + T * x * dv * (2 if has_gate else 1)
    return B * H * per + H * w * 4 * x


def traffic_entry(kernel):
    """HBM bytes per launch measured with rocprofv3 counters, if the kernel's
    source is unchanged since they were taken (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        table = json.load(f)
    e = table.get(kernel)
    if not e:
        return None
    src = os.path.join(ROOT, "gated_delta_rule_64_amd", "csrc", e["source"])
    if not os.path.exists(src):
        return None
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    return e["bytes_per_launch"] if sha == e["source_sha256"] else None


def roofline(kernel, bytes_per_launch, ms_per_launch):
    achieved = bytes_per_launch / (ms_per_launch * 1e-3) / 1e9
    return {"kernel": kernel, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_entry(kernel), "bytes_per_launch": int(bytes_per_launch),
            "us_per_launch": round(ms_per_launch * 1e3, 2)}


# ---------------------------------------------------------------------------

def bench_prefill(args):
    import torch
    from gated_delta_rule_64_amd import _lib, kda, synth

    w = synth.workload(args.workload)
    inp = synth.make(w)
    H, dk, dv, T, N = w.H, w.dk, w.dv, w.T_tot, w.N
    t = {k: dev(inp[k]) for k in ("q_in", "k_in", "v_in", "w_q", "w_k", "w_v", "g", "b")}
    z = dev(inp["z"]).view(T, H, dv) if inp["z"] is not None else None
    cu = dev(inp["cu_seqlens"])
    S0 = dev(inp["S0"]) if inp["S0"] is not None else None
    xdt = torch.bfloat16 if w.x_dtype == "bf16" else torch.float32
    pre_out = (torch.empty((T, H, dk), dtype=xdt, device="cuda"), torch.empty((T, H, dk), dtype=xdt, device="cuda"),
               torch.empty((T, H, dv), dtype=xdt, device="cuda"), torch.empty((T, H, dk), device="cuda"),
               torch.empty((T, H), device="cuda"))
    out = torch.empty((T, H, dv), dtype=xdt, device="cuda")
    S_out = torch.empty((N, H, dk, dv), device="cuda")
    x_code = 1 if w.x_dtype == "bf16" else 0
    ws = torch.empty(kda.kda_prefill_workspace_bytes(T, N, H, dk, dv, x_code), dtype=torch.uint8, device="cuda")

    def step_two_calls():
        q, k, v, la, beta = kda.kda_preprocess(t["q_in"], t["k_in"], t["v_in"], t["w_q"], t["w_k"], t["w_v"],
                                               t["g"], t["b"], H, dk, dv, cu_seqlens=cu, out=pre_out)
        kda.kda_prefill_chunked(q, k, v, la, beta, out_gate=z, initial_state=S0, final_state=S_out,
                                cu_seqlens=cu, workspace=ws, out=out)

    def step():
        kda.kda_prefill_layer(t["q_in"], t["k_in"], t["v_in"], t["w_q"], t["w_k"], t["w_v"], t["g"], t["b"],
                              H, dk, dv, out_gate=z, initial_state=S0, final_state=S_out, cu_seqlens=cu,
                              workspace=ws, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # second pass of the same K steps with per-kernel HIP events
    _lib.profile_enable(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed_ev = time.perf_counter() - t1
    _lib.profile_enable(False)
    times = _lib.profile_collect()

    # the same work as two calls (preprocess, then chunked prefill), for reference
    for _ in range(args.warmup):
        step_two_calls()
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(args.steps):
        step_two_calls()
    torch.cuda.synchronize()
    elapsed_two = time.perf_counter() - t2

    xb = 2 if w.x_dtype == "bf16" else 4
    rec = record_bytes(kda, T, N, H, dk, dv, x_code)
    kernels = {}
    for name, (n, ms) in times.items():
        per = ms / n
        b = prefill_kernel_bytes(name, w, xb, 4, rec, S0 is not None, z is not None)
        kernels[name] = {"launches": n, "us_per_launch": round(per * 1e3, 2),
                         "algorithmic_bytes": int(b), "gbs": round(b / (per * 1e-3) / 1e9, 1)}
    dom = max(times, key=lambda k: times[k][1])
    dn, dms = times[dom]
    roof = roofline(dom, kernels[dom]["algorithmic_bytes"], dms / dn)
    return {"w": w, "inp": inp, "elapsed": elapsed, "elapsed_events": elapsed_ev, "kernels": kernels,
            "roofline": roof, "elapsed_two_calls": elapsed_two}


def bench_decode(args):
    import torch
    from gated_delta_rule_64_amd import _lib, kda, synth

    inp = synth.make("decode_b256")
    H, dk, dv, B = inp["H"], inp["dk"], inp["dv"], inp["N"]
    cs = dev(inp["conv_state"])
    q, k, v, la, beta = kda.kda_preprocess(*(dev(inp[n]) for n in ("q_in", "k_in", "v_in", "w_q", "w_k", "w_v",
                                                                  "g", "b")), H, dk, dv,
                                           cu_seqlens=dev(inp["cu_seqlens"]), conv_state=cs)
    z = dev(inp["z"]).view(B, H, dv)
    state = dev(inp["S0"])
    out = torch.empty((B, H, dv), dtype=torch.bfloat16, device="cuda")
    for _ in range(args.warmup):
        kda.kda_decode_step(q, k, v, la, beta, state, out_gate=z, out=out)
    torch.cuda.synchronize()
    _lib.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(args.decode_steps):
        kda.kda_decode_step(q, k, v, la, beta, state, out_gate=z, out=out)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    _lib.profile_enable(False)
    n, ms = _lib.profile_collect()["decode"]
    per_ms = ms / n
    b = decode_bytes(B, H, dk, dv, 2, 4, True)
    return {"metric": "decode-step achieved HBM GB/s", "value": round(b / (per_ms * 1e-3) / 1e9, 1),
            "unit": "GB/s", "workload": "decode_b256", "B": B, "H": H, "dk": dk, "dv": dv,
            "steps": args.decode_steps, "us_per_step_events": round(per_ms * 1e3, 2),
            "us_per_step_wall": round(elapsed / args.decode_steps * 1e6, 2),
            "roofline": roofline("decode", b, per_ms)}


def bench_decode_layer(args):
    """The fused serving call (raw token -> output, history and state rolled in
    place) on the same 256 x 32 x 128^2 workload."""
    import torch
    from gated_delta_rule_64_amd import _lib, kda, synth

    inp = synth.make("decode_b256")
    H, dk, dv, B = inp["H"], inp["dk"], inp["dv"], inp["N"]
    raw = [dev(inp[n]) for n in ("q_in", "k_in", "v_in", "w_q", "w_k", "w_v", "g", "b")]
    cs = dev(inp["conv_state"])
    z = dev(inp["z"]).view(B, H, dv)
    state = dev(inp["S0"])
    out = torch.empty((B, H, dv), dtype=torch.bfloat16, device="cuda")
    for _ in range(args.warmup):
        kda.kda_decode_layer(*raw, H, dk, dv, cs, state, out_gate=z, out=out)
    torch.cuda.synchronize()
    _lib.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(args.decode_steps):
        kda.kda_decode_layer(*raw, H, dk, dv, cs, state, out_gate=z, out=out)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    _lib.profile_enable(False)
    n, ms = _lib.profile_collect()["decode_layer"]
    per_ms = ms / n
    b = decode_layer_bytes(B, H, dk, dv, 2, True)
    return {"metric": "fused decode-layer achieved HBM GB/s", "value": round(b / (per_ms * 1e-3) / 1e9, 1),
            "unit": "GB/s", "workload": "decode_b256", "B": B, "H": H, "dk": dk, "dv": dv,
            "steps": args.decode_steps, "us_per_step_events": round(per_ms * 1e3, 2),
            "us_per_step_wall": round(elapsed / args.decode_steps * 1e6, 2),
            "roofline": roofline("decode_layer", b, per_ms)}


def bench_spec(args):
    """Speculative verify on the same 256 x 32 x 128^2 workload, one token plus
    three drafts per call, every token of the previous call accepted (the
    most work a call does: 4 tokens committed, 4 verified)."""
    import torch
    from gated_delta_rule_64_amd import _lib, kda, synth

    T = 4
    inp = synth.make("decode_b256", lengths=(T,) * 256)
    H, dk, dv, B = inp["H"], inp["dk"], inp["dv"], inp["N"]
    tok = [dev(inp[n]).view(B, T, -1) for n in ("q_in", "k_in", "v_in")]
    w = [dev(inp[n]) for n in ("w_q", "w_k", "w_v")]
    g, b, z = (dev(inp[n]).view(B, T, -1) for n in ("g", "b", "z"))
    cs = dev(inp["conv_state"])
    state = dev(inp["S0"])
    drafts = torch.zeros(B * kda.kda_spec_draft_bytes(H, dk, dv, torch.bfloat16), dtype=torch.uint8, device="cuda")
    acc = torch.full((B,), T, dtype=torch.int32, device="cuda")
    out = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device="cuda")

    def call(accepted):
        kda.kda_spec_verify(*tok, *w, g, b, H, dk, dv, cs, state, drafts, accepted=accepted, out_gate=z, out=out)

    call(None)  # fills the draft buffer
    for _ in range(args.warmup):
        call(acc)
    torch.cuda.synchronize()
    _lib.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(args.decode_steps):
        call(acc)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    _lib.profile_enable(False)
    n, ms = _lib.profile_collect()["spec_verify"]
    per_ms = ms / n
    bts = spec_bytes(B, H, dk, dv, T, T, 2, True)
    return {"metric": "speculative verify (1 + 3 drafts, 4 committed) achieved HBM GB/s",
            "value": round(bts / (per_ms * 1e-3) / 1e9, 1), "unit": "GB/s", "workload": "decode_b256",
            "B": B, "H": H, "dk": dk, "dv": dv, "tokens_verified": T, "tokens_committed": T,
            "steps": args.decode_steps, "us_per_call_events": round(per_ms * 1e3, 2),
            "us_per_call_wall": round(elapsed / args.decode_steps * 1e6, 2),
            "roofline": roofline("spec_verify", bts, per_ms)}


def bench_backward(args):
    """Gradients of the chunked recurrence (kda_prefill_backward) on the
    4096-token layer: preprocessed q, k, v and gates of the bench's own
    inputs, dy ~ N(0, 1) in bf16, initial state and output gate given."""
    import torch
    from gated_delta_rule_64_amd import _lib, kda, synth

    inp = synth.make("layer_t4k")
    H, dk, dv, T = inp["H"], inp["dk"], inp["dv"], inp["T_tot"]
    q, k, v, la, beta = kda.kda_preprocess(*(dev(inp[n]) for n in ("q_in", "k_in", "v_in", "w_q", "w_k", "w_v",
                                                                  "g", "b")), H, dk, dv)
    z = dev(inp["z"]).view(T, H, dv)
    S0 = torch.randn((1, H, dk, dv), generator=torch.Generator().manual_seed(7)).mul_(0.02).cuda()
    dy = torch.randn((T, H, dv), generator=torch.Generator().manual_seed(8)).to(torch.bfloat16).cuda()
    ws = torch.empty(kda.kda_backward_workspace_bytes(T, 1, H, dk, dv), dtype=torch.uint8, device="cuda")
    steps = max(1, args.steps // 5)

    def call():
        return kda.kda_prefill_backward(q, k, v, la, beta, dy, out_gate=z, initial_state=S0, workspace=ws)

    for _ in range(max(1, args.warmup // 2)):
        call()
    torch.cuda.synchronize()
    _lib.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    _lib.profile_enable(False)
    prof = _lib.profile_collect()
    kern = {name: round(ms / n * 1e3, 2) for name, (n, ms) in prof.items()}
    # the dominant kernel, bwd_intra, is fp32 arithmetic: its dense 64-row products
    # on the fp32 matrix cores, the A/M tiles and their adjoint (decay-weighted sums)
    # on the vector ALUs, both with the same published 157.3 TFLOP/s peak.  Its
    # contractions, as executed, come to about 11.1 M multiply-adds per (chunk, head)
    # at d = 128
    units = (T // 64) * H
    flops = 2 * 11.1e6 * units
    n_i, ms_i = prof["bwd_intra"]
    achieved = flops / (ms_i / n_i * 1e-3) / 1e12
    roof = {"kernel": "bwd_intra", "bound": "mfma", "achieved": round(achieved, 2), "peak": FP32_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / FP32_PEAK_TFLOPS, 4), "traffic": traffic_entry("bwd_intra"),
            "flops_per_launch": int(flops), "us_per_launch": round(ms_i / n_i * 1e3, 2)}
    return {"metric": "backward tokens/s (dq, dk, dv, dlog_alpha, dbeta, dz, dS0)",
            "value": round(T * steps / elapsed, 1), "unit": "tokens/s", "workload": "layer_t4k",
            "steps": steps, "ms_per_step": round(elapsed / steps * 1e3, 3), "us_per_kernel": kern, "roofline": roof}


def cpu_baseline(res, min_seconds=10.0, max_passes=100):
    """The fp64 oracle (preprocess + token-by-token recurrence) on the bench's
    own inputs, repeated whole until at least ``min_seconds`` of CPU work."""
    import oracle
    from gated_delta_rule_64_amd import synth

    inp = res["inp"]
    w = res["w"]
    nth = threads_for_cpu()
    f = synth.to_f64
    o_in = {"q_in": f(inp["q_in"]), "k_in": f(inp["k_in"]), "v_in": f(inp["v_in"]), "w_q": f(inp["w_q"]),
            "w_k": f(inp["w_k"]), "w_v": f(inp["w_v"]), "g": f(inp["g"]), "b": f(inp["b"]),
            "z": f(inp["z"]) if inp["z"] is not None else None,
            "S0": f(inp["S0"]) if inp["S0"] is not None else None, "conv_state": None,
            "cu_seqlens": inp["cu_seqlens"].astype(np.int64), "H": w.H, "dk": w.dk, "dv": w.dv}
    oracle.build(force=False)
    passes = 0
    t0 = time.perf_counter()
    while passes < max_passes:
        oracle.layer(o_in, nthreads=nth)
        passes += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": round(w.T_tot * passes / dt, 1), "unit": "tokens/s", "cores": nth, "kind": "oracle",
            "sample": f"{passes} whole passes of the {w.name} workload ({w.T_tot} tokens x {w.H} heads, "
                      f"preprocess + recurrence, fp64) in {dt:.1f} s on {nth} threads"}


def copy_calibration(nbytes=1 << 30, reps=3):
    """A plain device copy of known size, for scaling HBM byte counters: its
    counter readings divided by ``nbytes`` read and written give the factor."""
    import torch
    src = torch.empty(nbytes // 2, dtype=torch.int16, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"bytes": nbytes, "reps": reps}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path shards over "
              "sequences and heads with no exchange, and no multi-GPU run is part of this build.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    from gated_delta_rule_64_amd import _lib
    _lib.lib()  # fail loudly if libkda is not built

    res = bench_prefill(args)
    w = res["w"]
    value = w.T_tot * args.steps / res["elapsed"]
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["elapsed"] / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.x_dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T_tot, "N": w.N, "H": w.H, "dk": w.dk, "dv": w.dv,
                   "chunk": 64, "out_gate": w.out_gate, "state": "fp32",
                   "step": "kda_prefill_layer (short conv, L2 norm, gates, chunked prefill, output gate)"},
        "roofline": res["roofline"],
        "kernels": res["kernels"],
        "ms_per_step_with_kernel_events": round(res["elapsed_events"] / args.steps * 1e3, 4),
        "ms_per_step_two_calls": round(res["elapsed_two_calls"] / args.steps * 1e3, 4),
    }
    line["decode"] = bench_decode(args)
    line["decode_layer"] = bench_decode_layer(args)
    line["spec_verify"] = bench_spec(args)
    line["backward"] = bench_backward(args)
    if args.copy_calibration:
        line["copy_calibration"] = copy_calibration()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(res)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
