#!/usr/bin/env python3
"""Benchmark of libkda on one MI355X.

One step = one pass of the whole prefill path over one batch: short conv,
L2 norm and gates, the chunked prefill and the output gate, as one
``kda_prefill_layer`` call (the preprocess runs inside the chunk kernel), on
the 4096-token, 32-head, d = 128 bf16 layer (``layer_t4k``), inputs already
resident in HBM.  ``value`` is prefill tokens/s over the K timed steps, run
back to back.  Beside it:

* ``roofline``: the kernel with the largest share of the step, priced on its
  algorithmic bytes (its share of the layer's own inputs and outputs, each
  counted once: raw q, k, v, decay logits and write logits for the chunk
  kernel; output-gate logits, output and states for the state pass) over its
  average launch time from HIP events recorded on the launch stream;
  ``traffic`` is the kernel's HBM bytes per launch from rocprofv3 counters
  (profiles/traffic.json), null once the kernel's source has changed;
* ``end_to_end``: the whole step against the layer's algorithmic bytes
  (1,538 B per token and head at d = 128 bf16), and the measured traffic of
  the step's kernels over those bytes;
* ``flushed``: the same step timed one at a time with the GPU caches
  (L2 and the 256 MB Infinity Cache) flushed before each, by a 1 GiB read
  outside the timed events (median);
* ``mfma``: the chunk kernel's matrix-core work (issued dense flops) against
  the bf16 peak, by wall clock and, from rocprofv3 counters
  (profiles/mfma_counters.json), as matrix-core busy cycles;
* ``peaks``: what this device sustains, measured here (a streaming read, a
  device copy, bf16 and fp32 matrix-core loops), beside the published peaks;
  they run first and also bring the GPU clock up from idle;
* ``large``: the 262,144-token sequence (with the state pass's time per
  chunk step) and the 64-sequence varlen batch, prefill tokens/s;
* ``decode``, ``decode_layer``, ``spec_verify``, ``backward``: the other
  entry points on their workloads;
* ``cpu_baseline``: the fp64 CPU oracle on a bounded sample of the same
  workload (rank 0, one GPU only).

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
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix cores, published
FP32_PEAK_TFLOPS = 157.3        # dense fp32 (matrix cores and vector ALUs), published
METRIC = "KDA prefill tokens/s @H32 d128 T4K; decode-step achieved HBM GB/s"
# matrix-core instructions (v_mfma_f32_16x16x32_bf16, 16,384 flops each) the
# chunk kernel issues per (chunk, head): A and M 80, W and U~ 96, Q' and M U~ 96
INTRA_MFMA_PER_UNIT = 272
MFMA_BF16_FLOPS = 2 * 16 * 16 * 32


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--decode-steps", type=int, default=50)
    p.add_argument("--flushed-steps", type=int, default=20)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-large", action="store_true", help="skip the 262,144-token and varlen configs")
    p.add_argument("--only-prefill", action="store_true", help="the headline prefill only (profiling runs)")
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


def host_threads():
    """Threads for the CPU oracle: the CPUs this process may run on, capped by
    OMP_NUM_THREADS when the environment sets it (the host's share for one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# ---------------------------------------------------------------------------
# algorithmic bytes (the layer's own inputs and outputs, each counted once)
# ---------------------------------------------------------------------------

def layer_bytes(T, H, dk, dv, N, x, has_gate, has_s0, want_state=True):
    """Whole prefill layer: raw q, k, v, decay logits, write logits and
    output-gate logits in, output out, states in and out."""
    per = x * (2 * dk + dv + dk + 1) + x * dv * (2 if has_gate else 1)
    state = N * H * dk * dv * 4
    return T * H * per + state * ((1 if has_s0 else 0) + (1 if want_state else 0))


def kernel_bytes(name, T, H, dk, dv, N, x, has_gate, has_s0):
    """A kernel's share of the layer's algorithmic bytes."""
    if name in ("mfma_prep_intra", "preprocess"):  # raw q, k, v, decay and write logits in
        return T * H * x * (2 * dk + dv + dk + 1)
    if name.startswith("mfma_state"):  # gate logits in, output out, states
        return T * H * x * dv * (2 if has_gate else 1) + N * H * dk * dv * 4 * (2 if has_s0 else 1)
    if name == "mfma_intra":  # its inputs are preprocessed tensors: nothing of the layer's own
        return 0
    if name == "chunk_map":
        return (N + 1) * 8
    raise KeyError(name)


def decode_bytes(B, H, dk, dv, x, g, has_gate):
    per = 2 * dk * dv * 4 + x * (2 * dk + dv) + g * (dk + 1) + x * dv * (2 if has_gate else 1)
    return B * H * per


def decode_layer_bytes(B, H, dk, dv, x, has_gate):
    """Per (sequence, head) the state read and written, the raw token (q, k,
    v, decay and write logits), the three-token conv history read and
    rewritten, the output (and gate); per call the conv taps once."""
    w = 2 * dk + dv
    per = 2 * dk * dv * 4 + x * (w + dk + 1) + 2 * 3 * w * 4 + x * dv * (2 if has_gate else 1)
    return B * H * per + H * w * 4 * x


def spec_bytes(B, H, dk, dv, T, na, x, has_gate):
    """Per (sequence, head) the state read and written once, the conv history
    read and written, na raw tokens read back from the draft buffer, T raw
    tokens read and written to it, T outputs (and gates); per call the conv
    taps once."""
    w = 2 * dk + dv
    raw = x * (w + dk + 1)
    per = 2 * dk * dv * 4 + 2 * 3 * w * 4 + (na + 2 * T) * raw + T * x * dv * (2 if has_gate else 1)
    return B * H * per + H * w * 4 * x


def backward_bytes(T, H, dk, dv, N, x):
    """The backward's own inputs (q, k, v, output-gate logits, dy in x; log
    decay and beta fp32; initial states) and outputs (fp32 gradients of all
    of them)."""
    reads = x * (2 * dk + dv) + 4 * dk + 4 + x * dv + x * dv
    writes = 4 * (2 * dk + dv) + 4 * dk + 4 + 4 * dv
    return T * H * (reads + writes) + 2 * N * H * dk * dv * 4


def _profile_entry(fname, kernel):
    """An entry of a profiles/*.json table, if the kernel's source is
    unchanged since the counters were taken (else None)."""
    path = os.path.join(ROOT, "profiles", fname)
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
    return e if sha == e["source_sha256"] else None


def traffic_entry(kernel):
    e = _profile_entry("traffic.json", kernel)
    return e["bytes_per_launch"] if e else None


def roofline(kernel, bytes_per_launch, ms_per_launch):
    achieved = bytes_per_launch / (ms_per_launch * 1e-3) / 1e9
    return {"kernel": kernel, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_entry(kernel), "bytes_per_launch": int(bytes_per_launch),
            "us_per_launch": round(ms_per_launch * 1e3, 2)}


# ---------------------------------------------------------------------------

def measure_peaks():
    """Streaming read and device copy of 1 GiB, bf16 and fp32 matrix-core
    loops on every CU, each timed with HIP events (best of a few)."""
    import torch
    from gated_delta_rule_64_amd import kda

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    blocks = cus * 8
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best(fn, reps=5):
        fn()
        ms = []
        for _ in range(reps):
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ms.append(e0.elapsed_time(e1))
        return min(ms)

    res = {}
    ms = best(lambda: kda.kda_probe_peak(2, blocks, 0, src=src, out=out))
    res["hbm_read_gbs"] = round(n / (ms * 1e-3) / 1e9, 1)
    ms = best(lambda: dst.copy_(src))
    res["hbm_copy_gbs"] = round(2 * n / (ms * 1e-3) / 1e9, 1)
    iters = 4096
    ms = best(lambda: kda.kda_probe_peak(0, blocks, iters, out=out))
    res["mfma_bf16_tflops"] = round(blocks * 4 * iters * 4 * MFMA_BF16_FLOPS / (ms * 1e-3) / 1e12, 1)
    ms = best(lambda: kda.kda_probe_peak(1, blocks, iters // 4, out=out))
    res["mfma_f32_tflops"] = round(blocks * 4 * (iters // 4) * 4 * 2048 / (ms * 1e-3) / 1e12, 1)
    res["published"] = {"hbm_gbs": HBM_PEAK_GBS, "mfma_bf16_tflops": MFMA_BF16_PEAK_TFLOPS,
                        "fp32_tflops": FP32_PEAK_TFLOPS}
    res["how"] = ("1 GiB streaming read (16-byte loads, grid-stride) and torch device copy (read + write "
                  "counted); loops of independent 16x16x32 bf16 / 16x16x4 fp32 matrix-core products, "
                  f"{blocks} workgroups of 4 waves; best of 5 event-timed runs")
    del src, dst
    torch.cuda.empty_cache()
    return res


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

    # one step at a time with cold caches: a 1 GiB read (L2 and the Infinity
    # Cache hold 32 MB and 256 MB) before each, outside the timed events
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(3)
    probe_out = torch.empty(2048 * 256, dtype=torch.float32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    flushed = []
    for _ in range(args.flushed_steps):
        kda.kda_probe_peak(2, 2048, 0, src=flush, out=probe_out)
        e0.record()
        step()
        e1.record()
        e1.synchronize()
        flushed.append(e0.elapsed_time(e1))
    del flush, probe_out

    # the same work as two calls (preprocess, then chunked prefill), for reference
    for _ in range(max(1, args.warmup // 4)):
        step_two_calls()
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(args.steps):
        step_two_calls()
    torch.cuda.synchronize()
    elapsed_two = time.perf_counter() - t2

    xb = 2 if w.x_dtype == "bf16" else 4
    has_gate, has_s0 = z is not None, S0 is not None
    kernels = {}
    for name, (n, ms) in times.items():
        per = ms / n
        b = kernel_bytes(name, T, H, dk, dv, N, xb, has_gate, has_s0)
        kernels[name] = {"launches": n, "us_per_launch": round(per * 1e3, 2), "algorithmic_bytes": int(b),
                         "gbs": round(b / (per * 1e-3) / 1e9, 1), "traffic": traffic_entry(name)}
    dom = max(times, key=lambda k: times[k][1])
    dn, dms = times[dom]
    roof = roofline(dom, kernels[dom]["algorithmic_bytes"], dms / dn)
    units = ((T + 63) // 64) * H if N == 1 else None
    return {"w": w, "inp": inp, "elapsed": elapsed, "elapsed_events": elapsed_ev, "kernels": kernels,
            "roofline": roof, "elapsed_two_calls": elapsed_two, "flushed_ms": flushed, "units": units,
            "layer_bytes": layer_bytes(T, H, dk, dv, N, xb, has_gate, has_s0)}


def mfma_report(res):
    """The chunk kernel's matrix-core work against the bf16 peak."""
    k = res["kernels"].get("mfma_prep_intra")
    if k is None or res["units"] is None:
        return None
    flops = INTRA_MFMA_PER_UNIT * MFMA_BF16_FLOPS * res["units"]
    tf = flops / (k["us_per_launch"] * 1e-6) / 1e12
    rep = {"kernel": "mfma_prep_intra", "dense_flops_per_launch": int(flops),
           "wall_tflops": round(tf, 1), "wall_frac_of_bf16_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
    c = _profile_entry("mfma_counters.json", "mfma_prep_intra")
    if c:
        rep["counters"] = {key: c[key] for key in c if key not in ("source", "source_sha256")}
    else:
        rep["counters"] = None
    return rep


def gpu_inputs(name, seed):
    """Inputs of a workload drawn on the GPU (seeded; distributions as the
    workload's: raw q, k, v, decay, write and gate logits N(0, 1) rounded to
    bf16, conv taps N(0, 0.5), initial states N(0, 0.02) as the workload
    places them), for timing only: the parity tests draw the same workloads
    on the host, where the oracle can read them."""
    import torch
    from gated_delta_rule_64_amd import synth

    w = synth.workload(name)
    H, dk, dv, T, N = w.H, w.dk, w.dv, w.T_tot, w.N
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)

    def randn(shape, std=1.0):
        x = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        rows = max(1, (1 << 28) // max(1, int(np.prod(shape[1:]))))
        flat = x.view(shape[0], -1)
        for r0 in range(0, shape[0], rows):  # in slabs, to bound the fp32 temporary
            r1 = min(shape[0], r0 + rows)
            flat[r0:r1] = (torch.randn((r1 - r0, flat.shape[1]), generator=gen, device="cuda") * std).to(
                torch.bfloat16)
        return x

    d = {"q_in": randn((T, H * dk)), "k_in": randn((T, H * dk)), "v_in": randn((T, H * dv)),
         "g": randn((T, H * dk)), "b": randn((T, H)), "z": randn((T, H, dv)),
         "w_q": randn((H * dk, 4), w.conv_w_std), "w_k": randn((H * dk, 4), w.conv_w_std),
         "w_v": randn((H * dv, 4), w.conv_w_std)}
    cu = np.zeros(N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(w.lengths)
    d["cu"] = torch.from_numpy(cu).cuda()
    if w.s0 == "zero":
        d["S0"] = None
    else:
        S0 = torch.randn((N, H, dk, dv), generator=gen, device="cuda") * w.s0_std
        if w.s0 == "alternate":
            S0[0::2] = 0
        d["S0"] = S0
    return w, d


def bench_large(name, steps, warmup):
    """Prefill tokens/s of a large workload (kda_prefill_layer), and the state
    pass's time per chunk step along its longest sequence."""
    import torch
    from gated_delta_rule_64_amd import _lib, kda

    w, d = gpu_inputs(name, seed={"long_t256k": 2, "varlen_64": 4}[name])
    H, dk, dv, T, N = w.H, w.dk, w.dv, w.T_tot, w.N
    out = torch.empty((T, H, dv), dtype=torch.bfloat16, device="cuda")
    S_out = torch.empty((N, H, dk, dv), device="cuda")
    ws = torch.empty(kda.kda_prefill_workspace_bytes(T, N, H, dk, dv, 1), dtype=torch.uint8, device="cuda")

    def step():
        kda.kda_prefill_layer(d["q_in"], d["k_in"], d["v_in"], d["w_q"], d["w_k"], d["w_v"], d["g"], d["b"],
                              H, dk, dv, out_gate=d["z"], initial_state=d["S0"], final_state=S_out,
                              cu_seqlens=d["cu"], workspace=ws, out=out)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    _lib.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    _lib.profile_enable(False)
    prof = _lib.profile_collect()
    kern = {k: round(ms / n * 1e3, 1) for k, (n, ms) in prof.items()}
    longest = max(w.lengths)
    chunks = (longest + 63) // 64
    res = {"workload": name, "T_tot": T, "N": N, "H": H, "steps": steps,
           "tokens_per_s": round(T * steps / elapsed, 1), "ms_per_step": round(elapsed / steps * 1e3, 3),
           "us_per_kernel": kern, "inputs": "drawn on the GPU (seeded), the workload's distributions"}
    if "mfma_state" in kern:
        res["state_us_per_chunk_step"] = round(kern["mfma_state"] / chunks, 3)
        res["longest_sequence_chunks"] = chunks
    lb = layer_bytes(T, H, dk, dv, N, 2, True, d["S0"] is not None)
    res["end_to_end_gbs"] = round(lb / (elapsed / steps) / 1e9, 1)
    del d, out, S_out, ws
    torch.cuda.empty_cache()
    return res


def _timed_loop(fn, warmup, steps, kernel):
    import torch
    from gated_delta_rule_64_amd import _lib
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    _lib.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    _lib.profile_enable(False)
    n, ms = _lib.profile_collect()[kernel]
    return ms / n, elapsed


def bench_decode(args):
    import torch
    from gated_delta_rule_64_amd import kda, synth

    inp = synth.make("decode_b256")
    H, dk, dv, B = inp["H"], inp["dk"], inp["dv"], inp["N"]
    cs = dev(inp["conv_state"])
    q, k, v, la, beta = kda.kda_preprocess(*(dev(inp[n]) for n in ("q_in", "k_in", "v_in", "w_q", "w_k", "w_v",
                                                                  "g", "b")), H, dk, dv,
                                           cu_seqlens=dev(inp["cu_seqlens"]), conv_state=cs)
    z = dev(inp["z"]).view(B, H, dv)
    state = dev(inp["S0"])
    out = torch.empty((B, H, dv), dtype=torch.bfloat16, device="cuda")
    per_ms, elapsed = _timed_loop(lambda: kda.kda_decode_step(q, k, v, la, beta, state, out_gate=z, out=out),
                                  args.warmup, args.decode_steps, "decode")
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
    from gated_delta_rule_64_amd import kda, synth

    inp = synth.make("decode_b256")
    H, dk, dv, B = inp["H"], inp["dk"], inp["dv"], inp["N"]
    raw = [dev(inp[n]) for n in ("q_in", "k_in", "v_in", "w_q", "w_k", "w_v", "g", "b")]
    cs = dev(inp["conv_state"])
    z = dev(inp["z"]).view(B, H, dv)
    state = dev(inp["S0"])
    out = torch.empty((B, H, dv), dtype=torch.bfloat16, device="cuda")
    per_ms, elapsed = _timed_loop(lambda: kda.kda_decode_layer(*raw, H, dk, dv, cs, state, out_gate=z, out=out),
                                  args.warmup, args.decode_steps, "decode_layer")
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
    from gated_delta_rule_64_amd import kda, synth

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
    per_ms, elapsed = _timed_loop(lambda: call(acc), args.warmup, args.decode_steps, "spec_verify")
    bts = spec_bytes(B, H, dk, dv, T, T, 2, True)
    roof = roofline("spec_verify", bts, per_ms)
    if roof["traffic"]:
        roof["achieved_on_measured_traffic"] = round(roof["traffic"] / (per_ms * 1e-3) / 1e9, 1)
        roof["frac_on_measured_traffic"] = round(roof["achieved_on_measured_traffic"] / HBM_PEAK_GBS, 4)
    return {"metric": "speculative verify (1 + 3 drafts, 4 committed) achieved HBM GB/s",
            "value": round(bts / (per_ms * 1e-3) / 1e9, 1), "unit": "GB/s", "workload": "decode_b256",
            "B": B, "H": H, "dk": dk, "dv": dv, "tokens_verified": T, "tokens_committed": T,
            "steps": args.decode_steps, "us_per_call_events": round(per_ms * 1e3, 2),
            "us_per_call_wall": round(elapsed / args.decode_steps * 1e6, 2), "roofline": roof}


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
    steps = max(2, args.steps // 5)

    def call():
        return kda.kda_prefill_backward(q, k, v, la, beta, dy, out_gate=z, initial_state=S0, workspace=ws)

    for _ in range(max(1, args.warmup // 4)):
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
    ab = backward_bytes(T, H, dk, dv, 1, 2)
    step_ms = elapsed / steps * 1e3
    dom = max(prof, key=lambda kk: prof[kk][1])
    n_d, ms_d = prof[dom]
    # the dominant kernel reads and writes nearly all of the backward's own
    # tensors; price it, and the whole step, on those algorithmic bytes
    roof = roofline(dom, ab, ms_d / n_d)
    return {"metric": "backward tokens/s (dq, dk, dv, dlog_alpha, dbeta, dz, dS0)",
            "value": round(T * steps / elapsed, 1), "unit": "tokens/s", "workload": "layer_t4k",
            "steps": steps, "ms_per_step": round(step_ms, 3), "us_per_kernel": kern,
            "algorithmic_bytes": int(ab),
            "end_to_end": {"achieved": round(ab / (step_ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                           "frac": round(ab / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
            "roofline": roof}


def cpu_baseline(res, min_seconds=12.0, max_passes=100):
    """The fp64 oracle (preprocess + token-by-token recurrence) on the bench's
    own inputs, repeated whole until at least ``min_seconds`` of CPU work."""
    import oracle
    from gated_delta_rule_64_amd import synth

    inp = res["inp"]
    w = res["w"]
    nth = host_threads()
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
    # the recurrence's fp64 work: decay d^2, u = S^T k 2 d^2, the write 2 d^2,
    # the read 2 d^2 flops per token and head
    flops = 7 * w.dk * w.dv * w.T_tot * w.H * passes
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = None
    return {"value": round(w.T_tot * passes / dt, 1), "unit": "tokens/s", "cores": nth, "kind": "oracle",
            "sample": f"{passes} whole passes of the {w.name} workload ({w.T_tot} tokens x {w.H} heads, "
                      f"preprocess + recurrence, fp64) in {dt:.1f} s on {nth} threads",
            "fp64_gflops": round(flops / dt / 1e9, 2), "threads": nth, "host_nproc": os.cpu_count(),
            "host_affinity_cpus": aff, "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "cpu_model": cpu_model()}


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

    peaks = measure_peaks()
    print(f"# peaks measured: {peaks['hbm_read_gbs']} GB/s read, {peaks['mfma_bf16_tflops']} TFLOP/s bf16",
          file=sys.stderr, flush=True)
    res = bench_prefill(args)
    w = res["w"]
    value = w.T_tot * args.steps / res["elapsed"]
    step_ms = res["elapsed"] / args.steps * 1e3
    flushed = sorted(res["flushed_ms"])
    med_flushed = flushed[len(flushed) // 2]
    step_traffic = [res["kernels"][k]["traffic"] for k in res["kernels"] if k != "chunk_map"]
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.x_dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T_tot, "N": w.N, "H": w.H, "dk": w.dk, "dv": w.dv,
                   "chunk": 64, "out_gate": w.out_gate, "state": "fp32",
                   "step": "kda_prefill_layer (short conv, L2 norm, gates, chunked prefill, output gate)"},
        "roofline": res["roofline"],
        "end_to_end": {
            "algorithmic_bytes": int(res["layer_bytes"]),
            "achieved": round(res["layer_bytes"] / (step_ms * 1e-3) / 1e9, 1), "unit": "GB/s",
            "frac": round(res["layer_bytes"] / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "measured_traffic": int(sum(step_traffic)) if all(step_traffic) else None,
            "traffic_over_algorithmic": round(sum(step_traffic) / res["layer_bytes"], 3)
            if all(step_traffic) else None},
        "flushed": {"ms_per_step_median": round(med_flushed, 4), "ms_min": round(flushed[0], 4),
                    "ms_max": round(flushed[-1], 4), "steps": len(flushed),
                    "tokens_per_s": round(w.T_tot / (med_flushed * 1e-3), 1),
                    "how": "1 GiB read before each step, outside its HIP events"},
        "kernels": res["kernels"],
        "mfma": mfma_report(res),
        "ms_per_step_with_kernel_events": round(res["elapsed_events"] / args.steps * 1e3, 4),
        "ms_per_step_two_calls": round(res["elapsed_two_calls"] / args.steps * 1e3, 4),
        "peaks": peaks,
    }
    if not args.only_prefill:
        if not args.no_large:
            line["large"] = {}
            for name in ("long_t256k", "varlen_64"):
                print(f"# large workload {name}", file=sys.stderr, flush=True)
                line["large"][name] = bench_large(name, steps=3, warmup=1)
        print("# decode, decode layer, speculative verify, backward", file=sys.stderr, flush=True)
        line["decode"] = bench_decode(args)
        line["decode_layer"] = bench_decode_layer(args)
        line["spec_verify"] = bench_spec(args)
        line["backward"] = bench_backward(args)
    if args.copy_calibration:
        line["copy_calibration"] = copy_calibration()
    if not args.no_cpu_baseline:
        print("# CPU oracle baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(res)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
