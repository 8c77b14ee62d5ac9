"""Shared test helpers: moving seeded inputs to the device, calling the
oracle on the same inputs, and the error metric.

Error metric (per output tensor): max |gpu - ref| / max |ref|, with no
non-finite value allowed.  Bars: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs
with fp32 accumulation and state.
"""

import numpy as np
import torch

from gated_delta_rule_64_amd import synth

TOL = {"f32": 1e-4, "bf16": 2e-2}


def to_dev(arr, device="cuda"):
    """numpy array (bf16 bit patterns as uint16, or float32/int32) -> device tensor."""
    if arr is None:
        return None
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(arr).to(device)


def to_host64(t):
    """device tensor -> fp64 numpy (exact widening)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def f64(arr):
    return None if arr is None else synth.to_f64(arr)


def oracle_layer_inputs(inp):
    """synth.make() dict -> the fp64 dict oracle.layer() takes."""
    H, dk, dv = inp["H"], inp["dk"], inp["dv"]
    return {"q_in": f64(inp["q_in"]), "k_in": f64(inp["k_in"]), "v_in": f64(inp["v_in"]),
            "w_q": f64(inp["w_q"]), "w_k": f64(inp["w_k"]), "w_v": f64(inp["w_v"]),
            "g": f64(inp["g"]), "b": f64(inp["b"]), "z": f64(inp["z"]),
            "S0": f64(inp["S0"]), "conv_state": f64(inp["conv_state"]),
            "cu_seqlens": inp["cu_seqlens"].astype(np.int64), "H": H, "dk": dk, "dv": dv}


def rel_err(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    if gpu.size == 0:
        return 0.0
    assert np.all(np.isfinite(gpu)), "non-finite values in GPU output"
    scale = np.max(np.abs(ref))
    if scale == 0.0:
        return float(np.max(np.abs(gpu)))
    return float(np.max(np.abs(gpu - ref)) / scale)


def assert_close(name, gpu, ref, tol):
    e = rel_err(gpu, ref)
    print(f"  {name}: max rel err {e:.3e} (bar {tol:.0e})", flush=True)
    assert e <= tol, f"{name}: max rel err {e:.3e} > {tol:.0e}"
    return e
