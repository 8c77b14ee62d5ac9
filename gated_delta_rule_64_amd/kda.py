"""Python binding of libkda: the same entry points, torch tensors in.

Argument marshalling only: shapes are read from the tensors, outputs that the
caller does not pass are allocated with torch (device memory is torch's
plumbing), and each call goes straight to the C ABI on torch's current HIP
stream.  Every step of the computation runs in libkda's kernels.
"""

from __future__ import annotations

import ctypes

import torch

from ._lib import KDA_BF16, KDA_F32, check, lib


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return KDA_F32
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; libkda takes float32 or bfloat16")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libkda takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libkda takes contiguous tensors")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device=None):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _n_seqs(cu_seqlens):
    if cu_seqlens is None:
        return 1
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    return cu_seqlens.numel() - 1


def kda_preprocess(q_in, k_in, v_in, w_q, w_k, w_v, g_alpha, b_beta, H, dk, dv,
                   cu_seqlens=None, conv_state=None, out=None):
    """Short conv + L2 norm + gates.  Inputs [T, H*d]; returns
    (q [T,H,dk], k [T,H,dk], v [T,H,dv], log_alpha fp32 [T,H,dk], beta fp32 [T,H]).
    ``conv_state`` (fp32 [N, 3, H*(2dk+dv)]) is read and rewritten in place."""
    T = q_in.shape[0]
    x = _dtype_code(q_in)
    dev = q_in.device
    if out is None:
        out = (torch.empty((T, H, dk), dtype=q_in.dtype, device=dev),
               torch.empty((T, H, dk), dtype=q_in.dtype, device=dev),
               torch.empty((T, H, dv), dtype=q_in.dtype, device=dev),
               torch.empty((T, H, dk), dtype=torch.float32, device=dev),
               torch.empty((T, H), dtype=torch.float32, device=dev))
    q_o, k_o, v_o, la_o, b_o = out
    check(lib().kda_preprocess(T, H, dk, dv, _ptr(cu_seqlens), _n_seqs(cu_seqlens), x,
                               _ptr(q_in), _ptr(k_in), _ptr(v_in), _ptr(w_q), _ptr(w_k), _ptr(w_v),
                               _ptr(g_alpha), _ptr(b_beta), _ptr(conv_state),
                               _ptr(q_o), _ptr(k_o), _ptr(v_o), _ptr(la_o), _ptr(b_o), _stream(dev)))
    return out


def kda_prefill_workspace_bytes(T_tot, N, H, dk, dv, x_dtype):
    if isinstance(x_dtype, torch.dtype):
        x_dtype = KDA_BF16 if x_dtype == torch.bfloat16 else KDA_F32
    return int(lib().kda_prefill_workspace_bytes(T_tot, N, H, dk, dv, x_dtype))


def _snap_buffers(snap_interval, T, N, H, dk, dv, dev, snapshots, snap_offsets):
    cap = T // snap_interval
    if snapshots is None:
        snapshots = torch.empty((max(cap, 1), H, dk, dv), dtype=torch.float32, device=dev)
    if snap_offsets is None:
        snap_offsets = torch.empty(N + 1, dtype=torch.int32, device=dev)
    return snapshots, snap_offsets


def kda_prefill_chunked(q, k, v, log_alpha, beta, out_gate=None, initial_state=None,
                        final_state=None, cu_seqlens=None, workspace=None, out=None,
                        want_final_state=True, snap_interval=None, snapshots=None, snap_offsets=None):
    """Chunked recurrence over preprocessed tokens q,k [T,H,dk], v [T,H,dv].
    Returns (out [T,H,dv], final_state fp32 [N,H,dk,dv] or None); with
    ``snap_interval`` (a multiple of 64) also (snapshots [C,H,dk,dv],
    snap_offsets int32 [N+1]): the state after every ``snap_interval`` tokens
    of each sequence, sequence n's m-th at row snap_offsets[n] + m - 1."""
    T, H, dk = q.shape
    dv = v.shape[2]
    N = _n_seqs(cu_seqlens)
    x = _dtype_code(q)
    g = _dtype_code(log_alpha)
    dev = q.device
    if out is None:
        out = torch.empty((T, H, dv), dtype=q.dtype, device=dev)
    if final_state is None and want_final_state:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    need = kda_prefill_workspace_bytes(T, N, H, dk, dv, x)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    if snap_interval is None:
        check(lib().kda_prefill_chunked(T, H, dk, dv, _ptr(cu_seqlens), N, x, g,
                                        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                        _ptr(out_gate), _ptr(initial_state), _ptr(final_state), _ptr(out),
                                        _ptr(workspace), workspace.numel(), _stream(dev)))
        return out, final_state
    snapshots, snap_offsets = _snap_buffers(snap_interval, T, N, H, dk, dv, dev, snapshots, snap_offsets)
    check(lib().kda_prefill_chunked_snap(T, H, dk, dv, _ptr(cu_seqlens), N, x, g,
                                         _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                         _ptr(out_gate), _ptr(initial_state), _ptr(final_state), _ptr(out),
                                         _ptr(workspace), workspace.numel(), snap_interval, _ptr(snapshots),
                                         snapshots.shape[0], _ptr(snap_offsets), _stream(dev)))
    return out, final_state, snapshots, snap_offsets


def kda_decode_step(q, k, v, log_alpha, beta, state, out_gate=None, out=None):
    """One token per sequence; ``state`` fp32 [B,H,dk,dv] is updated in place.
    Returns out [B,H,dv]."""
    B, H, dk = q.shape
    dv = v.shape[2]
    if out is None:
        out = torch.empty((B, H, dv), dtype=q.dtype, device=q.device)
    check(lib().kda_decode_step(B, H, dk, dv, _dtype_code(q), _dtype_code(log_alpha),
                                _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(out_gate),
                                _ptr(state), _ptr(out), _stream(q.device)))
    return out


def kda_prefill_layer(q_in, k_in, v_in, w_q, w_k, w_v, g_alpha, b_beta, H, dk, dv, out_gate=None,
                      initial_state=None, final_state=None, cu_seqlens=None, conv_state=None, workspace=None,
                      out=None, want_final_state=True, snap_interval=None, snapshots=None, snap_offsets=None):
    """kda_preprocess + kda_prefill_chunked in one call (bf16, dk = dv = 128):
    raw inputs [T, H*d] as for kda_preprocess, the rest as for
    kda_prefill_chunked.  Returns (out [T,H,dv], final_state fp32 [N,H,dk,dv] or None).
    ``conv_state`` (fp32 [N, 3, H*(2dk+dv)]) is read and rewritten in place."""
    T = q_in.shape[0]
    N = _n_seqs(cu_seqlens)
    x = _dtype_code(q_in)
    dev = q_in.device
    if out is None:
        out = torch.empty((T, H, dv), dtype=q_in.dtype, device=dev)
    if final_state is None and want_final_state:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    need = kda_prefill_workspace_bytes(T, N, H, dk, dv, x)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    if snap_interval is None:
        check(lib().kda_prefill_layer(T, H, dk, dv, _ptr(cu_seqlens), N, x,
                                      _ptr(q_in), _ptr(k_in), _ptr(v_in), _ptr(w_q), _ptr(w_k), _ptr(w_v),
                                      _ptr(g_alpha), _ptr(b_beta), _ptr(conv_state), _ptr(out_gate),
                                      _ptr(initial_state), _ptr(final_state), _ptr(out),
                                      _ptr(workspace), workspace.numel(), _stream(dev)))
        return out, final_state
    snapshots, snap_offsets = _snap_buffers(snap_interval, T, N, H, dk, dv, dev, snapshots, snap_offsets)
    check(lib().kda_prefill_layer_snap(T, H, dk, dv, _ptr(cu_seqlens), N, x,
                                       _ptr(q_in), _ptr(k_in), _ptr(v_in), _ptr(w_q), _ptr(w_k), _ptr(w_v),
                                       _ptr(g_alpha), _ptr(b_beta), _ptr(conv_state), _ptr(out_gate),
                                       _ptr(initial_state), _ptr(final_state), _ptr(out),
                                       _ptr(workspace), workspace.numel(), snap_interval, _ptr(snapshots),
                                       snapshots.shape[0], _ptr(snap_offsets), _stream(dev)))
    return out, final_state, snapshots, snap_offsets


def kda_prefill_layer_noalloc(q_in, k_in, v_in, w_q, w_k, w_v, g_alpha, b_beta, H, dk, dv, out_gate=None,
                              initial_state=None, final_state=None, cu_seqlens=None, conv_state=None, out=None,
                              want_final_state=True):
    """kda_prefill_layer without a workspace: the library's fixed scratch
    (KDA_NOALLOC_SCRATCH_BYTES per GPU) holds it.  Returns (out, final_state)."""
    T = q_in.shape[0]
    N = _n_seqs(cu_seqlens)
    x = _dtype_code(q_in)
    dev = q_in.device
    if out is None:
        out = torch.empty((T, H, dv), dtype=q_in.dtype, device=dev)
    if final_state is None and want_final_state:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    check(lib().kda_prefill_layer_noalloc(T, H, dk, dv, _ptr(cu_seqlens), N, x,
                                          _ptr(q_in), _ptr(k_in), _ptr(v_in), _ptr(w_q), _ptr(w_k), _ptr(w_v),
                                          _ptr(g_alpha), _ptr(b_beta), _ptr(conv_state), _ptr(out_gate),
                                          _ptr(initial_state), _ptr(final_state), _ptr(out), _stream(dev)))
    return out, final_state


def kda_decode_layer(q_in, k_in, v_in, w_q, w_k, w_v, g_alpha, b_beta, H, dk, dv, conv_state, state,
                     out_gate=None, state_indices=None, out=None):
    """One raw token per sequence through preprocess + decode step in one call.
    Inputs [B, H*d] (or [B, H, d]) as for kda_preprocess; ``conv_state`` fp32
    [S, 3, H*(2dk+dv)] and ``state`` fp32 [S, H, dk, dv] are pools updated in
    place, sequence b using row ``state_indices[b]`` (int32 [B]; row b when
    None, then S must be B; an index outside [0, S) marks a padding row whose
    output is zero).  Returns out [B, H, dv]."""
    B = q_in.shape[0]
    slots = state.shape[0]
    if state_indices is not None and state_indices.dtype != torch.int32:
        raise TypeError("state_indices must be int32")
    if out is None:
        out = torch.empty((B, H, dv), dtype=q_in.dtype, device=q_in.device)
    check(lib().kda_decode_layer(B, H, dk, dv, _dtype_code(q_in),
                                 _ptr(q_in), _ptr(k_in), _ptr(v_in), _ptr(w_q), _ptr(w_k), _ptr(w_v),
                                 _ptr(g_alpha), _ptr(b_beta), _ptr(conv_state), _ptr(out_gate),
                                 _ptr(state), slots, _ptr(state_indices), _ptr(out), _stream(q_in.device)))
    return out


def kda_spec_draft_bytes(H, dk, dv, x_dtype):
    """Bytes of draft buffer per pool slot for kda_spec_verify."""
    if isinstance(x_dtype, torch.dtype):
        x_dtype = KDA_BF16 if x_dtype == torch.bfloat16 else KDA_F32
    return int(lib().kda_spec_draft_bytes(H, dk, dv, x_dtype))


def kda_spec_verify(q_in, k_in, v_in, w_q, w_k, w_v, g_alpha, b_beta, H, dk, dv, conv_state, state, drafts,
                    accepted=None, out_gate=None, state_indices=None, out=None):
    """Commit ``accepted[b]`` tokens of the previous call, then run the T new
    raw tokens (inputs [B, T, H*d] or [B, T, H, d]) from that state without
    advancing it.  ``drafts`` is a device buffer of S * kda_spec_draft_bytes
    bytes (S = pool rows).  Returns out [B, T, H, dv]."""
    B, T = q_in.shape[0], q_in.shape[1]
    for t in (accepted, state_indices):
        if t is not None and t.dtype != torch.int32:
            raise TypeError("accepted and state_indices must be int32")
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=q_in.dtype, device=q_in.device)
    check(lib().kda_spec_verify(B, T, H, dk, dv, _dtype_code(q_in),
                                _ptr(q_in), _ptr(k_in), _ptr(v_in), _ptr(w_q), _ptr(w_k), _ptr(w_v),
                                _ptr(g_alpha), _ptr(b_beta), _ptr(conv_state), _ptr(out_gate),
                                _ptr(state), state.shape[0], _ptr(state_indices), _ptr(accepted),
                                _ptr(drafts), _ptr(out), _stream(q_in.device)))
    return out


def kda_backward_workspace_bytes(T_tot, N, H, dk, dv):
    return int(lib().kda_backward_workspace_bytes(T_tot, N, H, dk, dv))


def kda_prefill_backward(q, k, v, log_alpha, beta, dy, out_gate=None, initial_state=None, dS_final=None,
                         cu_seqlens=None, workspace=None, want_dS0=True):
    """Gradients of kda_prefill_chunked for output gradients dy [T,H,dv] (and
    dS_final on the final states).  Returns a dict of fp32 tensors dq, dk,
    dlog_alpha [T,H,dk], dv [T,H,dv], dbeta [T,H], dz (None without a gate)
    and dS0 [N,H,dk,dv] (None if not wanted)."""
    T, H, dk = q.shape
    dv = v.shape[2]
    N = _n_seqs(cu_seqlens)
    dev = q.device
    f32 = dict(dtype=torch.float32, device=dev)
    g = {"dq": torch.empty((T, H, dk), **f32), "dk": torch.empty((T, H, dk), **f32),
         "dv": torch.empty((T, H, dv), **f32), "dlog_alpha": torch.empty((T, H, dk), **f32),
         "dbeta": torch.empty((T, H), **f32),
         "dz": torch.empty((T, H, dv), **f32) if out_gate is not None else None,
         "dS0": torch.empty((N, H, dk, dv), **f32) if want_dS0 else None}
    need = kda_backward_workspace_bytes(T, N, H, dk, dv)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    check(lib().kda_prefill_backward(T, H, dk, dv, _ptr(cu_seqlens), N, _dtype_code(q), _dtype_code(log_alpha),
                                     _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(out_gate),
                                     _ptr(initial_state), _ptr(dy), _ptr(dS_final),
                                     _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dlog_alpha"]),
                                     _ptr(g["dbeta"]), _ptr(g["dz"]), _ptr(g["dS0"]),
                                     _ptr(workspace), workspace.numel(), _stream(dev)))
    return g


def kda_probe_peak(kind, blocks, iters=0, src=None, out=None):
    """Peak-rate probe (see kda.h): kind 0 bf16 matrix-core loop, 1 fp32
    matrix-core loop, 2 streaming read of ``src``.  Returns ``out``."""
    dev = src.device if src is not None else torch.device("cuda")
    if out is None:
        out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    nbytes = src.numel() * src.element_size() if src is not None else 0
    check(lib().kda_probe_peak(kind, blocks, iters, _ptr(src), nbytes, _ptr(out), _stream(dev)))
    return out
