"""The C ABI library: loads, exports every declared entry point, and rejects
bad arguments on the host before any device work (CPU only)."""

import ctypes
import os
import re

import pytest

from gated_delta_rule_64_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "kda.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.lib()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"kda_preprocess", "kda_prefill_chunked", "kda_prefill_workspace_bytes",
            "kda_decode_step", "kda_status_string", "kda_last_error_detail"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in kda.h but not exported"
        assert n in _lib.PROTOTYPES, f"{n} has no ctypes prototype"


def test_status_strings(lib):
    assert _lib.status_string(0) == "KDA_OK"
    assert _lib.status_string(3) == "KDA_ERR_WORKSPACE_TOO_SMALL"
    assert _lib.status_string(99) == "KDA_ERR_UNKNOWN"
    assert lib.kda_abi_version() == 104


def test_workspace_bytes_bound(lib):
    w = lib.kda_prefill_workspace_bytes
    assert w(4096, 1, 32, 128, 128, 1) > 0
    # grows with the slot bound ceil(T/64) + N
    assert w(4096, 2, 32, 128, 128, 1) > w(4096, 1, 32, 128, 128, 1)
    assert w(4160, 1, 32, 128, 128, 1) > w(4096, 1, 32, 128, 128, 1)
    assert w(0, 1, 2, 16, 16, 0) > 0
    # invalid or unsupported sizes give 0
    assert w(-1, 1, 32, 128, 128, 1) == 0
    assert w(64, 0, 32, 128, 128, 1) == 0
    assert w(64, 1, 32, 96, 128, 1) == 0
    assert w(64, 1, 32, 128, 128, 7) == 0


P = ctypes.c_void_p
FAKE = 1 << 40  # an aligned, never-dereferenced address: validation fails before any use


def decode(lib, **kw):
    a = dict(B=2, H=2, dk=16, dv=16, x=1, g=0, q=FAKE, k=FAKE + 4096, v=FAKE + 8192, la=FAKE + 12288,
             beta=FAKE + 16384, z=None, state=FAKE + 65536, out=FAKE + 2 * 65536)
    a.update(kw)
    return lib.kda_decode_step(a["B"], a["H"], a["dk"], a["dv"], a["x"], a["g"], P(a["q"]), P(a["k"]),
                               P(a["v"]), P(a["la"]), P(a["beta"]), P(a["z"]), P(a["state"]),
                               P(a["out"]), None)


def test_decode_rejects_bad_arguments(lib):
    assert decode(lib, dk=96) == _lib.KDA_ERR_UNSUPPORTED
    assert decode(lib, x=5) == _lib.KDA_ERR_INVALID_ARGUMENT
    assert decode(lib, q=None) == _lib.KDA_ERR_INVALID_ARGUMENT
    assert "q is NULL" in lib.kda_last_error_detail().decode()
    assert decode(lib, k=FAKE + 4) == _lib.KDA_ERR_INVALID_ARGUMENT
    assert "aligned" in lib.kda_last_error_detail().decode()
    assert decode(lib, out=FAKE + 65536 + 256) == _lib.KDA_ERR_INVALID_ARGUMENT  # overlaps state
    assert "overlaps" in lib.kda_last_error_detail().decode()
    assert decode(lib, H=0) == _lib.KDA_ERR_INVALID_ARGUMENT


def prefill(lib, **kw):
    a = dict(T=64, H=2, dk=16, dv=16, cu=None, N=1, x=0, g=0, q=FAKE, k=FAKE + 2**20, v=FAKE + 2 * 2**20,
             la=FAKE + 3 * 2**20, beta=FAKE + 4 * 2**20, z=None, s0=None, s1=None, out=FAKE + 5 * 2**20,
             ws=FAKE + 2**30, ws_bytes=None)
    a.update(kw)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = lib.kda_prefill_workspace_bytes(a["T"], a["N"], a["H"], a["dk"], a["dv"], a["x"])
    return lib.kda_prefill_chunked(a["T"], a["H"], a["dk"], a["dv"], P(a["cu"]), a["N"], a["x"], a["g"],
                                   P(a["q"]), P(a["k"]), P(a["v"]), P(a["la"]), P(a["beta"]), P(a["z"]),
                                   P(a["s0"]), P(a["s1"]), P(a["out"]), P(a["ws"]), a["ws_bytes"], None)


def test_prefill_rejects_bad_arguments(lib):
    assert prefill(lib, ws_bytes=1) == _lib.KDA_ERR_WORKSPACE_TOO_SMALL
    assert prefill(lib, ws=FAKE + 2**30 + 16) == _lib.KDA_ERR_INVALID_ARGUMENT  # not 256-aligned
    assert prefill(lib, N=2) == _lib.KDA_ERR_INVALID_ARGUMENT  # NULL cu_seqlens needs N = 1
    assert prefill(lib, T=-5) == _lib.KDA_ERR_INVALID_ARGUMENT
    assert prefill(lib, T=2**31) == _lib.KDA_ERR_INVALID_ARGUMENT
    assert prefill(lib, dv=48) == _lib.KDA_ERR_UNSUPPORTED
    assert prefill(lib, g=3) == _lib.KDA_ERR_INVALID_ARGUMENT
    assert prefill(lib, v=None) == _lib.KDA_ERR_INVALID_ARGUMENT
    assert prefill(lib, out=FAKE + 64) == _lib.KDA_ERR_INVALID_ARGUMENT  # overlaps q
    state = 2 * 2 * 16 * 16 * 4
    assert prefill(lib, s0=FAKE + 7 * 2**20, s1=FAKE + 7 * 2**20 + 256) == _lib.KDA_ERR_INVALID_ARGUMENT
    assert "partially overlaps" in lib.kda_last_error_detail().decode()
    assert state > 256


def test_preprocess_rejects_bad_arguments(lib):
    def call(**kw):
        a = dict(T=64, H=2, dk=16, dv=16, cu=None, N=1, x=1)
        a.update(kw)
        ptrs = [FAKE + i * 2**20 for i in range(14)]
        for key, idx in (("q_in", 0), ("cs", 8), ("q_out", 9)):
            if key in kw:
                ptrs[idx] = kw[key]
        return lib.kda_preprocess(a["T"], a["H"], a["dk"], a["dv"], P(a["cu"]), a["N"], a["x"],
                                  *[P(p) for p in ptrs[:8]], P(ptrs[8]), *[P(p) for p in ptrs[9:]], None)
    assert call(dk=8) == _lib.KDA_ERR_UNSUPPORTED
    assert call(x=2) == _lib.KDA_ERR_INVALID_ARGUMENT
    assert call(q_in=None) == _lib.KDA_ERR_INVALID_ARGUMENT
    assert call(q_out=FAKE + 64) == _lib.KDA_ERR_INVALID_ARGUMENT  # output overlaps q_in
    assert call(N=3) == _lib.KDA_ERR_INVALID_ARGUMENT


def test_decode_layer_rejects_bad_arguments(lib):
    def call(**kw):
        a = dict(B=2, H=2, dk=16, dv=16, x=1, slots=2, idx=None, z=None)
        names = ["q_in", "k_in", "v_in", "w_q", "w_k", "w_v", "g", "b", "cs", "state", "out"]
        ptrs = {n: FAKE + i * 2**20 for i, n in enumerate(names)}
        a.update(ptrs)
        a.update(kw)
        return lib.kda_decode_layer(a["B"], a["H"], a["dk"], a["dv"], a["x"],
                                    *[P(a[n]) for n in names[:8]], P(a["cs"]), P(a["z"]), P(a["state"]),
                                    a["slots"], P(a["idx"]), P(a["out"]), None)
    assert call(dk=8) == _lib.KDA_ERR_UNSUPPORTED
    assert call(x=3) == _lib.KDA_ERR_INVALID_ARGUMENT
    assert call(slots=5) == _lib.KDA_ERR_INVALID_ARGUMENT  # no indices: one slot per row
    assert "state_slots" in lib.kda_last_error_detail().decode()
    assert call(slots=-1, idx=FAKE + 2**30) == _lib.KDA_ERR_INVALID_ARGUMENT
    assert call(idx=FAKE + 2**30 + 2) == _lib.KDA_ERR_INVALID_ARGUMENT  # misaligned indices
    assert call(cs=None) == _lib.KDA_ERR_INVALID_ARGUMENT  # the conv history is required
    assert "conv_state is NULL" in lib.kda_last_error_detail().decode()
    assert call(state=FAKE + 8 * 2**20 + 256) == _lib.KDA_ERR_INVALID_ARGUMENT  # overlaps conv_state
    assert "overlaps" in lib.kda_last_error_detail().decode()
    assert call(b=None) == _lib.KDA_ERR_INVALID_ARGUMENT
    assert call(H=0) == _lib.KDA_ERR_INVALID_ARGUMENT
    # an empty batch touches nothing: NULL pools and tokens are fine
    assert call(B=0, slots=0, **{n: None for n in ["q_in", "k_in", "v_in", "w_q", "w_k", "w_v", "g", "b",
                                                   "cs", "state", "out"]}) == _lib.KDA_OK


def test_spec_verify_rejects_bad_arguments(lib):
    names = ["q_in", "k_in", "v_in", "w_q", "w_k", "w_v", "g", "b", "cs", "state", "acc", "drafts", "out"]

    def call(**kw):
        a = dict(B=2, T=4, H=2, dk=16, dv=16, x=1, slots=2, idx=None, z=None)
        a.update({n: FAKE + i * 2**20 for i, n in enumerate(names)})
        a.update(kw)
        return lib.kda_spec_verify(a["B"], a["T"], a["H"], a["dk"], a["dv"], a["x"],
                                   *[P(a[n]) for n in names[:8]], P(a["cs"]), P(a["z"]), P(a["state"]),
                                   a["slots"], P(a["idx"]), P(a["acc"]), P(a["drafts"]), P(a["out"]), None)
    per_slot = lib.kda_spec_draft_bytes(2, 16, 16, 1)
    assert per_slot == 8 * 2 * (3 * 16 + 16 + 8) * 2
    assert lib.kda_spec_draft_bytes(2, 16, 48, 1) == 0
    assert call(T=9) == _lib.KDA_ERR_INVALID_ARGUMENT
    assert "T=9" in lib.kda_last_error_detail().decode()
    assert call(T=-1) == _lib.KDA_ERR_INVALID_ARGUMENT
    assert call(dv=8) == _lib.KDA_ERR_UNSUPPORTED
    assert call(drafts=None) == _lib.KDA_ERR_INVALID_ARGUMENT
    assert call(drafts=FAKE + 9 * 2**20 + 2048) == _lib.KDA_ERR_INVALID_ARGUMENT  # overlaps state
    assert "overlaps" in lib.kda_last_error_detail().decode()
    assert call(acc=FAKE + 10 * 2**20 + 2) == _lib.KDA_ERR_INVALID_ARGUMENT  # misaligned
    assert call(slots=3) == _lib.KDA_ERR_INVALID_ARGUMENT  # NULL indices need one slot per row
    # a commit-only call (T = 0) needs no token inputs and no output
    assert call(B=0, T=0, slots=0, **{n: None for n in names}) == _lib.KDA_OK


def test_snapshot_requests_rejected(lib):
    def call(**kw):
        a = dict(T=1024, interval=128, snaps=FAKE + 2**32, cap=8, off=FAKE + 2**33)
        a.update(kw)
        ws = lib.kda_prefill_workspace_bytes(a["T"], 1, 2, 16, 16, 0)
        return lib.kda_prefill_chunked_snap(a["T"], 2, 16, 16, None, 1, 0, 0,
                                            *[P(FAKE + i * 2**22) for i in range(6)], None, None,
                                            P(FAKE + 2**31), P(FAKE + 2**34), ws, a["interval"],
                                            P(a["snaps"]), a["cap"], P(a["off"]), None)
    assert call(interval=100) == _lib.KDA_ERR_INVALID_ARGUMENT
    assert "multiple of 64" in lib.kda_last_error_detail().decode()
    assert call(interval=0) == _lib.KDA_ERR_INVALID_ARGUMENT
    assert call(cap=7) == _lib.KDA_ERR_INVALID_ARGUMENT  # 1024 / 128 = 8 rows needed
    assert "snap_capacity" in lib.kda_last_error_detail().decode()
    assert call(off=None) == _lib.KDA_ERR_INVALID_ARGUMENT
    assert call(snaps=FAKE + 2**31 + 64) == _lib.KDA_ERR_INVALID_ARGUMENT  # overlaps out
    assert "overlaps" in lib.kda_last_error_detail().decode()
