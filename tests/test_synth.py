"""The seeded input generator: formats and reproducibility (CPU only)."""

import numpy as np
import torch

from gated_delta_rule_64_amd import synth


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32) * 10.0,
                        np.array([0.0, -0.0, 1e-40, -1e-40, 3.3e38, -3.3e38, np.inf, -np.inf],
                                 dtype=np.float32)])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_workloads_are_reproducible_and_blocked():
    a = synth.make("layer_t4k", lengths=(5000,), H=2)
    b = synth.make("layer_t4k", lengths=(5000,), H=2)
    for key in ("q_in", "k_in", "v_in", "g", "b", "z", "w_q"):
        assert np.array_equal(a[key], b[key])
    # blocks of 4096 rows are seeded independently: the first block does not
    # depend on the total length
    c = synth.make("layer_t4k", lengths=(4096,), H=2)
    assert np.array_equal(a["q_in"][:4096], c["q_in"])
    assert a["q_in"].dtype == np.uint16 and a["q_in"].shape == (5000, 256)


def test_named_workload_shapes():
    w = synth.workload("varlen_64")
    assert w.N == 64 and all(1024 <= L <= 32768 for L in w.lengths)
    d = synth.make("decode_b256", H=2)
    assert d["conv_state"].shape == (256, 3, 2 * 384)
    assert d["S0"].shape == (256, 2, 128, 128)
    assert np.array_equal(d["cu_seqlens"], np.arange(257))
    t = synth.make("core_tiny")
    assert t["q_in"].dtype == np.float32 and t["z"] is None
    assert np.all(t["w_q"][:, :3] == 0) and np.all(t["w_q"][:, 3] == 1)
    s = synth.make("varlen_64", lengths=(3, 4, 5, 6), H=1)
    assert np.all(s["S0"][0] == 0) and np.all(s["S0"][2] == 0) and np.any(s["S0"][1] != 0)
