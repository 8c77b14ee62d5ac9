"""libkda: the Kimi Delta Attention token mixer on MI355X (gfx950).

``gated_delta_rule_64_amd.kda`` is the Python binding of the C ABI in
``include/kda.h`` (``kda_preprocess``, ``kda_prefill_chunked``,
``kda_prefill_workspace_bytes``, ``kda_decode_step``); importing it loads
``libkda.so`` lazily on first call and raises if it is not built.
``gated_delta_rule_64_amd.synth`` draws the seeded synthetic inputs.
"""

__all__ = ["kda", "synth", "build"]
