"""Kimi Delta Attention (KDA) forward hot path for AMD MI355X (gfx950).

The computation lives in the HIP library libkda.so (C ABI in include/kda.h);
this package holds its ctypes binding (`_lib`), the in-tree build script
(`build`) and the seeded synthetic input generator (`inputs`).

    from linear_attention_sequence_gate_amd import kda_gate, kda_chunk_fwd, kda_decode_step
"""
__all__ = ["kda_gate", "kda_chunk_fwd", "kda_chunk_fwd_workspace_size",
           "kda_chunk_fwd_gated", "kda_chunk_fwd_gated_workspace_size",
           "kda_chunk_fwd_gated_noalloc",
           "kda_chunk_fwd_varlen_pooled_gated",
           "kda_chunk_fwd_auto_segments", "kda_chunk_fwd_plan", "kda_decode_step", "kda_state_pool_reset",
           "kda_chunk_fwd_pooled", "kda_chunk_fwd_varlen_pooled", "kda_decode_step_pooled",
           "kda_chunk_bwd", "kda_chunk_bwd_workspace_size", "kda_chunk_bwd_workspace_size_flags",
           "kda_gate_bwd",
           "kda_gate_bwd_workspace_size", "kda_last_error", "kda_version",
           "KdaError"]


def __getattr__(name):
    # the binding (and torch) load on first use, so `inputs` and `build` stay light
    if name in __all__:
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(name)
