"""KDA (Kimi Delta Attention) recurrence on AMD MI355X: Python face of libkda.

    from linear_attention_rule_amd import chunk_prefill, recurrent_verify, commit_accepted

All calls run entirely in the HIP kernels of libkda.so (built in-tree by
``python -m linear_attention_rule_amd.build``); nothing falls back to the CPU.
"""

from ._binding import (KDAError, causal_conv1d_prefill, causal_conv1d_update,  # noqa: F401
                       chunk_prefill, chunk_prefill_noalloc, commit_accepted,
                       default_scale, gated_rmsnorm, header_entry_points, load_library,
                       noalloc_scratch_bytes, prefill_workspace_bytes, recurrent_verify,
                       recurrent_verify_gated)

__all__ = ["chunk_prefill", "chunk_prefill_noalloc", "noalloc_scratch_bytes", "recurrent_verify", "recurrent_verify_gated", "commit_accepted", "gated_rmsnorm",
           "causal_conv1d_prefill", "causal_conv1d_update", "load_library",
           "prefill_workspace_bytes", "KDAError", "default_scale", "header_entry_points"]
