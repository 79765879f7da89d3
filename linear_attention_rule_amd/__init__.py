"""KDA (Kimi Delta Attention) recurrence on AMD MI355X: Python face of libkda.

    from linear_attention_rule_amd import chunk_prefill, recurrent_verify, commit_accepted

All calls run entirely in the HIP kernels of libkda.so (built in-tree by
``python -m linear_attention_rule_amd.build``); nothing falls back to the CPU.
"""

from ._binding import (KDAError, chunk_prefill, commit_accepted, default_scale,  # noqa: F401
                       gated_rmsnorm, header_entry_points, load_library,
                       prefill_workspace_bytes, recurrent_verify)

__all__ = ["chunk_prefill", "recurrent_verify", "commit_accepted", "gated_rmsnorm",
           "load_library", "prefill_workspace_bytes", "KDAError", "default_scale",
           "header_entry_points"]
