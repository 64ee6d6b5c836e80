"""MI355X-native Kimi Delta Attention (KDA): chunkwise prefill and recurrent
decode behind the C ABI of ``include/kda.h`` (libkda.so, HIP for gfx950).

``prefill``, ``decode_step`` and ``decode_tokens`` marshal torch tensors to the library; the
library must be built (``python -m gated_delta_rule_prefill_amd.build``).
"""
from .kda import (KDAError, backward, backward_workspace_bytes, decode_step,  # noqa: F401
                  decode_tokens, num_chunk_states, prefill, prefill_kernel_times,
                  set_kernel_timing, workspace_bytes)

__all__ = ["prefill", "decode_step", "decode_tokens", "backward", "num_chunk_states",
           "workspace_bytes", "backward_workspace_bytes", "KDAError", "set_kernel_timing",
           "prefill_kernel_times"]
