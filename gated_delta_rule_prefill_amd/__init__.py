"""MI355X-native Kimi Delta Attention (KDA): chunkwise prefill and recurrent
decode behind the C ABI of ``include/kda.h`` (libkda.so, HIP for gfx950).

``prefill`` and ``decode_step`` marshal torch tensors to the library; the
library must be built (``python -m gated_delta_rule_prefill_amd.build``).
"""
from .kda import (KDAError, decode_step, prefill, prefill_kernel_times,  # noqa: F401
                  set_kernel_timing, workspace_bytes)

__all__ = ["prefill", "decode_step", "workspace_bytes", "KDAError", "set_kernel_timing",
           "prefill_kernel_times"]
