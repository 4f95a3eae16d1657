"""Gated DeltaNet recurrence on MI355X (gfx950): chunked prefill and decode
step as hand-written HIP kernels behind the C ABI of libgdn.so.

    from gated_deltanet_recurrent_delta_amd import prefill, decode_step
"""

from .binding import (GdnError, decode_step, prefill, prefill_prepare,  # noqa: F401
                      prefill_scan, prefill_workspace_bytes, status_str,
                      version)
