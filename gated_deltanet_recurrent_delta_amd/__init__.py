"""Gated DeltaNet recurrence on MI355X (gfx950): chunked prefill and decode
step as hand-written HIP kernels behind the C ABI of libgdn.so.

    from gated_deltanet_recurrent_delta_amd import prefill, decode_step

The binding (and with it libgdn.so) is loaded on first use of one of these
names, so `python -m gated_deltanet_recurrent_delta_amd.build` works before
the library exists.
"""

_EXPORTS = ("GdnError", "backward", "backward_workspace_bytes", "decode_step", "decode_step_qk", "drrqr_select", "gated_recurrent", "prefill",
            "prefill_prepare", "prefill_qk", "prefill_qk_workspace_bytes",
            "prefill_scan", "prefill_segments", "prefill_workspace_bytes",
            "status_str", "version")

__all__ = list(_EXPORTS)


def __getattr__(name):
    if name in _EXPORTS:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
