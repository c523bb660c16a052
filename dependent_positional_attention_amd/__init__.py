"""PaTH attention on MI355X (gfx950): hand-written HIP kernels behind a C ABI.

Public entry points (same names as the C ABI in include/path_attn.h):
    path_attn_fwd (= path_attn_prep + path_attn_scan), path_attn_fwd_workspace_bytes,
    path_attn_workspace_layout, path_attn_cache_from_prefill, path_decode_step,
    path_decode_workspace_bytes, path_decode_step_deferred, path_decode_deferred_state_bytes,
    path_attn_bwd, path_attn_bwd_workspace_bytes.
The seeded synthetic input generator is in ``synth``; it needs no GPU.
"""
from . import synth  # noqa: F401

__all__ = ["path_attn_fwd", "path_attn_prep", "path_attn_scan", "path_attn_fwd_workspace_bytes",
           "path_attn_workspace_layout", "path_attn_cache_from_prefill", "path_decode_step",
           "path_decode_workspace_bytes", "path_decode_step_deferred", "path_decode_deferred_state_bytes",
           "path_attn_bwd", "path_attn_bwd_workspace_bytes", "synth"]


def __getattr__(name):
    # The binding imports torch and loads the HIP library lazily, so that
    # ``synth`` stays usable without either.
    if name in __all__ and name != "synth":
        from . import native
        return getattr(native, name)
    raise AttributeError(name)
