"""Complex KDA (CKDA) recurrence on AMD Instinct MI355X (gfx950).

``forward``, ``kda_forward``, ``backward`` and ``decode_step`` are thin wrappers over the C-ABI library
``libckda.so`` (see ``include/ckda.h``); they marshal torch tensors and the
current HIP stream and nothing else.  The library is loaded on first use; if it
is missing the call raises instead of falling back to any other code.
"""
from . import workloads  # noqa: F401  (seeded input generators; no GPU needed)

__all__ = ["forward", "kda_forward", "backward", "decode_step", "forward_workspace_bytes",
           "backward_workspace_bytes", "library", "CkdaError", "workloads"]


def __getattr__(name):
    if name in ("forward", "kda_forward", "backward", "decode_step", "forward_workspace_bytes",
                "backward_workspace_bytes", "library", "CkdaError"):
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(name)
