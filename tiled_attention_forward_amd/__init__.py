"""MI355X-native fused attention forward (tiled, online softmax, HIP/gfx950).

The C-ABI library ``libfa.so`` (built from ``csrc/``) does all the work; the
Python names below only marshal arguments into it.  Importing this package
does not load the library: the first call does, and it raises if the library
is missing or does not load.
"""

from . import metrics, workloads  # noqa: F401

_BINDING_NAMES = ("fa_forward", "fa_forward_split", "fa_merge", "fa_backward", "fa_split_count",
                  "fa_split_workspace_bytes", "fa_backward_workspace_bytes", "fa_check_args",
                  "fa_status_string", "fa_version", "forward", "forward_split", "merge",
                  "backward", "FaError", "library_path", "load_library")


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
