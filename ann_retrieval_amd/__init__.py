"""IceCache hot path on MI355X: M-DCI semantic pages, top-k page selection and
sparse attention as hand-written HIP kernels behind a small C ABI
(``include/ice.h``). ``api.IceIndex`` is the Python binding.
"""
from . import _lib  # noqa: F401

__all__ = ["IceIndex", "make_params"]


def __getattr__(name):
    if name in ("IceIndex", "make_params", "ice_index_bytes", "ice_workspace_bytes"):
        from . import api
        return getattr(api, name)
    raise AttributeError(name)
