"""ctypes view of ``include/ice.h``: loads ``libice.so`` and declares every entry point.

There is no fallback: if the library is not built, importing the binding
raises, so nothing can silently run another implementation.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libice.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "ice.h")

c_i32, c_i64, c_u64, c_f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float
c_size, c_void_p, c_char_p = ctypes.c_size_t, ctypes.c_void_p, ctypes.c_char_p

ICE_OK, ICE_ERR_ARG, ICE_ERR_DTYPE, ICE_ERR_STATE, ICE_ERR_CAPACITY, ICE_ERR_HIP = 0, -1, -2, -3, -4, -5
ICE_F32, ICE_BF16 = 0, 1
ICE_HOST_POOL, ICE_SPLIT_RESORT, ICE_RESPLIT_MAX = 1, 2, 1024
ICE_PDCI_MAX_KEYS, ICE_PDCI_MAX_L = 16, 4
ICE_PAGE_CAP, ICE_MAX_LEVELS, ICE_MAX_GROUP, ICE_MAX_BEAM, ICE_MAX_RESIDENT = 16, 4, 16, 256, 4096
ICE_NOALLOC_SCRATCH_BYTES = 64 << 20
ICE_BUILD_PHASES, ICE_PHASE_LIFT, ICE_PHASE_OPERAND, ICE_PHASE_PARENT, ICE_PHASE_PACK, ICE_PHASE_COPY, ICE_PHASE_TOP = \
    14, 0, 1, 2, 3, 4, 13
(ICE_EXP_LEVEL, ICE_EXP_LIFT, ICE_EXP_PARENT, ICE_EXP_PAGE_TOK, ICE_EXP_PAGE_CNT, ICE_EXP_PAGE_NEXT,
 ICE_EXP_PAGE_OWNER, ICE_EXP_OWNER_FIRST, ICE_EXP_OWNER_TAIL, ICE_EXP_TOP, ICE_EXP_PAGE_K, ICE_EXP_PAGE_V,
 ICE_EXP_HEADER, ICE_EXP_OWNER_RUN, ICE_EXP_OWNER_COUNT) = range(15)


class IceParams(ctypes.Structure):
    _fields_ = [("n_heads", c_i32), ("group", c_i32), ("d", c_i32), ("dtype", c_i32), ("page_cap", c_i32),
                ("levels", c_i32), ("promote_log2", c_i32), ("capacity", c_i32), ("flags", ctypes.c_uint32),
                ("seed", c_u64), ("resident", c_i32)]


class IceHeadStats(ctypes.Structure):
    _fields_ = [("n_tokens", c_i32), ("top_level", c_i32), ("n_top", c_i32), ("n_pages", c_i32 * ICE_MAX_LEVELS),
                ("clamps", c_i32), ("splits", c_i32), ("near_ties", c_i32), ("overflow", c_i32),
                ("sync_timeouts", c_i32), ("n_resident", c_i32), ("dense", c_i32), ("M2", ctypes.c_double)]


_SIGNATURES = {
    "ice_index_bytes": (c_size, [ctypes.POINTER(IceParams)]),
    "ice_workspace_bytes": (c_size, [ctypes.POINTER(IceParams), c_i32]),
    "ice_create": (ctypes.c_int, [ctypes.POINTER(IceParams), c_void_p, c_size, ctypes.POINTER(c_void_p)]),
    "ice_destroy": (None, [c_void_p]),
    "ice_host_pool_bytes": (c_size, [ctypes.POINTER(IceParams)]),
    "ice_attach_host_pool": (ctypes.c_int, [c_void_p, c_void_p, c_size]),
    "ice_build": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, c_i32, c_i64, c_void_p, c_size, c_void_p]),
    "ice_build_noalloc": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, c_i32, c_i64, c_void_p]),
    "ice_build_timed": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, c_i32, c_i64, c_void_p, c_size, c_void_p,
                                       c_void_p]),
    "ice_build_pdci": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, c_i32, c_i64, c_void_p, c_i32, c_i32, c_i32, c_i32,
                                      c_void_p, c_size, c_void_p]),
    "ice_build_heads": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, c_i32, c_i64, c_i32, c_i32, c_void_p, c_size,
                                       c_void_p]),
    "ice_build_reuse": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, c_i32, c_i64, c_i32, c_i32, c_i32, c_void_p,
                                       c_size, c_void_p]),
    "ice_insert": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, c_i32, c_void_p, c_size, c_void_p]),
    "ice_select": (ctypes.c_int, [c_void_p, c_void_p, c_i32, c_i32, c_void_p, c_void_p, c_void_p, c_void_p,
                                  c_void_p, c_size, c_void_p]),
    "ice_attend": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_i32, c_f32, c_void_p, c_void_p,
                                  c_void_p, c_size, c_void_p]),
    "ice_decode": (ctypes.c_int, [c_void_p, c_void_p, c_i32, c_i32, c_void_p, c_void_p, c_void_p, c_f32, c_void_p,
                                  c_void_p, c_void_p, c_size, c_void_p]),
    "ice_set_resident": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, c_i32, c_i64, c_void_p]),
    "ice_set_dense": (ctypes.c_int, [c_void_p, c_void_p, c_void_p]),
    "ice_export_bytes": (c_size, [c_void_p, c_i32, c_i32]),
    "ice_export": (ctypes.c_int, [c_void_p, c_i32, c_i32, c_i32, c_void_p, c_size, c_void_p]),
    "ice_n_tokens": (c_i32, [c_void_p]),
    "ice_last_error": (c_char_p, []),
}

_lib = None


def header_functions() -> list[str]:
    """Names of every function ``include/ice.h`` declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ice_[a-z_0-9]+)\s*\(", text)))


def load() -> ctypes.CDLL:
    """The loaded library with its signatures declared; raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m ann_retrieval_amd.build` "
                          "(the HIP library is required, there is no fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class IceError(RuntimeError):
    def __init__(self, code: int, what: str):
        lib = load()
        msg = lib.ice_last_error().decode(errors="replace")
        super().__init__(f"{what} failed with status {code}: {msg}")
        self.code = code


def check(rc: int, what: str) -> None:
    if rc != ICE_OK:
        raise IceError(rc, what)
