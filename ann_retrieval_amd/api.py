"""Python binding over the C ABI: the same four calls, on torch tensors.

This layer only marshals arguments: it checks shapes and dtypes, allocates
the caller-owned device buffers with torch, and passes raw pointers and the
current HIP stream to ``libice.so``. Every step of the hot path runs in the
library's HIP kernels.
"""
from __future__ import annotations

import ctypes
import math

import numpy as np
import torch

from . import _lib
from ._lib import IceParams, IceHeadStats, check

_DT = {"f32": (_lib.ICE_F32, torch.float32), "bf16": (_lib.ICE_BF16, torch.bfloat16)}


def _stream_ptr(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


class PinnedHost:
    """Pinned host memory of an exact size from hipHostMalloc (mapped into the
    device address space), freed with hipHostFree. torch's pinned allocator
    rounds sizes up to powers of two, which doubles a multi-GB pool."""

    _hip = None

    def __init__(self, nbytes: int):
        if PinnedHost._hip is None:
            hip = ctypes.CDLL("libamdhip64.so")
            hip.hipHostMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t, ctypes.c_uint]
            hip.hipHostMalloc.restype = ctypes.c_int
            hip.hipHostFree.argtypes = [ctypes.c_void_p]
            hip.hipHostFree.restype = ctypes.c_int
            PinnedHost._hip = hip
        self.ptr = ctypes.c_void_p()
        self.nbytes = int(nbytes)
        rc = PinnedHost._hip.hipHostMalloc(ctypes.byref(self.ptr), max(self.nbytes, 1), 0)
        if rc != 0 or not self.ptr.value:
            raise MemoryError(f"hipHostMalloc of {self.nbytes} bytes failed with status {rc}")

    def data_ptr(self) -> int:
        return int(self.ptr.value)

    def __del__(self):
        if getattr(self, "ptr", None) is not None and self.ptr.value and PinnedHost._hip is not None:
            PinnedHost._hip.hipHostFree(self.ptr)
            self.ptr = None


def make_params(n_heads: int, group: int, d: int, dtype: str, capacity: int, levels: int = 3,
                promote_log2: int = 4, seed: int = 0, host_pool: bool = False, resident: int = 0,
                resort: bool = False) -> IceParams:
    flags = (_lib.ICE_HOST_POOL if host_pool else 0) | (_lib.ICE_SPLIT_RESORT if resort else 0)
    return IceParams(n_heads=n_heads, group=group, d=d, dtype=_DT[dtype][0], page_cap=_lib.ICE_PAGE_CAP,
                     levels=levels, promote_log2=promote_log2, capacity=capacity,
                     flags=flags, seed=seed, resident=resident)


def ice_index_bytes(p: IceParams) -> int:
    return int(_lib.load().ice_index_bytes(ctypes.byref(p)))


def ice_workspace_bytes(p: IceParams, max_budget_tokens: int) -> int:
    return int(_lib.load().ice_workspace_bytes(ctypes.byref(p), max_budget_tokens))


class IceIndex:
    """One index object: H independent heads, their device blob and workspace.

    ``ice_build`` / ``ice_insert`` / ``ice_select`` / ``ice_attend`` map one to
    one onto the C entry points of the same names. With ``host_pool=True`` the
    V pages live in a pinned host tensor (``self.pool``) and every attend
    gathers the union's pages over the host link first. ``resident`` reserves
    room for that many resident (sink and window) tokens per head, set with
    ``set_resident``; ``set_dense`` flags heads whose attention covers every
    indexed token. ``resort=True`` makes inserts split by re-sorting the
    owner's members over its pages (ICE_SPLIT_RESORT) instead of appending.
    """

    def __init__(self, n_heads: int, group: int, d: int, dtype: str, capacity: int, levels: int = 3,
                 promote_log2: int = 4, seed: int = 0, max_budget: int = 256, device="cuda",
                 host_pool: bool = False, resident: int = 0, resort: bool = False):
        self.lib = _lib.load()
        dev = torch.device(device)
        if dev.type == "cuda" and dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        self.device = dev
        self.dtype = dtype
        self.tdtype = _DT[dtype][1]
        self.p = make_params(n_heads, group, d, dtype, capacity, levels, promote_log2, seed, host_pool, resident,
                             resort)
        self.H, self.G, self.d, self.capacity, self.levels = n_heads, group, d, capacity, levels
        self.max_budget = max_budget
        nbytes = ice_index_bytes(self.p)
        if nbytes == 0:
            raise _lib.IceError(_lib.ICE_ERR_ARG, "ice_index_bytes")
        self.blob = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.ws_bytes = ice_workspace_bytes(self.p, max_budget)
        if self.ws_bytes == 0:
            raise _lib.IceError(_lib.ICE_ERR_ARG, "ice_workspace_bytes")
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        h = ctypes.c_void_p()
        check(self.lib.ice_create(ctypes.byref(self.p), _ptr(self.blob), nbytes, ctypes.byref(h)), "ice_create")
        self.handle = h
        self.pool = None
        if host_pool:
            pool_bytes = int(self.lib.ice_host_pool_bytes(ctypes.byref(self.p)))
            self.pool = PinnedHost(pool_bytes)
            check(self.lib.ice_attach_host_pool(self.handle, ctypes.c_void_p(self.pool.data_ptr()), pool_bytes),
                  "ice_attach_host_pool")

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            self.lib.ice_destroy(h)
            self.handle = None
        self.pool = None

    # ---- the four calls -------------------------------------------------
    def _check_kv(self, x: torch.Tensor, name: str):
        if x.device != self.device or x.dtype != self.tdtype:
            raise TypeError(f"{name} must be a {self.tdtype} tensor on {self.device}")
        if x.dim() != 3 or x.shape[0] != self.H or x.shape[2] != self.d:
            raise ValueError(f"{name} must have shape [H={self.H}, n, d={self.d}], got {tuple(x.shape)}")
        if x.stride(2) != 1 or x.stride(1) != self.d:
            raise ValueError(f"{name} rows must be contiguous")

    def ice_build(self, K: torch.Tensor, V: torch.Tensor) -> None:
        self._check_kv(K, "K")
        self._check_kv(V, "V")
        if K.shape != V.shape or K.stride() != V.stride():
            raise ValueError("K and V must have the same shape and strides")
        check(self.lib.ice_build(self.handle, _ptr(K), _ptr(V), K.shape[1], K.stride(0), _ptr(self.ws),
                                 self.ws_bytes, _stream_ptr(self.device)), "ice_build")

    def ice_build_noalloc(self, K: torch.Tensor, V: torch.Tensor) -> None:
        """ice_build with the library's fixed device scratch instead of this object's workspace (allocates
        nothing; see include/ice.h)."""
        self._check_kv(K, "K")
        self._check_kv(V, "V")
        if K.shape != V.shape or K.stride() != V.stride():
            raise ValueError("K and V must have the same shape and strides")
        check(self.lib.ice_build_noalloc(self.handle, _ptr(K), _ptr(V), K.shape[1], K.stride(0),
                                         _stream_ptr(self.device)), "ice_build_noalloc")

    def ice_build_timed(self, K: torch.Tensor, V: torch.Tensor) -> np.ndarray:
        """ice_build with per-phase times (ms, ICE_BUILD_PHASES entries; see include/ice.h), measured by events
        on the current stream; waits for the build to finish."""
        self._check_kv(K, "K")
        self._check_kv(V, "V")
        if K.shape != V.shape or K.stride() != V.stride():
            raise ValueError("K and V must have the same shape and strides")
        ms = np.zeros(_lib.ICE_BUILD_PHASES, dtype=np.float32)
        check(self.lib.ice_build_timed(self.handle, _ptr(K), _ptr(V), K.shape[1], K.stride(0), _ptr(self.ws),
                                       self.ws_bytes, _stream_ptr(self.device), ms.ctypes.data_as(ctypes.c_void_p)),
              "ice_build_timed")
        return ms

    def ice_build_pdci(self, K: torch.Tensor, V: torch.Tensor, dirs: torch.Tensor, m: int, l: int, visits: int,
                       cands: int) -> None:
        """ice_build with parents found by P-DCI: dirs is a float32 [m*l, d+1] device tensor of projection
        directions; m composite indices of l simple indices, `visits` visits and `cands` candidates per
        composite index."""
        self._check_kv(K, "K")
        self._check_kv(V, "V")
        if K.shape != V.shape or K.stride() != V.stride():
            raise ValueError("K and V must have the same shape and strides")
        if dirs.device != self.device or dirs.dtype != torch.float32 or tuple(dirs.shape) != (m * l, self.d + 1) \
                or not dirs.is_contiguous():
            raise ValueError(f"dirs must be a contiguous float32 [{m * l}, {self.d + 1}] tensor on {self.device}")
        check(self.lib.ice_build_pdci(self.handle, _ptr(K), _ptr(V), K.shape[1], K.stride(0), _ptr(dirs), m, l,
                                      visits, cands, _ptr(self.ws), self.ws_bytes, _stream_ptr(self.device)),
              "ice_build_pdci")

    def ice_build_heads(self, K: torch.Tensor, V: torch.Tensor, h0: int, stream=None) -> None:
        """Builds heads h0 .. h0 + K.shape[0] - 1 from their rows K, V [n_heads, n, d], on `stream`
        (a torch.cuda.Stream; the current stream if None)."""
        if K.device != self.device or K.dtype != self.tdtype or K.dim() != 3 or K.shape[2] != self.d:
            raise TypeError(f"K must be a {self.tdtype} [n_heads, n, {self.d}] tensor on {self.device}")
        if K.shape != V.shape or K.stride() != V.stride() or K.stride(2) != 1 or K.stride(1) != self.d:
            raise ValueError("K and V must have the same shape and strides, rows contiguous")
        s = _stream_ptr(self.device) if stream is None else ctypes.c_void_p(stream.cuda_stream)
        check(self.lib.ice_build_heads(self.handle, _ptr(K), _ptr(V), K.shape[1], K.stride(0), h0, K.shape[0],
                                       _ptr(self.ws), self.ws_bytes, s), "ice_build_heads")

    def ice_build_reuse(self, K: torch.Tensor, V: torch.Tensor, h0: int, src_h0: int, stream=None) -> None:
        """Heads h0 .. h0 + K.shape[0] - 1 take the layout of heads src_h0 .. and their own rows K, V."""
        if K.device != self.device or K.dtype != self.tdtype or K.dim() != 3 or K.shape[2] != self.d:
            raise TypeError(f"K must be a {self.tdtype} [n_heads, n, {self.d}] tensor on {self.device}")
        if K.shape != V.shape or K.stride() != V.stride() or K.stride(2) != 1 or K.stride(1) != self.d:
            raise ValueError("K and V must have the same shape and strides, rows contiguous")
        s = _stream_ptr(self.device) if stream is None else ctypes.c_void_p(stream.cuda_stream)
        check(self.lib.ice_build_reuse(self.handle, _ptr(K), _ptr(V), K.shape[1], K.stride(0), h0, K.shape[0], src_h0,
                                       _ptr(self.ws), self.ws_bytes, s), "ice_build_reuse")

    def ice_insert(self, k_new: torch.Tensor, v_new: torch.Tensor) -> None:
        self._check_kv(k_new, "k_new")
        self._check_kv(v_new, "v_new")
        if not (k_new.is_contiguous() and v_new.is_contiguous()) or k_new.shape != v_new.shape:
            raise ValueError("k_new and v_new must be contiguous [H, n_new, d]")
        check(self.lib.ice_insert(self.handle, _ptr(k_new), _ptr(v_new), k_new.shape[1], _ptr(self.ws),
                                  self.ws_bytes, _stream_ptr(self.device)), "ice_insert")

    def set_resident(self, K: torch.Tensor | None, V: torch.Tensor | None) -> None:
        """Resident tokens [H, n, d] (sink, then window) attended beside the pages; None clears them."""
        if K is None or V is None or K.shape[1] == 0:
            check(self.lib.ice_set_resident(self.handle, None, None, 0, 0, _stream_ptr(self.device)),
                  "ice_set_resident")
            return
        self._check_kv(K, "K")
        self._check_kv(V, "V")
        if K.shape != V.shape or K.stride() != V.stride():
            raise ValueError("K and V must have the same shape and strides")
        check(self.lib.ice_set_resident(self.handle, _ptr(K), _ptr(V), K.shape[1], K.stride(0),
                                        _stream_ptr(self.device)), "ice_set_resident")

    def set_dense(self, dense) -> None:
        """Per-head dense flags (a sequence of H booleans, or None for none)."""
        if dense is None:
            check(self.lib.ice_set_dense(self.handle, None, _stream_ptr(self.device)), "ice_set_dense")
            return
        flags = np.ascontiguousarray(np.asarray(dense, dtype=bool).astype(np.uint8))
        if flags.shape != (self.H,):
            raise ValueError(f"dense must have {self.H} entries")
        check(self.lib.ice_set_dense(self.handle, flags.ctypes.data_as(ctypes.c_void_p), _stream_ptr(self.device)),
              "ice_set_dense")

    def ice_select(self, Q: torch.Tensor, budget_tokens: int, beam: int | None = None, trace: bool = False):
        """Returns (sel [H,G,k], uni [H,G*k], n_uni [H]) int32 device tensors (+ trace [H,G,L,beam])."""
        self._check_q(Q)
        k = budget_tokens // _lib.ICE_PAGE_CAP
        beam = k if beam is None else beam
        sel = torch.empty(self.H, self.G, k, dtype=torch.int32, device=self.device)
        uni = torch.empty(self.H, self.G * k, dtype=torch.int32, device=self.device)
        n_uni = torch.empty(self.H, dtype=torch.int32, device=self.device)
        tr = torch.empty(self.H, self.G, self.levels, beam, dtype=torch.int32, device=self.device) if trace else None
        check(self.lib.ice_select(self.handle, _ptr(Q), budget_tokens, beam, _ptr(sel), _ptr(uni), _ptr(n_uni),
                                  _ptr(tr), _ptr(self.ws), self.ws_bytes, _stream_ptr(self.device)), "ice_select")
        return (sel, uni, n_uni, tr) if trace else (sel, uni, n_uni)

    def ice_attend(self, Q: torch.Tensor, uni: torch.Tensor, n_uni: torch.Tensor, scale: float | None = None,
                   out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
        """Returns (O [H,G,d] fp32, lse [H,G] fp32)."""
        self._check_q(Q)
        if uni.dtype != torch.int32 or n_uni.dtype != torch.int32 or not uni.is_contiguous():
            raise TypeError("uni and n_uni must be contiguous int32 tensors")
        scale = 1.0 / math.sqrt(self.d) if scale is None else scale
        O = torch.empty(self.H, self.G, self.d, dtype=torch.float32, device=self.device) if out is None else out
        L = torch.empty(self.H, self.G, dtype=torch.float32, device=self.device) if lse is None else lse
        check(self.lib.ice_attend(self.handle, _ptr(Q), _ptr(uni), _ptr(n_uni), uni.shape[1], scale, _ptr(O),
                                  _ptr(L), _ptr(self.ws), self.ws_bytes, _stream_ptr(self.device)), "ice_attend")
        return O, L

    def ice_decode(self, Q: torch.Tensor, budget_tokens: int, beam: int | None = None, scale: float | None = None):
        """One decode step (select + attend): returns (sel, uni, n_uni, O, lse)."""
        self._check_q(Q)
        k = budget_tokens // _lib.ICE_PAGE_CAP
        beam = k if beam is None else beam
        scale = 1.0 / math.sqrt(self.d) if scale is None else scale
        sel = torch.empty(self.H, self.G, k, dtype=torch.int32, device=self.device)
        uni = torch.empty(self.H, self.G * k, dtype=torch.int32, device=self.device)
        n_uni = torch.empty(self.H, dtype=torch.int32, device=self.device)
        O = torch.empty(self.H, self.G, self.d, dtype=torch.float32, device=self.device)
        L = torch.empty(self.H, self.G, dtype=torch.float32, device=self.device)
        check(self.lib.ice_decode(self.handle, _ptr(Q), budget_tokens, beam, _ptr(sel), _ptr(uni), _ptr(n_uni),
                                  scale, _ptr(O), _ptr(L), _ptr(self.ws), self.ws_bytes, _stream_ptr(self.device)),
              "ice_decode")
        return sel, uni, n_uni, O, L

    def _check_q(self, Q: torch.Tensor):
        if Q.device != self.device or Q.dtype != self.tdtype or tuple(Q.shape) != (self.H, self.G, self.d) \
                or not Q.is_contiguous():
            raise ValueError(f"Q must be a contiguous {self.tdtype} tensor [H, G, d] on {self.device}")

    # ---- inspection ------------------------------------------------------
    def n_tokens(self) -> int:
        return int(self.lib.ice_n_tokens(self.handle))

    def export(self, head: int, what: int, level: int = 0, np_dtype=np.int32) -> np.ndarray:
        n = int(self.lib.ice_export_bytes(self.handle, what, level))
        buf = np.empty(n, dtype=np.uint8)
        check(self.lib.ice_export(self.handle, head, what, level, buf.ctypes.data_as(ctypes.c_void_p), n,
                                  _stream_ptr(self.device)), "ice_export")
        return buf.view(np_dtype)

    def stats(self, head: int) -> dict:
        st = IceHeadStats()
        check(self.lib.ice_export(self.handle, head, _lib.ICE_EXP_HEADER, 0, ctypes.byref(st), ctypes.sizeof(st),
                                  _stream_ptr(self.device)), "ice_export")
        return dict(n_tokens=st.n_tokens, top_level=st.top_level, n_top=st.n_top, n_pages=list(st.n_pages),
                    clamps=st.clamps, splits=st.splits, near_ties=st.near_ties, overflow=st.overflow,
                    sync_timeouts=st.sync_timeouts, n_resident=st.n_resident, dense=st.dense, M2=st.M2)
