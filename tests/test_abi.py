"""The C-ABI library on the host (no GPU calls): it loads, exports every
function ``include/ice.h`` declares, sizes its blobs from the promotion draws,
and rejects bad arguments before enqueuing anything.
"""
import ctypes
import os

import numpy as np
import pytest

from ann_retrieval_amd import _lib as L
from ann_retrieval_amd.api import make_params
from oracle import icecache as ic


@pytest.fixture(scope="module")
def lib():
    return L.load()


def test_every_declared_function_is_exported(lib):
    names = L.header_functions()
    assert {"ice_build", "ice_insert", "ice_select", "ice_attend"} <= set(names)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_constants_match_the_header():
    import re
    text = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "ice.h")).read()
    defs = dict(re.findall(r"^#define (ICE_[A-Z0-9_]+)\s+\(?(-?\d+)u?\)?", text, flags=re.M))
    shared = [n for n in defs if hasattr(L, n)]
    assert {"ICE_HOST_POOL", "ICE_SPLIT_RESORT", "ICE_RESPLIT_MAX", "ICE_PAGE_CAP"} <= set(shared)
    for n in shared:
        assert getattr(L, n) == int(defs[n]), n


def test_binding_declares_every_function():
    assert set(L.header_functions()) == set(L._SIGNATURES)


def _fake_handle(lib, p):
    h = ctypes.c_void_p()
    n = lib.ice_index_bytes(ctypes.byref(p))
    rc = lib.ice_create(ctypes.byref(p), ctypes.c_void_p(1 << 20), n, ctypes.byref(h))
    assert rc == L.ICE_OK
    return h


@pytest.mark.parametrize("H,cap,levels,plog2", [(3, 5000, 3, 4), (2, 777, 4, 2), (1, 100, 1, 4), (4, 33, 2, 3)])
def test_page_tables_are_sized_by_the_promotion_draws(lib, H, cap, levels, plog2):
    p = make_params(H, 2, 128, "bf16", cap, levels, plog2, seed=11)
    h = _fake_handle(lib, p)
    try:
        # level counts from the oracle's own draws over every position
        lev = np.stack([ic.draw_levels(11, hh, 0, cap, levels, plog2) for hh in range(H)])
        ncap = [cap] + [int((lev >= l).sum(axis=1).max()) for l in range(1, levels)]
        ntab = max(1, levels - 1)
        for t in range(ntab):
            owners = ncap[t + 1] if t + 1 < levels else 0
            bound = (ncap[t] + 15 * max(owners, 1) + 15) // 16
            assert lib.ice_export_bytes(h, L.ICE_EXP_PAGE_TOK, t) == bound * 16 * 4
            assert lib.ice_export_bytes(h, L.ICE_EXP_PAGE_K, t) == bound * 16 * 128 * 2
        assert lib.ice_export_bytes(h, L.ICE_EXP_PAGE_TOK, ntab) == 0
        assert lib.ice_export_bytes(h, L.ICE_EXP_TOP, 0) == (max(ncap[1], 1) * 4 if levels >= 2 else 0)
    finally:
        lib.ice_destroy(h)


def test_invalid_params_give_zero_sizes(lib):
    for kw in [dict(d=96), dict(group=0), dict(group=17), dict(capacity=0), dict(levels=5)]:
        base = dict(n_heads=2, group=4, d=128, dtype="bf16", capacity=100)
        base.update(kw)
        p = make_params(**base)
        assert lib.ice_index_bytes(ctypes.byref(p)) == 0
    p = make_params(2, 4, 128, "bf16", 100)
    assert lib.ice_workspace_bytes(ctypes.byref(p), 24) == 0
    assert lib.ice_workspace_bytes(ctypes.byref(p), 256) > 0
    p.page_cap = 8
    assert lib.ice_index_bytes(ctypes.byref(p)) == 0
    assert b"page_cap" in lib.ice_last_error()
    # resident tokens: bounded, and only with the device V pool
    for kw in [dict(resident=-1), dict(resident=L.ICE_MAX_RESIDENT + 1), dict(resident=16, host_pool=True),
               dict(capacity=(1 << 26) + 1), dict(resort=True, host_pool=True)]:
        base = dict(n_heads=2, group=4, d=128, dtype="bf16", capacity=100)
        base.update(kw)
        assert lib.ice_index_bytes(ctypes.byref(make_params(**base))) == 0
    # the re-sort split is a flag of its own; unknown flag bits are refused
    n0 = lib.ice_index_bytes(ctypes.byref(make_params(2, 4, 128, "bf16", 100)))
    assert lib.ice_index_bytes(ctypes.byref(make_params(2, 4, 128, "bf16", 100, resort=True))) == n0
    p = make_params(2, 4, 128, "bf16", 100)
    p.flags = 4
    assert lib.ice_index_bytes(ctypes.byref(p)) == 0 and b"flags" in lib.ice_last_error()
    # resident pages add to the blob: 100 tokens -> 7 pages of K and V per head
    n0 = lib.ice_index_bytes(ctypes.byref(make_params(2, 4, 128, "bf16", 100)))
    n1 = lib.ice_index_bytes(ctypes.byref(make_params(2, 4, 128, "bf16", 100, resident=100)))
    assert n1 - n0 >= 2 * 7 * (2 * 16 * 128 * 2 + 4) and n1 - n0 <= 2 * (7 * (2 * 16 * 128 * 2 + 4) + 3 * 256)


def test_resident_and_dense_need_a_build(lib):
    p = make_params(1, 2, 64, "f32", 64, resident=16)
    h = _fake_handle(lib, p)
    try:
        assert lib.ice_set_resident(h, None, None, 0, 0, None) == L.ICE_ERR_STATE
        assert lib.ice_set_dense(h, None, None) == L.ICE_ERR_STATE
    finally:
        lib.ice_destroy(h)


def test_argument_checks_run_before_any_launch(lib):
    p = make_params(1, 2, 64, "f32", 64)
    h = _fake_handle(lib, p)
    try:
        fake = ctypes.c_void_p(1 << 20)
        ws_bytes = lib.ice_workspace_bytes(ctypes.byref(p), 64)
        # select / insert / attend before a build
        assert lib.ice_select(h, fake, 64, 4, fake, fake, fake, None, fake, ws_bytes, None) == L.ICE_ERR_STATE
        assert lib.ice_insert(h, fake, fake, 1, fake, ws_bytes, None) == L.ICE_ERR_STATE
        assert lib.ice_attend(h, fake, fake, fake, 8, 0.125, fake, None, fake, ws_bytes, None) == L.ICE_ERR_STATE
        # build: too many tokens, null inputs, small workspace, misaligned inputs
        assert lib.ice_build(h, fake, fake, 65, 65 * 64, fake, ws_bytes, None) == L.ICE_ERR_CAPACITY
        assert lib.ice_build(h, None, fake, 10, 640, fake, ws_bytes, None) == L.ICE_ERR_ARG
        assert lib.ice_build(h, fake, fake, 10, 640, fake, 16, None) == L.ICE_ERR_CAPACITY
        assert lib.ice_build(h, ctypes.c_void_p((1 << 20) + 4), fake, 10, 640, fake, ws_bytes, None) == L.ICE_ERR_ARG
        assert lib.ice_build(h, fake, fake, 10, 100, fake, ws_bytes, None) == L.ICE_ERR_ARG
        assert lib.ice_build(h, fake, fake, -1, 640, fake, ws_bytes, None) == L.ICE_ERR_ARG
        assert lib.ice_n_tokens(h) == 0
    finally:
        lib.ice_destroy(h)


def test_create_rejects_small_or_misaligned_blobs(lib):
    p = make_params(2, 2, 128, "bf16", 1000)
    n = lib.ice_index_bytes(ctypes.byref(p))
    h = ctypes.c_void_p()
    assert lib.ice_create(ctypes.byref(p), ctypes.c_void_p(1 << 20), n - 1, ctypes.byref(h)) == L.ICE_ERR_CAPACITY
    assert lib.ice_create(ctypes.byref(p), ctypes.c_void_p((1 << 20) + 64), n, ctypes.byref(h)) == L.ICE_ERR_ARG
    assert lib.ice_create(ctypes.byref(p), None, n, ctypes.byref(h)) == L.ICE_ERR_ARG


def test_host_pool_sizes_and_checks(lib):
    """Host-pool mode moves the level-0 V pages out of the device blob into a
    pinned host pool of exactly those bytes; the pool must be attached before a
    build, and only to an index created with the flag."""
    H, G, d, cap = 3, 4, 128, 5000
    dev = make_params(H, G, d, "bf16", cap)
    host = make_params(H, G, d, "bf16", cap, host_pool=True)
    assert lib.ice_host_pool_bytes(ctypes.byref(dev)) == 0
    pool = lib.ice_host_pool_bytes(ctypes.byref(host))
    hd = _fake_handle(lib, dev)
    try:
        pages0 = lib.ice_export_bytes(hd, L.ICE_EXP_PAGE_V, 0) // (16 * d * 2)
    finally:
        lib.ice_destroy(hd)
    per_head = -(-pages0 * 16 * d * 2 // 256) * 256
    assert pool == H * per_head
    # the blob shrinks by about the V pool; the workspace grows by the staging area
    shrink = lib.ice_index_bytes(ctypes.byref(dev)) - lib.ice_index_bytes(ctypes.byref(host))
    assert per_head * H <= shrink <= per_head * H + 256 * H
    grow = lib.ice_workspace_bytes(ctypes.byref(host), 256) - lib.ice_workspace_bytes(ctypes.byref(dev), 256)
    assert grow >= 0
    bad = make_params(H, G, d, "bf16", cap)
    bad.flags = 6
    assert lib.ice_index_bytes(ctypes.byref(bad)) == 0
    # attach: refused without the flag, with a small, misaligned or null pool
    hd = _fake_handle(lib, dev)
    try:
        assert lib.ice_attach_host_pool(hd, ctypes.c_void_p(1 << 20), pool) == L.ICE_ERR_STATE
    finally:
        lib.ice_destroy(hd)
    hh = _fake_handle(lib, host)
    try:
        fake = ctypes.c_void_p(1 << 20)
        ws_bytes = lib.ice_workspace_bytes(ctypes.byref(host), 256)
        assert lib.ice_attach_host_pool(hh, None, pool) == L.ICE_ERR_ARG
        assert lib.ice_attach_host_pool(hh, ctypes.c_void_p((1 << 20) + 64), pool) == L.ICE_ERR_ARG
        assert lib.ice_attach_host_pool(hh, fake, pool - 1) == L.ICE_ERR_CAPACITY
        # a build before the pool is attached
        assert lib.ice_build(hh, fake, fake, 10, 10 * d, fake, ws_bytes, None) == L.ICE_ERR_STATE
    finally:
        lib.ice_destroy(hh)


def test_reuse_can_outgrow_tables_sized_from_own_draws():
    """The sizing fact behind the reuse insert check: a head that takes its
    source's levels for its first 2048 tokens and its own draws after them
    can hold more level-1 points than any head's own draws over the whole
    capacity (the tables are sized from those). Seed 1, 2 heads, 2 levels,
    p = 1/16, capacity 4096: the reused head passes the 261-point bound at
    token 3992, which the GPU test of reuse inserts relies on."""
    cap, nb = 4096, 2048
    l0 = ic.draw_levels(1, 0, 0, cap, 2, 4)
    l1 = ic.draw_levels(1, 1, 0, cap, 2, 4)
    ncap = max(int((l0 >= 1).sum()), int((l1 >= 1).sum()))
    run = int((l0[:nb] >= 1).sum()) + np.cumsum(l1[nb:] >= 1)
    assert ncap == 261
    assert nb + int(np.nonzero(run > ncap)[0][0]) == 3992
