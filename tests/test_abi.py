"""C-ABI checks that need no GPU: the library loads, exports every function
include/wkv7.h declares, and rejects bad arguments on the host before any
HIP call (contract stated in include/wkv7.h)."""
import ctypes
import os
import re

import pytest

from rwkv_linear_attention_amd import build, wkv7

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wkv7.h")


@pytest.fixture(scope="module")
def L():
    build.build(force=False)
    return wkv7.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(wkv7_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert {"wkv7_fwd", "wkv7_fwd_varlen", "wkv7_gdn_fwd", "wkv7_bwd", "wkv7_bwd_workspace_bytes", "wkv7_gdn_step", "wkv7_gdn_fwd_varlen", "wkv7_gdn_bwd", "wkv7_gdn_bwd_workspace_bytes", "wkv7_bwd_varlen", "wkv7_bwd_varlen_workspace_bytes", "wkv7_gdn_bwd_varlen", "wkv7_gdn_bwd_varlen_workspace_bytes", "wkv7_step", "wkv7_strerror", "wkv7_fwd_path",
            "wkv7_version", "wkv7_set_wait_limit"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"{n} declared in wkv7.h but not exported"


def test_version_and_strerror(L):
    assert L.wkv7_version() == 201
    for code in range(5):
        assert len(L.wkv7_strerror(code)) > 0
    assert L.wkv7_strerror(99) == b"unknown status"


P = ctypes.c_void_p
GOOD = P(0x100000)       # 16-byte aligned stand-in; never dereferenced on the error paths
ODD = P(0x100002)


def fwd(L, dtype=1, B=1, T=4, H=1, K=64, V=64, ptrs=None, s0=None, n_state=None, mask=None, sf=None, algo=0):
    ptrs = ptrs or [GOOD] * 7
    r, w, k, v, a, b, o = ptrs
    if n_state is None:
        n_state = B if s0 is not None else 0
    return L.wkv7_fwd(dtype, B, T, H, K, V, r, w, k, v, a, b, s0, n_state, mask, o, sf, algo, None)


def step(L, dtype=1, B=1, H=1, K=64, V=64, ptrs=None):
    ptrs = ptrs or [GOOD] * 8
    return L.wkv7_step(dtype, B, H, K, V, *ptrs, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), wkv7.ERR_INVALID_ARG),
    (dict(dtype=-1), wkv7.ERR_INVALID_ARG),
    (dict(B=0), wkv7.ERR_INVALID_ARG),
    (dict(H=-3), wkv7.ERR_INVALID_ARG),
    (dict(T=-1), wkv7.ERR_INVALID_ARG),
    (dict(K=0), wkv7.ERR_INVALID_ARG),
    (dict(K=64, V=128), wkv7.ERR_UNSUPPORTED),
    (dict(K=32, V=32), wkv7.ERR_UNSUPPORTED),
    (dict(K=256, V=256), wkv7.ERR_UNSUPPORTED),
    (dict(algo=7), wkv7.ERR_INVALID_ARG),
])
def test_fwd_rejects(L, kw, code):
    assert fwd(L, **kw) == code


@pytest.mark.parametrize("slot", range(7))
def test_fwd_rejects_null_and_misaligned(L, slot):
    ptrs = [GOOD] * 7
    ptrs[slot] = None
    assert fwd(L, ptrs=ptrs) == wkv7.ERR_INVALID_ARG
    ptrs[slot] = ODD
    assert fwd(L, ptrs=ptrs) == wkv7.ERR_INVALID_ARG


def test_fwd_rejects_misaligned_states(L):
    assert fwd(L, s0=ODD) == wkv7.ERR_INVALID_ARG
    assert fwd(L, sf=ODD) == wkv7.ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [
    dict(B=2, s0=GOOD, n_state=0),             # state rows must be 1 or B
    dict(B=2, s0=GOOD, n_state=3),
    dict(B=2, s0=GOOD, n_state=1, sf=GOOD),    # a shared state overwritten by the finals
])
def test_fwd_state_rows(L, kw):
    assert fwd(L, **kw) == wkv7.ERR_INVALID_ARG


def test_wait_limit_hook(L):
    prev = L.wkv7_set_wait_limit(5)
    try:
        assert L.wkv7_set_wait_limit(0) == 5
        assert L.wkv7_set_wait_limit(-1) == 0       # negative: back to the default
        assert L.wkv7_set_wait_limit(-1) == 1 << 20
    finally:
        L.wkv7_set_wait_limit(prev)


@pytest.mark.parametrize("slot", range(8))
def test_step_rejects_null_and_misaligned(L, slot):
    ptrs = [GOOD] * 8
    ptrs[slot] = None
    assert step(L, ptrs=ptrs) == wkv7.ERR_INVALID_ARG
    ptrs[slot] = ODD
    assert step(L, ptrs=ptrs) == wkv7.ERR_INVALID_ARG


def test_step_rejects_sizes(L):
    assert step(L, B=1 << 15, H=1 << 14, K=128, V=128) == wkv7.ERR_UNSUPPORTED   # 4 B H waves exceed an int
    assert gdn_step(L, B=1 << 15, H=1 << 14, K=128, V=128) == wkv7.ERR_UNSUPPORTED
    assert step(L, B=0) == wkv7.ERR_INVALID_ARG
    assert step(L, K=64, V=32) == wkv7.ERR_UNSUPPORTED
    assert step(L, dtype=5) == wkv7.ERR_INVALID_ARG


def test_path_choice(L):
    R, C = wkv7.ALGO_RECURRENT, wkv7.ALGO_CHUNKED
    assert L.wkv7_fwd_path(1, 8, 4096, 64, 64, 64, 0) == C
    assert L.wkv7_fwd_path(1, 16, 4096, 32, 128, 128, 0) == C
    assert L.wkv7_fwd_path(0, 1, 15, 1, 64, 64, 0) == R          # fp32: short sequences
    assert L.wkv7_fwd_path(0, 1, 16, 1, 128, 128, 0) == C        # fp32 chunked from T = 16 (measured)
    assert L.wkv7_fwd_path(0, 8, 4096, 64, 64, 64, 0) == C
    assert L.wkv7_fwd_path(0, 1, 8, 1, 128, 128, 2) == C         # forced
    assert L.wkv7_fwd_path(1, 1, 8, 1, 64, 64, 0) == R           # very short sequences
    assert L.wkv7_fwd_path(1, 1, 15, 1, 128, 128, 0) == R
    assert L.wkv7_fwd_path(1, 1, 16, 1, 64, 64, 0) == C          # measured crossover
    assert L.wkv7_fwd_path(1, 1, 8, 1, 64, 64, 2) == C           # forced
    assert L.wkv7_fwd_path(1, 1, 4096, 1, 64, 64, 1) == R        # forced
    assert L.wkv7_fwd_path(1, 1, 4096, 1, 48, 48, 0) == -1


def varlen(L, dtype=1, N=2, TT=40, H=1, K=64, V=64, cu=GOOD, ptrs=None, s0=None, n_state=0, smap=None,
           mask=None, sf=None, algo=0):
    ptrs = ptrs or [GOOD] * 7
    r, w, k, v, a, b, o = ptrs
    return L.wkv7_fwd_varlen(dtype, N, TT, H, K, V, cu, r, w, k, v, a, b, s0, n_state, smap, mask, o, sf,
                             algo, None)


@pytest.mark.parametrize("kw,code", [
    (dict(N=0), wkv7.ERR_INVALID_ARG),
    (dict(TT=-1), wkv7.ERR_INVALID_ARG),
    (dict(cu=None), wkv7.ERR_INVALID_ARG),
    (dict(cu=P(0x100002)), wkv7.ERR_INVALID_ARG),                  # cu_seqlens not 4-byte aligned
    (dict(smap=P(0x100001)), wkv7.ERR_INVALID_ARG),                # state_map not 4-byte aligned
    (dict(s0=GOOD, n_state=0), wkv7.ERR_INVALID_ARG),              # pool without rows
    (dict(s0=GOOD, n_state=3), wkv7.ERR_INVALID_ARG),              # no map: pool must have N or 1 rows
    (dict(s0=GOOD, n_state=1, smap=GOOD, sf=GOOD), wkv7.ERR_INVALID_ARG),   # mapped pool aliased by output
    (dict(s0=GOOD, n_state=1, sf=GOOD), wkv7.ERR_INVALID_ARG),     # shared row aliased by output
    (dict(s0=ODD, n_state=2), wkv7.ERR_INVALID_ARG),
    (dict(ptrs=[GOOD] * 6 + [None]), wkv7.ERR_INVALID_ARG),
    (dict(K=64, V=128), wkv7.ERR_UNSUPPORTED),
    (dict(algo=7), wkv7.ERR_INVALID_ARG),
])
def test_varlen_validation(L, kw, code):
    assert varlen(L, **kw) == code


def test_varlen_accepts_empty_token_axis_without_launch_checks(L):
    # total_T == 0 needs no token buffers; the call would launch (so only the
    # argument checks are exercised here: a NULL token pointer is not an error)
    assert varlen(L, TT=0, ptrs=[None] * 7, cu=None) == wkv7.ERR_INVALID_ARG   # cu_seqlens still required


def gdn(L, dtype=1, B=2, T=4, H=1, K=64, V=64, ptrs=None, s0=None, n_state=0, sf=None, algo=0):
    ptrs = ptrs or [GOOD] * 6
    q, k, v, g, beta, o = ptrs
    return L.wkv7_gdn_fwd(dtype, B, T, H, K, V, q, k, v, g, beta, s0, n_state, o, sf, algo, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), wkv7.ERR_INVALID_ARG),
    (dict(T=-1), wkv7.ERR_INVALID_ARG),
    (dict(dtype=3), wkv7.ERR_INVALID_ARG),
    (dict(K=64, V=128), wkv7.ERR_UNSUPPORTED),
    (dict(dtype=0, algo=2), wkv7.ERR_UNSUPPORTED),
    (dict(algo=9), wkv7.ERR_INVALID_ARG),
    (dict(s0=GOOD, n_state=0), wkv7.ERR_INVALID_ARG),            # state rows must be 1 or B
    (dict(s0=GOOD, n_state=3), wkv7.ERR_INVALID_ARG),
    (dict(s0=GOOD, n_state=1, sf=GOOD), wkv7.ERR_INVALID_ARG),   # shared state overwritten by finals
    (dict(s0=ODD, n_state=2), wkv7.ERR_INVALID_ARG),
    (dict(sf=ODD), wkv7.ERR_INVALID_ARG),
])
def test_gdn_validation(L, kw, code):
    assert gdn(L, **kw) == code


@pytest.mark.parametrize("slot", range(6))
def test_gdn_rejects_null_and_misaligned(L, slot):
    ptrs = [GOOD] * 6
    ptrs[slot] = None
    assert gdn(L, ptrs=ptrs) == wkv7.ERR_INVALID_ARG
    ptrs[slot] = ODD
    assert gdn(L, ptrs=ptrs) == wkv7.ERR_INVALID_ARG


def bwd(L, dtype=1, B=1, T=20, H=1, K=64, V=64, ptrs=None, s0=None, n_state=None, mask=None, dsf=None,
        ds0=None, ws=GOOD, ws_bytes=None):
    ptrs = ptrs or [GOOD] * 13
    if ws_bytes is None:
        ws_bytes = L.wkv7_bwd_workspace_bytes(B, T, H, K, V)
    if n_state is None:
        n_state = B if s0 is not None else 0
    r, w, k, v, a, b, do, dr, dw, dk, dv, da, db = ptrs
    return L.wkv7_bwd(dtype, B, T, H, K, V, r, w, k, v, a, b, s0, n_state, mask, do, dsf,
                      dr, dw, dk, dv, da, db, ds0, ws, ws_bytes, None)


def test_bwd_workspace_size(L):
    # two fp32 states per 16-token chunk and sequence (rounded up to 256
    # bytes), then one state per sequence for a shared state's gradient
    assert L.wkv7_bwd_workspace_bytes(2, 33, 3, 64, 64) == 4 * 2 * 3 * 64 * 64 * 2 * 3 + 4 * 2 * 3 * 64 * 64
    assert L.wkv7_bwd_workspace_bytes(1, 16, 1, 128, 128) == 4 * 128 * 128 * 3
    assert L.wkv7_bwd_workspace_bytes(1, 16, 1, 64, 32) == 0
    assert L.wkv7_bwd_workspace_bytes(0, 16, 1, 64, 64) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), wkv7.ERR_INVALID_ARG),
    (dict(B=0), wkv7.ERR_INVALID_ARG),
    (dict(T=-1), wkv7.ERR_INVALID_ARG),
    (dict(K=64, V=128), wkv7.ERR_UNSUPPORTED),
    (dict(ws=None), wkv7.ERR_INVALID_ARG),
    (dict(ws=ODD), wkv7.ERR_INVALID_ARG),
    (dict(ws_bytes=1024), wkv7.ERR_INVALID_ARG),              # workspace too small
    (dict(s0=ODD), wkv7.ERR_INVALID_ARG),
    (dict(dsf=ODD), wkv7.ERR_INVALID_ARG),
    (dict(ds0=ODD), wkv7.ERR_INVALID_ARG),
    (dict(B=2, s0=GOOD, n_state=3), wkv7.ERR_INVALID_ARG),         # state rows must be 1 or B
    (dict(B=2, s0=GOOD, n_state=0), wkv7.ERR_INVALID_ARG),
    (dict(B=1 << 16, H=1 << 14, T=16), wkv7.ERR_UNSUPPORTED),      # 2 B H workgroups exceed the grid
    (dict(H=1 << 19, T=16), wkv7.ERR_UNSUPPORTED),                 # a chunk's H K D fp32 offsets reach 2^31
    (dict(H=1 << 18, K=128, V=128, T=16), wkv7.ERR_UNSUPPORTED),
])
def test_bwd_validation(L, kw, code):
    assert bwd(L, **kw) == code


@pytest.mark.parametrize("slot", range(13))
def test_bwd_rejects_null_and_misaligned(L, slot):
    ptrs = [GOOD] * 13
    ptrs[slot] = None
    assert bwd(L, ptrs=ptrs) == wkv7.ERR_INVALID_ARG
    ptrs[slot] = ODD
    assert bwd(L, ptrs=ptrs) == wkv7.ERR_INVALID_ARG


def gdn_bwd(L, dtype=1, B=2, T=20, H=1, K=64, V=64, ptrs=None, s0=None, n_state=0, dsf=None, ds0=None,
            ws=GOOD, ws_bytes=None):
    ptrs = ptrs or [GOOD] * 11
    if ws_bytes is None:
        ws_bytes = L.wkv7_gdn_bwd_workspace_bytes(B, T, H, K, V)
    q, k, v, g, beta, do, dq, dk, dv, dg, dbeta = ptrs
    return L.wkv7_gdn_bwd(dtype, B, T, H, K, V, q, k, v, g, beta, s0, n_state, do, dsf,
                          dq, dk, dv, dg, dbeta, ds0, ws, ws_bytes, None)


def test_gdn_bwd_workspace_size(L):
    # two state sets (a shared initial state expanded, and its per-sequence
    # gradients), then the WKV7 backward's workspace
    B, T, H, D = 2, 33, 3, 64
    states = -(-B * H * D * D * 4 // 256) * 256
    assert L.wkv7_gdn_bwd_workspace_bytes(B, T, H, D, D) == 2 * states + L.wkv7_bwd_workspace_bytes(B, T, H, D, D)
    assert L.wkv7_gdn_bwd_workspace_bytes(1, 16, 1, 64, 32) == 0
    assert L.wkv7_gdn_bwd_workspace_bytes(1, -1, 1, 64, 64) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), wkv7.ERR_INVALID_ARG),
    (dict(B=0), wkv7.ERR_INVALID_ARG),
    (dict(T=-1), wkv7.ERR_INVALID_ARG),
    (dict(K=128, V=64), wkv7.ERR_UNSUPPORTED),
    (dict(K=96, V=96), wkv7.ERR_UNSUPPORTED),
    (dict(ws=None), wkv7.ERR_INVALID_ARG),
    (dict(ws=ODD), wkv7.ERR_INVALID_ARG),
    (dict(ws_bytes=1024), wkv7.ERR_INVALID_ARG),              # workspace too small
    (dict(s0=GOOD, n_state=3), wkv7.ERR_INVALID_ARG),         # neither 1 nor B rows
    (dict(s0=GOOD, n_state=0), wkv7.ERR_INVALID_ARG),
    (dict(s0=ODD, n_state=2), wkv7.ERR_INVALID_ARG),
    (dict(dsf=ODD), wkv7.ERR_INVALID_ARG),
    (dict(ds0=ODD), wkv7.ERR_INVALID_ARG),
    (dict(B=1 << 16, H=1 << 14, T=16), wkv7.ERR_UNSUPPORTED),     # 2 B H workgroups exceed the grid
    (dict(B=1, H=1 << 19, T=16), wkv7.ERR_UNSUPPORTED),           # a chunk's H K D fp32 offsets reach 2^31
])
def test_gdn_bwd_validation(L, kw, code):
    assert gdn_bwd(L, **kw) == code


@pytest.mark.parametrize("slot", range(11))
def test_gdn_bwd_rejects_null_and_misaligned(L, slot):
    ptrs = [GOOD] * 11
    ptrs[slot] = None
    assert gdn_bwd(L, ptrs=ptrs) == wkv7.ERR_INVALID_ARG
    ptrs[slot] = ODD
    assert gdn_bwd(L, ptrs=ptrs) == wkv7.ERR_INVALID_ARG


def bwd_varlen(L, dtype=1, N=3, TT=50, H=1, K=64, V=64, cu=GOOD, ptrs=None, s0=None, n_state=0, smap=None,
               mask=None, dsf=None, ds0=None, ws=GOOD, ws_bytes=None):
    ptrs = ptrs or [GOOD] * 13
    if ws_bytes is None:
        ws_bytes = L.wkv7_bwd_varlen_workspace_bytes(N, TT, H, K, V)
    r, w, k, v, a, b, do, dr, dw, dk, dv, da, db = ptrs
    return L.wkv7_bwd_varlen(dtype, N, TT, H, K, V, cu, r, w, k, v, a, b, s0, n_state, smap, mask, do, dsf,
                             dr, dw, dk, dv, da, db, ds0, ws, ws_bytes, None)


def test_bwd_varlen_workspace_size(L):
    # two fp32 states per head for ceil(total_T / 16) + N chunks, then N + 1 offsets
    assert L.wkv7_bwd_varlen_workspace_bytes(3, 100, 2, 64, 64) == 4 * (7 + 3) * 2 * 64 * 64 * 2 + 4 * 4
    assert L.wkv7_bwd_varlen_workspace_bytes(1, 0, 1, 128, 128) == 4 * 1 * 128 * 128 * 2 + 8
    assert L.wkv7_bwd_varlen_workspace_bytes(1, 16, 1, 64, 32) == 0
    assert L.wkv7_bwd_varlen_workspace_bytes(0, 16, 1, 64, 64) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), wkv7.ERR_INVALID_ARG),
    (dict(N=0), wkv7.ERR_INVALID_ARG),
    (dict(TT=-1), wkv7.ERR_INVALID_ARG),
    (dict(K=64, V=128), wkv7.ERR_UNSUPPORTED),
    (dict(cu=None), wkv7.ERR_INVALID_ARG),
    (dict(cu=P(0x100002)), wkv7.ERR_INVALID_ARG),            # cu_seqlens not 4-byte aligned
    (dict(ws=None), wkv7.ERR_INVALID_ARG),
    (dict(ws_bytes=1024), wkv7.ERR_INVALID_ARG),              # workspace too small
    (dict(s0=GOOD, n_state=0), wkv7.ERR_INVALID_ARG),
    (dict(s0=GOOD, n_state=2), wkv7.ERR_INVALID_ARG),         # no map: N rows or one shared row
    (dict(s0=ODD, n_state=3), wkv7.ERR_INVALID_ARG),
    (dict(smap=P(0x100002)), wkv7.ERR_INVALID_ARG),
    (dict(dsf=ODD), wkv7.ERR_INVALID_ARG),
    (dict(ds0=ODD), wkv7.ERR_INVALID_ARG),
    (dict(N=1 << 16, H=1 << 14, TT=16), wkv7.ERR_UNSUPPORTED),    # 2 N H workgroups exceed the grid
    (dict(N=1, H=1 << 19, TT=16), wkv7.ERR_UNSUPPORTED),          # a chunk's H K D fp32 offsets reach 2^31
])
def test_bwd_varlen_validation(L, kw, code):
    assert bwd_varlen(L, **kw) == code


@pytest.mark.parametrize("slot", range(13))
def test_bwd_varlen_rejects_null_and_misaligned(L, slot):
    ptrs = [GOOD] * 13
    ptrs[slot] = None
    assert bwd_varlen(L, ptrs=ptrs) == wkv7.ERR_INVALID_ARG
    ptrs[slot] = ODD
    assert bwd_varlen(L, ptrs=ptrs) == wkv7.ERR_INVALID_ARG


def gdn_bwd_varlen(L, dtype=1, N=3, TT=50, H=1, K=64, V=64, cu=GOOD, ptrs=None, s0=None, n_state=0, smap=None,
                   dsf=None, ds0=None, ws=GOOD, ws_bytes=None):
    ptrs = ptrs or [GOOD] * 11
    if ws_bytes is None:
        ws_bytes = L.wkv7_gdn_bwd_varlen_workspace_bytes(N, TT, H, K, V)
    q, k, v, g, beta, do, dq, dk, dv, dg, dbeta = ptrs
    return L.wkv7_gdn_bwd_varlen(dtype, N, TT, H, K, V, cu, q, k, v, g, beta, s0, n_state, smap, do, dsf,
                                 dq, dk, dv, dg, dbeta, ds0, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), wkv7.ERR_INVALID_ARG),
    (dict(N=0), wkv7.ERR_INVALID_ARG),
    (dict(K=64, V=128), wkv7.ERR_UNSUPPORTED),
    (dict(cu=None), wkv7.ERR_INVALID_ARG),
    (dict(ws_bytes=1024), wkv7.ERR_INVALID_ARG),
    (dict(s0=GOOD, n_state=2), wkv7.ERR_INVALID_ARG),         # no map: N rows or one shared row
    (dict(N=1, H=1 << 19, TT=16), wkv7.ERR_UNSUPPORTED),      # a chunk's H K D fp32 offsets reach 2^31
])
def test_gdn_bwd_varlen_validation(L, kw, code):
    assert gdn_bwd_varlen(L, **kw) == code


def test_gdn_bwd_varlen_accepts_shared_row_without_launch(L):
    # total_T = 0 and no gradient to write: validation only, no HIP call
    assert gdn_bwd_varlen(L, TT=0, ws=None, ws_bytes=0, s0=GOOD, n_state=1) == wkv7.OK


@pytest.mark.parametrize("slot", range(11))
def test_gdn_bwd_varlen_rejects_null_and_misaligned(L, slot):
    ptrs = [GOOD] * 11
    ptrs[slot] = None
    assert gdn_bwd_varlen(L, ptrs=ptrs) == wkv7.ERR_INVALID_ARG
    ptrs[slot] = ODD
    assert gdn_bwd_varlen(L, ptrs=ptrs) == wkv7.ERR_INVALID_ARG


def gdn_step(L, dtype=1, B=2, H=1, K=64, V=64, ptrs=None, s_in=None, n_state=0, s_out=GOOD):
    ptrs = ptrs or [GOOD] * 6
    q, k, v, g, beta, o = ptrs
    return L.wkv7_gdn_step(dtype, B, H, K, V, q, k, v, g, beta, s_in, n_state, s_out, o, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), wkv7.ERR_INVALID_ARG),
    (dict(dtype=4), wkv7.ERR_INVALID_ARG),
    (dict(K=64, V=32), wkv7.ERR_UNSUPPORTED),
    (dict(s_out=None), wkv7.ERR_INVALID_ARG),
    (dict(s_out=ODD), wkv7.ERR_INVALID_ARG),
    (dict(s_in=ODD, n_state=2), wkv7.ERR_INVALID_ARG),
    (dict(s_in=GOOD, n_state=3), wkv7.ERR_INVALID_ARG),
    (dict(s_in=GOOD, n_state=1), wkv7.ERR_INVALID_ARG),     # shared state overwritten in place
])
def test_gdn_step_validation(L, kw, code):
    assert gdn_step(L, **kw) == code


@pytest.mark.parametrize("slot", range(6))
def test_gdn_step_rejects_null_and_misaligned(L, slot):
    ptrs = [GOOD] * 6
    ptrs[slot] = None
    assert gdn_step(L, ptrs=ptrs) == wkv7.ERR_INVALID_ARG
    ptrs[slot] = ODD
    assert gdn_step(L, ptrs=ptrs) == wkv7.ERR_INVALID_ARG


def gdn_varlen(L, dtype=1, N=2, TT=40, H=1, K=64, V=64, cu=GOOD, ptrs=None, s0=None, n_state=0, smap=None,
               sf=None, algo=0):
    ptrs = ptrs or [GOOD] * 6
    q, k, v, g, beta, o = ptrs
    return L.wkv7_gdn_fwd_varlen(dtype, N, TT, H, K, V, cu, q, k, v, g, beta, s0, n_state, smap, o, sf, algo,
                                 None)


@pytest.mark.parametrize("kw,code", [
    (dict(N=0), wkv7.ERR_INVALID_ARG),
    (dict(cu=None), wkv7.ERR_INVALID_ARG),
    (dict(cu=P(0x100002)), wkv7.ERR_INVALID_ARG),
    (dict(smap=P(0x100001)), wkv7.ERR_INVALID_ARG),
    (dict(s0=GOOD, n_state=0), wkv7.ERR_INVALID_ARG),
    (dict(s0=GOOD, n_state=3), wkv7.ERR_INVALID_ARG),             # no map: N rows or one shared row
    (dict(s0=GOOD, n_state=1, sf=GOOD), wkv7.ERR_INVALID_ARG),    # shared row overwritten
    (dict(s0=GOOD, n_state=4, smap=GOOD, sf=GOOD), wkv7.ERR_INVALID_ARG),   # mapped pool overwritten
    (dict(ptrs=[GOOD] * 5 + [None]), wkv7.ERR_INVALID_ARG),
    (dict(K=64, V=128), wkv7.ERR_UNSUPPORTED),
    (dict(dtype=0, algo=2), wkv7.ERR_UNSUPPORTED),
])
def test_gdn_varlen_validation(L, kw, code):
    assert gdn_varlen(L, **kw) == code


def bwd_noalloc(L, dtype=1, B=1, T=20, H=1, K=64, V=64, ptrs=None, s0=None, n_state=None, mask=None, dsf=None,
                ds0=None):
    ptrs = ptrs or [GOOD] * 13
    if n_state is None:
        n_state = B if s0 is not None else 0
    r, w, k, v, a, b, do, dr, dw, dk, dv, da, db = ptrs
    return L.wkv7_bwd_noalloc(dtype, B, T, H, K, V, r, w, k, v, a, b, s0, n_state, mask, do, dsf,
                              dr, dw, dk, dv, da, db, ds0, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), wkv7.ERR_INVALID_ARG),
    (dict(B=0), wkv7.ERR_INVALID_ARG),
    (dict(T=-1), wkv7.ERR_INVALID_ARG),
    (dict(K=64, V=128), wkv7.ERR_UNSUPPORTED),
    (dict(B=2, s0=GOOD, n_state=3), wkv7.ERR_INVALID_ARG),
    (dict(ds0=ODD), wkv7.ERR_INVALID_ARG),
    # the scratch holds B H (2 ceil(T/16) + 1) fp32 states: 4096 at d64, 1024 at d128
    (dict(B=1, H=8, T=4096), wkv7.ERR_TOO_LARGE),
    (dict(B=1, H=1, T=8192, K=128, V=128), wkv7.ERR_TOO_LARGE),
    (dict(B=64, H=64, T=16), wkv7.ERR_TOO_LARGE),
])
def test_bwd_noalloc_rejects_on_the_host(L, kw, code):
    assert bwd_noalloc(L, **kw) == code


@pytest.mark.parametrize("slot", range(13))
def test_bwd_noalloc_rejects_null_and_misaligned(L, slot):
    ptrs = [GOOD] * 13
    ptrs[slot] = None
    assert bwd_noalloc(L, ptrs=ptrs) == wkv7.ERR_INVALID_ARG
    ptrs[slot] = ODD
    assert bwd_noalloc(L, ptrs=ptrs) == wkv7.ERR_INVALID_ARG


def test_bwd_noalloc_bound_matches_workspace_size(L):
    """The largest accepted sizes are those whose wkv7_bwd workspace fits the
    fixed scratch: one more chunk or head does not."""
    limit = wkv7.NOALLOC_SCRATCH_BYTES
    assert L.wkv7_bwd_workspace_bytes(1, 4080, 8, 64, 64) <= limit < L.wkv7_bwd_workspace_bytes(1, 4096, 8, 64, 64)
    assert L.wkv7_bwd_workspace_bytes(1, 8176, 1, 128, 128) <= limit < L.wkv7_bwd_workspace_bytes(1, 8192, 1, 128, 128)
