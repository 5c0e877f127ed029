"""fp64 CPU oracle for the RWKV-7 WKV7 forward, its backward and the Gated
DeltaNet forward and backward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP product path never imports it,
and it imports nothing from the product package.

The arithmetic lives in ``wkv7_oracle.c`` (plain sequential fp64, libm
``exp``, no fast-math); this module only builds it with gcc, loads it with
ctypes and converts numpy arrays to contiguous float64.  The recurrence and
the reading of the pages it follows are documented in the C file's header
(rwkv-ops README, section "rwkv7op 使用方法" and section
"rwkv7_op_rnn 使用方法").
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wkv7_oracle.c")
_LIB = os.path.join(_HERE, "libwkv7_oracle.so")
_lib = None


def build(force=True):
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    cmd = ["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC",
           "-std=c99", _SRC, "-o", _LIB + ".tmp", "-lm"]
    if force or not os.path.exists(_LIB):
        subprocess.check_call(cmd)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    d = ctypes.c_void_p
    i = ctypes.c_int
    lib.wkv7_oracle_fwd.argtypes = [i, i, i, i, i] + [d] * 10
    lib.wkv7_oracle_fwd.restype = i
    lib.wkv7_oracle_step.argtypes = [i, i, i, i] + [d] * 8
    lib.wkv7_oracle_step.restype = i
    lib.wkv7_oracle_bwd.argtypes = [i, i, i, i, i] + [d] * 17
    lib.wkv7_oracle_bwd.restype = i
    lib.gdn_oracle_fwd.argtypes = [i, i, i, i, i] + [d] * 6 + [i, d, d]
    lib.gdn_oracle_fwd.restype = i
    lib.gdn_oracle_bwd.argtypes = [i, i, i, i, i] + [d] * 6 + [i] + [d] * 8
    lib.gdn_oracle_bwd.restype = i
    lib.wkv7_oracle_max_threads.restype = i
    lib.wkv7_oracle_set_threads.argtypes = [i]
    _lib = lib
    return lib


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def fwd(r, w, k, v, a, b, initial_state=None, mask=None):
    """WKV7 forward.  r,w,k,a,b: [B,T,H,K]; v: [B,T,H,V];
    initial_state: [B,H,K,V] or None (zeros); mask: [B,T] (nonzero updates)
    or None.  Returns (o [B,T,H,V], final_state [B,H,K,V]) in float64."""
    lib = _load()
    r, w, k, v, a, b = (_f64(x) for x in (r, w, k, v, a, b))
    B, T, H, K = r.shape
    V = v.shape[-1]
    for x in (w, k, a, b):
        assert x.shape == (B, T, H, K)
    assert v.shape == (B, T, H, V)
    s0 = None if initial_state is None else _f64(initial_state)
    if s0 is not None:
        assert s0.shape == (B, H, K, V)
    m = None
    if mask is not None:
        m = np.ascontiguousarray((np.asarray(mask) != 0).astype(np.uint8))
        assert m.shape == (B, T)
    o = np.zeros((B, T, H, V), np.float64)
    sf = np.zeros((B, H, K, V), np.float64)
    rc = lib.wkv7_oracle_fwd(B, T, H, K, V, _ptr(r), _ptr(w), _ptr(k), _ptr(v),
                             _ptr(a), _ptr(b), _ptr(s0), _ptr(m), _ptr(o), _ptr(sf))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return o, sf


def bwd(r, w, k, v, a, b, d_o, initial_state=None, mask=None, d_final_state=None):
    """Backward of fwd (reverse-mode derivative of the same recurrence; see
    the C file).  d_o: [B,T,H,V] gradient of the output; d_final_state:
    [B,H,K,V] or None (zero).  Returns a dict of float64 gradients r, w, k, v,
    a, b (input shapes) and s0 ([B,H,K,V])."""
    lib = _load()
    r, w, k, v, a, b, d_o = (_f64(x) for x in (r, w, k, v, a, b, d_o))
    B, T, H, K = r.shape
    V = v.shape[-1]
    for x in (w, k, a, b):
        assert x.shape == (B, T, H, K)
    assert v.shape == (B, T, H, V) and d_o.shape == (B, T, H, V)
    s0 = None if initial_state is None else _f64(initial_state)
    if s0 is not None:
        assert s0.shape == (B, H, K, V)
    dsf = None if d_final_state is None else _f64(d_final_state)
    if dsf is not None:
        assert dsf.shape == (B, H, K, V)
    m = None
    if mask is not None:
        m = np.ascontiguousarray((np.asarray(mask) != 0).astype(np.uint8))
        assert m.shape == (B, T)
    g = {n: np.zeros((B, T, H, K), np.float64) for n in ("r", "w", "k", "a", "b")}
    g["v"] = np.zeros((B, T, H, V), np.float64)
    g["s0"] = np.zeros((B, H, K, V), np.float64)
    rc = lib.wkv7_oracle_bwd(B, T, H, K, V, _ptr(r), _ptr(w), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                             _ptr(s0), _ptr(m), _ptr(d_o), _ptr(dsf),
                             *(_ptr(g[n]) for n in ("r", "w", "k", "v", "a", "b", "s0")))
    if rc != 0:
        raise ValueError("oracle rejected the arguments" if rc == -1 else "oracle ran out of memory")
    return g


def step(r, w, k, v, a, b, state):
    """One decode token.  r,w,k,a,b: [B,H,K]; v: [B,H,V]; state: [B,H,K,V].
    Returns (o [B,H,V], new_state) in float64; the input array is not
    modified."""
    lib = _load()
    r, w, k, v, a, b = (_f64(x) for x in (r, w, k, v, a, b))
    B, H, K = r.shape
    V = v.shape[-1]
    st = _f64(state).copy()
    assert st.shape == (B, H, K, V)
    o = np.zeros((B, H, V), np.float64)
    rc = lib.wkv7_oracle_step(B, H, K, V, _ptr(r), _ptr(w), _ptr(k), _ptr(v),
                              _ptr(a), _ptr(b), _ptr(st), _ptr(o))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return o, st


def gdn_fwd(q, k, v, g, beta, initial_state=None):
    """Gated DeltaNet forward (textbook gated delta rule; see the C file).
    q, k: [B,T,H,K]; v: [B,T,H,V]; g, beta: [B,T,H]; initial_state:
    [B,H,K,V], [1,H,K,V] (shared) or None.  Returns (o, final_state) in
    float64."""
    lib = _load()
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    B, T, H, K = q.shape
    V = v.shape[-1]
    assert k.shape == (B, T, H, K) and v.shape == (B, T, H, V)
    assert g.shape == (B, T, H) and beta.shape == (B, T, H)
    s0 = None if initial_state is None else _f64(initial_state)
    n_s0 = 0
    if s0 is not None:
        n_s0 = s0.shape[0]
        assert s0.shape == (n_s0, H, K, V) and n_s0 in (1, B)
    o = np.zeros((B, T, H, V), np.float64)
    sf = np.zeros((B, H, K, V), np.float64)
    rc = lib.gdn_oracle_fwd(B, T, H, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                            _ptr(s0), n_s0, _ptr(o), _ptr(sf))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return o, sf


def gdn_bwd(q, k, v, g, beta, d_o, initial_state=None, d_final_state=None):
    """Backward of gdn_fwd (reverse-mode derivative of the gated delta rule
    with the L2 normalisation of q and k; see the C file).  d_o: [B,T,H,V];
    d_final_state: [B,H,K,V] or None (zero).  Returns a dict of float64
    gradients q, k, v, g, beta (input shapes) and s0 ([n,H,K,V] with n the
    initial state's leading size, B when there is none)."""
    lib = _load()
    q, k, v, g, beta, d_o = (_f64(x) for x in (q, k, v, g, beta, d_o))
    B, T, H, K = q.shape
    V = v.shape[-1]
    assert k.shape == (B, T, H, K) and v.shape == (B, T, H, V) and d_o.shape == (B, T, H, V)
    assert g.shape == (B, T, H) and beta.shape == (B, T, H)
    s0 = None if initial_state is None else _f64(initial_state)
    n_s0 = B
    if s0 is not None:
        n_s0 = s0.shape[0]
        assert s0.shape == (n_s0, H, K, V) and n_s0 in (1, B)
    dsf = None if d_final_state is None else _f64(d_final_state)
    if dsf is not None:
        assert dsf.shape == (B, H, K, V)
    out = {"q": np.zeros((B, T, H, K)), "k": np.zeros((B, T, H, K)), "v": np.zeros((B, T, H, V)),
           "g": np.zeros((B, T, H)), "beta": np.zeros((B, T, H)), "s0": np.zeros((n_s0, H, K, V))}
    rc = lib.gdn_oracle_bwd(B, T, H, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                            _ptr(s0), n_s0 if s0 is not None else 0, _ptr(d_o), _ptr(dsf),
                            *(_ptr(out[n]) for n in ("q", "k", "v", "g", "beta", "s0")))
    if rc != 0:
        raise ValueError("oracle rejected the arguments" if rc == -1 else "oracle ran out of memory")
    return out


def max_threads():
    return _load().wkv7_oracle_max_threads()


def set_threads(n):
    _load().wkv7_oracle_set_threads(int(n))
