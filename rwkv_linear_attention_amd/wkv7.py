"""ctypes binding of libwkv7.so (C ABI declared in include/wkv7.h).

Argument marshalling only: shapes and dtypes are checked, torch allocates the
outputs, and the library enqueues its kernels on torch's current stream.
Nothing here computes any part of the operator; if the library is missing the
call raises instead of falling back.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwkv7.so")

F32, BF16 = 0, 1
ALGO_AUTO, ALGO_RECURRENT, ALGO_CHUNKED = 0, 1, 2
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_TOO_LARGE = 0, 1, 2, 3, 4
NOALLOC_SCRATCH_BYTES = 64 << 20   # WKV7_NOALLOC_SCRATCH_BYTES

_lib = None


def lib():
    """Load libwkv7.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing; build it with __graft_entry__.build() "
                           "or python -m rwkv_linear_attention_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    p, i = ctypes.c_void_p, ctypes.c_int
    L.wkv7_fwd.argtypes = [i, i, i, i, i, i] + [p] * 7 + [i] + [p] * 3 + [i, p]
    L.wkv7_fwd.restype = i
    L.wkv7_fwd_varlen.argtypes = [i, i, i, i, i, i, p] + [p] * 7 + [i, p, p, p, p, i, p]
    L.wkv7_fwd_varlen.restype = i
    L.wkv7_gdn_fwd.argtypes = [i, i, i, i, i, i] + [p] * 6 + [i, p, p, i, p]
    L.wkv7_gdn_fwd.restype = i
    L.wkv7_bwd.argtypes = [i, i, i, i, i, i] + [p] * 7 + [i] + [p] * 11 + [ctypes.c_size_t, p]
    L.wkv7_bwd.restype = i
    L.wkv7_bwd_noalloc.argtypes = [i, i, i, i, i, i] + [p] * 7 + [i] + [p] * 11
    L.wkv7_bwd_noalloc.restype = i
    L.wkv7_bwd_workspace_bytes.argtypes = [i] * 5
    L.wkv7_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.wkv7_bwd_varlen.argtypes = [i] * 6 + [p] * 7 + [p, i, p, p, p, p] + [p] * 8 + [ctypes.c_size_t, p]
    L.wkv7_bwd_varlen.restype = i
    L.wkv7_bwd_varlen_workspace_bytes.argtypes = [i] * 5
    L.wkv7_bwd_varlen_workspace_bytes.restype = ctypes.c_size_t
    L.wkv7_gdn_bwd_varlen.argtypes = [i] * 6 + [p] * 6 + [p, i, p, p, p] + [p] * 7 + [ctypes.c_size_t, p]
    L.wkv7_gdn_bwd_varlen.restype = i
    L.wkv7_gdn_bwd_varlen_workspace_bytes.argtypes = [i] * 5
    L.wkv7_gdn_bwd_varlen_workspace_bytes.restype = ctypes.c_size_t
    L.wkv7_gdn_bwd.argtypes = [i, i, i, i, i, i] + [p] * 6 + [i] + [p] * 9 + [ctypes.c_size_t, p]
    L.wkv7_gdn_bwd.restype = i
    L.wkv7_gdn_bwd_workspace_bytes.argtypes = [i] * 5
    L.wkv7_gdn_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.wkv7_gdn_fwd_varlen.argtypes = [i, i, i, i, i, i, p] + [p] * 6 + [i, p, p, p, i, p]
    L.wkv7_gdn_fwd_varlen.restype = i
    L.wkv7_gdn_step.argtypes = [i, i, i, i, i] + [p] * 6 + [i, p, p, p]
    L.wkv7_gdn_step.restype = i
    L.wkv7_step.argtypes = [i, i, i, i, i] + [p] * 8 + [p]
    L.wkv7_step.restype = i
    L.wkv7_strerror.argtypes = [i]
    L.wkv7_strerror.restype = ctypes.c_char_p
    L.wkv7_fwd_path.argtypes = [i] * 7
    L.wkv7_fwd_path.restype = i
    L.wkv7_version.restype = i
    L.wkv7_set_wait_limit.argtypes = [i]
    L.wkv7_set_wait_limit.restype = i
    _lib = L
    return L


class WKV7Error(ValueError):
    def __init__(self, status):
        self.status = status
        super().__init__(f"wkv7 status {status}: {lib().wkv7_strerror(status).decode()}")


def _dtype_code(t):
    if t == torch.float32:
        return F32
    if t == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t}; use float32 or bfloat16")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(t, name, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def fwd(r, w, k, v, a, b, initial_state=None, mask=None, output_final_state=True,
        algo=ALGO_AUTO, out=None, final_state=None):
    """WKV7 forward.  r, w, k, a, b: [B,T,H,K]; v: [B,T,H,V] (float32 or
    bfloat16, one device); initial_state: [B,H,K,V] or [1,H,K,V] (shared by
    every sequence) float32, or None (zeros); mask: [B,T] bool/uint8
    (nonzero = update) or None.  Returns (o [B,T,H,V] in the input dtype,
    final_state [B,H,K,V] float32 or None).  `final_state` may be passed as
    an output buffer, including a [B,H,K,V] initial_state tensor itself for
    in-place state passing."""
    dev = r.device
    B, T, H, K = r.shape
    V = v.shape[-1]
    dt = r.dtype
    code = _dtype_code(dt)
    for name, t in (("r", r), ("w", w), ("k", k), ("a", a), ("b", b)):
        _check(t, name, (B, T, H, K), dt, dev)
    _check(v, "v", (B, T, H, V), dt, dev)
    n_state = _state_rows(initial_state, B, H, K, V, dev)
    m = _mask_u8(mask)
    if m is not None:
        _check(m, "mask", (B, T), torch.uint8, dev)
    o = out if out is not None else torch.empty((B, T, H, V), dtype=dt, device=dev)
    _check(o, "out", (B, T, H, V), dt, dev)
    sf = None
    if output_final_state:
        sf = final_state if final_state is not None else torch.empty((B, H, K, V), dtype=torch.float32, device=dev)
        _check(sf, "final_state", (B, H, K, V), torch.float32, dev)
    st = lib().wkv7_fwd(code, B, T, H, K, V, _ptr(r), _ptr(w), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                        _ptr(initial_state), n_state, _ptr(m), _ptr(o), _ptr(sf), int(algo), _stream(dev))
    if st != OK:
        raise WKV7Error(st)
    return o, sf


def _state_rows(initial_state, B, H, K, V, dev):
    """Rows of an initial state with B rows or one shared row (0 for None)."""
    if initial_state is None:
        return 0
    n_state = initial_state.shape[0] if initial_state.dim() == 4 else -1
    if n_state not in (1, B):
        raise ValueError(f"initial_state must be [{B} or 1,H,K,V], got {tuple(initial_state.shape)}")
    _check(initial_state, "initial_state", (n_state, H, K, V), torch.float32, dev)
    return n_state


def _mask_u8(mask):
    if mask is None:
        return None
    if mask.dtype == torch.bool:
        return mask.view(torch.uint8)
    if mask.dtype == torch.uint8:
        return mask
    raise ValueError("mask must be bool or uint8")


def fwd_varlen(r, w, k, v, a, b, cu_seqlens, initial_state=None, state_map=None, mask=None,
               output_final_state=True, algo=ALGO_AUTO, out=None, final_state=None):
    """WKV7 forward over packed variable-length sequences.  r, w, k, a, b:
    [T_total,H,K] (or [1,T_total,H,K]); v: [T_total,H,V]; cu_seqlens: int32
    [N+1] token offsets (device); initial_state: [n_state,H,K,V] float32 pool
    or None; state_map: int32 [N] pool row per sequence (out of range: zero
    state) or None (row n, or the single row of a one-row pool); mask:
    [T_total] bool/uint8 or None.  Returns (o shaped like v, final_state
    [N,H,K,V] float32 or None).  A new o is zero-filled first, so tokens
    outside every sequence (trailing padding, gaps) read as zeros; a
    caller-provided `out` keeps whatever it holds there."""
    dev = r.device
    lead1 = r.dim() == 4
    if lead1:
        if r.shape[0] != 1:
            raise ValueError("packed inputs take a leading dimension of 1, or none")
        r, w, k, v, a, b = (t.squeeze(0) for t in (r, w, k, v, a, b))
    TT, H, K = r.shape
    V = v.shape[-1]
    dt = r.dtype
    code = _dtype_code(dt)
    for name, t in (("r", r), ("w", w), ("k", k), ("a", a), ("b", b)):
        _check(t, name, (TT, H, K), dt, dev)
    _check(v, "v", (TT, H, V), dt, dev)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be [N+1] with N >= 1")
    N = cu_seqlens.numel() - 1
    _check(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    n_state = 0
    if initial_state is not None:
        n_state = initial_state.shape[0]
        _check(initial_state, "initial_state", (n_state, H, K, V), torch.float32, dev)
    if state_map is not None:
        _check(state_map, "state_map", (N,), torch.int32, dev)
    m = _mask_u8(mask)
    if m is not None:
        _check(m, "mask", (TT,), torch.uint8, dev)
    if out is not None:
        o = out.squeeze(0) if (lead1 and out.dim() == 4) else out
    else:
        o = torch.zeros((TT, H, V), dtype=dt, device=dev)
    _check(o, "out", (TT, H, V), dt, dev)
    sf = None
    if output_final_state:
        sf = final_state if final_state is not None else torch.empty((N, H, K, V), dtype=torch.float32, device=dev)
        _check(sf, "final_state", (N, H, K, V), torch.float32, dev)
    st = lib().wkv7_fwd_varlen(code, N, TT, H, K, V, _ptr(cu_seqlens), _ptr(r), _ptr(w), _ptr(k), _ptr(v),
                               _ptr(a), _ptr(b), _ptr(initial_state), n_state, _ptr(state_map), _ptr(m),
                               _ptr(o), _ptr(sf), int(algo), _stream(dev))
    if st != OK:
        raise WKV7Error(st)
    return (o.unsqueeze(0) if lead1 else o), sf


def bwd_workspace_bytes(B, T, H, K, V):
    """Bytes of device workspace bwd needs (0 if the sizes are rejected)."""
    return int(lib().wkv7_bwd_workspace_bytes(B, T, H, K, V))


def bwd(r, w, k, v, a, b, d_o, initial_state=None, mask=None, d_final_state=None, workspace=None,
        need_initial_state_grad=True):
    """Gradients of fwd.  Inputs as for fwd; d_o: [B,T,H,V] in the input
    dtype; d_final_state: [B,H,K,V] float32 or None.  workspace: a uint8
    device tensor of at least bwd_workspace_bytes(...) bytes, or None to
    allocate one.  Returns a dict with r, w, k, v, a, b (input dtype) and s0
    (float32, shaped like initial_state, [B,H,K,V] without one: for a shared
    [1,H,K,V] state the sum over the sequences; None when
    need_initial_state_grad is False)."""
    dev = r.device
    B, T, H, K = r.shape
    V = v.shape[-1]
    dt = r.dtype
    code = _dtype_code(dt)
    for name, t in (("r", r), ("w", w), ("k", k), ("a", a), ("b", b)):
        _check(t, name, (B, T, H, K), dt, dev)
    _check(v, "v", (B, T, H, V), dt, dev)
    _check(d_o, "d_o", (B, T, H, V), dt, dev)
    n_state = _state_rows(initial_state, B, H, K, V, dev)
    if d_final_state is not None:
        _check(d_final_state, "d_final_state", (B, H, K, V), torch.float32, dev)
    m = _mask_u8(mask)
    if m is not None:
        _check(m, "mask", (B, T), torch.uint8, dev)
    need = bwd_workspace_bytes(B, T, H, K, V)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    elif workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the inputs' device")
    g = {n: torch.empty((B, T, H, K), dtype=dt, device=dev) for n in ("r", "w", "k", "a", "b")}
    g["v"] = torch.empty((B, T, H, V), dtype=dt, device=dev)
    g["s0"] = (torch.empty((n_state or B, H, K, V), dtype=torch.float32, device=dev)
               if need_initial_state_grad else None)
    st = lib().wkv7_bwd(code, B, T, H, K, V, _ptr(r), _ptr(w), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                        _ptr(initial_state), n_state, _ptr(m), _ptr(d_o), _ptr(d_final_state),
                        *(_ptr(g[n]) for n in ("r", "w", "k", "v", "a", "b", "s0")),
                        _ptr(workspace), workspace.numel(), _stream(dev))
    if st != OK:
        raise WKV7Error(st)
    return g


def bwd_noalloc(r, w, k, v, a, b, d_o, initial_state=None, mask=None, d_final_state=None,
                need_initial_state_grad=True, out=None):
    """Gradients of fwd through wkv7_bwd_noalloc: the library's fixed
    per-GPU scratch array instead of a workspace (bwd_workspace_bytes(...)
    must not exceed NOALLOC_SCRATCH_BYTES, else WKV7Error with
    ERR_TOO_LARGE).  Arguments and result as for bwd; out: optional dict of
    preallocated gradient tensors (r, w, k, v, a, b, s0), so that a caller can
    keep every allocation outside the call.  Calls that overlap in time on
    one GPU share the scratch and race."""
    dev = r.device
    B, T, H, K = r.shape
    V = v.shape[-1]
    dt = r.dtype
    code = _dtype_code(dt)
    for name, t in (("r", r), ("w", w), ("k", k), ("a", a), ("b", b)):
        _check(t, name, (B, T, H, K), dt, dev)
    _check(v, "v", (B, T, H, V), dt, dev)
    _check(d_o, "d_o", (B, T, H, V), dt, dev)
    n_state = _state_rows(initial_state, B, H, K, V, dev)
    if d_final_state is not None:
        _check(d_final_state, "d_final_state", (B, H, K, V), torch.float32, dev)
    m = _mask_u8(mask)
    if m is not None:
        _check(m, "mask", (B, T), torch.uint8, dev)
    if out is not None:
        g = dict(out)
        for n in ("r", "w", "k", "a", "b"):
            _check(g[n], "out[" + n + "]", (B, T, H, K), dt, dev)
        _check(g["v"], "out[v]", (B, T, H, V), dt, dev)
        if not need_initial_state_grad:
            g["s0"] = None
        elif g.get("s0") is not None:
            _check(g["s0"], "out[s0]", (n_state or B, H, K, V), torch.float32, dev)
    else:
        g = {n: torch.empty((B, T, H, K), dtype=dt, device=dev) for n in ("r", "w", "k", "a", "b")}
        g["v"] = torch.empty((B, T, H, V), dtype=dt, device=dev)
        g["s0"] = (torch.empty((n_state or B, H, K, V), dtype=torch.float32, device=dev)
                   if need_initial_state_grad else None)
    st = lib().wkv7_bwd_noalloc(code, B, T, H, K, V, _ptr(r), _ptr(w), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                                _ptr(initial_state), n_state, _ptr(m), _ptr(d_o), _ptr(d_final_state),
                                *(_ptr(g[n]) for n in ("r", "w", "k", "v", "a", "b", "s0")), _stream(dev))
    if st != OK:
        raise WKV7Error(st)
    return g


def bwd_varlen_workspace_bytes(N, total_T, H, K, V):
    """Bytes of device workspace bwd_varlen needs (0 if the sizes are rejected)."""
    return int(lib().wkv7_bwd_varlen_workspace_bytes(N, total_T, H, K, V))


def bwd_varlen(r, w, k, v, a, b, cu_seqlens, d_o, initial_state=None, state_map=None, mask=None,
               d_final_state=None, workspace=None, need_initial_state_grad=True, out=None):
    """Gradients of fwd_varlen.  Inputs as for fwd_varlen ([T_total,H,K] or
    [1,T_total,H,K]); d_o shaped like v; d_final_state: [N,H,K,V] float32 or
    None.  Returns a dict with r, w, k, v, a, b (shaped like the inputs;
    zero at tokens outside every sequence, which the forward does not read)
    and s0 ([N,H,K,V] float32: the gradient of each sequence's initial
    state, or None).  out: optional dict of preallocated gradient tensors
    (r, w, k, v, a, b as [T_total,...], s0), used as they are: tokens outside
    every sequence keep what they hold."""
    dev = r.device
    lead1 = r.dim() == 4
    if lead1:
        if r.shape[0] != 1:
            raise ValueError("packed inputs take a leading dimension of 1, or none")
        r, w, k, v, a, b, d_o = (t.squeeze(0) for t in (r, w, k, v, a, b, d_o))
    TT, H, K = r.shape
    V = v.shape[-1]
    dt = r.dtype
    code = _dtype_code(dt)
    for name, t in (("r", r), ("w", w), ("k", k), ("a", a), ("b", b)):
        _check(t, name, (TT, H, K), dt, dev)
    _check(v, "v", (TT, H, V), dt, dev)
    _check(d_o, "d_o", (TT, H, V), dt, dev)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be [N+1] with N >= 1")
    N = cu_seqlens.numel() - 1
    _check(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    n_state = 0
    if initial_state is not None:
        n_state = initial_state.shape[0]
        _check(initial_state, "initial_state", (n_state, H, K, V), torch.float32, dev)
    if state_map is not None:
        _check(state_map, "state_map", (N,), torch.int32, dev)
    if d_final_state is not None:
        _check(d_final_state, "d_final_state", (N, H, K, V), torch.float32, dev)
    m = _mask_u8(mask)
    if m is not None:
        _check(m, "mask", (TT,), torch.uint8, dev)
    need = bwd_varlen_workspace_bytes(N, TT, H, K, V)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    elif workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the inputs' device")
    if out is not None:
        g = dict(out)
        for n in ("r", "w", "k", "a", "b"):
            _check(g[n], "out[" + n + "]", (TT, H, K), dt, dev)
        _check(g["v"], "out[v]", (TT, H, V), dt, dev)
        if not need_initial_state_grad:
            g["s0"] = None
        elif g.get("s0") is not None:
            _check(g["s0"], "out[s0]", (N, H, K, V), torch.float32, dev)
    else:
        g = {n: torch.zeros((TT, H, K), dtype=dt, device=dev) for n in ("r", "w", "k", "a", "b")}
        g["v"] = torch.zeros((TT, H, V), dtype=dt, device=dev)
        g["s0"] = torch.empty((N, H, K, V), dtype=torch.float32, device=dev) if need_initial_state_grad else None
    st = lib().wkv7_bwd_varlen(code, N, TT, H, K, V, _ptr(cu_seqlens), _ptr(r), _ptr(w), _ptr(k), _ptr(v),
                               _ptr(a), _ptr(b), _ptr(initial_state), n_state, _ptr(state_map), _ptr(m),
                               _ptr(d_o), _ptr(d_final_state),
                               *(_ptr(g[n]) for n in ("r", "w", "k", "v", "a", "b", "s0")),
                               _ptr(workspace), workspace.numel(), _stream(dev))
    if st != OK:
        raise WKV7Error(st)
    if lead1:
        for n in ("r", "w", "k", "v", "a", "b"):
            g[n] = g[n].unsqueeze(0)
    return g


def gdn_fwd(q, k, v, g, beta, initial_state=None, output_final_state=True, algo=ALGO_AUTO,
            out=None, final_state=None):
    """Gated DeltaNet forward (q, k L2-normalised inside; gated delta rule).
    q, k: [B,T,H,K]; v: [B,T,H,V]; g, beta: [B,T,H] (one dtype, float32 or
    bfloat16); initial_state: [B,H,K,V] or [1,H,K,V] float32 (shared) or
    None.  Returns (o [B,T,H,V], final_state [B,H,K,V] float32 or None)."""
    dev = q.device
    B, T, H, K = q.shape
    V = v.shape[-1]
    dt = q.dtype
    code = _dtype_code(dt)
    _check(k, "k", (B, T, H, K), dt, dev)
    _check(v, "v", (B, T, H, V), dt, dev)
    _check(g, "g", (B, T, H), dt, dev)
    _check(beta, "beta", (B, T, H), dt, dev)
    n_state = 0
    if initial_state is not None:
        n_state = initial_state.shape[0]
        if n_state not in (1, B):
            raise ValueError(f"initial_state must have {B} or 1 rows, got {n_state}")
        _check(initial_state, "initial_state", (n_state, H, K, V), torch.float32, dev)
    o = out if out is not None else torch.empty((B, T, H, V), dtype=dt, device=dev)
    _check(o, "out", (B, T, H, V), dt, dev)
    sf = None
    if output_final_state:
        sf = final_state if final_state is not None else torch.empty((B, H, K, V), dtype=torch.float32, device=dev)
        _check(sf, "final_state", (B, H, K, V), torch.float32, dev)
    st = lib().wkv7_gdn_fwd(code, B, T, H, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                            _ptr(initial_state), n_state, _ptr(o), _ptr(sf), int(algo), _stream(dev))
    if st != OK:
        raise WKV7Error(st)
    return o, sf


def gdn_bwd_workspace_bytes(B, T, H, K, V):
    """Bytes of device workspace gdn_bwd needs (0 if the sizes are rejected)."""
    return int(lib().wkv7_gdn_bwd_workspace_bytes(B, T, H, K, V))


def gdn_bwd(q, k, v, g, beta, d_o, initial_state=None, d_final_state=None, workspace=None,
            need_initial_state_grad=True):
    """Gradients of gdn_fwd.  Inputs as for gdn_fwd; d_o: [B,T,H,V] in the
    input dtype; d_final_state: [B,H,K,V] float32 or None.  workspace: a
    uint8 device tensor of at least gdn_bwd_workspace_bytes(...) bytes, or
    None to allocate one.  Returns a dict with q, k, v, g, beta (input dtype)
    and s0 (float32, shaped like initial_state, [B,H,K,V] without one; None
    when need_initial_state_grad is False)."""
    dev = q.device
    B, T, H, K = q.shape
    V = v.shape[-1]
    dt = q.dtype
    code = _dtype_code(dt)
    _check(k, "k", (B, T, H, K), dt, dev)
    _check(v, "v", (B, T, H, V), dt, dev)
    _check(g, "g", (B, T, H), dt, dev)
    _check(beta, "beta", (B, T, H), dt, dev)
    _check(d_o, "d_o", (B, T, H, V), dt, dev)
    n_state = B
    if initial_state is not None:
        n_state = initial_state.shape[0]
        if n_state not in (1, B):
            raise ValueError(f"initial_state must have {B} or 1 rows, got {n_state}")
        _check(initial_state, "initial_state", (n_state, H, K, V), torch.float32, dev)
    if d_final_state is not None:
        _check(d_final_state, "d_final_state", (B, H, K, V), torch.float32, dev)
    need = gdn_bwd_workspace_bytes(B, T, H, K, V)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    elif workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the inputs' device")
    out = {"q": torch.empty((B, T, H, K), dtype=dt, device=dev), "k": torch.empty((B, T, H, K), dtype=dt, device=dev),
           "v": torch.empty((B, T, H, V), dtype=dt, device=dev), "g": torch.empty((B, T, H), dtype=dt, device=dev),
           "beta": torch.empty((B, T, H), dtype=dt, device=dev)}
    out["s0"] = (torch.empty((n_state, H, K, V), dtype=torch.float32, device=dev)
                 if need_initial_state_grad else None)
    st = lib().wkv7_gdn_bwd(code, B, T, H, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                            _ptr(initial_state), n_state if initial_state is not None else 0,
                            _ptr(d_o), _ptr(d_final_state),
                            *(_ptr(out[n]) for n in ("q", "k", "v", "g", "beta", "s0")),
                            _ptr(workspace), workspace.numel(), _stream(dev))
    if st != OK:
        raise WKV7Error(st)
    return out


def gdn_fwd_varlen(q, k, v, g, beta, cu_seqlens, initial_state=None, state_map=None,
                   output_final_state=True, algo=ALGO_AUTO, out=None, final_state=None):
    """Gated DeltaNet forward over packed variable-length sequences.  q, k:
    [T_total,H,K] (or [1,T_total,H,K]); v: [T_total,H,V]; g, beta:
    [T_total,H]; cu_seqlens: int32 [N+1] token offsets (device);
    initial_state: [n_state,H,K,V] float32 pool or None; state_map: int32 [N]
    pool row per sequence (out of range: zero state) or None (row n, or the
    single shared row).  Returns (o shaped like v, final_state [N,H,K,V])."""
    dev = q.device
    lead1 = q.dim() == 4
    if lead1:
        if q.shape[0] != 1:
            raise ValueError("packed inputs take a leading dimension of 1, or none")
        q, k, v, g, beta = (t.squeeze(0) for t in (q, k, v, g, beta))
    TT, H, K = q.shape
    V = v.shape[-1]
    dt = q.dtype
    code = _dtype_code(dt)
    _check(k, "k", (TT, H, K), dt, dev)
    _check(v, "v", (TT, H, V), dt, dev)
    _check(g, "g", (TT, H), dt, dev)
    _check(beta, "beta", (TT, H), dt, dev)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be [N+1] with N >= 1")
    N = cu_seqlens.numel() - 1
    _check(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    n_state = 0
    if initial_state is not None:
        n_state = initial_state.shape[0]
        _check(initial_state, "initial_state", (n_state, H, K, V), torch.float32, dev)
    if state_map is not None:
        _check(state_map, "state_map", (N,), torch.int32, dev)
    if out is not None:
        o = out.squeeze(0) if (lead1 and out.dim() == 4) else out
    else:
        o = torch.zeros((TT, H, V), dtype=dt, device=dev)
    _check(o, "out", (TT, H, V), dt, dev)
    sf = None
    if output_final_state:
        sf = final_state if final_state is not None else torch.empty((N, H, K, V), dtype=torch.float32, device=dev)
        _check(sf, "final_state", (N, H, K, V), torch.float32, dev)
    st = lib().wkv7_gdn_fwd_varlen(code, N, TT, H, K, V, _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                   _ptr(beta), _ptr(initial_state), n_state, _ptr(state_map), _ptr(o), _ptr(sf),
                                   int(algo), _stream(dev))
    if st != OK:
        raise WKV7Error(st)
    return (o.unsqueeze(0) if lead1 else o), sf


def gdn_bwd_varlen(q, k, v, g, beta, cu_seqlens, d_o, initial_state=None, state_map=None, d_final_state=None,
                   workspace=None, need_initial_state_grad=True):
    """Gradients of gdn_fwd_varlen.  Inputs as for gdn_fwd_varlen; d_o
    shaped like v; d_final_state: [N,H,K,V] float32 or None.  Returns a dict
    with q, k, v, g, beta (shaped like the inputs; zero at tokens outside
    every sequence) and s0 ([N,H,K,V] float32: the gradient of each
    sequence's initial state, or None)."""
    dev = q.device
    lead1 = q.dim() == 4
    if lead1:
        if q.shape[0] != 1:
            raise ValueError("packed inputs take a leading dimension of 1, or none")
        q, k, v, g, beta, d_o = (t.squeeze(0) for t in (q, k, v, g, beta, d_o))
    TT, H, K = q.shape
    V = v.shape[-1]
    dt = q.dtype
    code = _dtype_code(dt)
    _check(k, "k", (TT, H, K), dt, dev)
    _check(v, "v", (TT, H, V), dt, dev)
    _check(g, "g", (TT, H), dt, dev)
    _check(beta, "beta", (TT, H), dt, dev)
    _check(d_o, "d_o", (TT, H, V), dt, dev)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be [N+1] with N >= 1")
    N = cu_seqlens.numel() - 1
    _check(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    n_state = 0
    if initial_state is not None:
        n_state = initial_state.shape[0]
        _check(initial_state, "initial_state", (n_state, H, K, V), torch.float32, dev)
    if state_map is not None:
        _check(state_map, "state_map", (N,), torch.int32, dev)
    if d_final_state is not None:
        _check(d_final_state, "d_final_state", (N, H, K, V), torch.float32, dev)
    need = int(lib().wkv7_gdn_bwd_varlen_workspace_bytes(N, TT, H, K, V))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    elif workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the inputs' device")
    out = {"q": torch.zeros((TT, H, K), dtype=dt, device=dev), "k": torch.zeros((TT, H, K), dtype=dt, device=dev),
           "v": torch.zeros((TT, H, V), dtype=dt, device=dev), "g": torch.zeros((TT, H), dtype=dt, device=dev),
           "beta": torch.zeros((TT, H), dtype=dt, device=dev)}
    out["s0"] = torch.empty((N, H, K, V), dtype=torch.float32, device=dev) if need_initial_state_grad else None
    st = lib().wkv7_gdn_bwd_varlen(code, N, TT, H, K, V, _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                   _ptr(beta), _ptr(initial_state), n_state, _ptr(state_map), _ptr(d_o),
                                   _ptr(d_final_state), *(_ptr(out[n]) for n in ("q", "k", "v", "g", "beta", "s0")),
                                   _ptr(workspace), workspace.numel(), _stream(dev))
    if st != OK:
        raise WKV7Error(st)
    if lead1:
        for n in ("q", "k", "v", "g", "beta"):
            out[n] = out[n].unsqueeze(0)
    return out


def gdn_step(q, k, v, g, beta, state=None, out=None, next_state=None):
    """One Gated DeltaNet decode token.  q, k: [B,H,K]; v: [B,H,V]; g, beta:
    [B,H]; state: [B,H,K,V] or [1,H,K,V] float32 (shared) or None (zeros).
    The next state goes to next_state ([B,H,K,V] float32); by default a state
    with B rows is updated in place and otherwise a new tensor is returned.
    Returns (o [B,H,V], next_state)."""
    dev = q.device
    B, H, K = q.shape
    V = v.shape[-1]
    dt = q.dtype
    code = _dtype_code(dt)
    _check(k, "k", (B, H, K), dt, dev)
    _check(v, "v", (B, H, V), dt, dev)
    _check(g, "g", (B, H), dt, dev)
    _check(beta, "beta", (B, H), dt, dev)
    n_state = 0
    if state is not None:
        n_state = state.shape[0]
        if n_state not in (1, B):
            raise ValueError(f"state must have {B} or 1 rows, got {n_state}")
        _check(state, "state", (n_state, H, K, V), torch.float32, dev)
    if next_state is None:
        next_state = state if (state is not None and n_state == B) else \
            torch.empty((B, H, K, V), dtype=torch.float32, device=dev)
    _check(next_state, "next_state", (B, H, K, V), torch.float32, dev)
    o = out if out is not None else torch.empty((B, H, V), dtype=dt, device=dev)
    _check(o, "out", (B, H, V), dt, dev)
    st = lib().wkv7_gdn_step(code, B, H, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                             _ptr(state), n_state, _ptr(next_state), _ptr(o), _stream(dev))
    if st != OK:
        raise WKV7Error(st)
    return o, next_state


def step(r, w, k, v, a, b, state, out=None):
    """One decode token.  r, w, k, a, b: [B,H,K]; v: [B,H,V]; state:
    [B,H,K,V] float32, updated in place.  Returns o [B,H,V] (input dtype)."""
    dev = r.device
    B, H, K = r.shape
    V = v.shape[-1]
    dt = r.dtype
    code = _dtype_code(dt)
    for name, t in (("r", r), ("w", w), ("k", k), ("a", a), ("b", b)):
        _check(t, name, (B, H, K), dt, dev)
    _check(v, "v", (B, H, V), dt, dev)
    _check(state, "state", (B, H, K, V), torch.float32, dev)
    o = out if out is not None else torch.empty((B, H, V), dtype=dt, device=dev)
    _check(o, "out", (B, H, V), dt, dev)
    st = lib().wkv7_step(code, B, H, K, V, _ptr(r), _ptr(w), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                         _ptr(state), _ptr(o), _stream(dev))
    if st != OK:
        raise WKV7Error(st)
    return o


def fwd_path(dtype, B, T, H, K, V, algo=ALGO_AUTO):
    """Kernel wkv7_fwd would launch (ALGO_RECURRENT / ALGO_CHUNKED), or -1."""
    return lib().wkv7_fwd_path(_dtype_code(dtype), B, T, H, K, V, int(algo))


def set_wait_limit(polls):
    """Test hook (wkv7_set_wait_limit): polls a chunked-forward wave makes on
    a hand-off counter before it gives up and poisons its results with NaN;
    0 gives up at once, a negative value restores the default.  Returns the
    previous limit."""
    return int(lib().wkv7_set_wait_limit(int(polls)))
