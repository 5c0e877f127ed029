"""Entry points in the shape of the rwkv-ops interface.

The rwkv-ops README lists, in section "rwkv7op 使用方法", the trainable
``generalized_delta_rule(r, w, k, v, a, b, initial_state=None,
output_final_state=True, head_first=False, mask=None) -> (o, final_state)``
(also named ``rwkv7_op``) and its gradient-free twin
``generalized_delta_rule_inference``; in section "rwkv7_op_rnn 使用方法" the
one-token ``rwkv7_op_rnn`` on (B, 1, H, K) inputs; in sections
"gdn_recurrent 使用方法" and "gdn_chunk 使用方法" the Gated DeltaNet entries
``gated_delta_net_recurrent`` (trainable), ``..._inference``,
``..._single_step`` and ``gated_delta_net_chunk``.  These wrappers map them
onto libwkv7.so and torch.autograd: the forward calls wkv7_fwd /
wkv7_gdn_fwd, the backward wkv7_bwd / wkv7_gdn_bwd, the one-token forms
wkv7_step / wkv7_gdn_step.  They compute nothing themselves and have no CPU
path: inputs must be contiguous device tensors in the seq-first layout
(head_first=True is rejected rather than served by a hidden layout copy; the
single-token Gated DeltaNet form is [B,H,K] by definition).
"""
import torch

from . import wkv7


def _require_device(tensors):
    for name, t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} is on {t.device}: the operator runs on the GPU only (no CPU path)")


def _head_first(head_first):
    if head_first:
        raise NotImplementedError("only the seq-first layout [B,T,H,K] is supported (head_first=False)")


class _GeneralizedDeltaRule(torch.autograd.Function):
    @staticmethod
    def forward(ctx, r, w, k, v, a, b, initial_state, mask):
        o, sf = wkv7.fwd(r, w, k, v, a, b, initial_state=initial_state, mask=mask, output_final_state=True)
        ctx.save_for_backward(r, w, k, v, a, b, initial_state, mask)
        ctx.s0_grad = initial_state is not None and initial_state.requires_grad
        return o, sf

    @staticmethod
    def backward(ctx, d_o, d_sf):
        r, w, k, v, a, b, s0, mask = ctx.saved_tensors
        if d_o is None:
            d_o = torch.zeros_like(v)
        g = wkv7.bwd(r, w, k, v, a, b, d_o.contiguous(), initial_state=s0, mask=mask,
                     d_final_state=None if d_sf is None else d_sf.contiguous(),
                     need_initial_state_grad=ctx.s0_grad)
        return g["r"], g["w"], g["k"], g["v"], g["a"], g["b"], g["s0"], None


def _pool_grad(per_seq, pool, smap):
    """Gradient of a pool of initial states from the per-sequence ones: row
    n without a map (N rows), the sum over the sequences for one shared row,
    else the sum over the sequences mapped to each row (a map entry outside
    the pool started from zeros)."""
    if smap is None:
        return per_seq if pool.shape[0] == per_seq.shape[0] else per_seq.sum(dim=0, keepdim=True)
    ok = (smap >= 0) & (smap < pool.shape[0])
    return torch.zeros_like(pool).index_add_(0, smap[ok].long(), per_seq[ok])


class _GeneralizedDeltaRulePacked(torch.autograd.Function):
    @staticmethod
    def forward(ctx, r, w, k, v, a, b, initial_state, cu_seqlens, state_map, mask):
        o, sf = wkv7.fwd_varlen(r, w, k, v, a, b, cu_seqlens, initial_state=initial_state, state_map=state_map,
                                mask=mask, output_final_state=True)
        ctx.save_for_backward(r, w, k, v, a, b, initial_state, cu_seqlens, state_map, mask)
        ctx.s0_grad = initial_state is not None and initial_state.requires_grad
        return o, sf

    @staticmethod
    def backward(ctx, d_o, d_sf):
        r, w, k, v, a, b, s0, cu, smap, mask = ctx.saved_tensors
        if d_o is None:
            d_o = torch.zeros_like(v)
        g = wkv7.bwd_varlen(r, w, k, v, a, b, cu, d_o.contiguous(), initial_state=s0, state_map=smap, mask=mask,
                            d_final_state=None if d_sf is None else d_sf.contiguous(),
                            need_initial_state_grad=ctx.s0_grad)
        ds0 = _pool_grad(g["s0"], s0, smap) if ctx.s0_grad else None
        return g["r"], g["w"], g["k"], g["v"], g["a"], g["b"], ds0, None, None, None


def generalized_delta_rule(r, w, k, v, a, b, initial_state=None, output_final_state=True, head_first=False,
                           mask=None, cu_seqlens=None, state_map=None):
    """WKV7 generalized delta rule with gradients.  r, w, k, a, b: [B,T,H,K];
    v: [B,T,H,V] (float32 or bfloat16); initial_state: [B,H,K,V] float32,
    [1,H,K,V] (one state shared by every sequence; its gradient is the sum
    over them) or None; mask: [B,T] (nonzero = update) or None.  Returns (o, final_state or
    None); gradients flow to r, w, k, v, a, b and initial_state.

    Packed sequences: with cu_seqlens (int32 [N+1] token offsets) the inputs
    are [1,T,H,K] (N sequences back to back), mask is [T] or [1,T],
    initial_state is [N,H,K,V], [1,H,K,V] (shared) or, with state_map
    (int32 [N]), a pool of rows; final_state is [N,H,K,V].  Tokens outside
    every sequence get a zero output and zero gradients."""
    _head_first(head_first)
    _require_device([("r", r), ("w", w), ("k", k), ("v", v), ("a", a), ("b", b),
                     ("initial_state", initial_state), ("mask", mask), ("cu_seqlens", cu_seqlens),
                     ("state_map", state_map)])
    tensors = (r, w, k, v, a, b) + (() if initial_state is None else (initial_state,))
    grad = torch.is_grad_enabled() and any(t.requires_grad for t in tensors)
    if cu_seqlens is not None:
        if mask is not None and mask.dim() == 2:
            mask = mask.reshape(-1)
        if grad:
            o, sf = _GeneralizedDeltaRulePacked.apply(r, w, k, v, a, b, initial_state, cu_seqlens, state_map, mask)
        else:
            o, sf = wkv7.fwd_varlen(r, w, k, v, a, b, cu_seqlens, initial_state=initial_state,
                                    state_map=state_map, mask=mask, output_final_state=True)
    elif state_map is not None:
        raise ValueError("state_map needs cu_seqlens (packed sequences)")
    elif grad:
        o, sf = _GeneralizedDeltaRule.apply(r, w, k, v, a, b, initial_state, mask)
    else:
        o, sf = wkv7.fwd(r, w, k, v, a, b, initial_state=initial_state, mask=mask, output_final_state=True)
    return o, (sf if output_final_state else None)


class _GatedDeltaNet(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, g, beta, initial_state):
        o, sf = wkv7.gdn_fwd(q, k, v, g, beta, initial_state=initial_state, output_final_state=True)
        ctx.save_for_backward(q, k, v, g, beta, initial_state)
        ctx.s0_grad = initial_state is not None and initial_state.requires_grad
        return o, sf

    @staticmethod
    def backward(ctx, d_o, d_sf):
        q, k, v, g, beta, s0 = ctx.saved_tensors
        if d_o is None:
            d_o = torch.zeros_like(v)
        gr = wkv7.gdn_bwd(q, k, v, g, beta, d_o.contiguous(), initial_state=s0,
                          d_final_state=None if d_sf is None else d_sf.contiguous(),
                          need_initial_state_grad=ctx.s0_grad)
        return gr["q"], gr["k"], gr["v"], gr["g"], gr["beta"], gr["s0"]


class _GatedDeltaNetPacked(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, g, beta, initial_state, cu_seqlens, state_map):
        o, sf = wkv7.gdn_fwd_varlen(q, k, v, g, beta, cu_seqlens, initial_state=initial_state,
                                    state_map=state_map, output_final_state=True)
        ctx.save_for_backward(q, k, v, g, beta, initial_state, cu_seqlens, state_map)
        ctx.s0_grad = initial_state is not None and initial_state.requires_grad
        return o, sf

    @staticmethod
    def backward(ctx, d_o, d_sf):
        q, k, v, g, beta, s0, cu, smap = ctx.saved_tensors
        if d_o is None:
            d_o = torch.zeros_like(v)
        gr = wkv7.gdn_bwd_varlen(q, k, v, g, beta, cu, d_o.contiguous(), initial_state=s0, state_map=smap,
                                 d_final_state=None if d_sf is None else d_sf.contiguous(),
                                 need_initial_state_grad=ctx.s0_grad)
        ds0 = _pool_grad(gr["s0"], s0, smap) if ctx.s0_grad else None
        return gr["q"], gr["k"], gr["v"], gr["g"], gr["beta"], ds0, None, None


def gated_delta_net(q, k, v, g, beta, initial_state=None, output_final_state=True, head_first=False,
                    cu_seqlens=None, state_map=None):
    """Gated DeltaNet with gradients (q and k are L2-normalised inside).
    q, k: [B,T,H,K]; v: [B,T,H,V]; g, beta: [B,T,H]; initial_state:
    [B,H,K,V] or [1,H,K,V] (shared) float32, or None.  Returns (o,
    final_state or None); gradients flow to q, k, v, g, beta and
    initial_state.

    Packed sequences: with cu_seqlens (int32 [N+1]) the inputs are
    [1,T,H,K] and g, beta [1,T,H]; initial_state is [N,H,K,V], one shared
    row, or with state_map (int32 [N]) a pool; final_state is [N,H,K,V]."""
    _head_first(head_first)
    _require_device([("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("initial_state", initial_state),
                     ("cu_seqlens", cu_seqlens), ("state_map", state_map)])
    tensors = (q, k, v, g, beta) + (() if initial_state is None else (initial_state,))
    grad = torch.is_grad_enabled() and any(t.requires_grad for t in tensors)
    if cu_seqlens is not None:
        if grad:
            o, sf = _GatedDeltaNetPacked.apply(q, k, v, g, beta, initial_state, cu_seqlens, state_map)
        else:
            o, sf = wkv7.gdn_fwd_varlen(q, k, v, g, beta, cu_seqlens, initial_state=initial_state,
                                        state_map=state_map, output_final_state=True)
    elif state_map is not None:
        raise ValueError("state_map needs cu_seqlens (packed sequences)")
    elif grad:
        o, sf = _GatedDeltaNet.apply(q, k, v, g, beta, initial_state)
    else:
        o, sf = wkv7.gdn_fwd(q, k, v, g, beta, initial_state=initial_state, output_final_state=True)
    return o, (sf if output_final_state else None)


rwkv7_op = generalized_delta_rule


def generalized_delta_rule_inference(r, w, k, v, a, b, initial_state=None, output_final_state=True,
                                     head_first=False, mask=None, cu_seqlens=None, state_map=None):
    """generalized_delta_rule without gradients."""
    with torch.no_grad():
        return generalized_delta_rule(r, w, k, v, a, b, initial_state, output_final_state, head_first, mask,
                                      cu_seqlens, state_map)


def rwkv7_op_rnn(r, w, k, v, a, b, initial_state=None, output_final_state=True, head_first=False):
    """One token of the WKV7 recurrence (no gradients).  r, w, k, a, b:
    [B,1,H,K]; v: [B,1,H,V]; initial_state: [B,H,K,V] float32 or None
    (zeros), not modified.  Returns (o [B,1,H,V], next_state or None)."""
    _head_first(head_first)
    _require_device([("r", r), ("w", w), ("k", k), ("v", v), ("a", a), ("b", b),
                     ("initial_state", initial_state)])
    if r.dim() != 4 or r.shape[1] != 1:
        raise ValueError(f"r must be [B,1,H,K], got {tuple(r.shape)}")
    B, _, H, K = r.shape
    V = v.shape[-1]
    state = initial_state.clone() if initial_state is not None else \
        torch.zeros((B, H, K, V), dtype=torch.float32, device=r.device)
    with torch.no_grad():
        o = wkv7.step(*(x[:, 0] for x in (r, w, k, v, a, b)), state)
    return o.unsqueeze(1), (state if output_final_state else None)


def gated_delta_net_recurrent(q, k, v, g, beta, initial_state=None, output_final_state=True, head_first=False,
                              cu_seqlens=None, state_map=None):
    """gated_delta_net (with gradients); the kernel is chosen by size."""
    return gated_delta_net(q, k, v, g, beta, initial_state, output_final_state, head_first, cu_seqlens, state_map)


def gated_delta_net_recurrent_inference(q, k, v, g, beta, initial_state=None, output_final_state=True,
                                        head_first=False):
    """gated_delta_net without gradients."""
    with torch.no_grad():
        return gated_delta_net(q, k, v, g, beta, initial_state, output_final_state, head_first)


def gated_delta_net_chunk(q, k, v, g, beta, initial_state=None, output_final_state=True, chunk_size=16):
    """gated_delta_net (with gradients).  The interface's chunk_size must
    divide T; the kernels' own chunk length is fixed (16 tokens) and does not
    change the result beyond rounding."""
    if chunk_size <= 0 or q.shape[1] % chunk_size:
        raise ValueError(f"chunk_size {chunk_size} must divide T = {q.shape[1]}")
    return gated_delta_net(q, k, v, g, beta, initial_state, output_final_state)


def gated_delta_net_recurrent_single_step(q, k, v, g, beta, initial_state=None, output_final_state=True,
                                          head_first=True):
    """One Gated DeltaNet token (no gradients).  q, k: [B,H,K]; v: [B,H,V];
    g, beta: [B,H]; initial_state: [B,H,K,V] or [1,H,K,V] float32 or None
    (zeros), not modified.  Returns (o [B,H,V], next_state or None)."""
    if not head_first:
        raise NotImplementedError("the single-token form takes [B,H,K] inputs (head_first=True)")
    _require_device([("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("initial_state", initial_state)])
    B, H, K = q.shape
    nxt = torch.empty((B, H, K, v.shape[-1]), dtype=torch.float32, device=q.device)
    with torch.no_grad():
        o, nxt = wkv7.gdn_step(q, k, v, g, beta, state=initial_state, next_state=nxt)
    return o, (nxt if output_final_state else None)
