"""Tensor-level wrappers over the C ABI (checks and allocation only).

``attention`` and ``dconv`` validate torch tensors, allocate the output (and,
if asked, a workspace), and call the library on the current torch stream.
``attention_train`` is the same forward with autograd: its backward is the
library's exact backward pass, started from the state the forward kept.
They raise ``NystromError`` on any non-zero return code.
"""
from __future__ import annotations

import torch
from torch.autograd.function import once_differentiable

from . import _lib

_DTYPES = {torch.float32: _lib.NYS_F32, torch.bfloat16: _lib.NYS_BF16}


class NystromError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {_lib.nystrom_strerror(code)} (code {code})")
        self.code = code


def _check_io(*ts):
    t0 = ts[0]
    if t0.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t0.dtype}; use float32 or bfloat16")
    for t in ts:
        if t.device.type != "cuda":
            raise ValueError("tensors must live on the GPU")
        if t.dtype != t0.dtype or t.shape != t0.shape:
            raise ValueError("Q, K, V must share shape and dtype")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    if t0.dim() != 4:
        raise ValueError("expected [batch, heads, n, d]")


def workspace_bytes(batch, heads, n, d, m) -> int:
    return _lib.nystrom_attn_workspace_bytes(batch, heads, n, d, m)


def new_workspace(batch, heads, n, d, m, device="cuda") -> torch.Tensor:
    nbytes = workspace_bytes(batch, heads, n, d, m)
    if nbytes == 0:
        raise NystromError(_lib.NYS_EUNSUPPORTED, "workspace")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def attention(Q, K, V, m, iters=6, conv_w=None, out=None, workspace=None, stream=None, lengths=None):
    """Nyström attention forward.  Q, K, V: [batch, heads, n, d] (fp32 or bf16);
    conv_w: fp32 [heads, d, k] or None; lengths: None, or int32 [batch] on
    the GPU, the tokens of each right-padded sequence (key-padding mask).
    Returns ``out`` (same shape/dtype)."""
    _check_io(Q, K, V)
    batch, heads, n, d = Q.shape
    conv_k = 0
    if conv_w is not None:
        if conv_w.dtype != torch.float32 or conv_w.dim() != 3 or tuple(conv_w.shape[:2]) != (heads, d):
            raise ValueError("conv_w must be float32 [heads, d, k]")
        if not conv_w.is_contiguous() or conv_w.device.type != "cuda":
            raise ValueError("conv_w must be a contiguous GPU tensor")
        conv_k = conv_w.shape[2]
    if out is None:
        out = torch.empty_like(Q)
    if stream is None:
        stream = torch.cuda.current_stream()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if lengths is None:
        rc = _lib.nystrom_attn_fwd(Q, K, V, conv_w, n, d, m, heads, iters, out, batch, conv_k, _DTYPES[Q.dtype],
                                   workspace, ws_bytes, stream)
        if rc != _lib.NYS_OK:
            raise NystromError(rc, "nystrom_attn_fwd")
        return out
    if (lengths.dtype != torch.int32 or tuple(lengths.shape) != (batch,) or lengths.device.type != "cuda"
            or not lengths.is_contiguous()):
        raise ValueError("lengths must be a contiguous int32 GPU tensor of shape [batch]")
    rc = _lib.nystrom_attn_fwd_masked(Q, K, V, conv_w, n, d, m, heads, iters, out, batch, conv_k,
                                      _DTYPES[Q.dtype], lengths, workspace, ws_bytes, stream)
    if rc != _lib.NYS_OK:
        raise NystromError(rc, "nystrom_attn_fwd_masked")
    return out


def _conv_k(conv_w, heads, d) -> int:
    if conv_w is None:
        return 0
    if conv_w.dtype != torch.float32 or conv_w.dim() != 3 or tuple(conv_w.shape[:2]) != (heads, d):
        raise ValueError("conv_w must be float32 [heads, d, k]")
    if not conv_w.is_contiguous() or conv_w.device.type != "cuda":
        raise ValueError("conv_w must be a contiguous GPU tensor")
    return conv_w.shape[2]


class _NystromAttention(torch.autograd.Function):
    """Forward: nystrom_attn_fwd_save, which keeps the landmark-side state in
    a buffer held by the autograd context (the state alone, not the
    backward's scratch); backward: nystrom_attn_bwd_from_state from that state
    with a scratch buffer that lives only during the call (gradients of Q, K,
    V and the filters)."""

    @staticmethod
    def forward(ctx, Q, K, V, conv_w, m, iters):
        _check_io(Q, K, V)
        batch, heads, n, d = Q.shape
        conv_k = _conv_k(conv_w, heads, d)
        nbytes = _lib.nystrom_attn_bwd_state_bytes(batch, heads, n, d, m, iters, conv_k)
        if nbytes == 0:
            raise NystromError(_lib.NYS_EUNSUPPORTED, "nystrom_attn_bwd_state_bytes")
        saved = torch.empty(nbytes, dtype=torch.uint8, device=Q.device)
        out = torch.empty_like(Q)
        rc = _lib.nystrom_attn_fwd_save(Q, K, V, conv_w, n, d, m, heads, iters, out, batch, conv_k,
                                        _DTYPES[Q.dtype], saved, nbytes, torch.cuda.current_stream())
        if rc != _lib.NYS_OK:
            raise NystromError(rc, "nystrom_attn_fwd_save")
        ctx.save_for_backward(Q, K, V, conv_w)
        ctx.state, ctx.nbytes, ctx.m, ctx.iters, ctx.conv_k = saved, nbytes, m, iters, conv_k
        return out

    @staticmethod
    @once_differentiable
    def backward(ctx, dO):
        # The gradients come from the library, outside autograd: a second
        # derivative through them (create_graph=True) raises instead of
        # silently missing terms.
        Q, K, V, conv_w = ctx.saved_tensors
        batch, heads, n, d = Q.shape
        dO = dO.to(Q.dtype).contiguous()
        dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
        dW = torch.empty_like(conv_w) if conv_w is not None and ctx.needs_input_grad[3] else None
        total = _lib.nystrom_attn_bwd_workspace_bytes(batch, heads, n, d, ctx.m, ctx.iters, ctx.conv_k)
        scratch = torch.empty(total - ctx.nbytes, dtype=torch.uint8, device=Q.device)
        rc = _lib.nystrom_attn_bwd_from_state(Q, K, V, conv_w, dO, n, d, ctx.m, heads, ctx.iters, dQ, dK, dV, dW,
                                              batch, ctx.conv_k, _DTYPES[Q.dtype], ctx.state, ctx.nbytes, scratch,
                                              scratch.numel(), torch.cuda.current_stream())
        if rc != _lib.NYS_OK:
            raise NystromError(rc, "nystrom_attn_bwd_from_state")
        return dQ, dK, dV, dW, None, None


class _NystromAttentionMasked(torch.autograd.Function):
    """Under a key-padding mask: forward nystrom_attn_fwd_masked, backward
    nystrom_attn_bwd_masked (which recomputes the landmark side)."""

    @staticmethod
    def forward(ctx, Q, K, V, conv_w, m, iters, lengths):
        _conv_k(conv_w, Q.shape[1], Q.shape[3])
        out = attention(Q, K, V, m, iters, conv_w=conv_w, lengths=lengths)
        ctx.save_for_backward(Q, K, V, conv_w, lengths)
        ctx.m, ctx.iters = m, iters
        return out

    @staticmethod
    @once_differentiable
    def backward(ctx, dO):
        Q, K, V, conv_w, lengths = ctx.saved_tensors
        batch, heads, n, d = Q.shape
        conv_k = _conv_k(conv_w, heads, d)
        dO = dO.to(Q.dtype).contiguous()
        dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
        dW = torch.empty_like(conv_w) if conv_w is not None and ctx.needs_input_grad[3] else None
        nbytes = _lib.nystrom_attn_bwd_workspace_bytes(batch, heads, n, d, ctx.m, ctx.iters, conv_k)
        if nbytes == 0:
            raise NystromError(_lib.NYS_EUNSUPPORTED, "nystrom_attn_bwd_workspace_bytes")
        ws = torch.empty(nbytes, dtype=torch.uint8, device=Q.device)
        rc = _lib.nystrom_attn_bwd_masked(Q, K, V, conv_w, dO, n, d, ctx.m, heads, ctx.iters, dQ, dK, dV, dW, batch,
                                          conv_k, _DTYPES[Q.dtype], lengths, ws, nbytes,
                                          torch.cuda.current_stream())
        if rc != _lib.NYS_OK:
            raise NystromError(rc, "nystrom_attn_bwd_masked")
        return dQ, dK, dV, dW, None, None, None


def attention_train(Q, K, V, m, iters=6, conv_w=None, lengths=None):
    """Nyström attention forward with autograd.  Q, K, V: [batch, heads, n, d]
    (fp32 or bf16, m <= 64); conv_w: fp32 [heads, d, k] (k <= 33) or None.
    Backpropagating through the result runs the library's exact backward
    pass from the state this forward kept (no recompute).  lengths: None, or
    a contiguous int32 GPU tensor [batch] of sequence lengths (key-padding
    mask, as for ``attention``); the backward then recomputes the landmark
    side, and the gradients of every pad row are zero."""
    if lengths is not None:
        return _NystromAttentionMasked.apply(Q, K, V, conv_w, m, iters, lengths)
    return _NystromAttention.apply(Q, K, V, conv_w, m, iters)


def dconv(V, conv_w, out=None, stream=None):
    """Depthwise-conv skip alone: out = DConv(V)."""
    _check_io(V)
    batch, heads, n, d = V.shape
    if out is None:
        out = torch.empty_like(V)
    if stream is None:
        stream = torch.cuda.current_stream()
    rc = _lib.nystrom_dconv_fwd(V, conv_w, n, d, heads, batch, conv_w.shape[2], _DTYPES[V.dtype], out, stream)
    if rc != _lib.NYS_OK:
        raise NystromError(rc, "nystrom_dconv_fwd")
    return out


def read_intermediate(workspace: torch.Tensor, which: int, batch, heads, n, d, m) -> torch.Tensor:
    """View of an fp32 intermediate (NYS_WS_*) inside a workspace after a call."""
    off = _lib.nystrom_attn_workspace_offset(which, batch, heads, n, d, m)
    if off < 0:
        raise NystromError(_lib.NYS_EINVAL, "workspace offset")
    cols = m if which in (_lib.NYS_WS_A, _lib.NYS_WS_Z) else d
    count = batch * heads * m * cols
    flat = workspace[off:off + 4 * count].view(torch.float32)
    return flat.view(batch, heads, m, cols)
