"""Helpers for the GPU tests: move seeded inputs to the device, run the HIP
path through the C ABI, bring results back as float32/float64 NumPy."""
from __future__ import annotations

import numpy as np

from efficient_transformer_attention_mean_amd import _lib
from efficient_transformer_attention_mean_amd.workloads import bf16_bits, bf16_bits_to_f32


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def to_dev(x, dtype: str):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()


def to_host(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f32(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    return t.float().cpu().numpy()


def dtype_code(dtype: str) -> int:
    return _lib.NYS_BF16 if dtype == "bf16" else _lib.NYS_F32


_UNSET = object()


def run_forward(inp, m, iters, dtype, use_conv=True, own_workspace=True, stream=None, lengths=_UNSET):
    """Run nystrom_attn_fwd on the seeded inputs, or nystrom_attn_fwd_masked
    when ``lengths`` is given (a sequence of per-entry lengths, or None for a
    NULL lengths pointer); returns (out, intermediates dict)."""
    import torch
    Q, K, V = (to_dev(inp[k], dtype) for k in ("Q", "K", "V"))
    B, H, n, d = inp["Q"].shape
    w = inp["conv_w"] if use_conv else None
    wdev = None if w is None else torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda()
    conv_k = 0 if w is None else w.shape[2]
    out = torch.empty_like(Q)
    ws = None
    nbytes = 0
    if own_workspace:
        nbytes = _lib.nystrom_attn_workspace_bytes(B, H, n, d, m)
        assert nbytes > 0
        ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream() if stream is None else stream
    if lengths is _UNSET:
        rc = _lib.nystrom_attn_fwd(Q, K, V, wdev, n, d, m, H, iters, out, B, conv_k, dtype_code(dtype), ws, nbytes,
                                   s)
    else:
        lens = None if lengths is None else torch.tensor(list(lengths), dtype=torch.int32, device="cuda")
        rc = _lib.nystrom_attn_fwd_masked(Q, K, V, wdev, n, d, m, H, iters, out, B, conv_k, dtype_code(dtype), lens,
                                          ws, nbytes, s)
    assert rc == _lib.NYS_OK, _lib.nystrom_strerror(rc)
    torch.cuda.synchronize()
    inter = {}
    if ws is not None:
        for name, which, cols in (("Qt", _lib.NYS_WS_QT, d), ("Kt", _lib.NYS_WS_KT, d), ("A", _lib.NYS_WS_A, m),
                                  ("Z", _lib.NYS_WS_Z, m), ("BV", _lib.NYS_WS_BV, d), ("W", _lib.NYS_WS_W, d)):
            off = _lib.nystrom_attn_workspace_offset(which, B, H, n, d, m)
            cnt = B * H * m * cols
            inter[name] = ws[off:off + 4 * cnt].view(torch.float32).view(B, H, m, cols).cpu().numpy()
    return to_host(out), inter
