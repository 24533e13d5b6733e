"""Graph capture of the forward and backward calls through the C ABI.

One call is captured into a HIP graph (torch.cuda.graph) and replayed three
times; between replays the outputs are overwritten with NaN by an eager fill
kernel.  Every replay must reproduce the eager call's outputs bit for bit.
The bf16 backward at d = 64 forks part of its work onto the library's second
stream and joins it back by events, and the capture has to follow that fork."""
import numpy as np
import pytest
import torch

from efficient_transformer_attention_mean_amd import _lib
from efficient_transformer_attention_mean_amd.workloads import WORKLOADS, make_inputs

from ._gpu_util import dtype_code, to_dev
from .test_gpu_backward import upstream

pytestmark = pytest.mark.gpu

# Headline layout (bf16, d = 64, m = 64, conv 33) at a size that captures quickly.
WL = WORKLOADS["headline"].with_(name="graph", batch=1, heads=2, n=2048)


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _check_graph(call, outs):
    assert call() == _lib.NYS_OK
    torch.cuda.synchronize()
    ref = [_bits(o).clone() for o in outs]
    # Warm-up on another stream before capture, then capture on torch's
    # capture stream (the current stream inside the context).
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        assert call() == _lib.NYS_OK
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rc = call()
    assert rc == _lib.NYS_OK
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(_bits(o), r), f"replay {rep} differs from the eager call"


def _inputs():
    inp = make_inputs(WL)
    Q, K, V = (to_dev(inp[k], WL.dtype) for k in ("Q", "K", "V"))
    w = torch.from_numpy(np.ascontiguousarray(inp["conv_w"], np.float32)).cuda()
    return inp, Q, K, V, w


def test_forward_graph_replay():
    _, Q, K, V, w = _inputs()
    O = torch.empty_like(Q)
    nbytes = _lib.nystrom_attn_workspace_bytes(WL.batch, WL.heads, WL.n, WL.d, WL.m)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def call():
        return _lib.nystrom_attn_fwd(Q, K, V, w, WL.n, WL.d, WL.m, WL.heads, WL.iters, O, WL.batch, WL.conv_k,
                                     dtype_code(WL.dtype), ws, nbytes, torch.cuda.current_stream())

    _check_graph(call, [O])


def test_backward_graph_replay():
    inp, Q, K, V, w = _inputs()
    G = to_dev(upstream(WL, 11), WL.dtype)
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    dW = torch.empty_like(w)
    nbytes = _lib.nystrom_attn_bwd_workspace_bytes(WL.batch, WL.heads, WL.n, WL.d, WL.m, WL.iters, WL.conv_k)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def call():
        return _lib.nystrom_attn_bwd(Q, K, V, w, G, WL.n, WL.d, WL.m, WL.heads, WL.iters, dQ, dK, dV, dW, WL.batch,
                                     WL.conv_k, dtype_code(WL.dtype), ws, nbytes, torch.cuda.current_stream())

    _check_graph(call, [dQ, dK, dV, dW])
