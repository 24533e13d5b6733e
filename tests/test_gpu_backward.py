"""Parity of the HIP backward pass (through the C ABI) against the fp64 CPU
oracle of the gradients (itself pinned by finite differences).

Bars (relative L2 over each whole gradient tensor): 1e-4 for fp32 I/O and
2e-2 for bf16 I/O, the forward's output bars.  The bf16 path inherits the
forward's single-bf16 landmark-side products (B's row statistics and BV,
about 2^-9 relative) and rounds every gradient to bf16 (2^-9 relative), so
its error is of the order 1e-3; the fp32 path runs its n-sized passes in
fp32 and the pseudoinverse backward with three-way split products."""
import numpy as np
import pytest
import torch

from efficient_transformer_attention_mean_amd import _lib
from efficient_transformer_attention_mean_amd.workloads import WORKLOADS, make_inputs, round_to_bf16
from oracle import nystrom_attention_backward

from ._checks import Bars, Gate
from ._gpu_util import dtype_code, to_dev, to_host

pytestmark = pytest.mark.gpu

# Gradient gates (tests/_checks.py): relative L2 over each tensor and each
# (b, h) at the forward's output bars, the same per 64-row tile, and an
# elementwise bound.  bf16: each gradient is rounded to bf16 (<= 2^-9 |x|)
# after fp32 arithmetic with single-bf16 n-sized products, whose error is a
# few 1e-3 of the gradient's rms; fp32: ~1e-6 relative.
GRAD_BARS = {
    "f32": Bars(rel=1e-4, tile=1e-4, rtol=1e-4, atol=1e-4),
    "bf16": Bars(rel=2e-2, tile=2e-2, rtol=2.0 ** -7, atol=5e-2),
}
# The filter gradient is a sum over every row of the batch: no tiles.
DW_BARS = {
    "f32": Bars(rel=1e-4, tile=1e-4, rtol=1e-4, atol=1e-4),
    "bf16": Bars(rel=2e-2, tile=2e-2, rtol=2.0 ** -7, atol=5e-2),
}


def upstream(wl, seed):
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((wl.batch, wl.heads, wl.n, wl.d)).astype(np.float32)
    return round_to_bf16(g) if wl.dtype == "bf16" else g


def run_backward(inp, dO, m, iters, dtype, use_conv=True, own_workspace=True, want_dw=True, lengths=False):
    """lengths: False = nystrom_attn_bwd; None or a sequence = nystrom_attn_bwd_masked
    with no lengths or those lengths."""
    Q, K, V, G = (to_dev(x, dtype) for x in (inp["Q"], inp["K"], inp["V"], dO))
    B, H, n, d = inp["Q"].shape
    w = inp["conv_w"] if use_conv else None
    wdev = None if w is None else torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda()
    conv_k = 0 if w is None else w.shape[2]
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    dW = None if (w is None or not want_dw) else torch.full_like(wdev, 7.0)
    ws, nbytes = None, 0
    if own_workspace:
        nbytes = _lib.nystrom_attn_bwd_workspace_bytes(B, H, n, d, m, iters, conv_k)
        assert nbytes > 0
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    if lengths is False:
        rc = _lib.nystrom_attn_bwd(Q, K, V, wdev, G, n, d, m, H, iters, dQ, dK, dV, dW, B, conv_k,
                                   dtype_code(dtype), ws, nbytes, torch.cuda.current_stream())
    else:
        lens = None if lengths is None else torch.tensor(list(lengths), dtype=torch.int32, device="cuda")
        rc = _lib.nystrom_attn_bwd_masked(Q, K, V, wdev, G, n, d, m, H, iters, dQ, dK, dV, dW, B, conv_k,
                                          dtype_code(dtype), lens, ws, nbytes, torch.cuda.current_stream())
    assert rc == _lib.NYS_OK, _lib.nystrom_strerror(rc)
    torch.cuda.synchronize()
    return to_host(dQ), to_host(dK), to_host(dV), None if dW is None else dW.cpu().numpy()


CASES = [
    # (batch, heads, n, d, m, iters, conv_k, dtype)
    (1, 1, 64, 16, 8, 6, 3, "f32"),
    (2, 2, 100, 16, 10, 6, 5, "bf16"),      # ragged n: padded segments
    (1, 2, 256, 32, 32, 6, 33, "f32"),
    (2, 2, 1000, 64, 64, 6, 33, "bf16"),    # one segment of pad only
    (1, 1, 96, 128, 16, 6, 0, "f32"),       # d = 128, no skip
    (1, 2, 512, 64, 64, 0, 9, "f32"),       # iters = 0: the start only
    (1, 1, 64, 32, 64, 8, 3, "f32"),        # m = n
    (2, 12, 512, 64, 64, 6, 33, "f32"),     # BERT-base-shaped layer
    (1, 3, 777, 32, 48, 6, 33, "bf16"),     # m = 48 (padded to 64), ragged
    (2, 12, 8192, 64, 64, 6, 33, "bf16"),   # headline shape
    (1, 2, 512, 64, 64, 6, 0, "bf16"),      # matrix-core path without the skip
    (2, 2, 300, 32, 16, 6, 1, "bf16"),      # matrix-core path, one-tap skip, ragged n
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}H{c[1]}n{c[2]}d{c[3]}m{c[4]}it{c[5]}k{c[6]}{c[7]}"
                                             for c in CASES])
def test_backward_parity(case):
    B, H, n, d, m, iters, k, dt = case
    wl = WORKLOADS["tiny"].with_(name=f"bwd{case}", batch=B, heads=H, n=n, d=d, m=m, iters=iters, conv_k=k,
                                 dtype=dt, seed=300 + n + m)
    inp = make_inputs(wl)
    dO = upstream(wl, 900 + n)
    ref = nystrom_attention_backward(inp["Q"], inp["K"], inp["V"], m, iters, dO, inp["conv_w"])
    got = run_backward(inp, dO, m, iters, dt, use_conv=k > 0)
    g = Gate(f"backward {case}")
    for nm, x, r in zip(("dQ", "dK", "dV"), got, ref):
        g(nm, x, r, GRAD_BARS[dt])
    if ref[3] is not None:
        g("dconv_w", got[3], ref[3], DW_BARS[dt])
    g.close()


# One-token sequences (fp32): largest absolute error against the rms gradient
# of the batch's other entries.
ONE_TOKEN_TOL = {"f32": 1e-4}

MASKED = [
    # (batch, heads, n, d, m, iters, conv_k, dtype, lengths)
    (3, 2, 300, 64, 16, 6, 33, "bf16", (300, 173, 40)),      # matrix-core path
    (2, 2, 1000, 32, 64, 6, 33, "f32", (1000, 517)),
    (4, 1, 256, 16, 8, 6, 5, "f32", (3, 999, 129, 64)),      # 3 < m; 999 clamped to n
    (4, 2, 512, 64, 64, 6, 33, "bf16", (0, 17, 63, 512)),    # empty, and two sequences shorter than m
    (2, 2, 4096, 32, 32, 6, 0, "bf16", (2, 4096)),           # matrix-core d = 32, no skip, two tokens
    (3, 2, 1024, 32, 32, 6, 3, "f32", (1, 2, 1000)),         # one and two tokens
    (2, 2, 300, 128, 16, 6, 9, "bf16", (300, 100)),          # bf16 on the vector path
    (2, 12, 8192, 64, 64, 6, 33, "bf16", (8192, 5000)),      # headline shape, one entry padded
]


@pytest.mark.parametrize("case", MASKED, ids=[f"B{c[0]}H{c[1]}n{c[2]}d{c[3]}m{c[4]}k{c[6]}{c[7]}L{'-'.join(map(str, c[8]))}"
                                              for c in MASKED])
def test_masked_backward_parity(case):
    """Gradients under a key-padding mask against the masked oracle, with NaN
    in every pad row of Q, K, V and dO (never read); pad rows of dQ, dK and
    dV must be exactly zero.

    A one-token sequence is gated in fp32, against the gradient scale of the
    batch's other entries instead of its own: its landmarks are the token and
    m - 1 zero vectors, so A~ is singular (m - 1 equal rows) and the output
    hardly depends on the token's q and k.  Its dQ and dK are a remainder of
    about 1e-3 of the terms the softmax backward of A~ sums (the oracle gives
    |dA| ~ 9 against |dS_A| ~ 0.01 and |dQ| ~ 2e-3), so rounding is a large
    share of so small a result.  In bf16 it is larger still: with one key
    every row of B~ is exactly 1 and dS_B is exactly 0, but the backward's
    single-bf16 scores differ from the forward's row statistics by 2^-8,
    which leaves B~ = 1 + O(2^-8) and a dS_B of that order; the bf16 cases
    start at two tokens."""
    B, H, n, d, m, iters, k, dt, lengths = case
    wl = WORKLOADS["tiny"].with_(name=f"bwd_masked{case}", batch=B, heads=H, n=n, d=d, m=m, iters=iters, conv_k=k,
                                 dtype=dt, seed=400 + n + m)
    inp = dict(make_inputs(wl))
    dO = np.array(upstream(wl, 700 + n), copy=True)
    eff = [min(max(L, 0), n) for L in lengths]
    for key in ("Q", "K", "V"):
        x = np.array(inp[key], copy=True)
        for b, L in enumerate(eff):
            x[b, :, L:] = np.nan
        inp[key] = x
    for b, L in enumerate(eff):
        dO[b, :, L:] = np.nan
    ref = nystrom_attention_backward(inp["Q"], inp["K"], inp["V"], m, iters, dO, inp["conv_w"], lengths=lengths)
    got = run_backward(inp, dO, m, iters, dt, use_conv=k > 0, lengths=lengths)
    for x in got[:3]:
        for b, L in enumerate(eff):
            assert np.all(x[b, :, L:] == 0.0), b
    one = [b for b, L in enumerate(eff) if L == 1]
    rest = [b for b in range(B) if b not in one]
    rows = np.arange(n)[None, :] < np.array([eff[b] for b in rest])[:, None]  # live rows of `rest`
    g = Gate(f"masked backward {case}")
    for nm, x, r in zip(("dQ", "dK", "dV"), got, ref):
        g(nm, x[rest], r[rest], GRAD_BARS[dt])
        if one:
            scale = float(np.sqrt(np.mean(r[rest].transpose(0, 2, 1, 3)[rows] ** 2)))
            err = float(np.max(np.abs(x[one] - r[one])))
            assert err <= ONE_TOKEN_TOL[dt] * scale, (nm, err, scale)
    if ref[3] is not None:
        g("dconv_w", got[3], ref[3], DW_BARS[dt])
    g.close()


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_masked_backward_full_lengths_equal_unmasked_bitwise(dt):
    wl = WORKLOADS["long"].with_(name=f"bwd_masked_full_{dt}", batch=2, heads=3, n=1500, dtype=dt)
    inp = make_inputs(wl)
    dO = upstream(wl, 23)
    a = run_backward(inp, dO, wl.m, wl.iters, dt)
    b = run_backward(inp, dO, wl.m, wl.iters, dt, lengths=None)
    c = run_backward(inp, dO, wl.m, wl.iters, dt, lengths=(1500, 1500))
    for x, y, z in zip(a, b, c):
        assert np.array_equal(x, y) and np.array_equal(x, z)


def test_backward_deterministic_and_workspace_forms():
    wl = WORKLOADS["long"].with_(name="bwd_det", batch=1, heads=3, n=1500)
    inp = make_inputs(wl)
    dO = upstream(wl, 5)
    a = run_backward(inp, dO, wl.m, wl.iters, wl.dtype)
    b = run_backward(inp, dO, wl.m, wl.iters, wl.dtype, own_workspace=False)
    c = run_backward(inp, dO, wl.m, wl.iters, wl.dtype, want_dw=False)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    for x, y in zip(a[:3], c[:3]):
        assert np.array_equal(x, y)
    assert c[3] is None


def test_backward_rejects_unsupported():
    Q = torch.zeros(1, 1, 128, 16, device="cuda")
    out = torch.empty_like(Q)
    # m > 64 is outside the backward kernels; the forward accepts it.
    rc = _lib.nystrom_attn_bwd(Q, Q, Q, None, Q, 128, 16, 80, 1, 6, out, out, out, None, 1, 0, _lib.NYS_F32,
                               None, 0, None)
    assert rc == _lib.NYS_EUNSUPPORTED
    assert _lib.nystrom_attn_bwd_workspace_bytes(1, 1, 128, 16, 80, 6, 0) == 0


def test_backward_two_host_threads():
    """Two host threads call the bf16 d = 64 backward at once, each on its own
    stream with its own buffers.  The library shares one side stream per
    device between them, and enqueues each call's fork and join under a lock.
    Every result must equal the single-thread result bit for bit."""
    import threading

    wl = WORKLOADS["headline"].with_(name="bwd_threads", batch=1, heads=2, n=2048)
    inp = make_inputs(wl)
    dO = upstream(wl, 17)
    ref = run_backward(inp, dO, wl.m, wl.iters, wl.dtype)
    nbytes = _lib.nystrom_attn_bwd_workspace_bytes(wl.batch, wl.heads, wl.n, wl.d, wl.m, wl.iters, wl.conv_k)
    results, errors = {}, []

    def worker(tid):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                Q, K, V, G = (to_dev(x, wl.dtype) for x in (inp["Q"], inp["K"], inp["V"], dO))
                w = torch.from_numpy(np.ascontiguousarray(inp["conv_w"], np.float32)).cuda()
                dQ, dK, dV, dW = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V), torch.empty_like(w)
                ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
                outs = []
                for _ in range(4):
                    rc = _lib.nystrom_attn_bwd(Q, K, V, w, G, wl.n, wl.d, wl.m, wl.heads, wl.iters, dQ, dK, dV, dW,
                                               wl.batch, wl.conv_k, dtype_code(wl.dtype), ws, nbytes, stream)
                    assert rc == _lib.NYS_OK, _lib.nystrom_strerror(rc)
                    stream.synchronize()
                    outs.append((to_host(dQ), to_host(dK), to_host(dV), dW.cpu().numpy()))
                results[tid] = outs
        except Exception as exc:  # reported by the main thread
            errors.append(repr(exc))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=90)
    assert not errors, errors
    assert sorted(results) == [0, 1]
    for outs in results.values():
        for got in outs:
            for x, y in zip(got, ref):
                assert np.array_equal(x, y)


@pytest.mark.parametrize("case", [(2, 2, 1000, 64, 64, 6, 33, "bf16"), (1, 2, 256, 32, 32, 6, 33, "f32")],
                         ids=["bf16_d64", "f32_d32"])
def test_saved_forward_pair_matches_plain_calls(case):
    """nystrom_attn_fwd_save + nystrom_attn_bwd_saved give the plain forward's
    output and the plain backward's gradients bit for bit (the same kernels
    on the same data; the backward only skips recomputing the forward's
    landmark side), also when the backward runs twice on one saved forward."""
    from ._gpu_util import run_forward

    B, H, n, d, m, iters, k, dt = case
    wl = WORKLOADS["tiny"].with_(name="saved", batch=B, heads=H, n=n, d=d, m=m, iters=iters, conv_k=k, dtype=dt,
                                 seed=41)
    inp = make_inputs(wl)
    dO = upstream(wl, 43)
    ref_grads = run_backward(inp, dO, m, iters, dt)
    ref_out = run_forward(inp, m, iters, dt)[0]

    Q, K, V, G = (to_dev(x, dt) for x in (inp["Q"], inp["K"], inp["V"], dO))
    w = torch.from_numpy(np.ascontiguousarray(inp["conv_w"], np.float32)).cuda()
    O = torch.empty_like(Q)
    dQ, dK, dV, dW = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V), torch.empty_like(w)
    nbytes = _lib.nystrom_attn_bwd_workspace_bytes(B, H, n, d, m, iters, k)
    saved = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream()
    rc = _lib.nystrom_attn_fwd_save(Q, K, V, w, n, d, m, H, iters, O, B, k, dtype_code(dt), saved, nbytes, st)
    assert rc == _lib.NYS_OK, _lib.nystrom_strerror(rc)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(O), ref_out)
    for _ in range(2):
        for t in (dQ, dK, dV, dW):
            t.fill_(float("nan"))
        rc = _lib.nystrom_attn_bwd_saved(Q, K, V, w, G, n, d, m, H, iters, dQ, dK, dV, dW, B, k, dtype_code(dt),
                                         saved, nbytes, st)
        assert rc == _lib.NYS_OK, _lib.nystrom_strerror(rc)
        torch.cuda.synchronize()
        got = (to_host(dQ), to_host(dK), to_host(dV), dW.cpu().numpy())
        for x, y in zip(got, ref_grads):
            assert np.array_equal(x, y)

    # The state alone (a buffer of exactly its size) and the scratch apart,
    # given by the caller or allocated by the library: the same bits.
    sbytes = _lib.nystrom_attn_bwd_state_bytes(B, H, n, d, m, iters, k)
    state = torch.empty(sbytes, dtype=torch.uint8, device="cuda")
    rc = _lib.nystrom_attn_fwd_save(Q, K, V, w, n, d, m, H, iters, O, B, k, dtype_code(dt), state, sbytes, st)
    assert rc == _lib.NYS_OK, _lib.nystrom_strerror(rc)
    scratch = torch.empty(nbytes - sbytes, dtype=torch.uint8, device="cuda")
    for sc in (scratch, None):
        for t in (dQ, dK, dV, dW):
            t.fill_(float("nan"))
        rc = _lib.nystrom_attn_bwd_from_state(Q, K, V, w, G, n, d, m, H, iters, dQ, dK, dV, dW, B, k,
                                              dtype_code(dt), state, sbytes, sc, 0 if sc is None else sc.numel(), st)
        assert rc == _lib.NYS_OK, _lib.nystrom_strerror(rc)
        torch.cuda.synchronize()
        got = (to_host(dQ), to_host(dK), to_host(dV), dW.cpu().numpy())
        for x, y in zip(got, ref_grads):
            assert np.array_equal(x, y)


def test_attention_train_autograd_matches_plain_backward():
    """api.attention_train under torch autograd: the output equals the plain
    forward and the gradients equal nystrom_attn_bwd, bit for bit."""
    from efficient_transformer_attention_mean_amd import api
    from ._gpu_util import run_forward

    wl = WORKLOADS["tiny"].with_(name="autograd", batch=2, heads=2, n=1000, d=64, m=64, iters=6, conv_k=33,
                                 dtype="bf16", seed=51)
    inp = make_inputs(wl)
    dO = upstream(wl, 53)
    ref_grads = run_backward(inp, dO, wl.m, wl.iters, wl.dtype)
    ref_out = run_forward(inp, wl.m, wl.iters, wl.dtype)[0]
    Q, K, V = (to_dev(inp[k], wl.dtype).requires_grad_() for k in ("Q", "K", "V"))
    w = torch.from_numpy(np.ascontiguousarray(inp["conv_w"], np.float32)).cuda().requires_grad_()
    out = api.attention_train(Q, K, V, wl.m, wl.iters, conv_w=w)
    out.backward(to_dev(dO, wl.dtype))
    torch.cuda.synchronize()
    assert np.array_equal(to_host(out.detach()), ref_out)
    got = (to_host(Q.grad), to_host(K.grad), to_host(V.grad), w.grad.cpu().numpy())
    for x, y in zip(got, ref_grads):
        assert np.array_equal(x, y)


def test_attention_train_masked_matches_masked_calls():
    """api.attention_train with lengths: the output equals
    nystrom_attn_fwd_masked and the gradients equal nystrom_attn_bwd_masked,
    bit for bit; pad rows of every gradient are zero."""
    from efficient_transformer_attention_mean_amd import api
    from ._gpu_util import run_forward

    lengths = (1000, 357)
    wl = WORKLOADS["tiny"].with_(name="autograd_masked", batch=2, heads=2, n=1000, d=64, m=64, iters=6, conv_k=33,
                                 dtype="bf16", seed=57)
    inp = make_inputs(wl)
    dO = upstream(wl, 59)
    ref_grads = run_backward(inp, dO, wl.m, wl.iters, wl.dtype, lengths=lengths)
    ref_out = run_forward(inp, wl.m, wl.iters, wl.dtype, lengths=lengths)[0]
    Q, K, V = (to_dev(inp[k], wl.dtype).requires_grad_() for k in ("Q", "K", "V"))
    w = torch.from_numpy(np.ascontiguousarray(inp["conv_w"], np.float32)).cuda().requires_grad_()
    lens = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    out = api.attention_train(Q, K, V, wl.m, wl.iters, conv_w=w, lengths=lens)
    out.backward(to_dev(dO, wl.dtype))
    torch.cuda.synchronize()
    assert np.array_equal(to_host(out.detach()), ref_out)
    got = (to_host(Q.grad), to_host(K.grad), to_host(V.grad), w.grad.cpu().numpy())
    for x, y in zip(got, ref_grads):
        assert np.array_equal(x, y)
    assert np.all(got[0][1, :, 357:] == 0.0)


def test_attention_train_rejects_second_derivatives():
    """The gradients are computed by the library outside autograd; asking for
    a derivative of them (create_graph=True, then backward through the
    gradient) must raise, not return a silently incomplete result."""
    from efficient_transformer_attention_mean_amd import api

    wl = WORKLOADS["tiny"].with_(name="twice", batch=1, heads=1, n=128, d=32, m=16, conv_k=0, dtype="f32", seed=3)
    inp = make_inputs(wl)
    Q, K, V = (to_dev(inp[k], wl.dtype).requires_grad_() for k in ("Q", "K", "V"))
    out = api.attention_train(Q, K, V, wl.m, wl.iters)
    (gq,) = torch.autograd.grad(out.square().sum(), Q, create_graph=True)
    with pytest.raises(RuntimeError):
        gq.sum().backward()
