"""Parity of the HIP path (through the C ABI) against the fp64 CPU oracle.

Every comparison gates four figures (tests/_checks.py): relative L2 over the
whole tensor and over each (b, h), per 64-row tile, and an elementwise bound.
Output bars: relative L2 <= 1e-4 for fp32 I/O and <= 2e-2 for bf16 I/O (the
method's stated tolerances), the same per tile; intermediates to the bars in
INTER_BARS, derived from the arithmetic each one goes through.  Every
workload is compared in full (the oracle finishes each in seconds), with the
conv skip and without it (attention-only), so the skip cannot hide attention
errors."""
import numpy as np
import pytest

from efficient_transformer_attention_mean_amd import _lib
from efficient_transformer_attention_mean_amd.workloads import WORKLOADS, make_inputs
from oracle import depthwise_conv_skip, exact_attention, nystrom_attention

from ._checks import OUT_BARS, Bars, Gate
from ._gpu_util import dtype_code, rel_l2, run_forward, to_dev, to_host

pytestmark = pytest.mark.gpu


def _bars(rel, elem):
    return Bars(rel=rel, tile=rel, rtol=elem, atol=elem)


# Intermediate gates.  Each is about three times the largest value measured
# over every parity case of this file (relative L2 per tensor, per (b, h) and
# per tile; the elementwise bound |d| <= e (|ref| + rms(ref)) about twice the
# largest measured ratio), with the arithmetic that sets the measured size:
#  Qt, Kt: fp32 sums of exact inputs (measured <= 9e-8 fp32 I/O, 3e-8 bf16).
#  A: scores from split-bf16 matrix-core products (fp32-grade for fp32 I/O,
#     bf16x3 ~2^-17 for bf16 I/O) then an fp32 softmax (<= 2.4e-7 / 1.8e-6).
#  Z: 4 products per iteration; errors in the directions of small singular
#     values of A grow by up to 13/4 per step (the slope of the iteration map
#     at 0): <= 6.1e-6 (three-way split) / 1.3e-3 (bf16x3).
#  BV: fp32 I/O: split-fp32 products (<= 6.5e-6).  bf16 I/O: single bf16
#     products with fp32 accumulation, as in bf16 attention kernels: every
#     probability is rounded to bf16 (relative error <= 2^-9, RMS
#     2^-9/sqrt(3) ~ 1.1e-3), and the weighted average of V keeps that
#     relative size (<= 2.1e-3, gate 5e-3).
#  W = Z BV: sums with cancellation (|Z| entries up to ~300 when A is
#     ill-conditioned), so it inherits BV's and Z's errors times that growth
#     (fp32 I/O: <= 2.4e-4 at m = n with 30 iterations, where Z is close to
#     the inverse of an ill-conditioned A, elementwise 1.5 e with e = 8e-4;
#     bf16: <= 8.5e-3 at the stress shape, gate 2e-2).
INTER_BARS = {
    "f32": {"Qt": _bars(3e-7, 1e-6), "Kt": _bars(3e-7, 1e-6), "A": _bars(1e-6, 2e-6), "Z": _bars(2e-5, 3e-5),
            "BV": _bars(2e-5, 4e-5), "W": _bars(7e-4, 3e-3)},
    "bf16": {"Qt": _bars(1e-7, 2e-7), "Kt": _bars(1e-7, 2e-7), "A": _bars(6e-6, 2e-5), "Z": _bars(4e-3, 7e-3),
             "BV": _bars(5e-3, 1.5e-2), "W": _bars(2e-2, 6e-2)},
}

_cache = {}


def oracle_for(wl):
    if wl.name not in _cache:
        inp = make_inputs(wl)
        O, inter = nystrom_attention(inp["Q"], inp["K"], inp["V"], wl.m, wl.iters, inp["conv_w"],
                                     with_intermediates=True)
        _cache[wl.name] = (inp, O, inter)
    return _cache[wl.name]


def gate_forward(title, inp, O, inter, m, iters, dt, use_conv=True, lengths=None, live=None):
    """Run the forward with and without the skip and gate the output, the
    attention-only output and every documented intermediate.  ``live``: batch
    entries whose intermediates are defined (all by default)."""
    kw = {} if lengths is None else {"lengths": lengths}
    out, got = run_forward(inp, m, iters, dt, use_conv=use_conv, **kw)
    out_att, _ = run_forward(inp, m, iters, dt, use_conv=False, **kw)
    g = Gate(title)
    g("out", out, O, OUT_BARS[dt])
    g("out_att_only", out_att, inter["O_att"], OUT_BARS[dt])
    sel = slice(None) if live is None else live
    for k, bars in INTER_BARS[dt].items():
        g(k, got[k][sel], inter[k][sel], bars)
    return out, g.close()


def check(wl):
    inp, O, inter = oracle_for(wl)
    return gate_forward(wl.name, inp, O, inter, wl.m, wl.iters, wl.dtype)[1]


@pytest.mark.parametrize("name", ["tiny", "bert", "long", "headline", "headline_ragged", "headline_m32", "stress"])
def test_workload_parity(name):
    check(WORKLOADS[name])


def test_m_equals_n_matches_exact_attention():
    # m = n with a converged pseudoinverse: the method is exact attention (Lemma 2).
    wl = WORKLOADS["tiny_m_eq_n"]
    errs = check(wl)
    inp = oracle_for(wl)[0]
    out, _ = run_forward(inp, wl.m, wl.iters, wl.dtype, use_conv=False)
    ex = exact_attention(inp["Q"], inp["K"], inp["V"])
    assert rel_l2(out, ex) <= 1e-4, errs


EDGE = [
    # (batch, heads, n, d, m, iters, conv_k, dtype)
    (1, 1, 96, 32, 12, 6, 3, "f32"),      # n not a multiple of the 64-row tile
    (2, 3, 100, 16, 10, 6, 5, "bf16"),    # ragged n, m = 10, d = 16
    (1, 2, 48, 64, 3, 6, 0, "f32"),       # odd m, no skip
    (1, 1, 64, 128, 1, 6, 1, "bf16"),     # m = 1 (rank one), k = 1
    (1, 1, 640, 64, 80, 6, 33, "f32"),    # m > 64: global pseudoinverse path, m not a multiple of 32
    (1, 2, 512, 32, 256, 8, 9, "bf16"),   # m = 256, segment length 2
    (1, 1, 256, 64, 128, 6, 33, "f32"),   # m = 128
    (2, 2, 128, 16, 32, 0, 7, "f32"),     # iters = 0: Z is the start Z0
    (1, 1, 16, 16, 16, 30, 3, "f32"),     # m = n, tiny
    (1, 1, 33, 16, 33, 30, 0, "f32"),     # m = n = 33, odd
    (3, 1, 200, 64, 40, 6, 33, "bf16"),   # conv halo wider than the ragged tail
    (1, 2, 256, 128, 64, 6, 33, "f32"),   # d = 128
    (1, 2, 256, 32, 64, 6, 33, "bf16"),   # d = 32
    (1, 1, 4096, 64, 64, 6, 33, "f32"),   # many key chunks in fp32
    (2, 2, 222, 64, 6, 6, 33, "bf16"),    # n = 2 mod 4: the last group of 4 staged rows crosses the head's end
    (1, 3, 134, 32, 2, 6, 33, "f32"),     # the same with fp32 rows
    # n not a multiple of m: zero pad to m*ceil(n/m), pad keys masked
    (2, 2, 100, 16, 8, 6, 5, "f32"),      # l = 13, last segment 9 real rows
    (1, 2, 1000, 64, 64, 6, 33, "bf16"),  # l = 16, one segment of pad only
    (1, 1, 203, 32, 10, 6, 7, "f32"),     # l = 21, 14 real rows in the last segment
    (1, 2, 777, 128, 96, 8, 33, "f32"),   # m > 64 path, l = 9
    (1, 1, 500, 32, 75, 6, 5, "f32"),     # m > 64 path, m odd: rows not 16-byte aligned
    (2, 1, 600, 64, 130, 7, 33, "bf16"),  # m > 64 path, three 64-landmark tiles, m = 2 mod 4
    (1, 1, 300, 16, 70, 0, 0, "f32"),     # m > 64 path, iters = 0: Z is the start Z0
    (2, 3, 8191, 64, 64, 6, 33, "bf16"),  # headline shape less one row
    (1, 2, 4097, 64, 32, 6, 33, "f32"),   # one real row in the last segment
    (1, 1, 130, 32, 64, 6, 3, "bf16"),    # l = 3: 20 segments of pad only (equal rows in A)
]


@pytest.mark.parametrize("case", EDGE, ids=[f"B{c[0]}H{c[1]}n{c[2]}d{c[3]}m{c[4]}it{c[5]}k{c[6]}{c[7]}" for c in EDGE])
def test_edge_parity(case):
    B, H, n, d, m, iters, k, dt = case
    wl = WORKLOADS["tiny"].with_(name=f"edge{case}", batch=B, heads=H, n=n, d=d, m=m, iters=iters, conv_k=k,
                                 dtype=dt, seed=100 + n + m)
    check(wl)


def test_determinism_bitwise():
    wl = WORKLOADS["long"].with_(name="det", batch=1, heads=4, n=2048)
    inp = make_inputs(wl)
    a, ia = run_forward(inp, wl.m, wl.iters, wl.dtype)
    b, ib = run_forward(inp, wl.m, wl.iters, wl.dtype)
    assert np.array_equal(a, b)
    for k in ia:
        assert np.array_equal(ia[k], ib[k]), k


def test_null_workspace_matches_caller_workspace():
    wl = WORKLOADS["long"].with_(name="nullws", batch=1, heads=2, n=1024)
    inp = make_inputs(wl)
    a, _ = run_forward(inp, wl.m, wl.iters, wl.dtype, own_workspace=True)
    b, _ = run_forward(inp, wl.m, wl.iters, wl.dtype, own_workspace=False)
    assert np.array_equal(a, b)


def test_side_stream():
    import torch
    wl = WORKLOADS["bert"].with_(name="stream", batch=1, heads=3)
    inp, O, _ = oracle_for(wl)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out, _ = run_forward(inp, wl.m, wl.iters, wl.dtype, stream=s)
    g = Gate("side stream")
    g("out", out, O, OUT_BARS["f32"])
    g.close()


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n,d,k", [(100, 16, 1), (257, 64, 33), (64, 128, 5), (1000, 32, 33)])
def test_dconv_standalone(dt, n, d, k):
    import torch
    rng = np.random.default_rng(n + d + k)
    from efficient_transformer_attention_mean_amd.workloads import round_to_bf16
    B, H = 2, 3
    V = rng.standard_normal((B, H, n, d)).astype(np.float32)
    if dt == "bf16":
        V = round_to_bf16(V)
    w = rng.normal(0, 0.5, (H, d, k)).astype(np.float32)
    Vd = to_dev(V, dt)
    out = torch.empty_like(Vd)
    wd = torch.from_numpy(w).cuda()
    rc = _lib.nystrom_dconv_fwd(Vd, wd, n, d, H, B, k, dtype_code(dt), out, torch.cuda.current_stream())
    assert rc == 0
    torch.cuda.synchronize()
    ref = np.stack([np.stack([depthwise_conv_skip(V[b, h], w[h]) for h in range(H)]) for b in range(B)])
    # fp32: fp32 FMAs (~1e-7); bf16: taps split hi/lo (~2^-17), then the
    # output rounded to bf16 (<= 2^-9 |x| per element).
    bars = Bars(rel=1e-6, tile=1e-6, rtol=1e-6, atol=1e-6) if dt == "f32" else \
        Bars(rel=8e-3, tile=8e-3, rtol=2.0 ** -8, atol=1e-4)
    g = Gate(f"dconv {dt} n={n} d={d} k={k}")
    g("out", to_host(out), ref, bars)
    g.close()


def test_invalid_calls_leave_output_untouched():
    import torch
    Q = torch.randn(1, 1, 64, 16, device="cuda")
    out = torch.full_like(Q, 7.0)
    for kw, code in ((dict(m=65), _lib.NYS_EINVAL), (dict(d=24), _lib.NYS_EUNSUPPORTED)):
        args = dict(n=64, d=16, m=8)
        args.update(kw)
        rc = _lib.nystrom_attn_fwd(Q, Q, Q, None, args["n"], args["d"], args["m"], 1, 6, out, 1, 0, _lib.NYS_F32,
                                   None, 0, None)
        assert rc == code
    ws = torch.zeros(8, dtype=torch.uint8, device="cuda")
    rc = _lib.nystrom_attn_fwd(Q, Q, Q, None, 64, 16, 8, 1, 6, out, 1, 0, _lib.NYS_F32, ws, 8, None)
    assert rc == _lib.NYS_EWORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


# Key-padding mask: a batch of right-padded sequences, one length per entry.
# Every row at or past an entry's length in Q, K and V is filled with NaN, so
# any read of them would show in the output; the output's pad rows must come
# back exactly zero.
MASKED = [
    # (batch, heads, n, d, m, iters, conv_k, dtype, lengths)
    (3, 2, 300, 64, 16, 6, 33, "bf16", (300, 173, 40)),
    (2, 2, 1000, 32, 64, 6, 33, "f32", (1000, 517)),
    (4, 1, 256, 16, 8, 6, 5, "f32", (3, 999, 129, 64)),      # 3 < m: landmarks of pad; 999 clamped to n
    (2, 3, 640, 128, 80, 6, 33, "f32", (640, 333)),          # m > 64 path
    (2, 12, 8192, 64, 64, 6, 33, "bf16", (8192, 5000)),      # headline shape, one entry padded
    (2, 2, 4096, 64, 32, 6, 0, "bf16", (1, 4096)),           # no skip; a one-token sequence
    (4, 2, 512, 64, 64, 6, 33, "bf16", (0, 17, 63, 512)),    # empty, and two sequences shorter than m
    (3, 1, 300, 128, 96, 8, 9, "f32", (95, 0, 300)),         # m > 64 path, shorter than m, empty
    (2, 2, 1500, 128, 256, 8, 33, "bf16", (1500, 700)),      # stress layout: 16-wave key pass, 12-wave output stage
    (3, 1, 600, 128, 256, 8, 33, "bf16", (600, 200, 0)),     # the same, shorter than m, empty
]


@pytest.mark.parametrize("case", MASKED, ids=[f"B{c[0]}H{c[1]}n{c[2]}d{c[3]}m{c[4]}k{c[6]}{c[7]}L{'-'.join(map(str, c[8]))}"
                                              for c in MASKED])
def test_masked_parity(case):
    B, H, n, d, m, iters, k, dt, lengths = case
    wl = WORKLOADS["tiny"].with_(name=f"masked{case}", batch=B, heads=H, n=n, d=d, m=m, iters=iters, conv_k=k,
                                 dtype=dt, seed=200 + n + m)
    inp = dict(make_inputs(wl))
    eff = [min(max(L, 0), n) for L in lengths]
    for key in ("Q", "K", "V"):
        x = np.array(inp[key], copy=True)
        for b, L in enumerate(eff):
            x[b, :, L:] = np.nan
        inp[key] = x
    O, inter = nystrom_attention(inp["Q"], inp["K"], inp["V"], m, iters, inp["conv_w"], with_intermediates=True,
                                 lengths=lengths)
    live = [b for b, L in enumerate(eff) if L > 0]
    out, _ = gate_forward(f"masked {case}", inp, O, inter, m, iters, dt, use_conv=k > 0, lengths=lengths, live=live)
    for b, L in enumerate(eff):
        assert np.all(out[b, :, L:] == 0.0), b


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_masked_full_lengths_equal_unmasked_bitwise(dt):
    wl = WORKLOADS["long"].with_(name=f"masked_full_{dt}", batch=2, heads=3, n=1500, dtype=dt)
    inp = make_inputs(wl)
    a, ia = run_forward(inp, wl.m, wl.iters, dt)
    b, ib = run_forward(inp, wl.m, wl.iters, dt, lengths=None)
    c, ic = run_forward(inp, wl.m, wl.iters, dt, lengths=(1500, 1500))
    assert np.array_equal(a, b) and np.array_equal(a, c)
    for key in ia:
        assert np.array_equal(ia[key], ib[key]) and np.array_equal(ia[key], ic[key]), key
