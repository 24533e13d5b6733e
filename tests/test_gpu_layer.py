"""Parity of the full layer (nystrom_layer_fwd: QKV projection, heads,
Nyström attention with the skip, output projection) against the fp64 layer
oracle.  Bars: 1e-4 (fp32 I/O) and 2e-2 (bf16 I/O) relative L2 on Y; the bf16
path also rounds the projected Q, K, V and the attention output to bf16
(about 2^-9 relative each), which the oracle does not."""
import numpy as np
import pytest
import torch

from efficient_transformer_attention_mean_amd import _lib
from efficient_transformer_attention_mean_amd.workloads import round_to_bf16
from oracle import nystrom_layer

from ._checks import Bars, Gate
from ._gpu_util import dtype_code, to_dev, to_host

pytestmark = pytest.mark.gpu

# Y gates (tests/_checks.py): relative L2 over Y and over each batch entry at
# the attention's output bars, the same per 64-row tile, and an elementwise
# bound.  bf16 rounds Q, K, V, the attention output and Y to bf16 (2^-9
# relative each), and the projections sum E = heads * d such terms, so the
# elementwise error is a few 1e-3 of Y's rms.
BARS = {
    "f32": Bars(rel=1e-4, tile=1e-4, rtol=1e-4, atol=1e-4),
    "bf16": Bars(rel=2e-2, tile=2e-2, rtol=2.0 ** -7, atol=5e-2),
}


def layer_inputs(B, n, H, d, k, dt, seed):
    """X ~ N(0, 1); projections ~ N(0, 1/E) so that Q, K, V ~ N(0, 1);
    filters ~ N(0, 0.02)."""
    rng = np.random.default_rng(seed)
    E = H * d
    X = rng.standard_normal((B, n, E)).astype(np.float32)
    Wqkv = (rng.standard_normal((E, 3 * E)) / np.sqrt(E)).astype(np.float32)
    Wo = (rng.standard_normal((E, E)) / np.sqrt(E)).astype(np.float32)
    w = rng.normal(0, 0.02, (H, d, k)).astype(np.float32) if k else None
    if dt == "bf16":
        X, Wqkv, Wo = round_to_bf16(X), round_to_bf16(Wqkv), round_to_bf16(Wo)
    return X, Wqkv, Wo, w


def run_layer(X, Wqkv, Wo, w, H, d, m, iters, dt, own_workspace=True):
    B, n, E = X.shape
    Xd, Wd, Wod = to_dev(X, dt), to_dev(Wqkv, dt), to_dev(Wo, dt)
    wd = None if w is None else torch.from_numpy(w).cuda()
    Y = torch.empty_like(Xd)
    ws, nbytes = None, 0
    if own_workspace:
        nbytes = _lib.nystrom_layer_workspace_bytes(B, H, n, d, m, dtype_code(dt))
        assert nbytes > 0
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    rc = _lib.nystrom_layer_fwd(Xd, Wd, Wod, wd, n, d, m, H, iters, Y, B, 0 if w is None else w.shape[2],
                                dtype_code(dt), ws, nbytes, torch.cuda.current_stream())
    assert rc == _lib.NYS_OK, _lib.nystrom_strerror(rc)
    torch.cuda.synchronize()
    return to_host(Y)


CASES = [
    # (batch, n, heads, d, m, iters, conv_k, dtype)
    (1, 64, 1, 16, 8, 6, 3, "f32"),
    (2, 100, 3, 32, 10, 6, 5, "bf16"),     # ragged n
    (2, 256, 4, 64, 64, 6, 33, "f32"),
    (8, 512, 12, 64, 64, 6, 33, "bf16"),   # BERT-base-shaped layer
    (1, 300, 2, 128, 32, 6, 0, "bf16"),    # d = 128, no skip
    (2, 300, 3, 64, 64, 6, 33, "bf16"),    # Q, K, V read in place, ragged n (5-row segments, 60-row tail)
    (1, 512, 2, 64, 128, 6, 33, "bf16"),   # m > 64: heads copied out of the QKV product first
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}n{c[1]}H{c[2]}d{c[3]}m{c[4]}k{c[6]}{c[7]}" for c in CASES])
def test_layer_parity(case):
    B, n, H, d, m, iters, k, dt = case
    X, Wqkv, Wo, w = layer_inputs(B, n, H, d, k, dt, 400 + n + H)
    ref = nystrom_layer(X, Wqkv, Wo, H, m, iters, w)
    got = run_layer(X, Wqkv, Wo, w, H, d, m, iters, dt)
    g = Gate(f"layer {case}")
    g("Y", got, ref, BARS[dt])
    g.close()


def test_layer_null_workspace_and_determinism():
    X, Wqkv, Wo, w = layer_inputs(2, 200, 4, 32, 9, "bf16", 7)
    a = run_layer(X, Wqkv, Wo, w, 4, 32, 16, 6, "bf16")
    b = run_layer(X, Wqkv, Wo, w, 4, 32, 16, 6, "bf16", own_workspace=False)
    assert np.array_equal(a, b)
