"""CPU oracle of the full self-attention layer around the Nyström attention
(fp64 NumPy).  TEST INFRASTRUCTURE ONLY, like the rest of this package.

[NF] "Standard Self-Attention" defines the learned projections Q = X W_Q,
K = X W_K, V = X W_V (no bias term is written); its discussion of the skip
connection refers to the attention-output projection.  Readings taken: the
layer is multi-head -- E = heads * d columns, head h owning columns
h*d .. h*d+d-1 of each projection -- each head runs ``nystrom_attention``
(with its DConv skip), the heads are concatenated in order and multiplied by
W_O; no biases.  The three projections are one product with the column
blocks [W_Q | W_K | W_V].

Pinned in ``tests/test_oracle_layer_pins.py``.
"""
from __future__ import annotations

import numpy as np

from .nystrom_oracle import nystrom_attention

__all__ = ["split_heads", "merge_heads", "nystrom_layer"]


def split_heads(M, heads):
    """(batch, n, heads*d) -> (batch, heads, n, d): head h takes columns h*d .. h*d+d-1."""
    M = np.asarray(M, dtype=np.float64)
    b, n, e = M.shape
    return M.reshape(b, n, heads, e // heads).transpose(0, 2, 1, 3)


def merge_heads(O):
    """(batch, heads, n, d) -> (batch, n, heads*d), heads concatenated in order."""
    O = np.asarray(O, dtype=np.float64)
    b, h, n, d = O.shape
    return O.transpose(0, 2, 1, 3).reshape(b, n, h * d)


def nystrom_layer(X, Wqkv, Wo, heads, m, iters, conv_w=None):
    """Y = merge(Nyström attention of the heads of X W_Q, X W_K, X W_V) W_O.

    X: (batch, n, E); Wqkv: (E, 3E) = [W_Q | W_K | W_V]; Wo: (E, E);
    conv_w: (heads, E/heads, k) or None.  Returns Y (batch, n, E) in fp64."""
    X, Wqkv, Wo = (np.asarray(a, dtype=np.float64) for a in (X, Wqkv, Wo))
    E = X.shape[2]
    QKV = X @ Wqkv
    Q, K, V = (split_heads(QKV[..., i * E:(i + 1) * E], heads) for i in range(3))
    O = nystrom_attention(Q, K, V, m, iters, conv_w)
    return merge_heads(O) @ Wo
