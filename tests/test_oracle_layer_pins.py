"""Pins for the layer oracle: closed forms and symmetries that a wrong column
block, a transposed head split or a missing output projection would break."""
import numpy as np

from oracle import depthwise_conv_skip, merge_heads, nystrom_head, nystrom_layer, split_heads


def test_split_and_merge_by_hand():
    M = np.arange(2 * 3 * 4, dtype=float).reshape(1, 3, 8)[:, :, :8]  # batch 1, n 3, E 8
    S = split_heads(M, 2)
    assert S.shape == (1, 2, 3, 4)
    np.testing.assert_array_equal(S[0, 1, 2], M[0, 2, 4:8])  # head 1, row 2 = columns 4..7 of row 2
    np.testing.assert_array_equal(merge_heads(S), M)


def test_one_head_is_the_composition():
    rng = np.random.default_rng(50)
    n, d, m = 24, 4, 4
    X = rng.standard_normal((1, n, d))
    Wq, Wk, Wv, Wo = (rng.standard_normal((d, d)) / 2 for _ in range(4))
    w = rng.standard_normal((1, d, 3)) * 0.2
    Y = nystrom_layer(X, np.concatenate([Wq, Wk, Wv], axis=1), Wo, 1, m, 6, w)
    O, _ = nystrom_head(X[0] @ Wq, X[0] @ Wk, X[0] @ Wv, m, 6, w[0])
    np.testing.assert_allclose(Y[0], O @ Wo, atol=1e-12)


def test_zero_key_projection_gives_the_mean_value():
    # W_K = 0 makes every score zero: every softmax is uniform and each head's
    # attention output is the mean of its value rows (see the forward pins),
    # so Y = mean_j(X_j W_V) W_O in every row (no skip).  A wrong column block
    # order would zero Q or V instead.
    rng = np.random.default_rng(51)
    B, n, H, d, m = 2, 20, 3, 4, 5
    E = H * d
    X = rng.standard_normal((B, n, E))
    Wq, Wv, Wo = (rng.standard_normal((E, E)) / np.sqrt(E) for _ in range(3))
    Y = nystrom_layer(X, np.concatenate([Wq, np.zeros((E, E)), Wv], axis=1), Wo, H, m, 6)
    for b in range(B):
        np.testing.assert_allclose(Y[b], np.broadcast_to((X[b] @ Wv).mean(0) @ Wo, (n, E)), atol=1e-12)


def test_head_permutation_invariance():
    # Renumbering the heads consistently in every projection (and the filters)
    # leaves Y unchanged.
    rng = np.random.default_rng(52)
    B, n, H, d, m = 1, 16, 3, 4, 4
    E = H * d
    X = rng.standard_normal((B, n, E))
    Wqkv = rng.standard_normal((E, 3 * E)) / np.sqrt(E)
    Wo = rng.standard_normal((E, E)) / np.sqrt(E)
    w = rng.standard_normal((H, d, 5)) * 0.2
    perm = np.array([2, 0, 1])
    cols = np.concatenate([np.arange(p * d, (p + 1) * d) for p in perm])
    Wqkv_p = np.concatenate([Wqkv[:, i * E:(i + 1) * E][:, cols] for i in range(3)], axis=1)
    Y = nystrom_layer(X, Wqkv, Wo, H, m, 6, w)
    Yp = nystrom_layer(X, Wqkv_p, Wo[cols], H, m, 6, w[perm])
    np.testing.assert_allclose(Yp, Y, atol=1e-12)


def test_skip_only_layer():
    # W_Q = W_K = 0 and a filter that is the centred delta: each head returns
    # mean(V) + V, so Y = (mean_j X_j W_V + X W_V) W_O.
    rng = np.random.default_rng(53)
    B, n, H, d, m = 1, 12, 2, 4, 3
    E = H * d
    X = rng.standard_normal((B, n, E))
    Wv, Wo = rng.standard_normal((E, E)), rng.standard_normal((E, E))
    w = np.zeros((H, d, 3))
    w[:, :, 1] = 1.0
    Y = nystrom_layer(X, np.concatenate([np.zeros((E, 2 * E)), Wv], axis=1), Wo, H, m, 6, w)
    V = X[0] @ Wv
    np.testing.assert_allclose(Y[0], (V.mean(0) + V) @ Wo, atol=1e-11)
    assert depthwise_conv_skip(V[:, :d], w[0]).shape == (n, d)
