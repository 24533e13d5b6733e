"""Pins for the backward oracle: each check ties its gradients to something
other than the reverse-mode code itself -- central finite differences of the
forward oracle, closed forms at Q = 0, the textbook gradient of exact softmax
attention at m = n, and linearity -- so that a dropped term, a transposed
factor or a wrong sign in any step fails at least one of them."""
import numpy as np
import pytest

from oracle import (
    conv_skip_backward,
    depthwise_conv_skip,
    iterative_pinv,
    nystrom_attention,
    nystrom_attention_backward,
    nystrom_head,
    nystrom_head_backward,
    pinv_backward,
    segment_means,
    segment_means_backward,
)


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / np.linalg.norm(np.asarray(b)))


def _fd(f, X, h=1e-6):
    """Central differences of the scalar f at X, entry by entry."""
    G = np.zeros_like(X)
    it = np.nditer(X, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        x0 = X[i]
        X[i] = x0 + h
        fp = f(X)
        X[i] = x0 - h
        fm = f(X)
        X[i] = x0
        G[i] = (fp - fm) / (2 * h)
    return G


@pytest.mark.parametrize("n,d,m,iters,k", [(12, 3, 4, 6, 3), (10, 2, 3, 3, 5), (9, 4, 9, 2, 1), (16, 4, 4, 0, 3)])
def test_head_gradients_match_finite_differences(n, d, m, iters, k):
    rng = np.random.default_rng(40 + n + m)
    Q, K, V = (rng.standard_normal((n, d)) for _ in range(3))
    w = rng.standard_normal((d, k)) * 0.3
    dO = rng.standard_normal((n, d))

    def loss(Q_=Q, K_=K, V_=V, w_=w):
        O, _ = nystrom_head(Q_, K_, V_, m, iters, w_)
        return float((O * dO).sum())

    dQ, dK, dV, dw = nystrom_head_backward(Q, K, V, m, iters, dO, w)
    assert rel(dQ, _fd(lambda X: loss(Q_=X), Q.copy())) < 1e-6
    assert rel(dK, _fd(lambda X: loss(K_=X), K.copy())) < 1e-6
    assert rel(dV, _fd(lambda X: loss(V_=X), V.copy())) < 1e-6
    assert rel(dw, _fd(lambda X: loss(w_=X), w.copy())) < 1e-6


def test_pinv_backward_matches_finite_differences():
    rng = np.random.default_rng(41)
    m = 5
    # Positive, rows not normalised: both maxima have a unique maximiser (a
    # softmax's rows all sum to 1, a tie at which a difference quotient of
    # max(row sums) is not a derivative).
    A = np.exp(rng.standard_normal((m, m))) / m
    G = rng.standard_normal((m, m))
    for iters in (0, 1, 4):
        dA = pinv_backward(A, iters, G)
        fd = _fd(lambda X: float((iterative_pinv(X, iters) * G).sum()), A.copy())
        assert rel(dA, fd) < 1e-6, iters


def test_segment_and_conv_backward_by_hand():
    # segment means of 5 rows into 2 landmarks (l = 3, one pad row): the
    # gradient of landmark j is spread as 1/3 over its real rows.
    dXt = np.array([[3.0], [6.0]])
    np.testing.assert_array_equal(segment_means_backward(dXt, 5), [[1.0], [1.0], [1.0], [2.0], [2.0]])
    # Adjoint identity <conv(V), G> = <V, conv^T(G)> and <conv_w(V), G> linear in w.
    rng = np.random.default_rng(42)
    V, G = rng.standard_normal((7, 2)), rng.standard_normal((7, 2))
    w = rng.standard_normal((2, 3))
    dV, dw = conv_skip_backward(V, w, G)
    assert abs((depthwise_conv_skip(V, w) * G).sum() - (V * dV).sum()) < 1e-12
    assert abs((depthwise_conv_skip(V, w) * G).sum() - (w * dw).sum()) < 1e-12
    # Impulse: a single dO entry at row 3 of feature 0 sends w[0, t] to row 3 + t - 1.
    G = np.zeros((7, 2))
    G[3, 0] = 1.0
    dV, _ = conv_skip_backward(np.zeros((7, 2)), np.array([[1.0, 2.0, 3.0], [0.0, 0.0, 0.0]]), G)
    np.testing.assert_array_equal(dV[:, 0], [0, 0, 1, 2, 3, 0, 0])


def test_zero_queries_closed_forms():
    # Q = 0 makes the attention output the mean of the value rows for every K
    # (see the forward pins), so dK = 0 and the attention part of dV is the
    # column sum of dO over n in every row.
    rng = np.random.default_rng(43)
    n, d, m = 23, 3, 5
    K, V, dO = (rng.standard_normal((n, d)) for _ in range(3))
    dQ, dK, dV, _ = nystrom_head_backward(np.zeros((n, d)), K, V, m, 6, dO)
    np.testing.assert_allclose(dK, 0.0, atol=1e-13)
    np.testing.assert_allclose(dV, np.broadcast_to(dO.sum(0) / n, (n, d)), rtol=0, atol=1e-13)
    assert np.abs(dQ).max() > 1e-3  # the queries still move the output


def _exact_attention_grads(Q, K, V, dO):
    """Gradients of softmax(Q K^T / sqrt d) V written out from its textbook
    form (loops over rows, no shared code with the oracle)."""
    n, d = Q.shape
    s = 1.0 / np.sqrt(d)
    dQ, dK, dV = np.zeros((n, d)), np.zeros((n, d)), np.zeros((n, d))
    for i in range(n):
        sc = s * (K @ Q[i])
        p = np.exp(sc - sc.max())
        p /= p.sum()
        dp = V @ dO[i]
        ds = p * (dp - p @ dp)
        dQ[i] = s * ds @ K
        dK += s * np.outer(ds, Q[i])
        dV += np.outer(p, dO[i])
    return dQ, dK, dV


def test_m_equals_n_converged_is_exact_attention_gradient():
    rng = np.random.default_rng(44)
    n, d = 10, 3
    Q, K, V, dO = (rng.standard_normal((n, d)) for _ in range(4))
    dQ, dK, dV, _ = nystrom_head_backward(Q, K, V, n, 60, dO)
    eQ, eK, eV = _exact_attention_grads(Q, K, V, dO)
    assert rel(dQ, eQ) < 1e-9 and rel(dK, eK) < 1e-9 and rel(dV, eV) < 1e-9


def test_batched_backward_linear_in_dO_and_sums_filters():
    rng = np.random.default_rng(45)
    Bt, H, n, d, m = 2, 2, 12, 3, 4
    Q, K, V, G1, G2 = (rng.standard_normal((Bt, H, n, d)) for _ in range(5))
    w = rng.standard_normal((H, d, 3)) * 0.2
    a = nystrom_attention_backward(Q, K, V, m, 6, G1, w)
    b = nystrom_attention_backward(Q, K, V, m, 6, G2, w)
    c = nystrom_attention_backward(Q, K, V, m, 6, 2.0 * G1 - G2, w)
    for x, y, z in zip(a, b, c):
        np.testing.assert_allclose(z, 2.0 * x - y, atol=1e-11)
    per = [nystrom_head_backward(Q[bb, 1], K[bb, 1], V[bb, 1], m, 6, G1[bb, 1], w[1])[3] for bb in range(Bt)]
    np.testing.assert_allclose(a[3][1], per[0] + per[1], atol=1e-13)
    # The forward used by the finite differences above is the batched one's head.
    O = nystrom_attention(Q, K, V, m, 6, w)
    np.testing.assert_allclose(O[1, 0], nystrom_head(Q[1, 0], K[1, 0], V[1, 0], m, 6, w[0])[0], atol=1e-14)
    assert segment_means(Q[0, 0], m).shape == (m, d)


@pytest.mark.parametrize("lengths,m", [((7, 12), 4), ((3, 0), 4), ((12, 5), 6)])
def test_masked_backward_matches_finite_differences(lengths, m):
    """The masked backward against central differences of the masked forward
    oracle (a sequence shorter than m, one m does not divide, an empty one),
    with NaN in every pad row of Q, K, V and dO: the pad rows must not be
    read, their gradients are exactly zero, and the filter gradient sums the
    real rows of every entry only."""
    rng = np.random.default_rng(46 + sum(lengths) + m)
    Bt, H, n, d, k, iters = 2, 2, 12, 3, 3, 6
    Q, K, V, dO = (rng.standard_normal((Bt, H, n, d)) for _ in range(4))
    w = rng.standard_normal((H, d, k)) * 0.3
    lens = np.array(lengths)
    pad = np.arange(n)[None, None, :, None] >= lens[:, None, None, None]
    Qn, Kn, Vn, dOn = (np.where(pad, np.nan, X) for X in (Q, K, V, dO))
    dQ, dK, dV, dw = nystrom_attention_backward(Qn, Kn, Vn, m, iters, dOn, w, lengths=lens)
    for G in (dQ, dK, dV):
        assert np.all(G[np.broadcast_to(pad, G.shape)] == 0.0)
    assert np.all(np.isfinite(dw))

    def loss(Q_=Q, K_=K, V_=V, w_=w):
        O = nystrom_attention(Q_, K_, V_, m, iters, w_, lengths=lens)
        return float((np.where(pad, 0.0, O) * np.where(pad, 0.0, dO)).sum())

    live = ~np.broadcast_to(pad, Q.shape)
    for G, X, key in ((dQ, Q, "Q_"), (dK, K, "K_"), (dV, V, "V_")):
        fd = _fd(lambda Y: loss(**{key: Y}), X.copy())
        assert rel(G[live], fd[live]) < 1e-6
        assert np.all(np.abs(fd[~live]) < 1e-9)  # the forward does not depend on the pad rows
    assert rel(dw, _fd(lambda Y: loss(w_=Y), w.copy())) < 1e-6
