"""Pins for the CPU oracle: each check ties an oracle function to something
other than itself (a closed form, exact rational arithmetic, brute force on a
tiny input, or a library routine), chosen so that a plausible slip -- a
dropped 1/sqrt(d), a divisor m instead of l, A instead of A^T in the start,
the wrong softmax axis, a flipped filter -- fails at least one of them."""
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

from oracle import (
    depthwise_conv_skip,
    exact_attention,
    iterative_pinv,
    landmark_kernels,
    nystrom_attention,
    nystrom_head,
    pinv_init,
    row_softmax,
    segment_means,
)


def rel_l2(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / np.linalg.norm(np.asarray(b)))


# ---------------------------------------------------------------- segment means

def test_segment_means_closed_form():
    # X[i, c] = i + 10 c; with l = 4 the mean of rows 4j..4j+3 is 4j + 1.5 + 10c.
    n, d, m = 12, 3, 3
    X = np.arange(n)[:, None] + 10.0 * np.arange(d)[None, :]
    expect = np.array([[4 * j + 1.5 + 10 * c for c in range(d)] for j in range(m)])
    np.testing.assert_array_equal(segment_means(X, m), expect)


def test_segment_means_brute_force():
    rng = np.random.default_rng(11)
    n, d, m = 20, 3, 5
    X = rng.standard_normal((n, d))
    seg = n // m
    expect = np.zeros((m, d))
    for j in range(m):
        for c in range(d):
            acc = 0.0
            for i in range(j * seg, (j + 1) * seg):
                acc += X[i, c]
            expect[j, c] = acc / seg
    np.testing.assert_allclose(segment_means(X, m), expect, rtol=0, atol=1e-15)


def test_segment_means_special_cases():
    rng = np.random.default_rng(12)
    X = rng.standard_normal((16, 4))
    np.testing.assert_array_equal(segment_means(X, 16), X)          # l = 1: identity
    np.testing.assert_allclose(segment_means(X, 1)[0], X.mean(0), atol=1e-15)
    # Constant segments give their own value back (a divisor m != l would not).
    C = np.repeat(rng.standard_normal((2, 4)), 8, axis=0)
    np.testing.assert_allclose(segment_means(C, 2), C[::8], atol=1e-15)
    # More landmarks than rows (only a key-padding mask asks for it): l = 1,
    # the rows themselves, then landmarks of pad only.
    np.testing.assert_array_equal(segment_means(X, 17), np.vstack([X, np.zeros((1, 4))]))
    with pytest.raises(ValueError):
        segment_means(X, 0)
    with pytest.raises(ValueError):
        segment_means(X[:0], 4)


def test_segment_means_padded_by_hand():
    # n not a multiple of m: zero rows are appended up to m * ceil(n/m) and
    # every segment is divided by the padded length (a divisor counting only
    # the real rows of the last segment would give 4.5 below).
    X = np.array([[1.0], [2.0], [3.0], [4.0], [5.0]])
    np.testing.assert_array_equal(segment_means(X, 2), [[2.0], [3.0]])              # l = 3
    np.testing.assert_array_equal(segment_means(X, 3), [[1.5], [3.5], [2.5]])       # l = 2
    np.testing.assert_array_equal(segment_means(X, 4), [[1.5], [3.5], [2.5], [0.0]])  # a segment of pad only
    np.testing.assert_array_equal(segment_means(X, 5), X)                            # divisible: no pad


def test_segment_means_padded_brute_force():
    rng = np.random.default_rng(14)
    for n, m in ((23, 5), (100, 8), (65, 64), (130, 64)):
        d = 3
        X = rng.standard_normal((n, d))
        seg = -(-n // m)
        expect = np.zeros((m, d))
        for j in range(m):
            for c in range(d):
                acc = 0.0
                for i in range(j * seg, (j + 1) * seg):
                    acc += X[i, c] if i < n else 0.0
                expect[j, c] = acc / seg
        np.testing.assert_allclose(segment_means(X, m), expect, rtol=0, atol=1e-15)


# ---------------------------------------------------------------- softmax

def test_row_softmax_closed_form_and_library():
    np.testing.assert_allclose(row_softmax(np.array([[0.0, math.log(3.0)]])), [[0.25, 0.75]], atol=1e-15)
    np.testing.assert_allclose(row_softmax(np.array([[1000.0, 1000.0]])), [[0.5, 0.5]], atol=1e-15)
    rng = np.random.default_rng(13)
    S = rng.standard_normal((7, 9)) * 3
    P = row_softmax(S)
    np.testing.assert_allclose(P, scipy.special.softmax(S, axis=1), atol=1e-15)
    np.testing.assert_allclose(P.sum(1), 1.0, atol=1e-15)
    np.testing.assert_allclose(row_softmax(S + rng.standard_normal((7, 1))), P, atol=1e-15)


def test_kernels_scale_closed_form():
    # d = 4, l = 1: score = q.k / sqrt(4).  q = (2 ln 3, 0, 0, 0), keys 0 and e1:
    # scores (0, ln 3) -> (1/4, 3/4).  Without the 1/sqrt(d) it would be (1/10, 9/10).
    ln3 = math.log(3.0)
    Q = np.array([[2 * ln3, 0, 0, 0], [0, 0, 0, 0]], float)
    K = np.array([[0, 0, 0, 0], [1, 0, 0, 0]], float)
    F, A, B = landmark_kernels(Q, K, Q, K)
    np.testing.assert_allclose(F[0], [0.25, 0.75], atol=1e-15)
    np.testing.assert_allclose(F[1], [0.5, 0.5], atol=1e-15)
    np.testing.assert_allclose(A, F, atol=1e-15)
    np.testing.assert_allclose(B, F, atol=1e-15)


def test_kernels_brute_force_and_axes():
    rng = np.random.default_rng(14)
    n, d, m = 6, 3, 2
    Q, K = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    Qt, Kt = segment_means(Q, m), segment_means(K, m)
    F, A, B = landmark_kernels(Q, K, Qt, Kt)

    def soft(rows_x, cols_y):
        out = []
        for x in rows_x:
            e = [math.exp(sum(x[c] * y[c] for c in range(d)) / math.sqrt(d)) for y in cols_y]
            out.append([v / sum(e) for v in e])
        return np.array(out)

    np.testing.assert_allclose(F, soft(Q, Kt), atol=1e-14)
    np.testing.assert_allclose(A, soft(Qt, Kt), atol=1e-14)
    np.testing.assert_allclose(B, soft(Qt, K), atol=1e-14)
    # B is normalised over the n keys (rows sum to 1), not over landmarks.
    np.testing.assert_allclose(B.sum(1), 1.0, atol=1e-15)
    assert B.shape == (m, n)


# ---------------------------------------------------------------- pseudoinverse

def test_pinv_init_hand():
    # ||A||_1 = max column sum = 6, ||A||_inf = max row sum = 7 -> Z0 = A^T / 42.
    A = np.array([[1.0, 2.0], [3.0, 4.0]])
    np.testing.assert_allclose(pinv_init(A), np.array([[1.0, 3.0], [2.0, 4.0]]) / 42.0, atol=1e-16)
    np.testing.assert_array_equal(iterative_pinv(A, 0), pinv_init(A))


def _closed_form_iterates(A, iters):
    """With A = U diag(s) V^T and Z0 = c A^T, every iterate is
    Z_t = V diag(y_t) U^T where x_t = s * y_t follows the scalar map
    x -> 1 - (1 - x)^3 (4 - x) / 4 (the iteration acts on each singular
    value separately), y_0 = c s, y_{t+1} = y_t * g(x_t),
    g(x) = (13 - 15 x + 7 x^2 - x^3) / 4."""
    U, s, Vt = np.linalg.svd(A)
    c = 1.0 / (np.abs(A).sum(0).max() * np.abs(A).sum(1).max())
    y = c * s
    x = s * y
    for _ in range(iters):
        g = (13 - 15 * x + 7 * x ** 2 - x ** 3) / 4
        y = y * g
        x = s * y
    return Vt.T @ np.diag(y) @ U.T, s, x


@pytest.mark.parametrize("iters", [0, 1, 2, 6, 10])
def test_pinv_matches_svd_closed_form(iters):
    rng = np.random.default_rng(15)
    A = row_softmax(rng.standard_normal((8, 8)) * 2.0)   # non-symmetric, like A~
    Zc, _, _ = _closed_form_iterates(A, iters)
    assert rel_l2(iterative_pinv(A, iters), Zc) < 1e-11


def test_pinv_diagonal_exact_rationals():
    # For a diagonal matrix every iterate is diagonal; run the scalar map in
    # exact rational arithmetic.  c = 1 / (max col sum * max row sum) = 1.
    sig = [Fraction(1), Fraction(1, 2), Fraction(1, 5)]
    A = np.diag([float(s) for s in sig])
    iters = 4
    zs = []
    for s in sig:
        z = s  # z0 = c * s
        for _ in range(iters):
            x = s * z
            z = z * (13 - 15 * x + 7 * x ** 2 - x ** 3) / 4
        zs.append(float(z))
    np.testing.assert_allclose(np.diag(iterative_pinv(A, iters)), zs, rtol=1e-14)
    np.testing.assert_allclose(iterative_pinv(A, iters) - np.diag(np.diag(iterative_pinv(A, iters))), 0, atol=0)


def test_pinv_converges_to_library_pinv():
    rng = np.random.default_rng(16)
    A = row_softmax(rng.standard_normal((10, 10)) * 2.0)
    np.testing.assert_allclose(iterative_pinv(A, 60), np.linalg.pinv(A), rtol=0, atol=1e-9 * np.abs(np.linalg.pinv(A)).max())
    # Rank-deficient: two equal rows.  In exact arithmetic zero singular values
    # stay zero, so the limit is the Moore-Penrose inverse.  In floating point
    # the null direction holds rounding noise that the map multiplies by its
    # slope at 0 (13/4) every step, so the check stops at 20 steps: the range
    # has converged (cubically) and the noise is still ~1e-16 * 3.25^20.
    R = A.copy()
    R[3] = R[5]
    P = np.linalg.pinv(R, rcond=1e-12)
    assert rel_l2(iterative_pinv(R, 20), P) < 1e-6


def test_pinv_residual_matches_closed_form():
    rng = np.random.default_rng(17)
    A = row_softmax(rng.standard_normal((12, 12)) * 1.5)
    for iters in (3, 6):
        Z = iterative_pinv(A, iters)
        _, s, x = _closed_form_iterates(A, iters)
        expect = math.sqrt(float(np.sum(s ** 2 * (1 - x) ** 2)))
        got = np.linalg.norm(A @ Z @ A - A)
        assert abs(got - expect) <= 1e-10 * max(1.0, expect)


# ---------------------------------------------------------------- depthwise conv skip

def test_conv_matches_numpy_correlate():
    rng = np.random.default_rng(18)
    n, d, k = 40, 5, 9
    V = rng.standard_normal((n, d))
    w = rng.standard_normal((d, k))
    expect = np.stack([np.correlate(V[:, c], w[c], mode="same") for c in range(d)], axis=1)
    np.testing.assert_allclose(depthwise_conv_skip(V, w), expect, atol=1e-13)


def test_conv_impulse_response_hand():
    # V = impulse at row p in feature 0: out[i] = w[p - i + r], i.e. the filter
    # appears reversed around row p (cross-correlation, no flip).
    n, k, p = 11, 5, 5
    r = (k - 1) // 2
    V = np.zeros((n, 1))
    V[p, 0] = 1.0
    w = np.array([[1.0, 2.0, 3.0, 4.0, 5.0]])
    out = depthwise_conv_skip(V, w)[:, 0]
    expect = np.zeros(n)
    for t in range(k):
        expect[p - t + r] = w[0, t]
    np.testing.assert_array_equal(out, expect)
    np.testing.assert_array_equal(out[p - r:p + r + 1], [5, 4, 3, 2, 1])


def test_conv_special_filters():
    rng = np.random.default_rng(19)
    V = rng.standard_normal((16, 3))
    w1 = rng.standard_normal((3, 1))
    np.testing.assert_allclose(depthwise_conv_skip(V, w1), V * w1[:, 0], atol=1e-15)
    delta = np.zeros((3, 7))
    delta[:, 3] = 1.0
    np.testing.assert_array_equal(depthwise_conv_skip(V, delta), V)
    # Zero padding at the ends: a filter that reads only the next row.
    nxt = np.zeros((3, 3))
    nxt[:, 2] = 1.0
    out = depthwise_conv_skip(V, nxt)
    np.testing.assert_array_equal(out[:-1], V[1:])
    np.testing.assert_array_equal(out[-1], 0.0)


# ---------------------------------------------------------------- whole pipeline

def _brute_exact_attention(Q, K, V):
    n, d = Q.shape
    out = np.zeros_like(V)
    for i in range(n):
        e = [math.exp(sum(Q[i, c] * K[j, c] for c in range(d)) / math.sqrt(d)) for j in range(n)]
        z = sum(e)
        for j in range(n):
            out[i] += (e[j] / z) * V[j]
    return out


def test_exact_attention_brute_force():
    rng = np.random.default_rng(20)
    Q, K, V = (rng.standard_normal((9, 3)) for _ in range(3))
    full = _brute_exact_attention(Q, K, V)
    np.testing.assert_allclose(exact_attention(Q, K, V, row_chunk=4), full, atol=1e-14)
    rows = np.array([1, 4, 8])  # a subset of query rows against all keys
    np.testing.assert_allclose(exact_attention(Q[rows], K, V, row_chunk=2), full[rows], atol=1e-14)


def test_lemma2_m_equals_n_is_exact():
    # m = n: F = A = B = S and, with a converged pseudoinverse, F A^+ B V = S V.
    rng = np.random.default_rng(21)
    n, d = 12, 4
    Q, K, V = (rng.standard_normal((n, d)) for _ in range(3))
    O, inter = nystrom_head(Q, K, V, m=n, iters=60)
    np.testing.assert_allclose(inter["F"], inter["A"], atol=1e-15)
    np.testing.assert_allclose(inter["B"], inter["A"], atol=1e-15)
    assert rel_l2(O, _brute_exact_attention(Q, K, V)) < 1e-10
    # Six iterations alone are not converged at this size: the gap is visible.
    O6, _ = nystrom_head(Q, K, V, m=n, iters=6)
    assert rel_l2(O6, exact_attention(Q, K, V)) > 1e-6


def test_segment_constant_inputs_are_exact():
    # If Q and K are constant on each segment then S = E A E^T / l with E the
    # segment indicator, and F A^+ B = E A A^+ A E^T / l = S: the approximation
    # is exact for any m dividing n (a wrong segment divisor or a missing scale
    # breaks this).
    rng = np.random.default_rng(22)
    n, d, m = 24, 4, 4
    Q = np.repeat(rng.standard_normal((m, d)) * 1.5, n // m, axis=0)
    K = np.repeat(rng.standard_normal((m, d)) * 1.5, n // m, axis=0)
    V = rng.standard_normal((n, d))
    O, _ = nystrom_head(Q, K, V, m=m, iters=60)
    assert rel_l2(O, _brute_exact_attention(Q, K, V)) < 1e-10


def test_zero_queries_give_the_mean_of_the_real_values():
    # Q = 0 makes every softmax uniform: A = 11^T/m is idempotent with unit
    # norms, so Z0 = A and Lemma 1 maps A to A; BV rows are the mean of the
    # value rows over the keys, and O = F Z BV is that mean in every row, for
    # any K.  With n not a multiple of m the pad keys must not count: taking
    # them as zero-valued keys would give sum(V) / (m ceil(n/m)) instead.
    rng = np.random.default_rng(27)
    for n, m in ((23, 5), (100, 8), (65, 64), (24, 4)):
        d = 3
        K, V = rng.standard_normal((n, d)), rng.standard_normal((n, d))
        O, inter = nystrom_head(np.zeros((n, d)), K, V, m, 6)
        assert inter["B"].shape == (m, n)
        np.testing.assert_allclose(O, np.broadcast_to(V.mean(0), (n, d)), rtol=0, atol=1e-13)


def test_key_shift_invariance():
    # K -> K + 1 c^T adds a per-row constant to every score matrix (row-wise
    # softmax does not see it).  Column-wise normalisation of B would.
    rng = np.random.default_rng(23)
    n, d, m = 32, 4, 4
    Q, K, V = (rng.standard_normal((n, d)) for _ in range(3))
    c = rng.standard_normal(d) * 3
    O1, _ = nystrom_head(Q, K, V, m, 6)
    O2, _ = nystrom_head(Q, K + c, V, m, 6)
    assert rel_l2(O2, O1) < 1e-12


def test_permutation_equivariance():
    rng = np.random.default_rng(24)
    n, d, m = 32, 4, 4
    seg = n // m
    Q, K, V = (rng.standard_normal((n, d)) for _ in range(3))
    O, _ = nystrom_head(Q, K, V, m, 6)
    # Shuffle rows inside each segment: landmarks unchanged, output rows follow.
    p = np.concatenate([j * seg + rng.permutation(seg) for j in range(m)])
    Op, _ = nystrom_head(Q[p], K[p], V[p], m, 6)
    assert rel_l2(Op, O[p]) < 1e-12
    # Permute whole segments.
    sp = rng.permutation(m)
    p2 = np.concatenate([np.arange(s * seg, (s + 1) * seg) for s in sp])
    Op2, _ = nystrom_head(Q[p2], K[p2], V[p2], m, 6)
    assert rel_l2(Op2, O[p2]) < 1e-12


def test_linearity_in_v_and_skip_is_added():
    rng = np.random.default_rng(25)
    n, d, m = 32, 4, 8
    Q, K, V1, V2 = (rng.standard_normal((n, d)) for _ in range(4))
    w = rng.standard_normal((d, 5)) * 0.1
    a, b = 0.7, -1.3
    O1, _ = nystrom_head(Q, K, V1, m, 6, w)
    O2, _ = nystrom_head(Q, K, V2, m, 6, w)
    O12, inter = nystrom_head(Q, K, a * V1 + b * V2, m, 6, w)
    assert rel_l2(O12, a * O1 + b * O2) < 1e-12
    np.testing.assert_allclose(O12, inter["O_att"] + depthwise_conv_skip(a * V1 + b * V2, w), atol=1e-14)


def test_association_orders_agree():
    rng = np.random.default_rng(26)
    n, d, m = 64, 8, 8
    Q, K, V = (rng.standard_normal((n, d)) for _ in range(3))
    _, it = nystrom_head(Q, K, V, m, 6)
    F, Z, B = it["F"], it["Z"], it["B"]
    ours = F @ (Z @ (B @ V))
    assert rel_l2((F @ Z) @ (B @ V), ours) < 1e-12     # blog-post excerpt order
    assert rel_l2(F @ ((Z @ B) @ V), ours) < 1e-12     # paper's "Putting It Together" order


def test_batch_of_heads_equals_per_head():
    rng = np.random.default_rng(27)
    Bt, H, n, d, m, k = 2, 3, 16, 4, 4, 3
    Q, K, V = (rng.standard_normal((Bt, H, n, d)) for _ in range(3))
    w = rng.standard_normal((H, d, k))
    O, inter = nystrom_attention(Q, K, V, m, 6, w, with_intermediates=True)
    for b in range(Bt):
        for h in range(H):
            Oh, ih = nystrom_head(Q[b, h], K[b, h], V[b, h], m, 6, w[h])
            np.testing.assert_array_equal(O[b, h], Oh)
            np.testing.assert_array_equal(inter["Z"][b, h], ih["Z"])


def test_approximation_error_is_reported_not_gated():
    # Random Gaussian Q/K are neither low rank nor local, so m < n is far from
    # exact; the check only asks for a finite, bounded report.
    rng = np.random.default_rng(28)
    Q, K, V = (rng.standard_normal((64, 16)) for _ in range(3))
    O, _ = nystrom_head(Q, K, V, 8, 6)
    err = rel_l2(O, exact_attention(Q, K, V))
    assert np.isfinite(err) and 0.0 < err < 10.0


# ---------------------------------------------------------------- key-padding mask

def test_lengths_zero_queries_give_the_mean_of_each_sequence():
    # As in the zero-query case above, per batch entry: rows below L_b are the
    # mean of that entry's first L_b value rows, rows from L_b on are zero.
    rng = np.random.default_rng(28)
    Bt, H, n, d, m = 3, 2, 40, 3, 4
    K, V = rng.standard_normal((Bt, H, n, d)), rng.standard_normal((Bt, H, n, d))
    lengths = [40, 23, 9]
    O = nystrom_attention(np.zeros((Bt, H, n, d)), K, V, m, 6, lengths=lengths)
    for b, L in enumerate(lengths):
        for h in range(H):
            np.testing.assert_allclose(O[b, h, :L], np.broadcast_to(V[b, h, :L].mean(0), (L, d)), rtol=0, atol=1e-13)
            assert not O[b, h, L:].any()


def test_lengths_pad_rows_are_never_read():
    rng = np.random.default_rng(29)
    Bt, H, n, d, m = 2, 2, 48, 4, 8
    Q, K, V = (rng.standard_normal((Bt, H, n, d)) for _ in range(3))
    w = rng.standard_normal((H, d, 5)) * 0.2
    lengths = [30, 48]
    O1, i1 = nystrom_attention(Q, K, V, m, 6, w, with_intermediates=True, lengths=lengths)
    Q2, K2, V2 = Q.copy(), K.copy(), V.copy()
    for X in (Q2, K2, V2):
        X[0, :, 30:] = np.nan
    O2, i2 = nystrom_attention(Q2, K2, V2, m, 6, w, with_intermediates=True, lengths=lengths)
    np.testing.assert_array_equal(O1, O2)
    for key in i1:
        np.testing.assert_array_equal(i1[key], i2[key])
    # The skip sees zeros past L_b: its last output row differs from the
    # unmasked call's, which reads the rows past 30.
    O3 = nystrom_attention(Q, K, V, m, 6, w)
    assert not np.allclose(O1[0, :, 29], O3[0, :, 29])
    np.testing.assert_array_equal(O1[1], O3[1])  # full length: same as no mask


def test_lengths_are_clamped_to_zero_and_n():
    rng = np.random.default_rng(30)
    Bt, H, n, d, m = 3, 1, 20, 2, 5
    Q, K, V = (rng.standard_normal((Bt, H, n, d)) for _ in range(3))
    np.testing.assert_array_equal(nystrom_attention(Q, K, V, m, 6, lengths=[-3, 99, 2]),
                                  nystrom_attention(Q, K, V, m, 6, lengths=[0, 20, 2]))


def test_lengths_below_m_pad_the_landmarks_by_hand():
    # L_b = 3 < m = 5: padded to m rows (l = 1), so the landmarks are the three
    # rows and two zero vectors; B~ spans the three real keys.  Written out
    # here with explicit loops (softmaxes by hand) on one head.
    rng = np.random.default_rng(31)
    n, d, m, L = 12, 2, 5, 3
    Q, K, V = (rng.standard_normal((1, 1, n, d)) for _ in range(3))
    O, inter = nystrom_attention(Q, K, V, m, 30, with_intermediates=True, lengths=[L])
    q, k, v = Q[0, 0], K[0, 0], V[0, 0]
    lm_q = np.zeros((m, d))
    lm_k = np.zeros((m, d))
    lm_q[:L], lm_k[:L] = q[:L], k[:L]
    np.testing.assert_array_equal(inter["Qt"][0, 0], lm_q)
    np.testing.assert_array_equal(inter["Kt"][0, 0], lm_k)
    s = 1.0 / math.sqrt(d)

    def softmax_row(x):
        e = [math.exp(t - max(x)) for t in x]
        return [t / sum(e) for t in e]

    F = np.array([softmax_row([s * float(q[i] @ lm_k[j]) for j in range(m)]) for i in range(L)])
    A = np.array([softmax_row([s * float(lm_q[i] @ lm_k[j]) for j in range(m)]) for i in range(m)])
    B = np.array([softmax_row([s * float(lm_q[i] @ k[j]) for j in range(L)]) for i in range(m)])
    np.testing.assert_allclose(inter["A"][0, 0], A, rtol=0, atol=1e-15)
    # 30 steps converge, so the pseudoinverse is the library's.
    expect = F @ np.linalg.pinv(A) @ (B @ v[:L])
    np.testing.assert_allclose(O[0, 0, :L], expect, rtol=0, atol=1e-9)
    assert not O[0, 0, L:].any()


def test_lengths_below_m_zero_queries_and_nan_pad():
    # Zero queries: every softmax is uniform, the pseudoinverse of the uniform
    # m x m matrix is itself, and each output row below L_b is the mean of the
    # L_b real value rows (counting the zero landmarks' pad rows as keys would
    # not give this).  The pad rows hold NaN and must never be read.
    rng = np.random.default_rng(32)
    Bt, H, n, d, m = 4, 2, 24, 3, 8
    K, V = rng.standard_normal((Bt, H, n, d)), rng.standard_normal((Bt, H, n, d))
    lengths = [5, 1, 0, 24]
    Q = np.zeros((Bt, H, n, d))
    for X in (Q, K, V):
        for b, L in enumerate(lengths):
            X[b, :, L:] = np.nan
    O = nystrom_attention(Q, K, V, m, 6, lengths=lengths)
    assert np.all(np.isfinite(O))
    for b, L in enumerate(lengths):
        for h in range(H):
            if L:
                np.testing.assert_allclose(O[b, h, :L], np.broadcast_to(V[b, h, :L].mean(0), (L, d)),
                                           rtol=0, atol=1e-13)
            assert not O[b, h, L:].any()


def test_empty_sequence_has_zero_output_and_undefined_intermediates():
    rng = np.random.default_rng(33)
    Q, K, V = (rng.standard_normal((2, 1, 16, 2)) for _ in range(3))
    w = rng.standard_normal((1, 2, 3))
    O, inter = nystrom_attention(Q, K, V, 4, 6, w, with_intermediates=True, lengths=[0, 16])
    assert not O[0].any()
    assert np.all(np.isnan(inter["Z"][0])) and np.all(np.isfinite(inter["Z"][1]))
    np.testing.assert_array_equal(O[1], nystrom_attention(Q[1:], K[1:], V[1:], 4, 6, w)[0])


# ---------------------------------------------------------------- approximation error

def test_approximation_error_special_cases():
    from oracle import approximation_error
    rng = np.random.default_rng(60)
    n, d = 16, 4
    Q, K, V = (rng.standard_normal((1, 2, n, d)) for _ in range(3))
    # m = n with a converged pseudoinverse is exact attention (Lemma 2).
    assert approximation_error(Q, K, V, n, 60).max() < 1e-10
    # Segment-constant queries and keys: exact for m dividing n.
    m = 4
    Qc = np.repeat(rng.standard_normal((1, 2, m, d)), n // m, axis=2)
    Kc = np.repeat(rng.standard_normal((1, 2, m, d)), n // m, axis=2)
    assert approximation_error(Qc, Kc, V, m, 60).max() < 1e-10
    # Otherwise a visible error, equal to its definition on one head.
    e = approximation_error(Q, K, V, 4, 6)
    O, _ = nystrom_head(Q[0, 1], K[0, 1], V[0, 1], 4, 6)
    ex = _brute_exact_attention(Q[0, 1], K[0, 1], V[0, 1])
    assert abs(e[0, 1] - np.linalg.norm(O - ex) / np.linalg.norm(ex)) < 1e-12
    assert e.min() > 1e-3
