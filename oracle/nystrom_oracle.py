"""CPU oracle for the Nyströmformer self-attention forward pass (fp64 NumPy).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this module; only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
constant with the HIP library: it is a plain, slow, step-by-step restatement
of what the method computes, written so that each step can be checked against
the pages by eye.

Sources (cited by page title and the section / equation on that page):

* [NF] "Nyströmformer: A Nyström-Based Algorithm for Approximating
  Self-Attention" (paper deep-dive page on arXiv 2102.03902), section
  3.4 "Detailed, sentence-based technical breakdown" and its sub-parts
  "Standard Self-Attention" (Eq. 2), "Moore-Penrose Pseudoinverse
  Computation" (Lemma 1 and the initialisation), "Landmark Selection:
  Segment-Means" (Eq. 16 and the note on its divisor), "Putting It
  Together" (Eq. 13 / Eq. 17, the association order, the DConv skip of
  Figure 4), and "Complexity Analysis".
* [HF] "Approximating self-attention in linear time and memory via the
  Nyström method" (Hugging Face blog post), sections "How can we adapt
  the Nyström method to approximate self-attention?", "How do we select
  landmarks?" and "How is Nyströmformer implemented?".

Readings taken where the pages are silent or garbled (each is also listed in
the design notes):

* Segment means divide by the segment length l = n/m over contiguous blocks
  of l rows ([NF] Eq. 16 prints a divisor m; the page itself calls that a
  typo, and [HF]'s reshape-and-mean agrees).
* All three softmaxes use the scale 1/sqrt(d), d = head dimension ([NF]
  Eq. 13; [HF] says its excerpt leaves the normalisation out).
* Every softmax is over the last axis (row-wise); for B~ that is over the n
  keys, as in [NF] Eq. 13 and [HF]'s ``softmax(dim=-1)``.
* The pseudoinverse runs exactly ``iters`` steps of Lemma 1 from the
  Pan-Schreiber start; the matrix norms are taken per (batch, head).
* Product order F~ (Z (B~ V)); in exact arithmetic this equals the orders
  of [NF] "Putting It Together" and [HF]'s excerpt.
* The skip is a depthwise 1-D cross-correlation along the sequence with one
  odd-length filter per (head, feature): weights ``conv_w[h, c, t]``, "same"
  zero padding of (k-1)/2 on each side, no flip, no bias ([NF] "Putting It
  Together", Figure 4 "DConv k x 1"; [HF] "How do we select landmarks?").
* n not a multiple of m: the sequence is padded at its end with zero rows
  to n' = m * ceil(n/m) ([NF] "Landmark Selection: Segment-Means" assumes
  divisibility and says padding provides it).  Every segment, the last one
  included, is divided by its padded length l = n'/m, so the pad rows count
  as zeros in the means.  The pad rows are not tokens: they are masked out
  as keys (B~ spans the n real keys only) and produce no output rows.
* Key-padding mask ([HF] leaves masking out of its excerpt): a batch of
  right-padded sequences is given by one length L_b per batch entry, and
  entry b is the method on its first L_b rows alone; its pad rows are never
  read and their output rows are zero (``nystrom_attention``'s ``lengths``).
  A sequence shorter than m is zero-padded to m rows like any other (l = 1):
  its first L_b landmarks are its rows, the rest are zero vectors, and B~
  spans its L_b keys.  An empty sequence (L_b = 0) has no output rows.

Parity pins: every function here is pinned in ``tests/test_oracle_pins.py``
against closed forms, brute force on tiny inputs, or library routines.
No function is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "segment_means",
    "row_softmax",
    "landmark_kernels",
    "pinv_init",
    "iterative_pinv",
    "depthwise_conv_skip",
    "nystrom_head",
    "nystrom_attention",
    "exact_attention",
    "approximation_error",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def segment_means(X, m):
    """Landmarks by segment means ([NF] "Landmark Selection: Segment-Means",
    Eq. 16, with the divisor read as the segment length; [HF] "How do we
    select landmarks?").

    X: (n, d), n >= 1, m >= 1.  X is first padded at its end with zero rows
    to n' = m * ceil(n/m) (the section assumes n divisible by m and says
    padding ensures it); with l = n'/m, row j of the result is the mean of
    padded rows j*l .. j*l+l-1.  For n divisible by m there is no pad; for
    n < m, l = 1 and rows n .. m-1 of the result are zero (landmarks of pad
    only, which only a key-padding mask produces: the unmasked entry point
    asks for m <= n).
    """
    X = _f64(X)
    n, d = X.shape
    if m < 1 or n < 1:
        raise ValueError("need m >= 1 and n >= 1")
    seg = -(-n // m)
    Xp = np.zeros((m * seg, d))
    Xp[:n] = X
    return Xp.reshape(m, seg, d).mean(axis=1)


def row_softmax(S):
    """Softmax along the last axis, subtracting the row maximum first
    ([NF] Eq. 2 / Eq. 13 apply softmax row-wise)."""
    S = _f64(S)
    E = np.exp(S - S.max(axis=-1, keepdims=True))
    return E / E.sum(axis=-1, keepdims=True)


def landmark_kernels(Q, K, Qt, Kt):
    """The three softmax kernels of [NF] Eq. 13 / [HF] "How can we adapt ...":

    F = softmax(Q Kt^T / sqrt(d))   (n x m)
    A = softmax(Qt Kt^T / sqrt(d))  (m x m)   -- before pseudo-inversion
    B = softmax(Qt K^T / sqrt(d))   (m x n)
    """
    Q, K, Qt, Kt = map(_f64, (Q, K, Qt, Kt))
    d = Q.shape[1]
    s = 1.0 / np.sqrt(d)
    F = row_softmax(s * (Q @ Kt.T))
    A = row_softmax(s * (Qt @ Kt.T))
    B = row_softmax(s * (Qt @ K.T))
    return F, A, B


def pinv_init(A):
    """Pan-Schreiber start Z0 = A^T / (||A||_1 ||A||_inf) ([NF] "Moore-Penrose
    Pseudoinverse Computation", initialisation scheme): ||A||_1 is the largest
    absolute column sum, ||A||_inf the largest absolute row sum."""
    A = _f64(A)
    norm_1 = np.abs(A).sum(axis=0).max()
    norm_inf = np.abs(A).sum(axis=1).max()
    return A.T / (norm_1 * norm_inf)


def iterative_pinv(A, iters):
    """Lemma 1 of [NF] ("Moore-Penrose Pseudoinverse Computation"):

    Z_{j+1} = 1/4 Z_j (13 I - A Z_j (15 I - A Z_j (7 I - A Z_j)))

    run exactly ``iters`` times from ``pinv_init(A)``.  ``iters = 0`` returns
    the start itself.
    """
    A = _f64(A)
    if iters < 0:
        raise ValueError("iters must be >= 0")
    I = np.eye(A.shape[0])
    Z = pinv_init(A)
    for _ in range(iters):
        AZ = A @ Z
        Z = 0.25 * Z @ (13.0 * I - AZ @ (15.0 * I - AZ @ (7.0 * I - AZ)))
    return Z


def depthwise_conv_skip(V, w):
    """Depthwise 1-D convolution skip on V ([NF] "Putting It Together",
    Figure 4's "DConv k x 1" path; [HF] "How do we select landmarks?").

    V: (n, d); w: (d, k), k odd.  out[i, c] = sum_t w[c, t] V[i + t - r, c],
    r = (k-1)/2, rows outside [0, n) read as zero (cross-correlation, "same"
    length, no bias).
    """
    V, w = _f64(V), _f64(w)
    n, d = V.shape
    dw, k = w.shape
    if dw != d or k % 2 == 0:
        raise ValueError("w must be (d, k) with k odd")
    r = (k - 1) // 2
    out = np.zeros((n, d))
    for t in range(k):
        shift = t - r  # output row i reads input row i + shift
        lo = max(0, -shift)
        hi = min(n, n - shift)
        if lo < hi:
            out[lo:hi] += V[lo + shift:hi + shift] * w[:, t]
    return out


def nystrom_head(Q, K, V, m, iters, w=None):
    """One (batch, head) of Nyström attention, step by step.

    Steps ([NF] section 3.2 "Big-picture architecture" and "Putting It
    Together", Eq. 17):
      1. Qt, Kt = segment means of Q and K (Eq. 16).
      2. F, A, B = the three softmax kernels (Eq. 13).
      3. Z = ``iters`` steps of Lemma 1 on A.
      4. BV = B V;  W = Z BV;  O = F W   (never forms n x n).
      5. O += DConv(V) if a filter is given.

    When n is not a multiple of m, step 1 sees the zero-padded sequence;
    step 2 takes the n real rows only, so the pad is masked out of B's keys
    and has no rows in F or O.

    Returns (O, dict of intermediates).
    """
    Q, K, V = map(_f64, (Q, K, V))
    Qt = segment_means(Q, m)
    Kt = segment_means(K, m)
    F, A, B = landmark_kernels(Q, K, Qt, Kt)
    Z = iterative_pinv(A, iters)
    BV = B @ V
    W = Z @ BV
    O_att = F @ W
    O = O_att.copy()
    if w is not None:
        O += depthwise_conv_skip(V, w)
    inter = dict(Qt=Qt, Kt=Kt, F=F, A=A, B=B, Z=Z, BV=BV, W=W, O_att=O_att)
    return O, inter


def nystrom_attention(Q, K, V, m, iters, conv_w=None, with_intermediates=False, lengths=None):
    """Nyström attention over a batch of heads.

    Q, K, V: (batch, heads, n, d).  conv_w: (heads, d, k) or None.
    lengths: None, or one sequence length per batch entry for a batch of
    right-padded sequences (a key-padding mask).  The pages leave masking
    out ([HF] "How is Nyströmformer implemented?"); the reading taken is
    that padding tokens are not part of the sequence: entry b is the method
    on its first L_b rows alone (with the zero padding to a multiple of m of
    ``segment_means`` when m does not divide L_b, to m rows when L_b < m),
    its rows L_b .. n-1 are never read, and its output rows there are zero.
    Each L_b is clamped to [0, n]; an entry with L_b = 0 has an all-zero
    output and NaN intermediates (it has no keys, so B~ is undefined).
    Returns O of shape (batch, heads, n, d) in fp64 and, if asked, a dict of
    stacked intermediates (each with leading (batch, heads) axes).
    """
    Q, K, V = map(_f64, (Q, K, V))
    Bt, H, n, d = Q.shape
    if lengths is None and m > n:
        raise ValueError("need m <= n without a key-padding mask")
    O = np.zeros((Bt, H, n, d))
    inter_all = {}
    shapes = dict(Qt=(m, d), Kt=(m, d), A=(m, m), Z=(m, m), BV=(m, d), W=(m, d))
    for b in range(Bt):
        L = n if lengths is None else int(min(max(int(lengths[b]), 0), n))
        if L == 0:
            if with_intermediates:
                for key, shp in shapes.items():
                    inter_all.setdefault(key, np.empty((Bt, H) + shp))[b] = np.nan
                inter_all.setdefault("O_att", np.zeros((Bt, H, n, d)))
            continue
        for h in range(H):
            w = None if conv_w is None else _f64(conv_w)[h]
            O[b, h, :L], inter = nystrom_head(Q[b, h, :L], K[b, h, :L], V[b, h, :L], m, iters, w)
            if with_intermediates:
                for key, val in inter.items():
                    if key in ("F", "B"):  # n x m / m x n: skipped to save memory
                        continue
                    if key == "O_att":  # rows past L_b stay zero, as in O
                        inter_all.setdefault(key, np.zeros((Bt, H, n, d)))[b, h, :L] = val
                    else:
                        inter_all.setdefault(key, np.empty((Bt, H) + val.shape))[b, h] = val
    if with_intermediates:
        return O, inter_all
    return O


def exact_attention(Q, K, V, row_chunk=1024):
    """Standard softmax attention softmax(Q K^T / sqrt(d)) V ([NF] Eq. 2),
    evaluated in row chunks so the n x n matrix is never held at once.

    Q: (..., nq, d) query rows (a subset of rows is allowed); K, V: (..., n, d).
    Used only to report how far the approximation is from exact attention,
    and for the m = n check of Lemma 2.
    """
    Q, K, V = map(_f64, (Q, K, V))
    lead = Q.shape[:-2]
    nq, d = Q.shape[-2:]
    n = K.shape[-2]
    Qf = Q.reshape((-1, nq, d))
    Kf = K.reshape((-1, n, d))
    Vf = V.reshape((-1, n, V.shape[-1]))
    out = np.empty(Vf.shape[:1] + (nq, V.shape[-1]))
    s = 1.0 / np.sqrt(d)
    for g in range(Qf.shape[0]):
        for i0 in range(0, nq, row_chunk):
            S = s * (Qf[g, i0:i0 + row_chunk] @ Kf[g].T)
            out[g, i0:i0 + row_chunk] = row_softmax(S) @ Vf[g]
    return out.reshape(lead + (nq, V.shape[-1]))


def approximation_error(Q, K, V, m, iters):
    """Per-(batch, head) relative error of the method's attention output
    against exact softmax attention ([NF] Eq. 2 for the exact output; the
    page's closing discussion proposes measuring ||S - S^|| per example):
    ||O_att - O_exact||_F / ||O_exact||_F, skip excluded (it is exact).

    Q, K, V: (batch, heads, n, d).  Returns (batch, heads) fp64."""
    Q, K, V = map(_f64, (Q, K, V))
    Bt, H = Q.shape[:2]
    err = np.empty((Bt, H))
    for b in range(Bt):
        for h in range(H):
            O, _ = nystrom_head(Q[b, h], K[b, h], V[b, h], m, iters)
            ex = exact_attention(Q[b, h], K[b, h], V[b, h])
            err[b, h] = np.linalg.norm(O - ex) / np.linalg.norm(ex)
    return err
