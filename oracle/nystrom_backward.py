"""CPU oracle for the gradients of the Nyströmformer self-attention forward
pass (fp64 NumPy).

TEST INFRASTRUCTURE ONLY, like the forward oracle beside it: only the test
suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it, and it shares nothing with the HIP library.

The pages do not print a backward pass.  They say the model is trained end to
end with the pseudoinverse iterations inside the graph, so that gradients flow
through the fixed number of Lemma-1 steps ([NF] "Moore-Penrose Pseudoinverse
Computation" and the complexity discussion of the iterations).  What is
computed here is therefore the exact derivative of the forward oracle
(``nystrom_head``) with respect to Q, K, V and the skip filters, taken by
reverse-mode differentiation of its steps in reverse order:

  O = F W + DConv(V),  W = Z BV,  BV = B V,  Z = Lemma-1 iterates of A,
  F, A, B = row softmaxes of s Q Kt^T, s Qt Kt^T, s Qt K^T,  Qt, Kt = segment means.

Readings taken where differentiation needs one (each listed in the design
notes):

* The Pan-Schreiber start Z0 = A^T / (||A||_1 ||A||_inf) divides by two
  maxima.  The derivative of a maximum is taken at its first maximiser (a
  subgradient; the entries of A are positive, so the absolute values are
  smooth).  For ||A||_inf the choice does not matter: every row of a softmax
  sums to 1, so that term is constant along a row and the softmax's backward
  removes it.
* Segment means with zero padding (n not a multiple of m): the gradient of
  landmark j goes to the real rows of segment j, divided by the padded length.
* The skip filters are shared by the batch: their gradient sums over batch
  entries and positions.
* Key-padding mask: as in the forward oracle, entry b is the method on its
  first L_b rows (zero-padded to m rows when L_b < m), so its gradients are
  the gradients of that problem, and zero on its pad rows.

Parity pins (``tests/test_oracle_backward_pins.py``): central finite
differences of the forward oracle, closed forms at Q = 0, the exact-attention
gradient at m = n with a converged pseudoinverse, and linearity in dO.
"""
from __future__ import annotations

import numpy as np

from .nystrom_oracle import iterative_pinv, landmark_kernels, pinv_init, segment_means

__all__ = [
    "softmax_rows_backward",
    "segment_means_backward",
    "pinv_backward",
    "conv_skip_backward",
    "nystrom_head_backward",
    "nystrom_attention_backward",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def softmax_rows_backward(P, dP):
    """Gradient of the scores of a row-wise softmax P, given dL/dP:
    dS = P * (dP - rowsum(dP * P))."""
    P, dP = _f64(P), _f64(dP)
    return P * (dP - (dP * P).sum(axis=-1, keepdims=True))


def segment_means_backward(dXt, n):
    """Gradient of ``segment_means`` (n rows, zero padding to m*ceil(n/m)):
    real row i receives dXt[i // l] / l with l = ceil(n/m)."""
    dXt = _f64(dXt)
    m, d = dXt.shape
    seg = -(-n // m)
    rows = np.arange(n) // seg
    return dXt[rows] / seg


def pinv_backward(A, iters, dZ):
    """Gradient with respect to A of ``iterative_pinv(A, iters)``, given dL/dZ.

    The forward iterates are recomputed; each step
      X = A Z_k, P1 = 7I - X, T1 = X P1, P2 = 15I - T1, T2 = X P2,
      P3 = 13I - T2, Z_{k+1} = Z_k P3 / 4
    is differentiated in reverse, then the start Z0 = c A^T with
    c = 1 / (max column sum * max row sum)."""
    A, dZ = _f64(A), _f64(dZ)
    m = A.shape[0]
    I = np.eye(m)
    Zs = [pinv_init(A)]
    for _ in range(iters):
        Zk = Zs[-1]
        X = A @ Zk
        Zs.append(0.25 * Zk @ (13.0 * I - X @ (15.0 * I - X @ (7.0 * I - X))))
    dA = np.zeros_like(A)
    for k in reversed(range(iters)):
        Zk = Zs[k]
        X = A @ Zk
        P1 = 7.0 * I - X
        T1 = X @ P1
        P2 = 15.0 * I - T1
        T2 = X @ P2
        P3 = 13.0 * I - T2
        dZk = 0.25 * dZ @ P3.T          # through the factor Z_k
        dT2 = -0.25 * Zk.T @ dZ         # through P3 = 13I - T2
        dX = dT2 @ P2.T                 # T2 = X P2
        dT1 = -(X.T @ dT2)              # P2 = 15I - T1
        dX += dT1 @ P1.T                # T1 = X P1
        dX -= X.T @ dT1                 # P1 = 7I - X
        dA += dX @ Zk.T                 # X = A Z_k
        dZk += A.T @ dX
        dZ = dZk
    col = A.sum(axis=0)
    row = A.sum(axis=1)
    n1, ninf = col.max(), row.max()
    c = 1.0 / (n1 * ninf)
    dA += c * dZ.T
    dc = float((dZ * A.T).sum())
    dA[:, int(np.argmax(col))] += dc * (-c / n1)
    dA[int(np.argmax(row)), :] += dc * (-c / ninf)
    return dA


def conv_skip_backward(V, w, dO):
    """Gradients of ``depthwise_conv_skip(V, w)`` given dL/dout: returns
    (dV, dw).  out[i, c] = sum_t w[c, t] V[i + t - r, c] gives
    dV[j, c] = sum_t w[c, t] dO[j - t + r, c] and
    dw[c, t] = sum_i dO[i, c] V[i + t - r, c] (rows outside [0, n) are zero)."""
    V, w, dO = _f64(V), _f64(w), _f64(dO)
    n, d = V.shape
    k = w.shape[1]
    r = (k - 1) // 2
    dV = np.zeros((n, d))
    dw = np.zeros((d, k))
    for t in range(k):
        shift = t - r
        lo, hi = max(0, -shift), min(n, n - shift)
        if lo < hi:
            dV[lo + shift:hi + shift] += dO[lo:hi] * w[:, t]
            dw[:, t] += (dO[lo:hi] * V[lo + shift:hi + shift]).sum(axis=0)
    return dV, dw


def nystrom_head_backward(Q, K, V, m, iters, dO, w=None):
    """Gradients of one (batch, head) of ``nystrom_head`` with respect to Q,
    K, V (and the filters w if given), for the upstream gradient dO = dL/dO.

    Returns (dQ, dK, dV, dw or None)."""
    Q, K, V, dO = map(_f64, (Q, K, V, dO))
    n, d = Q.shape
    s = 1.0 / np.sqrt(d)
    Qt, Kt = segment_means(Q, m), segment_means(K, m)
    F, A, B = landmark_kernels(Q, K, Qt, Kt)
    Z = iterative_pinv(A, iters)
    BV = B @ V
    W = Z @ BV
    # O_att = F W
    dW = F.T @ dO
    dF = dO @ W.T
    # W = Z BV
    dZ = dW @ BV.T
    dBV = Z.T @ dW
    # BV = B V
    dB = dBV @ V.T
    dV = B.T @ dBV
    # the three softmaxes
    dSF = softmax_rows_backward(F, dF)
    dSB = softmax_rows_backward(B, dB)
    dSA = softmax_rows_backward(A, pinv_backward(A, iters, dZ))
    dQ = s * dSF @ Kt
    dKt = s * dSF.T @ Q + s * dSA.T @ Qt
    dQt = s * dSB @ K + s * dSA @ Kt
    dK = s * dSB.T @ Qt
    # segment means
    dQ += segment_means_backward(dQt, n)
    dK += segment_means_backward(dKt, n)
    dw = None
    if w is not None:
        dVc, dw = conv_skip_backward(V, w, dO)
        dV += dVc
    return dQ, dK, dV, dw


def nystrom_attention_backward(Q, K, V, m, iters, dO, conv_w=None, lengths=None):
    """Batched gradients: Q, K, V, dO of shape (batch, heads, n, d), conv_w
    (heads, d, k) or None.  Returns (dQ, dK, dV, dconv_w or None); dconv_w
    sums over the batch.

    lengths: None, or one sequence length per batch entry, as for the
    forward oracle's key-padding mask.  Entry b's forward is the method on
    its first L_b rows alone, so its gradients are those of that shorter
    problem on rows 0 .. L_b-1 and exactly zero on the pad rows, whose
    values (and dO there) are never read; an empty entry contributes nothing,
    to the filter gradient included."""
    Q, K, V, dO = map(_f64, (Q, K, V, dO))
    Bt, H, n, d = Q.shape
    dQ, dK, dV = (np.zeros((Bt, H, n, d)) for _ in range(3))
    dW = None if conv_w is None else np.zeros(np.shape(conv_w))
    for b in range(Bt):
        L = n if lengths is None else int(min(max(int(lengths[b]), 0), n))
        if L == 0:
            continue
        for h in range(H):
            w = None if conv_w is None else _f64(conv_w)[h]
            dQ[b, h, :L], dK[b, h, :L], dV[b, h, :L], dw = nystrom_head_backward(
                Q[b, h, :L], K[b, h, :L], V[b, h, :L], m, iters, dO[b, h, :L], w)
            if dw is not None:
                dW[h] += dw
    return dQ, dK, dV, dW
