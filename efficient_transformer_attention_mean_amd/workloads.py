"""Seeded synthetic workloads for Nyström attention.

This module only draws random inputs and rounds them to the I/O precision.
It holds none of the method's arithmetic, so both the HIP path (through the
tests and the bench) and the CPU oracle can be fed from it.

The shapes are those of the workloads the method is measured on: random
Q/K/V tensors (the paper's efficiency table times the attention module alone
on random inputs), a BERT-base-shaped layer, long sequences, and a stress
case with sharpened keys.  No dataset is used or imitated.

Recipe (fixed, so every run sees the same numbers):
  rng = numpy.random.default_rng(seed)
  Q, K, V = three draws of rng.standard_normal((batch, heads, n, d)), in order
  conv_w  = rng.normal(0, 0.02, (heads, d, k))          (if the workload has a skip)
  sharpen: for each (b, h) in order, idx = rng.choice(n, n // 10, replace=False),
           K[b, h, idx] *= 4                              (stress workload only)
  then every tensor is rounded to fp32 (or to bf16, round-to-nearest-even).
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_inputs", "round_to_bf16", "bf16_bits", "bf16_bits_to_f32"]


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    n: int
    d: int
    m: int
    iters: int
    conv_k: int          # 0 = no depthwise-conv skip
    dtype: str           # "f32" or "bf16": the I/O precision of Q, K, V and the output
    seed: int
    sharpen_keys: bool = False
    note: str = ""

    @property
    def heads_total(self) -> int:
        return self.batch * self.heads

    @property
    def tokens(self) -> int:
        return self.batch * self.n

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def compulsory_bytes(self) -> int:
        """Read Q, K, V once and write O once, plus the conv weights."""
        b = 4 * self.batch * self.heads * self.n * self.d * self.elem_bytes
        if self.conv_k:
            b += 4 * self.heads * self.d * self.conv_k
        return b

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 64, 16, 8, 6, 0, "f32", 0,
                     note="tiny fp32 case, segment length 8, no skip"),
    "tiny_m_eq_n": Workload("tiny_m_eq_n", 1, 1, 64, 16, 64, 30, 0, "f32", 0,
                            note="m = n = 64: with a converged pseudoinverse this is exact attention"),
    "bert": Workload("bert", 8, 12, 512, 64, 64, 6, 33, "f32", 1,
                     note="BERT-base-shaped layer, fp32 I/O"),
    "bert_bf16": Workload("bert_bf16", 8, 12, 512, 64, 64, 6, 33, "bf16", 1,
                          note="BERT-base-shaped layer, bf16 I/O"),
    "long": Workload("long", 4, 12, 4096, 64, 64, 6, 33, "bf16", 2,
                     note="long sequence, bf16 I/O"),
    "headline": Workload("headline", 2, 12, 8192, 64, 64, 6, 33, "bf16", 3,
                         note="n=8192, m=64, d=64, bf16 I/O"),
    "headline_ragged": Workload("headline_ragged", 2, 12, 8191, 64, 64, 6, 33, "bf16", 3,
                                note="the headline shape less one row: m does not divide n"),
    "headline_m32": Workload("headline_m32", 2, 12, 8192, 64, 32, 6, 33, "bf16", 3,
                             note="n=8192, m=32, d=64, bf16 I/O"),
    "stress": Workload("stress", 1, 16, 32768, 128, 256, 8, 33, "bf16", 4, sharpen_keys=True,
                       note="n=32768, d=128, m=256; 10% of key rows scaled by 4"),
}


def round_to_bf16(x) -> np.ndarray:
    """Round to the nearest bf16 value (ties to even); returned as float32."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = ((u + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    return u.view(np.float32).reshape(f.shape)


def bf16_bits(x) -> np.ndarray:
    """The bf16 bit patterns (uint16) of values already representable in bf16."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("values are not bf16-representable; round them first")
    return (u >> 16).astype(np.uint16).reshape(f.shape)


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).reshape(b.shape)


def make_inputs(wl: Workload, seed: int | None = None):
    """Draw the workload's inputs.

    Returns a dict with float32 arrays Q, K, V of shape (batch, heads, n, d)
    whose values are exactly representable in ``wl.dtype``, and ``conv_w``
    (heads, d, k) float32 or None.
    """
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    shape = (wl.batch, wl.heads, wl.n, wl.d)
    Q = rng.standard_normal(shape)
    K = rng.standard_normal(shape)
    V = rng.standard_normal(shape)
    conv_w = None
    if wl.conv_k:
        conv_w = rng.normal(0.0, 0.02, (wl.heads, wl.d, wl.conv_k)).astype(np.float32)
    if wl.sharpen_keys:
        for b in range(wl.batch):
            for h in range(wl.heads):
                idx = rng.choice(wl.n, wl.n // 10, replace=False)
                K[b, h, idx] *= 4.0
    out = {}
    for name, X in (("Q", Q), ("K", K), ("V", V)):
        X32 = X.astype(np.float32)
        out[name] = round_to_bf16(X32) if wl.dtype == "bf16" else X32
    out["conv_w"] = conv_w
    return out
