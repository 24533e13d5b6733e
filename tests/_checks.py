"""Parity checks of a device result against the oracle, finer than one norm.

One relative L2 over a whole tensor hides local damage: at 196,608 output
rows a 64-row tile written as zeros moves it by only sqrt(64 / 196608) ~ 0.018.
So every comparison here gates four figures for an array shaped
[..., rows, cols], whose leading axes are (batch, head) or a subset of them:

* ``rel``   relative L2 over the whole tensor (the method's stated measure);
* ``slice`` the largest relative L2 of one leading-axes slice, one (b, h);
* ``tile``  the largest relative L2 of one 64-row tile of a slice, where the
  tile's reference norm is floored at its even share of the slice's norm
  (sqrt(tile rows / rows) * ||ref slice||), so that a tile of near-zero
  values is not held to a relative bar it cannot meet;
* ``elem``  the largest ratio |got - ref| / (rtol |ref| + atol rms(ref slice))
  over all elements; it must stay <= 1.

NumPy only: the tests of the checker itself run on the CPU.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

TILE_ROWS = 64


@dataclass(frozen=True)
class Bars:
    """Gates for one quantity: relative L2 over the tensor and per slice
    (``rel``), per 64-row tile (``tile``), and the elementwise bound
    |d| <= rtol |ref| + atol rms(ref slice)."""
    rel: float
    tile: float
    rtol: float
    atol: float


def _as3(x):
    """View as [slices, rows, cols] (a 1-D array is one slice of one column)."""
    x = np.asarray(x, np.float64)
    if x.ndim == 1:
        return x.reshape(1, -1, 1)
    if x.ndim == 2:
        return x.reshape(1, *x.shape)
    return x.reshape(-1, *x.shape[-2:])


def parity_metrics(got, ref, tile_rows: int = TILE_ROWS, rtol: float = 0.0, atol: float = 0.0) -> dict:
    """The four figures described in the module docstring (``elem`` only when
    rtol or atol is positive), plus where the worst tile and element are."""
    g, r = _as3(got), _as3(ref)
    if g.shape != r.shape:
        raise ValueError(f"shape mismatch: {np.shape(got)} vs {np.shape(ref)}")
    d = g - r
    out = {}
    tot = float(np.linalg.norm(r))
    out["rel"] = float(np.linalg.norm(d) / max(tot, 1e-300))
    if not np.all(np.isfinite(g)):
        out.update(slice=np.inf, tile=np.inf, elem=np.inf, nonfinite=int(np.sum(~np.isfinite(g))))
        return out
    S, R, C = r.shape
    rn = np.sqrt(np.sum(r * r, axis=(1, 2)))
    dn = np.sqrt(np.sum(d * d, axis=(1, 2)))
    out["slice"] = float(np.max(np.where(dn == 0, 0.0, dn / np.maximum(rn, 1e-300))))
    nt = -(-R // tile_rows)
    pad = nt * tile_rows - R
    if pad:
        r = np.concatenate([r, np.zeros((S, pad, C))], axis=1)
        d = np.concatenate([d, np.zeros((S, pad, C))], axis=1)
    rt = np.sqrt(np.sum(r.reshape(S, nt, tile_rows, C) ** 2, axis=(2, 3)))
    dt = np.sqrt(np.sum(d.reshape(S, nt, tile_rows, C) ** 2, axis=(2, 3)))
    share = rn[:, None] * np.sqrt(min(tile_rows, R) / R)
    den = np.maximum(np.maximum(rt, share), 1e-300)
    tr = dt / den
    worst = np.unravel_index(int(np.argmax(tr)), tr.shape)
    out["tile"] = float(tr[worst])
    out["tile_at"] = (int(worst[0]), int(worst[1]) * tile_rows)
    if rtol > 0 or atol > 0:
        g3, r3 = _as3(got), _as3(ref)
        # rms over the rows that hold values (the all-zero rows of a padded
        # sequence would deflate it).
        live = np.maximum(np.sum(np.any(r3 != 0, axis=2), axis=1) * r3.shape[2], 1)
        rms = np.sqrt(np.sum(r3 * r3, axis=(1, 2)) / live)[:, None, None]
        bound = rtol * np.abs(r3) + atol * rms
        ratio = np.abs(g3 - r3) / np.maximum(bound, 1e-300)
        # Exact matches (zeros of masked rows included) never fail.
        ratio = np.where(g3 == r3, 0.0, ratio)
        at = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        out["elem"] = float(ratio[at])
        out["elem_at"] = tuple(int(i) for i in at)
    return out


def parity_failures(m: dict, bars: Bars) -> list:
    """Which gates ``m`` (from parity_metrics) fails under ``bars``."""
    bad = []
    if not m["rel"] <= bars.rel:
        bad.append(f"rel {m['rel']:.3e} > {bars.rel:.1e}")
    if not m["slice"] <= bars.rel:
        bad.append(f"slice {m['slice']:.3e} > {bars.rel:.1e}")
    if not m["tile"] <= bars.tile:
        bad.append(f"tile {m['tile']:.3e} > {bars.tile:.1e} at {m.get('tile_at')}")
    if "elem" in m and not m["elem"] <= 1.0:
        bad.append(f"elem {m['elem']:.3e} > 1 at {m.get('elem_at')}")
    return bad


class Gate:
    """Collects the figures and failures of several comparisons, so that one
    run reports every quantity before ``close`` raises for the failed ones."""

    def __init__(self, title: str, report=print):
        self.title, self.report, self.bad, self.figures = title, report, [], {}
        report(title)

    def __call__(self, name: str, got, ref, bars: Bars) -> dict:
        m = parity_metrics(got, ref, rtol=bars.rtol, atol=bars.atol)
        self.figures[name] = m
        self.report(f"  {name}: rel={m['rel']:.2e} slice={m['slice']:.2e} tile={m['tile']:.2e}"
                    + (f" elem={m['elem']:.2f}" if "elem" in m else ""))
        self.bad += [f"{name}: {b}" for b in parity_failures(m, bars)]
        return m

    def close(self) -> dict:
        assert not self.bad, f"{self.title}: " + "; ".join(self.bad)
        return self.figures


def check_parity(got, ref, bars: Bars, name: str = "", report=print) -> dict:
    """Gate one comparison; raises AssertionError naming every failed gate."""
    g = Gate(name, report)
    g(name, got, ref, bars)
    return g.close()[name]


# Output bars.  rel: the method's stated tolerances (relative L2 1e-4 for fp32
# I/O, 2e-2 for bf16 I/O), applied to the whole tensor and to every (b, h).
# tile: the same bar per 64-row tile (rounding errors are relative per element,
# so a tile's relative error is the tensor's up to sampling noise).
# Elementwise: the bf16 output is rounded to nearest (<= 2^-9 |x|) after fp32
# arithmetic whose single-bf16 attention products (F~ and W rounded to bf16)
# leave an error of order 2^-9 times the magnitude of the terms summed over
# the landmarks, which can exceed |O| where they cancel: measured up to
# 1.5e-2 rms(O) on the small parity shapes, so |d| <= 2^-7 |ref| + 3e-2 rms.
# fp32: every product keeps about 2^-17 or better (measured |d| up to about
# 1e-4 (|ref| + rms)), so |d| <= 2e-4 |ref| + 2e-4 rms(ref).
OUT_BARS = {
    "f32": Bars(rel=1e-4, tile=1e-4, rtol=2e-4, atol=2e-4),
    "bf16": Bars(rel=2e-2, tile=2e-2, rtol=2.0 ** -7, atol=3e-2),
}
