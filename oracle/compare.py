"""Result comparison used by the parity tests, smoke() and the bench's check.

TEST INFRASTRUCTURE ONLY (see ``oracle/interpreter.py``).

Matching rule:

* exact class (the last writer of the element is COPY, GATHER, ADD, MUL,
  SCALE, RELU or ROPE, or the element was never written): the bit patterns
  must be equal, except that any NaN matches any NaN;
* tolerance class (EXP, reductions, dot products, SILU_MUL): both values must
  have the same class (NaN, +inf, -inf, finite) and finite values must satisfy
  ``|g - o| <= max(rtol * max(|o|, s), 2 * u)`` where ``s`` is the oracle's
  error scale for the element (sum of |terms| for sums and dot products),
  ``rtol`` is 1e-5 for fp32 outputs, 1e-2 for bf16 and 2e-3 for fp16 (two
  units in the last place of an 11-bit significand), and ``u`` is the
  spacing of the output type's subnormal numbers (2**-149 for fp32, 2**-133
  for bf16, 2**-24 for fp16).  Below the normal range a format keeps a fixed absolute
  spacing and ever fewer significant bits, so no relative bound is reachable
  there; a result within two subnormal steps of the exact value is accepted.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .interpreter import bf16_to_f32

RTOL = {"f32": 1e-5, "bf16": 1e-2, "f16": 2e-3}
# spacing of the subnormal numbers of each output type
SUBNORMAL_STEP = {"f32": 2.0 ** -149, "bf16": 2.0 ** -133, "f16": 2.0 ** -24}


@dataclass
class Mismatch:
    count: int
    total: int
    first_index: int = -1
    got: float = 0.0
    want: float = 0.0
    worst_rel: float = 0.0

    @property
    def ok(self) -> bool:
        return self.count == 0

    def __str__(self) -> str:
        if self.ok:
            return f"ok ({self.total} elements, worst rel {self.worst_rel:.3g})"
        return (f"{self.count}/{self.total} mismatches; first at {self.first_index}: "
                f"got {self.got!r} want {self.want!r}; worst rel {self.worst_rel:.3g}")


def _as_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_to_f32(a)
    if dtype == "i32":
        return a.astype(np.float64)
    return a.astype(np.float32)


def compare(got: np.ndarray, want: np.ndarray, dtype: str,
            scale: Optional[np.ndarray] = None, rtol: Optional[float] = None) -> Mismatch:
    """Compares a GPU buffer with the oracle's buffer element by element."""
    got = np.asarray(got)
    want = np.asarray(want)
    if got.shape != want.shape:
        raise ValueError(f"shape {got.shape} vs {want.shape}")
    total = got.shape[0]
    if rtol is None:
        rtol = RTOL.get(dtype, 0.0)
    if scale is None:
        tol_mask = np.zeros(total, bool)
    else:
        tol_mask = ~np.isnan(scale)
    bad = np.zeros(total, bool)
    worst = 0.0
    # exact elements: bit equality, NaN == NaN
    ex = ~tol_mask
    if ex.any():
        if dtype == "i32":
            bad[ex] = got[ex] != want[ex]
        else:
            bits = np.uint16 if dtype in ("bf16", "f16") else np.uint32
            g = got.view(bits)[ex]
            w = want.view(bits)[ex]
            gf = _as_f32(got[ex], dtype)
            wf = _as_f32(want[ex], dtype)
            both_nan = np.isnan(gf) & np.isnan(wf)
            bad[ex] = (g != w) & ~both_nan
    if tol_mask.any():
        gf = _as_f32(got[tol_mask], dtype).astype(np.float64)
        wf = _as_f32(want[tol_mask], dtype).astype(np.float64)
        s = scale[tol_mask]
        cls_g = np.where(np.isnan(gf), 0, np.where(np.isposinf(gf), 1, np.where(np.isneginf(gf), 2, 3)))
        cls_w = np.where(np.isnan(wf), 0, np.where(np.isposinf(wf), 1, np.where(np.isneginf(wf), 2, 3)))
        fin = (cls_g == 3) & (cls_w == 3)
        err = np.zeros_like(gf)
        with np.errstate(invalid="ignore"):
            bound = rtol * np.maximum(np.abs(wf), np.where(np.isfinite(s), s, 0.0))
            bound = np.maximum(bound, 2.0 * SUBNORMAL_STEP.get(dtype, 0.0))
            err[fin] = np.abs(gf[fin] - wf[fin])
            rel = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
        b = (cls_g != cls_w) | (fin & (err > bound))
        bad[tol_mask] = b
        if fin.any():
            worst = float(np.max(rel[fin]) * rtol)
    cnt = int(bad.sum())
    if cnt:
        i = int(np.argmax(bad))
        return Mismatch(cnt, total, i, float(_as_f32(got[i:i + 1], dtype)[0]),
                        float(_as_f32(want[i:i + 1], dtype)[0]), worst)
    return Mismatch(0, total, worst_rel=worst)


@dataclass
class EndToEnd:
    """Outcome of an end-to-end comparison of a final buffer.

    ``count`` elements lie outside the bound, ``bit_equal`` are bit-identical
    (any NaN matching any NaN), ``rel_l2`` is ||g - o||_2 / ||o||_2 over the
    elements finite on both sides and ``max_rel`` the largest |g - o| / |o|
    there (0 where both are 0)."""

    count: int
    total: int
    bit_equal: int
    rel_l2: float
    max_rel: float

    @property
    def fraction(self) -> float:
        return self.count / self.total if self.total else 0.0

    def __str__(self) -> str:
        return (f"{self.count}/{self.total} outside the bound ({self.fraction:.3%}), "
                f"{self.bit_equal} bit-identical, rel L2 {self.rel_l2:.3g}, max rel {self.max_rel:.3g}")


def end_to_end(got: np.ndarray, want: np.ndarray, dtype: str, rtol: Optional[float] = None) -> EndToEnd:
    """Compares a final buffer of a long queue with the oracle's run of the
    same queue.  Every element, whichever op wrote it last, must satisfy the
    relative bound of its type, ``|g - o| <= rtol * |o|`` (two subnormal steps
    near zero) with the same class (NaN, +inf, -inf, finite): along a chain of
    ops, the rounding differences that tolerance-class ops are allowed reach
    the later exact ops too, so the exact-class bit test does not apply to
    them.  The caller states how many elements may fall outside the bound."""
    got = np.asarray(got)
    want = np.asarray(want)
    m = compare(got, want, dtype, np.zeros(got.shape[0]), rtol)
    gf = _as_f32(got, dtype).astype(np.float64)
    wf = _as_f32(want, dtype).astype(np.float64)
    if dtype == "i32":
        same = got == want
    else:
        bits = np.uint16 if dtype in ("bf16", "f16") else np.uint32
        same = (got.view(bits) == want.view(bits)) | (np.isnan(gf) & np.isnan(wf))
    fin = np.isfinite(gf) & np.isfinite(wf)
    diff = np.abs(gf[fin] - wf[fin])
    ref = np.abs(wf[fin])
    norm = float(np.sqrt(np.sum(ref * ref)))
    rel_l2 = float(np.sqrt(np.sum(diff * diff))) / norm if norm > 0 else float(np.any(diff > 0))
    with np.errstate(invalid="ignore", divide="ignore"):
        rel = np.where(ref > 0, diff / np.where(ref > 0, ref, 1.0), np.where(diff > 0, np.inf, 0.0))
    return EndToEnd(m.count, m.total, int(same.sum()), rel_l2, float(rel.max()) if rel.size else 0.0)
