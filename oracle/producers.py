"""CPU oracle for the producer-fused int8 linear: the op that produces X
(RMSNorm with adaptive modulation, or tanh-form GELU) followed by the LLM.int8
linear of ``w8ref`` with a bias added to the output.

TEST INFRASTRUCTURE, like ``w8ref``: only the test suite, ``smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; it shares no code with the
HIP path.

X is the 16-bit value (the type of H) that a separate producer op would store:

  RMSNorm + modulation (RMSNorm: Zhang and Sennrich, 2019; the x(1+scale)+shift
  modulation of adaptive layer norm: Peebles and Xie, "Scalable Diffusion
  Models with Transformers", 2023), a fixed sequence of float32 operations,
  each rounded to nearest even, none fused:
      ss   = sum_k h[m,k]^2, the exact sum rounded once to float64
      ms   = fl32(ss / K)                   (float64 division, then to float32)
      rstd = fl32(1 / fl32(sqrt(fl32(ms + eps))))
      w[k] = fl32(gamma[k] * fl32(1 + scale[k]))
      x    = fl32(fl32(h * rstd) * w[k]),  then  x = fl32(x + shift[k])
  gamma, scale, shift may each be absent (1, 0, no addition); X = x rounded to
  nearest even in the 16-bit type.

  GELU, tanh form (Hendrycks and Gimpel, "Gaussian Error Linear Units", 2016):
      gelu(h) = 0.5 h (1 + tanh(u)) = h / (1 + exp(-2u)),
      u = sqrt(2/pi) (h + 0.044715 h^3),
  and X = gelu(h) correctly rounded (to nearest, ties to even) in the 16-bit
  type: a function of the 16-bit input alone, evaluated here with 60-digit
  decimal arithmetic and an exact rounding step.

The sum of squares is taken exactly (math.fsum rounds the exact sum once), so
ss does not depend on a summation order. A kernel that adds the squares in
float64 in its own order may land on the neighbouring float64 value; when that
moves rstd, both rstd values are correct readings of the definition above, and
the tests accept exactly those rows (see ``rstd_alternatives``).
"""
from __future__ import annotations

import decimal
import math
from decimal import Decimal

import numpy as np

from . import w8ref

F32 = np.float32

# ---------------------------------------------------------------------------
# GELU, correctly rounded to the 16-bit type
# ---------------------------------------------------------------------------

_CTX = decimal.Context(prec=60, Emin=-10 ** 6, Emax=10 ** 6)


def _pi() -> Decimal:
    """pi to the context's precision by Machin's formula,
    pi = 16 atan(1/5) - 4 atan(1/239), each arctangent by its Taylor series."""
    with decimal.localcontext(_CTX) as ctx:
        ctx.prec += 10

        def atan_inv(n: int) -> Decimal:
            x2 = Decimal(n * n)
            term = Decimal(1) / n
            total, k, sign = term, 1, -1
            eps = Decimal(10) ** -(ctx.prec + 2)
            while True:
                term /= x2
                t = term / (2 * k + 1)
                if t < eps:
                    return total
                total += sign * t
                sign, k = -sign, k + 1

        return +(16 * atan_inv(5) - 4 * atan_inv(239))


_SQRT_2_OVER_PI = None


def gelu_decimal(h: float) -> Decimal:
    """tanh-form GELU of a finite float, as h / (1 + exp(-2u)) in 60-digit
    decimal arithmetic (h itself converts exactly)."""
    global _SQRT_2_OVER_PI
    with decimal.localcontext(_CTX):
        if _SQRT_2_OVER_PI is None:
            _SQRT_2_OVER_PI = (Decimal(2) / _pi()).sqrt()
        d = Decimal(h)
        if d == 0:
            return d                                        # keeps the sign of zero
        u = _SQRT_2_OVER_PI * (d + Decimal("0.044715") * d * d * d)
        a = -2 * u
        if a > 5000:                                        # exp(a) > 10^2000: |gelu| < |h| 10^-2000
            return Decimal(0).copy_sign(d)                  # -> a signed zero after rounding
        if a < -5000:                                       # exp(a) < 10^-2000: gelu = h (1 - tiny),
            return d                                        # which rounds to h itself
        return d / (1 + a.exp())


def _bits16_value(bits: int, dtype: str) -> float:
    return float(w8ref.decode16(np.array([bits], np.uint16), dtype)[0])


def round_decimal_to16(g: Decimal, dtype: str) -> int:
    """Bits of the 16-bit value nearest to ``g`` (ties to the even pattern).

    A float64 first guess rounded to the 16-bit type can be off by one step
    (double rounding), so the guess and its two neighbours are compared with
    ``g`` exactly."""
    with decimal.localcontext(decimal.Context(prec=2000, Emin=-10 ** 6, Emax=10 ** 6)):
        # every difference below is exact at this precision (the 16-bit
        # values have at most a few hundred significant decimal digits)
        return _round_decimal_to16_exact(g, dtype)


def _round_decimal_to16_exact(g: Decimal, dtype: str) -> int:
    neg = g.is_signed()
    a = abs(g)
    guess = float(a)
    if dtype == "f16":
        with np.errstate(over="ignore"):
            c = int(np.array([guess], np.float64).astype(np.float16).view(np.uint16)[0])
        top = 0x7C00                                        # +inf
    else:
        c = int(w8ref.round_to_bf16(np.array([guess]))[0])
        top = 0x7F80
    best, best_d = None, None
    for b in (c - 1, c, c + 1):
        if b < 0 or b > top:
            continue
        v = _bits16_value(b, dtype)
        d = abs(Decimal(v) - a) if math.isfinite(v) else None
        if d is None:
            continue
        if best is None or d < best_d or (d == best_d and b % 2 == 0):
            best, best_d = b, d
    if best == top - 1 and a > Decimal(_bits16_value(top - 1, dtype)):
        # beyond the largest finite value: overflow to inf when past the
        # midpoint to the next (unrepresentable) step
        step = Decimal(_bits16_value(top - 1, dtype)) - Decimal(_bits16_value(top - 2, dtype))
        if a >= Decimal(_bits16_value(top - 1, dtype)) + step / 2:
            best = top
    return best | (0x8000 if neg else 0)


_GELU_TABLE: dict = {}


def gelu16(h_bits: np.ndarray, dtype: str) -> np.ndarray:
    """X bits = gelu(H) correctly rounded in H's 16-bit type, element by
    element (a function of the 16-bit pattern; evaluated once per distinct
    pattern). NaN and infinite inputs are outside the contract."""
    h_bits = np.ascontiguousarray(h_bits, dtype=np.uint16)
    table = _GELU_TABLE.setdefault(dtype, {})
    uniq = np.unique(h_bits)
    vals = w8ref.decode16(uniq, dtype)
    assert np.all(np.isfinite(vals)), "non-finite input"
    for b, v in zip(uniq.tolist(), vals.tolist()):
        if b not in table:
            table[b] = round_decimal_to16(gelu_decimal(v), dtype)
    out = np.array([table[b] for b in uniq.tolist()], dtype=np.uint16)
    return out[np.searchsorted(uniq, h_bits)]


def _rstd_of_ss(ss: np.ndarray, K: int, eps: float) -> np.ndarray:
    """rstd = fl32(1 / fl32(sqrt(fl32(fl32(ss / K) + eps)))) of float64 sums."""
    ms = (np.asarray(ss, np.float64) / K).astype(F32)
    v = (ms + F32(eps)).astype(F32)
    return (F32(1.0) / np.sqrt(v).astype(F32)).astype(F32)


def rstd_alternatives(h: np.ndarray, eps: float = 1e-6):
    """(rstd_a, rstd_b) float32 [M]: the rstd values that a float64 sum of a
    row's squares, added in any order, can lead to. The squares are positive,
    so any order's sum lies within (K-1) 2^-53 / (1 - (K-1) 2^-53) of the exact
    sum (Higham, "Accuracy and Stability of Numerical Algorithms", 2002,
    section 4.2); rstd is monotone in ss, so the ends of that interval give
    the only candidates (equal on almost every row)."""
    h = np.asarray(h, dtype=F32)
    K = h.shape[1]
    S = np.array([math.fsum(r) for r in (h.astype(np.float64) ** 2)], dtype=np.float64)
    g = (K - 1) * 2.0 ** -53
    g = g / (1.0 - g)
    lo = np.nextafter(S * (1.0 - g), -np.inf)
    hi = np.nextafter(S * (1.0 + g), np.inf)
    return _rstd_of_ss(hi, K, eps), _rstd_of_ss(lo, K, eps)


def rmsnorm_modulate32(h: np.ndarray, gamma=None, scale=None, shift=None, eps: float = 1e-6, rstd=None):
    """RMSNorm with modulation of float32 rows [M, K]; returns (x float32 [M, K],
    rstd float32 [M]). ``rstd``: use these per-row values instead (one of the
    readings ``rstd_alternatives`` allows)."""
    h = np.asarray(h, dtype=F32)
    K = h.shape[1]
    # each square of a 16-bit value is exact in float64; fsum rounds the
    # exact sum of the row once
    if rstd is None:
        ss = np.array([math.fsum(r) for r in (h.astype(np.float64) ** 2)], dtype=np.float64)
        rstd = _rstd_of_ss(ss, K, eps)
    rstd = np.asarray(rstd, dtype=F32)
    one = np.ones(K, dtype=F32)
    g = one if gamma is None else np.asarray(gamma, dtype=F32)
    sc = np.zeros(K, dtype=F32) if scale is None else np.asarray(scale, dtype=F32)
    w = (g * (F32(1.0) + sc).astype(F32)).astype(F32)
    x = (h * rstd[:, None]).astype(F32)
    x = (x * w[None, :]).astype(F32)
    if shift is not None:
        x = (x + np.asarray(shift, dtype=F32)[None, :]).astype(F32)
    return x, rstd


def to16(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> 16-bit patterns, round to nearest even (single rounding)."""
    x64 = np.asarray(x, dtype=F32).astype(np.float64)
    return w8ref.round_to_bf16(x64) if dtype == "bf16" else w8ref.round_to_f16(x64)


def produce(h_bits, h_dtype: str, kind: str, gamma=None, scale=None, shift=None, eps: float = 1e-6, rstd=None):
    """X (16-bit patterns, the type of H) from H by producer ``kind``:
    "none", "rmsnorm" or "gelu". ``rstd``: RMSNorm's per-row values, if given."""
    h = w8ref.decode16(h_bits, h_dtype)
    if kind == "none":
        return np.ascontiguousarray(h_bits, dtype=np.uint16)
    if kind == "rmsnorm":
        x, _ = rmsnorm_modulate32(h, gamma, scale, shift, eps, rstd)
    elif kind == "gelu":
        return gelu16(h_bits, h_dtype)
    else:
        raise ValueError(kind)
    return to16(x, h_dtype)


def fused_int8_linear(h_bits, h_dtype, kind, wq, sw, threshold, bias=None, out_dtype="f16", rows=None,
                      gamma=None, scale=None, shift=None, eps: float = 1e-6, x_bits=None):
    """Y = producer(H) W^T + bias under the LLM.int8 decomposition.

    The producer gives X exactly as a separate producer op would store it (16-bit);
    the linear is ``w8ref.int8_mixed_linear``; bias (float32 [N]) is added to the
    float64 result before the single final rounding. ``x_bits``: X already made
    by ``produce`` with the same arguments (saves recomputing it)."""
    if x_bits is None:
        x_bits = produce(h_bits, h_dtype, kind, gamma, scale, shift, eps)
    ref = w8ref.int8_mixed_linear(x_bits, h_dtype, wq, sw, threshold, out_dtype, rows=rows)
    y = ref["y"]
    if bias is not None:
        y = y + np.asarray(bias, dtype=F32).astype(np.float64)[None, :]
    ref = dict(ref)
    ref["x_bits"] = x_bits
    ref["y"] = y
    ref["Y"] = w8ref.round_output(y, out_dtype)
    return ref
