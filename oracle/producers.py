"""CPU oracle for the producer-fused int8 linear: the op that produces X
(RMSNorm with adaptive modulation, or tanh-form GELU) followed by the LLM.int8
linear of ``w8ref`` with a bias added to the output.

TEST INFRASTRUCTURE, like ``w8ref``: only the test suite, ``smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; it shares no code with the
HIP path.

The producers are defined in float32, the precision the library computes
them in, as a fixed sequence of single IEEE operations (each rounded to
nearest even, none fused), so that the 16-bit X they produce, and with it
every int8 code, is reproduced exactly:

  RMSNorm + modulation (RMSNorm: Zhang and Sennrich, 2019; the x(1+scale)+shift
  modulation of adaptive layer norm: Peebles and Xie, "Scalable Diffusion
  Models with Transformers", 2023):
      ss   = sum_k h[m,k]^2                 (float64; each square is exact)
      ms   = fl32(ss / K)                   (float64 division, then to float32)
      rstd = fl32(1 / fl32(sqrt(fl32(ms + eps))))
      w[k] = fl32(gamma[k] * fl32(1 + scale[k]))
      x    = fl32(fl32(h * rstd) * w[k]),  then  x = fl32(x + shift[k])
  gamma, scale, shift may each be absent (1, 0, no addition).

  GELU, tanh form (Hendrycks and Gimpel, "Gaussian Error Linear Units", 2016):
      gelu(h) = h / (1 + exp(-2u)),  u = sqrt(2/pi) (h + 0.044715 h^3),
  which equals 0.5 h (1 + tanh(u)) and stays accurate for negative h; exp is
  the Cody-Waite reduced Taylor form of ``exp32`` below.

X is then the producer's float32 result rounded to nearest even in the 16-bit
type of H. Parity of the float32 definitions with the true functions is pinned
separately against float64 references.
"""
from __future__ import annotations

import numpy as np

from . import w8ref

F32 = np.float32

# exp32: exp(x) = 2^k * p(r), k = rint(x * log2(e)), r = x - k*ln2 computed in
# two parts (Cody and Waite, "Software Manual for the Elementary Functions",
# 1980): LN2_HI has 9 significant bits, so k * LN2_HI is exact for |k| < 2^15;
# p is the degree-6 Taylor polynomial of exp on |r| <= ln(2)/2 (truncation
# below 1.2e-7 relative), evaluated by Horner's rule.
LOG2E = F32(1.4426950408889634)
LN2_HI = F32(0.693359375)
LN2_LO = F32(-2.12194440e-4)
EXP_COEF = [F32(1.0 / 720.0), F32(1.0 / 120.0), F32(1.0 / 24.0), F32(1.0 / 6.0), F32(0.5), F32(1.0), F32(1.0)]
GELU_C = F32(0.7978845608028654)      # sqrt(2 / pi)
GELU_A = F32(0.044715)


def exp32(x: np.ndarray) -> np.ndarray:
    """exp of float32 values, in float32 operations in the order above."""
    x = np.asarray(x, dtype=F32)
    with np.errstate(over="ignore", under="ignore", invalid="ignore"):
        k = np.rint(x * LOG2E).astype(F32)
        r = (x - k * LN2_HI).astype(F32)
        r = (r - k * LN2_LO).astype(F32)
        p = EXP_COEF[0]
        for c in EXP_COEF[1:]:
            p = ((p * r).astype(F32) + c).astype(F32)
        # 2^k p: clamp k to keep ldexp in range; results then overflow to inf
        # or underflow to 0 exactly as the scaled value would
        kk = np.clip(k, -300, 300).astype(np.int32)
        out = np.ldexp(p.astype(F32), kk).astype(F32)
    return out


def gelu32(h: np.ndarray) -> np.ndarray:
    """tanh-form GELU of float32 values, float32 operations in fixed order."""
    h = np.asarray(h, dtype=F32)
    with np.errstate(over="ignore", under="ignore", invalid="ignore"):
        h3 = ((h * h).astype(F32) * h).astype(F32)
        inner = (h + (GELU_A * h3).astype(F32)).astype(F32)
        u = (GELU_C * inner).astype(F32)
        e = exp32((u * F32(-2.0)).astype(F32))
        den = (F32(1.0) + e).astype(F32)
        return (h / den).astype(F32)


def rmsnorm_modulate32(h: np.ndarray, gamma=None, scale=None, shift=None, eps: float = 1e-6):
    """RMSNorm with modulation of float32 rows [M, K]; returns (x float32 [M, K],
    rstd float32 [M])."""
    h = np.asarray(h, dtype=F32)
    K = h.shape[1]
    ss = (h.astype(np.float64) ** 2).sum(axis=1)
    ms = (ss / K).astype(F32)
    v = (ms + F32(eps)).astype(F32)
    rstd = (F32(1.0) / np.sqrt(v).astype(F32)).astype(F32)
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


def produce(h_bits, h_dtype: str, kind: str, gamma=None, scale=None, shift=None, eps: float = 1e-6):
    """X (16-bit patterns, the type of H) from H by producer ``kind``:
    "none", "rmsnorm" or "gelu"."""
    h = w8ref.decode16(h_bits, h_dtype)
    if kind == "none":
        return np.ascontiguousarray(h_bits, dtype=np.uint16)
    if kind == "rmsnorm":
        x, _ = rmsnorm_modulate32(h, gamma, scale, shift, eps)
    elif kind == "gelu":
        x = gelu32(h)
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
