"""CPU oracle: LLM.int8 mixed-precision linear and FP8-E4M3 W8A8 linear.

TEST INFRASTRUCTURE. Only the test suite, the smoke check in
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this module. The library never does, and this module shares no code
with the HIP path: it has its own 16-bit decoders, its own E4M3 table, its
own rounding.

Plain numpy, slow and literal. Every quantisation decision is made in float32
with IEEE round-to-nearest-even, the precision the encodings are defined in.
Integer contractions are exact. Floating epilogues are float64 with a single
final rounding to the output type.

Sources (the pages the method is taken from, and the published algorithm the
first of them names):
  [INT8]  "Image21-INT8" model card, section "Quantization": bitsandbytes
          LLM.int8 on the eligible linears, outlier threshold 6.0; outliers are
          handled in floating point; no calibration. Section "Installation and
          loading": the INT8 weights are stored once and never re-quantised.
  [LLM8]  LLM.int8() (Dettmers et al., 2022), the algorithm bitsandbytes
          implements: vector-wise absmax int8 for activation rows and weight
          rows, int32 accumulation, dequantisation by the outer product of the
          two scale vectors over 127^2, plus a 16-bit product over the input
          columns that hold an outlier.
  [FP8D]  "Qwen-Image-2.1 Text Encoder: FP8" card, section "Format": E4M3
          weights with one bf16 scale per output channel ([out, 1]);
          activations quantised per token at run time; the dequantised weight
          is the FP8 value times its scale, in bf16, for a weight-only
          loader that computes in bf16 (section "How it was tested" measures
          that weight-only mode beside W8A8).
  [FP8S]  "Darkstar-Qwen-Image-2.1-Base-ModelOpt-FP8" card, sections
          "Precision map" and "Provenance": E4M3 with static fp32 per-tensor
          weight and input scales, calibrated with the "max" algorithm.
  [OFP8]  OCP 8-bit floating point specification, format E4M3 (the "FN"
          flavour: bias 7, no infinities, S.1111.111 is NaN, max 448).

Readings where the pages are silent (each is listed with its reason in the
project's design notes):
  * outlier test is strict (|x| > t); the outlier set is taken column-wise
    over all rows of the call and listed in ascending order;
  * a row's int8 scale is the absmax over the non-outlier columns only;
  * codes: r = fl32(127 / s) once per row, q = rne(fl32(x * r)), clamped to
    [-127, 127]; s == 0 or x == 0 gives 0; outlier columns get code 0;
  * the floating side path multiplies the outlier columns of X by the
    dequantised int8 weights (Wq * sw / 127), since no float weight exists
    at inference;
  * FP8: s = fl32(amax / 448), q = e4m3(fl32(x / s)) with saturation to
    +-448 and the sign of zero kept; the weight scale is rounded to bf16
    before encoding with it.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32

# ---------------------------------------------------------------------------
# 16-bit storage formats (IEEE binary16 and bfloat16)
# ---------------------------------------------------------------------------


def decode16(bits: np.ndarray, dtype: str) -> np.ndarray:
    """16-bit patterns -> exact float32 values."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == "bf16":
        # bfloat16 is the top half of a binary32 pattern.
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float32)  # widening is exact
    raise ValueError(dtype)


def round_to_f16(y) -> np.ndarray:
    """float64 -> binary16 bits, IEEE round to nearest even, overflow to inf."""
    with np.errstate(over="ignore"):
        return np.asarray(y, dtype=np.float64).astype(np.float16).view(np.uint16)


def round_to_bf16(y) -> np.ndarray:
    """float64 -> bfloat16 bits, round to nearest even, overflow to inf.

    bfloat16 keeps 8 significant bits; below 2**-126 its spacing is fixed at
    2**-133. Scale |y| so the last kept bit is the units digit, round the
    (exactly scaled) value to an integer with ties to even, scale back.
    """
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    _, e = np.frexp(a)                      # a = m * 2**e, 0.5 <= m < 1
    unit_exp = np.maximum(e - 8, -133)      # exponent of the last kept bit
    r = np.ldexp(np.rint(np.ldexp(a, -unit_exp)), unit_exp)
    with np.errstate(over="ignore"):
        r32 = r.astype(np.float32)          # exact unless it overflows -> inf
    bits = (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(np.signbit(y), bits | np.uint16(0x8000), bits)
    return bits.astype(np.uint16)


def round_to_f32(y) -> np.ndarray:
    return np.asarray(y, dtype=np.float64).astype(np.float32)


def round_output(y: np.ndarray, out_dtype: str) -> np.ndarray:
    """Final IEEE RNE rounding of a float64 result; returns the stored array
    (uint16 patterns for 16-bit types, float32 values for f32)."""
    if out_dtype == "f16":
        return round_to_f16(y)
    if out_dtype == "bf16":
        return round_to_bf16(y)
    if out_dtype == "f32":
        return round_to_f32(y)
    raise ValueError(out_dtype)


def stored_to_f64(stored: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    return decode16(stored, dtype).astype(np.float64)


# ---------------------------------------------------------------------------
# Symmetric absmax int8 encoding [LLM8]
# ---------------------------------------------------------------------------


def absmax_int8(v: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Encode each row of float32 ``v`` with its float32 absmax ``s``.

    r = fl32(127 / s); q = rne(fl32(v * r)) clamped to [-127, 127].
    Rows with s == 0 and elements equal to 0 encode to 0 (0 * r would be
    NaN when r overflows to inf for a subnormal s).
    """
    v = np.asarray(v, dtype=F32)
    s = np.asarray(s, dtype=F32)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        r = F32(127.0) / s                         # one IEEE fp32 division per row
        p = v * r[:, None]                         # IEEE fp32 product
        q = np.clip(np.rint(p), -127.0, 127.0)     # rint: ties to even
    zero = (s == 0)[:, None] | (v == 0)
    q = np.where(zero, 0.0, q)
    return q.astype(np.int8)


def quantize_weight_int8(w: np.ndarray):
    """Rowwise int8 weight quantisation [INT8 stored weights; LLM8 rowwise].

    w: float32 [N, K] (exact values of the 16-bit weights).
    Returns (Wq int8 [N, K], sw float32 [N]) with sw[n] = max_k |w[n, k]|.
    No outlier threshold applies to weights.
    """
    w = np.asarray(w, dtype=F32)
    sw = np.abs(w).max(axis=1).astype(F32) if w.shape[1] else np.zeros(w.shape[0], F32)
    return absmax_int8(w, sw), sw


# ---------------------------------------------------------------------------
# LLM.int8 mixed-precision decomposition [INT8, LLM8]
# ---------------------------------------------------------------------------


def outlier_columns(xf: np.ndarray, threshold: float) -> np.ndarray:
    """Ascending indices of the columns where some row has |x| > t (strict)."""
    t = F32(threshold)
    return np.flatnonzero((np.abs(xf) > t).any(axis=0)).astype(np.int64)


def quantize_activations_int8(xf: np.ndarray, threshold: float, rows=None):
    """Split X into outlier columns and an int8-coded remainder.

    xf: float32 [M, K]. The outlier set always comes from all M rows; ``rows``
    (optional index array) restricts the returned scales and codes.
    Returns (O, sx [R], q int8 [R, K]).
    """
    xf = np.asarray(xf, dtype=F32)
    O = outlier_columns(xf, threshold)
    sel = xf if rows is None else xf[np.asarray(rows)]
    keep = np.ones(xf.shape[1], dtype=bool)
    keep[O] = False
    if keep.any():
        sx = np.abs(sel[:, keep]).max(axis=1).astype(F32)
    else:
        sx = np.zeros(sel.shape[0], dtype=F32)
    q = absmax_int8(sel, sx)
    q[:, O] = 0
    return O, sx, q


def int8_contract(q: np.ndarray, wq: np.ndarray) -> np.ndarray:
    """acc[m, n] = sum_k q[m, k] * wq[n, k], exact, as int64.

    Computed with a float64 matrix product: each product is an integer of
    magnitude <= 127**2 and, for K <= 133144, every partial sum stays below
    2**31, far inside the 2**53 range where float64 integer addition is exact
    in any order.
    """
    assert q.shape[1] == wq.shape[1]
    assert q.shape[1] <= 133144
    acc = q.astype(np.float64) @ wq.astype(np.float64).T
    out = acc.astype(np.int64)
    assert np.all(np.abs(out) < 2**31)
    return out


def int8_mixed_linear(x_bits, x_dtype, wq, sw, threshold, out_dtype="f16", rows=None):
    """Y = X W^T under the LLM.int8 decomposition.

    x_bits: uint16 [M, K] (f16 or bf16 patterns); wq: int8 [N, K];
    sw: float32 [N]. ``rows`` optionally restricts the output to a subset of
    token rows (the outlier set still comes from all rows).

    Steps:
      1. O = outlier columns of X (all rows);
      2. sx[m] = absmax of row m over columns not in O;
      3. q = int8 codes of X with column set O zeroed;
      4. acc = q . wq^T exactly (int32 range);
      5. outl = X[:, O] . wq[:, O]^T (float side path on dequantised weights,
         the common 1/127 * sw factor applied below);
      6. y = (sw/127) * ((sx/127) * acc + outl) in float64;
      7. Y = round(y) to the output type.
    Returns a dict with every intermediate.
    """
    xf = decode16(x_bits, x_dtype)
    O, sx, q = quantize_activations_int8(xf, threshold, rows)
    sel = xf if rows is None else xf[np.asarray(rows)]
    acc = int8_contract(q, wq)
    outl = sel[:, O].astype(np.float64) @ wq[:, O].astype(np.float64).T
    sw64 = np.asarray(sw, dtype=np.float32).astype(np.float64)
    sx64 = sx.astype(np.float64)
    y = (sw64[None, :] / 127.0) * ((sx64[:, None] / 127.0) * acc + outl)
    return {"O": O, "sx": sx, "q": q, "acc": acc, "outl": outl, "y": y,
            "Y": round_output(y, out_dtype)}


# ---------------------------------------------------------------------------
# FP8 E4M3 (OCP "FN" flavour) [OFP8]
# ---------------------------------------------------------------------------


def e4m3_decode_table() -> np.ndarray:
    """Value of each of the 256 codes (float64; NaN for 0x7F and 0xFF).

    Bits S EEEE MMM, exponent bias 7. E == 0: subnormal M * 2**-9.
    Otherwise (1 + M/8) * 2**(E - 7). E == 15, M == 7 is NaN (no infinities).
    """
    c = np.arange(256)
    s = c >> 7
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where(s == 1, -mag, mag)
    val[0x7F] = np.nan
    val[0xFF] = np.nan
    return val


_E4M3 = e4m3_decode_table()
_E4M3_POS = _E4M3[:0x7F]        # codes 0x00..0x7E, strictly increasing 0 .. 448
E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """float32 -> E4M3 codes: round to nearest, ties to the even code,
    saturating: |v| >= 448 (an fp32 overflow to +-inf included) gives +-448;
    the sign of zero is kept. NaN is outside the contract."""
    v = np.asarray(v, dtype=np.float32)
    assert not np.any(np.isnan(v)), "NaN input"
    a = np.minimum(np.abs(v).astype(np.float64), E4M3_MAX)
    i = np.searchsorted(_E4M3_POS, a, side="right") - 1      # pos[i] <= a
    i = np.clip(i, 0, 0x7E)
    j = np.minimum(i + 1, 0x7E)
    lo, hi = _E4M3_POS[i], _E4M3_POS[j]
    d_lo, d_hi = a - lo, hi - a                                # exact in float64
    up = (d_hi < d_lo) | ((d_hi == d_lo) & (i % 2 == 1))
    code = np.where(up, j, i).astype(np.uint8)
    return np.where(np.signbit(v), code | np.uint8(0x80), code).astype(np.uint8)


def quantize_weight_fp8(w: np.ndarray):
    """E4M3 weights with one per-output-channel scale [FP8D].

    amax = max_k |w|; sw = bf16(fl32(amax / 448)) (the card stores the scale
    as bf16); codes = e4m3(fl32(w / sw)), all zero when sw == 0.
    Returns (codes uint8 [N, K], sw float32 [N] holding bf16 values).
    """
    w = np.asarray(w, dtype=F32)
    amax = np.abs(w).max(axis=1).astype(F32)
    s32 = amax / F32(E4M3_MAX)
    sw = decode16(round_to_bf16(s32.astype(np.float64)), "bf16")
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = w / sw[:, None]                               # IEEE fp32 division
    ratio = np.where((sw == 0)[:, None], F32(0.0), ratio).astype(F32)
    codes = e4m3_encode(ratio)
    codes = np.where((sw == 0)[:, None], np.uint8(0), codes).astype(np.uint8)
    return codes, sw


def fp8_activation_scales(xf: np.ndarray, act_scale=None) -> np.ndarray:
    """Per-token dynamic scale fl32(amax / 448) [FP8D], or the static
    per-tensor input scale broadcast to every token [FP8S]."""
    xf = np.asarray(xf, dtype=F32)
    if act_scale is None:
        return (np.abs(xf).max(axis=1).astype(F32) / F32(E4M3_MAX)).astype(F32)
    return np.full(xf.shape[0], F32(act_scale), dtype=F32)


def quantize_activations_fp8(xf: np.ndarray, act_scale=None):
    """Returns (codes uint8 [M, K], sx float32 [M]); codes = e4m3(fl32(x / sx)),
    all zero on rows whose scale is 0."""
    xf = np.asarray(xf, dtype=F32)
    sx = fp8_activation_scales(xf, act_scale)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        ratio = xf / sx[:, None]
    ratio = np.where((sx == 0)[:, None], F32(0.0), ratio).astype(F32)
    codes = e4m3_encode(ratio)
    codes = np.where((sx == 0)[:, None], np.uint8(0), codes).astype(np.uint8)
    return codes, sx


def fp8_contract(xq: np.ndarray, wq8: np.ndarray) -> np.ndarray:
    """sum_k dec(xq[m,k]) * dec(wq8[n,k]) in float64, exact.

    E4M3 values have at most 4 significant bits and lie on the 2**-9 grid
    below 2**9, so every product is a multiple of 2**-18 below 2**18 and, for
    K <= 2**14, every partial sum is a multiple of 2**-18 below 2**32: 50
    bits, exact in float64 whatever the summation order.
    """
    return e4m3_decode(xq) @ e4m3_decode(wq8).T


def fp8_w8a8_linear(x_bits, x_dtype, wq8, sw, act_scale=None, out_dtype="bf16"):
    """Y = sx[m] * sw[n] * sum_k dec(xq) dec(wq8)   [FP8D, FP8S]."""
    xf = decode16(x_bits, x_dtype)
    xq, sx = quantize_activations_fp8(xf, act_scale)
    acc = fp8_contract(xq, wq8)
    y = sx.astype(np.float64)[:, None] * np.asarray(sw, np.float32).astype(np.float64)[None, :] * acc
    return {"xq": xq, "sx": sx, "acc": acc, "y": y, "Y": round_output(y, out_dtype)}


# ---------------------------------------------------------------------------
# FP8 weight-only (W8A16) [FP8D]: the card's weight-only loader dequantises
# each weight to bf16 as the FP8 value times its channel scale and runs the
# linear in bf16.
# ---------------------------------------------------------------------------


def dequantize_weight_fp8_bf16(wq8: np.ndarray, sw: np.ndarray) -> np.ndarray:
    """bfloat16 bits of the dequantised weight, rne_bf16(dec(wq8[n,k]) * sw[n]).

    sw holds bf16 values. An E4M3 value has at most 4 significant bits and a
    bf16 scale 8, so the float64 product is exact and this is the one rounding
    of a bf16 multiply (float product, rounded to bf16)."""
    w = e4m3_decode(wq8) * np.asarray(sw, dtype=F32).astype(np.float64)[:, None]
    return round_to_bf16(w)


def fp8_w8a16_linear(x_bits, x_dtype, wq8, sw, out_dtype="bf16", rows=None):
    """Y = X W_deq^T with W_deq = dequantize_weight_fp8_bf16(wq8, sw): the
    16-bit X times the bf16 weights, summed in float64, one final rounding.
    ``rows``: compute only these rows of Y."""
    w_bits = dequantize_weight_fp8_bf16(wq8, sw)
    xf = decode16(x_bits, x_dtype).astype(np.float64)
    if rows is not None:
        xf = xf[np.asarray(rows)]
    y = xf @ decode16(w_bits, "bf16").astype(np.float64).T
    return {"w_bits": w_bits, "y": y, "Y": round_output(y, out_dtype)}


# ---------------------------------------------------------------------------
# Error metrics of the FP8 text-encoder card ("How it was tested")
# ---------------------------------------------------------------------------


def relative_l2(a: np.ndarray, ref: np.ndarray) -> float:
    """||a - ref||_F / ||ref||_F (the card's relative L2 over a matrix)."""
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(a - ref) / den) if den > 0 else float(np.linalg.norm(a))


def mean_token_cosine(a: np.ndarray, ref: np.ndarray) -> float:
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = (a * ref).sum(axis=1)
    den = np.linalg.norm(a, axis=1) * np.linalg.norm(ref, axis=1)
    return float(np.mean(num / np.where(den == 0, 1.0, den)))
