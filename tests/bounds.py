"""Element-wise output bounds for the GPU parity tests (test-only).

The GPU epilogues compute in float32 and round once into the output type. For
each output element the bound on |Y_gpu - y| (y: the oracle's float64 value
before its final rounding) is half a unit in the last place of the output
type at max(|Y_gpu|, |y|), plus the float32 error of that path, derived
from its sequence of roundings (u = 2^-24 per rounding, gamma_n = n u for n
accumulated terms), with a factor 2 of slack. The terms use magnitudes from
the oracle's exact intermediates, so a wrong scale, bias or outlier term in
one column moves that column far outside its bound even when a norm over the
row would not notice it.
"""
from __future__ import annotations

import numpy as np

from oracle import w8ref as o

U = 2.0 ** -24


def half_ulp(v: np.ndarray, dtype: str) -> np.ndarray:
    """Half the spacing of the output format at |v| (its subnormal spacing
    below the normal range)."""
    mant, emin = {"f16": (11, -14), "bf16": (8, -126), "f32": (24, -126)}[dtype]
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** emin)))
    return 0.5 * np.exp2(e - (mant - 1))


def assert_elementwise(y_stored: np.ndarray, out_dtype: str, y_exact: np.ndarray, err32: np.ndarray, label) -> None:
    """|Y - y| <= half_ulp(max(|Y|, |y|)) + 2 err32 + a float64 hair, element
    by element."""
    got = o.stored_to_f64(y_stored, out_dtype)
    y_exact = np.asarray(y_exact, np.float64)
    assert got.shape == y_exact.shape, label
    assert np.all(np.isfinite(got)), label
    big = np.maximum(np.abs(got), np.abs(y_exact))
    bound = half_ulp(big, out_dtype) + 2.0 * np.asarray(err32, np.float64) + 1e-12 * big
    over = np.abs(got - y_exact) > bound
    if over.any():
        i = np.argwhere(over)[:5]
        raise AssertionError((label, int(over.sum()), [(tuple(ix), got[tuple(ix)], y_exact[tuple(ix)],
                                                        bound[tuple(ix)]) for ix in i]))


def int8_err32(ref: dict, x_bits, x_dtype: str, wq: np.ndarray, sw: np.ndarray, bias=None, rows=None) -> np.ndarray:
    """float32 error of the int8 epilogue ((acc sx/127 + side) sw/127 + bias):
    acc converted (u), sx/127 and sw/127 each rounded once (u), the side
    product summed over nO outlier columns in float32 (nO u of the sum of
    |products|, each product exact), two fused multiply-adds (u each)."""
    xf = o.decode16(x_bits, x_dtype).astype(np.float64)
    if rows is not None:
        xf = xf[np.asarray(rows)]
    O = ref["O"]
    nO = len(O)
    A = np.abs(ref["acc"].astype(np.float64)) * (ref["sx"].astype(np.float64)[:, None] / 127.0)
    S = np.abs(xf[:, O]) @ np.abs(wq[:, O].astype(np.float64)).T if nO else np.zeros_like(A)
    c = np.asarray(sw, np.float64)[None, :] / 127.0
    b = np.zeros((1, A.shape[1])) if bias is None else np.abs(np.asarray(bias, np.float64))[None, :]
    y = np.abs(ref["y"])
    return U * (c * (5.0 * A + (nO + 3) * S) + y + b)


def fp8_err32(ref: dict, wq8: np.ndarray, sw: np.ndarray, K: int) -> np.ndarray:
    """float32 error of the FP8 GEMM: K products (exact) accumulated in
    float32 (gamma_K of the sum of |products|), then scaled by sx and sw (two
    roundings of |y|)."""
    a = np.abs(o.e4m3_decode(ref["xq"]))
    w = np.abs(o.e4m3_decode(wq8))
    P = a @ w.T
    s = ref["sx"].astype(np.float64)[:, None] * np.asarray(sw, np.float64)[None, :]
    return U * (K * s * P + 3.0 * np.abs(ref["y"]))


def dense_err32(x_abs: np.ndarray, w_abs: np.ndarray, y: np.ndarray, K: int) -> np.ndarray:
    """float32 error of a 16-bit product with float32 accumulation: gamma_K of
    the sum of |products| plus one rounding of |y|."""
    return U * (K * (x_abs @ w_abs.T) + np.abs(y))


def w4a8_err32(ref: dict, sw4: np.ndarray) -> np.ndarray:
    """float32 error of the W4A8 fold: each group's exact int32 sum times its
    scale (sw/7/16 rounded twice, one fused multiply-add: about 3 u per
    group) accumulated over G groups (gamma_G), then times sx/127 (two
    roundings)."""
    acc = np.abs(ref["acc"].astype(np.float64))               # [M, N, G]
    s = np.asarray(sw4, np.float64).T[None, :, :] / 7.0       # [1, N, G]
    G = acc.shape[2]
    mag = (acc * s).sum(axis=2) * (ref["sx"].astype(np.float64)[:, None] / 127.0)
    return U * ((G + 6.0) * mag + np.abs(ref["y"]))
