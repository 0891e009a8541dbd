"""Pins for the LLM.int8 part of the oracle.

The oracle is checked against: a hand-worked example (exact rationals), an
independent brute force on Python Fractions, closed forms for the special
thresholds (t = +inf: plain vector-wise int8; t = 0: the float GEMM with the
dequantised weights), a quantisation error bound, and invariances that a
wrong index, sign or transposition would break.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import w8ref as o
from tests.exact import to_f16, to_f32


def bf16(a):
    return synth.encode16(np.asarray(a, np.float32), "bf16")


# --------------------------------------------------------------------------
# Independent brute force (exact rationals, pure Python)
# --------------------------------------------------------------------------

def brute_int8_mixed(X, Wq, sw, t):
    """X: list of rows of exact floats, Wq: int rows, sw: floats, t: float."""
    M, K, N = len(X), len(X[0]), len(Wq)
    Xf = [[Fraction(v) for v in row] for row in X]
    if math.isinf(t):
        O = []
    else:
        tf = Fraction(t)
        O = [k for k in range(K) if any(abs(Xf[m][k]) > tf for m in range(M))]
    Oset = set(O)
    sx, q = [], []
    for m in range(M):
        rest = [abs(Xf[m][k]) for k in range(K) if k not in Oset]
        s = max(rest) if rest else Fraction(0)
        sx.append(s)
        row = [0] * K
        if s != 0:
            r = to_f32(Fraction(127) / s)
            for k in range(K):
                if k in Oset or Xf[m][k] == 0:
                    continue
                p = to_f32(Xf[m][k] * r)
                row[k] = max(-127, min(127, round(p)))
        q.append(row)
    acc = [[sum(q[m][k] * int(Wq[n][k]) for k in range(K)) for n in range(N)] for m in range(M)]
    y = []
    for m in range(M):
        yr = []
        for n in range(N):
            outl = sum(Xf[m][k] * int(Wq[n][k]) for k in O)
            swn = Fraction(float(sw[n]))
            yr.append(swn / 127 * (sx[m] / 127 * acc[m][n] + outl))
        y.append(yr)
    return O, sx, q, acc, y


def _tiny_case(rng, M, K, N):
    pool = np.concatenate([
        rng.standard_normal(64) * 3,
        [6.0, -6.0, 6.03125, -6.03125, 8.0, -20.0, 0.0, 1.015625, 3.96875, 0.5, 63.5 / 32],
    ]).astype(np.float32)
    x = rng.choice(pool, size=(M, K)).astype(np.float32)
    if M > 2:
        x[rng.integers(M)] = 0.0                       # an all-zero row
    xb = bf16(x)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    wq, sw = o.quantize_weight_int8(o.decode16(bf16(w), "bf16"))
    return xb, wq, sw


@pytest.mark.parametrize("seed", range(12))
def test_oracle_matches_rational_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    M, K, N = rng.integers(1, 9), rng.integers(1, 13), rng.integers(1, 7)
    xb, wq, sw = _tiny_case(rng, M, K, N)
    t = float(rng.choice([6.0, 0.0, math.inf, 2.5]))
    X = o.decode16(xb, "bf16").astype(np.float64).tolist()
    O, sx, q, acc, y = brute_int8_mixed(X, wq.tolist(), sw, t)
    r = o.int8_mixed_linear(xb, "bf16", wq, sw, t, "f16")
    assert r["O"].tolist() == O
    assert [Fraction(float(v)) for v in r["sx"]] == sx
    assert r["q"].tolist() == q
    assert r["acc"].tolist() == acc
    for m in range(M):
        for n in range(N):
            exact = y[m][n]
            got = r["y"][m, n]
            assert abs(Fraction(float(got)) - exact) <= abs(exact) * Fraction(1, 2 ** 50), (m, n)
            ref16 = to_f16(exact)
            g16 = float(o.decode16(r["Y"][m:m + 1, n], "f16")[0])
            # one rounding of the float64 y: equal to the exact rounding,
            # except that an exact tie may be resolved either way
            assert g16 == float(ref16) or (
                abs(Fraction(g16) - exact) <= abs(Fraction(ref16) - exact) * (1 + Fraction(1, 2 ** 40)))


# --------------------------------------------------------------------------
# Hand-worked examples
# --------------------------------------------------------------------------

def test_hand_example_split_scale_ties_and_side_path():
    """X 2x4, t = 6. Column 0 holds 8.0 > 6 in row 0, so it is an outlier
    column for every row (row 1's 5.0 included).
      sx = [max(.5,.25,0), max(1,2,.5)] = [0.5, 2.0]   (not 5.0: the outlier
      column is excluded from the scale)
      r  = [127/0.5, 127/2] = [254, 63.5]               (exact in fp32)
      q0 = [0, .5*254, .25*254 -> 63.5 -> 64, 0]        (tie to even)
      q1 = [0, 63.5 -> 64, -127, 31.75 -> 32]
      acc = q Wq^T ; outl = X[:,0] Wq[:,0]^T = [[8,-8],[5,-5]]
      y  = sw/127 * (sx/127 * acc + outl)
    """
    X = np.array([[8.0, 0.5, 0.25, 0.0], [5.0, 1.0, -2.0, 0.5]], np.float32)
    Wq = np.array([[1, 2, 3, 4], [-1, 0, 127, -127]], np.int8)
    sw = np.array([127.0, 254.0], np.float32)
    r = o.int8_mixed_linear(bf16(X), "bf16", Wq, sw, 6.0, "f16")
    assert r["O"].tolist() == [0]
    assert r["sx"].tolist() == [0.5, 2.0]
    assert r["q"].tolist() == [[0, 127, 64, 0], [0, 64, -127, 32]]
    acc = [[127 * 2 + 64 * 3, 64 * 127], [64 * 2 - 127 * 3 + 32 * 4, -127 * 127 - 32 * 127]]
    assert r["acc"].tolist() == acc == [[446, 8128], [-125, -20193]]
    F = Fraction
    y = [[F(127, 127) * (F(1, 2) / 127 * 446 + 8), F(254, 127) * (F(1, 2) / 127 * 8128 - 8)],
         [F(127, 127) * (F(2) / 127 * -125 + 5), F(254, 127) * (F(2) / 127 * -20193 - 5)]]
    assert y == [[F(1239, 127), F(48)], [F(385, 127), F(-646)]]
    assert np.allclose(r["y"], np.array([[float(v) for v in row] for row in y]), rtol=1e-15)
    Y = o.decode16(r["Y"], "f16").tolist()
    assert Y == [[float(to_f16(v)) for v in row] for row in y] == [[9.7578125, 48.0], [3.03125, -646.0]]


def test_hand_example_tie_rounds_to_even():
    # s = 127/32 (exact): r = fl32(127/s) = 32, and 1.015625 * 32 = 32.5 -> 32.
    X = np.array([[127 / 32, 1.015625, 1.046875]], np.float32)   # 1.046875*32 = 33.5 -> 34
    O, sx, q = o.quantize_activations_int8(o.decode16(bf16(X), "bf16"), 6.0)
    assert O.size == 0 and sx.tolist() == [3.96875]
    assert q.tolist() == [[127, 32, 34]]


def test_hand_example_threshold_is_strict():
    # A column whose largest |x| is exactly t stays on the int8 path.
    X = np.array([[6.0, 1.0], [-6.0, 0.5]], np.float32)
    O, sx, q = o.quantize_activations_int8(o.decode16(bf16(X), "bf16"), 6.0)
    assert O.size == 0 and sx.tolist() == [6.0, 6.0]
    assert q[:, 0].tolist() == [127, -127]
    O2, _, _ = o.quantize_activations_int8(o.decode16(bf16(X), "bf16"), 5.999)
    assert O2.tolist() == [0]


# --------------------------------------------------------------------------
# Closed forms and bounds
# --------------------------------------------------------------------------

def _mid_case(seed, M=24, K=96, N=40, n_out=3):
    c = synth.random_linear(M, K, N, seed, "bf16", outlier_cols=n_out)
    xf = o.decode16(c.x_bits, "bf16")
    wq, sw = o.quantize_weight_int8(o.decode16(c.w_bits, "bf16"))
    return c, xf, wq, sw


def test_infinite_threshold_is_plain_vectorwise_int8():
    c, xf, wq, sw = _mid_case(1)
    r = o.int8_mixed_linear(c.x_bits, "bf16", wq, sw, math.inf, "f32")
    assert r["O"].size == 0
    assert np.array_equal(r["sx"], np.abs(xf).max(axis=1))
    # each row's largest element maps to +-127
    am = np.abs(xf).argmax(axis=1)
    assert np.array_equal(np.abs(r["q"][np.arange(c.M), am]), np.full(c.M, 127))
    # |x - q sx/127| <= sx (1/254 + 2^-23) elementwise
    err = np.abs(xf - r["q"] * (r["sx"][:, None] / 127.0))
    assert np.all(err <= r["sx"][:, None] * (1 / 254 + 2.0 ** -23))


def test_zero_threshold_equals_float_gemm_with_dequantised_weights():
    c, xf, wq, sw = _mid_case(2)
    xf[:, 5] = 0.0                                   # an all-zero column stays int8
    xb = bf16(xf)
    r = o.int8_mixed_linear(xb, "bf16", wq, sw, 0.0, "f32")
    assert 5 not in r["O"].tolist() and r["O"].size == c.K - 1
    assert not r["q"].any()
    wdeq = wq.astype(np.float64) * (sw.astype(np.float64)[:, None] / 127.0)
    ref = xf.astype(np.float64) @ wdeq.T
    assert np.allclose(r["y"], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", [3, 4, 5])
def test_output_error_bound_against_float_gemm(seed):
    """y differs from X.Wdeq^T only through the int8 coding of the
    non-outlier columns: |y - X Wdeq^T| <= sx (1/254 + 2^-23) sum_k |Wdeq|."""
    c, xf, wq, sw = _mid_case(seed, n_out=4)
    r = o.int8_mixed_linear(c.x_bits, "bf16", wq, sw, 6.0, "f32")
    assert r["O"].tolist() == sorted(c.injected_cols)
    wdeq = wq.astype(np.float64) * (sw.astype(np.float64)[:, None] / 127.0)
    ref = xf.astype(np.float64) @ wdeq.T
    bound = (r["sx"].astype(np.float64)[:, None] * (1 / 254 + 2.0 ** -23)) * np.abs(wdeq).sum(axis=1)[None, :]
    assert np.all(np.abs(r["y"] - ref) <= bound * (1 + 1e-9) + 1e-12)


def test_zero_row_gives_zero_output_row():
    c, xf, wq, sw = _mid_case(6)
    xf[7] = 0.0
    r = o.int8_mixed_linear(bf16(xf), "bf16", wq, sw, 6.0, "f16")
    assert r["sx"][7] == 0 and not r["q"][7].any()
    assert not r["y"][7].any() and not r["Y"][7].any()


def test_contraction_is_exact_integer_product():
    rng = np.random.default_rng(12)
    q = rng.integers(-127, 128, size=(5, 300)).astype(np.int8)
    w = rng.integers(-127, 128, size=(4, 300)).astype(np.int8)
    acc = o.int8_contract(q, w)
    ref = [[sum(int(a) * int(b) for a, b in zip(qr, wr)) for wr in w] for qr in q]
    assert acc.tolist() == ref
    full = np.full((1, 16384), 127, np.int8)
    assert o.int8_contract(full, -full)[0, 0] == -(127 * 127 * 16384)


def test_power_of_two_scaling_equivariance():
    c, xf, wq, sw = _mid_case(7)
    base = o.quantize_activations_int8(xf, 6.0)
    for e in (-3, 5):
        O, sx, q = o.quantize_activations_int8(xf * np.float32(2.0 ** e), 6.0 * 2.0 ** e)
        assert np.array_equal(O, base[0]) and np.array_equal(q, base[2])
        assert np.array_equal(sx, base[1] * np.float32(2.0 ** e))


def test_permutation_invariances():
    c, xf, wq, sw = _mid_case(8)
    r = o.int8_mixed_linear(bf16(xf), "bf16", wq, sw, 6.0, "f32")
    perm = np.random.default_rng(13).permutation(c.K)
    rp = o.int8_mixed_linear(bf16(xf[:, perm]), "bf16", wq[:, perm], sw, 6.0, "f32")
    assert np.array_equal(np.sort(perm[rp["O"]]), r["O"])
    assert np.array_equal(rp["q"], r["q"][:, perm])
    assert np.array_equal(rp["acc"], r["acc"])
    rows = np.random.default_rng(14).permutation(c.M)
    rr = o.int8_mixed_linear(bf16(xf[rows]), "bf16", wq, sw, 6.0, "f32")
    assert np.array_equal(rr["O"], r["O"]) and np.array_equal(rr["q"], r["q"][rows])


def test_sampled_rows_equal_full_result():
    c, xf, wq, sw = _mid_case(9)
    full = o.int8_mixed_linear(c.x_bits, "bf16", wq, sw, 6.0, "f16")
    rows = np.array([0, 5, 23, 11])
    part = o.int8_mixed_linear(c.x_bits, "bf16", wq, sw, 6.0, "f16", rows=rows)
    assert np.array_equal(part["O"], full["O"])
    for key in ("sx", "q", "acc", "Y"):
        assert np.array_equal(part[key], full[key][rows])


# --------------------------------------------------------------------------
# Weight quantisation
# --------------------------------------------------------------------------

def test_weight_quantisation_bound_and_scales():
    rng = np.random.default_rng(15)
    w = o.decode16(bf16(rng.standard_normal((33, 257)) * 0.02), "bf16")
    w[4] = 0.0
    wq, sw = o.quantize_weight_int8(w)
    assert np.all(np.abs(wq.astype(int)) <= 127)
    assert np.array_equal(sw, np.abs(w).max(axis=1))
    assert sw[4] == 0 and not wq[4].any()
    nz = sw > 0
    assert np.all(np.isfinite(sw)) and np.all(sw[nz] > 0)     # no degenerate scale
    am = np.abs(w).argmax(axis=1)
    assert np.all(np.abs(wq[nz, am[nz]].astype(int)) == 127)
    err = np.abs(w - wq * (sw[:, None] / 127.0))
    assert np.all(err <= sw[:, None] * (1 / 254 + 2.0 ** -23))


def test_fp32_steps_are_the_fl32_of_exact_values():
    # r = fl32(127/s) and p = fl32(x r) are single IEEE roundings.
    rng = np.random.default_rng(16)
    s = o.decode16(bf16(np.abs(rng.standard_normal(50)) + 0.1), "bf16")
    x = o.decode16(bf16(rng.standard_normal(50)), "bf16")
    r = np.float32(127.0) / s
    for si, ri, xi in zip(s, r, x):
        assert Fraction(float(ri)) == to_f32(Fraction(127) / Fraction(float(si)))
        assert Fraction(float(np.float32(xi) * ri)) == to_f32(Fraction(float(xi)) * Fraction(float(ri)))


# --------------------------------------------------------------------------
# The seeded workloads carry the structure they claim
# --------------------------------------------------------------------------

def test_tiny_workload_outliers_are_the_injected_columns():
    c = synth.tiny_int8()
    xf = o.decode16(c.x_bits, "f16")
    assert o.outlier_columns(xf, 6.0).tolist() == list(c.injected_cols)
    for col in c.injected_cols:
        big = np.abs(xf[:, col]) > 6
        assert np.flatnonzero(big).tolist() == list(c.injected_rows)
        assert np.all((np.abs(xf[big, col]) >= 8) & (np.abs(xf[big, col]) <= 20))
