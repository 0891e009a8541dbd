"""Pins of the producer oracle (oracle/producers.py) against references that
do not share its arithmetic: float64 library routines (numpy exp, torch's
tanh-form GELU and RMSNorm), closed forms and special values."""
import math

import numpy as np
import pytest
import torch

from oracle import producers as P
from oracle import w8ref as o


def _all_finite(dtype):
    bits = np.arange(65536, dtype=np.uint16)
    return bits[np.isfinite(o.decode16(bits, dtype))]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_gelu16_is_float64_gelu_rounded_once(dtype):
    """Every finite 16-bit input: the oracle's X equals the float64 value
    h * sigmoid(2u) (scipy's expit, which stays accurate where 1 + tanh(u)
    cancels) rounded once to the 16-bit type, and lies within one 16-bit step
    of torch's float64 tanh-form GELU where that is not in cancellation. The
    exact values stay at least 2.6e-8 (relative) away from every 16-bit
    rounding midpoint, far more than float64's error, with one class of
    exceptions: bf16 inputs with |h| < 2^-125, where gelu(h) = h/2 +
    sqrt(2/pi) h^2 / 2 + O(h^4) sits just above h/2 and h/2 (a subnormal) can
    be a midpoint. float64 loses the h^2 term there, so those inputs are
    checked against the series: h/2 rounded with ties toward +inf."""
    from scipy.special import expit
    bits = _all_finite(dtype)
    got = P.gelu16(bits, dtype)
    h = o.decode16(bits, dtype).astype(np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        u = np.sqrt(2.0 / np.pi) * (h + 0.044715 * h ** 3)
        ref = h * expit(2.0 * u)
    ref = np.where(np.isnan(ref), np.copysign(0.0, h), ref)       # h^3 overflow at the bf16 extremes
    r16 = o.round_to_f16(ref) if dtype == "f16" else o.round_to_bf16(ref)
    tg = torch.nn.functional.gelu(torch.from_numpy(h), approximate="tanh").numpy()
    ok = np.abs(tg) > 1e-3
    gv = o.decode16(got, dtype).astype(np.float64)
    step = 2.0 ** -10 if dtype == "f16" else 2.0 ** -7
    assert np.all(np.abs(gv[ok] - tg[ok]) <= step * np.abs(tg[ok]))
    tiny = np.abs(h) < 2.0 ** -125
    if dtype == "f16":
        assert np.array_equal(got, r16)
        return
    assert np.array_equal(got[~tiny], r16[~tiny])
    # series form for the subnormal inputs, with exact rationals
    from fractions import Fraction
    from tests.exact import to_bf16
    for b, g in zip(bits[tiny].tolist(), got[tiny].tolist()):
        hv = Fraction(float(o.decode16(np.array([b], np.uint16), "bf16")[0]))
        half = hv / 2
        want = to_bf16(half + abs(half) * Fraction(1, 2 ** 40))   # just above h/2
        gv = Fraction(float(o.decode16(np.array([g], np.uint16), "bf16")[0]))
        assert gv == want, (b, g, float(want))
        assert (g >> 15) == (b >> 15)                              # sign kept, -0 included


def test_gelu16_special_values():
    f16 = o.round_to_f16(np.array([0.0, -0.0, 1.0, -1.0, 20.0, -20.0, 65504.0, -65504.0, 3.0, -9.5]))
    g = o.decode16(P.gelu16(f16, "f16"), "f16")
    assert g[0] == 0.0 and not np.signbit(g[0])
    assert g[1] == 0.0 and np.signbit(g[1])
    assert g[2] == np.float16(0.8411919906082768)                # tanh-form GELU(1) in fp16
    assert g[3] == np.float16(-0.15880800939172324)
    assert g[4] == 20.0 and g[6] == 65504.0                      # large positive h: h itself
    assert g[5] == 0.0 and np.signbit(g[5]) and np.signbit(g[7])  # large negative h: -0
    assert g[8] == np.float16(2.9963627)                          # 3 Phi-like: just below 3
    bf = o.round_to_bf16(np.array([1.0, -3.0e38, 3.0e38]))
    gb = o.decode16(P.gelu16(bf, "bf16"), "bf16")
    assert gb[0] == o.decode16(o.round_to_bf16(np.array([0.8411919906082768])), "bf16")[0]
    assert gb[1] == 0.0 and np.signbit(gb[1]) and gb[2] == o.decode16(bf[2:], "bf16")[0]


def test_gelu16_odd_part_identity():
    """gelu(h) - gelu(-h) = h exactly for the tanh form (sigma(z) + sigma(-z)
    = 1): checked on the decimal values before rounding."""
    for h in [0.5, 1.0, 2.75, 4.0, 0.001, 7.5]:
        d = P.gelu_decimal(h) - P.gelu_decimal(-h)
        assert abs(float(d) - h) <= 1e-40 * max(1.0, h)


def test_decimal_rounding_matches_exact_rationals():
    """round_decimal_to16 (the oracle's last step) against the Fraction-based
    rounding of tests/exact.py, at midpoints, just off them and at random."""
    import decimal
    from decimal import Decimal
    from fractions import Fraction
    from tests.exact import to_bf16, to_f16
    rng = np.random.default_rng(5)
    vals = [Fraction(1) + Fraction(1, 2 ** 11), Fraction(1) + Fraction(3, 2 ** 11), Fraction(1, 2 ** 25),
            Fraction(3, 2 ** 25), Fraction(65504) + Fraction(16), Fraction(65520), Fraction(1, 2 ** 134)]
    vals += [Fraction(float(v)) for v in rng.standard_normal(200) * 10.0 ** rng.integers(-8, 5, 200)]
    for v in vals:
        for dtype, ref in (("f16", to_f16), ("bf16", to_bf16)):
            for sgn in (1, -1):
                fr = sgn * v
                with decimal.localcontext(decimal.Context(prec=2000)):
                    d = Decimal(fr.numerator) / Decimal(fr.denominator)   # exact: a dyadic rational
                got = P.round_decimal_to16(d, dtype)
                gv = float(o.decode16(np.array([got], np.uint16), dtype)[0])
                want = ref(fr)
                assert gv == float(want), (dtype, float(fr), gv, float(want))


@pytest.mark.parametrize("K", [64, 4096])
def test_rmsnorm_matches_float64_reference(K):
    rng = np.random.default_rng(K)
    h = (rng.standard_normal((32, K)) * rng.uniform(0.1, 30.0, size=(32, 1))).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, K).astype(np.float32)
    x, rstd = P.rmsnorm_modulate32(h, gamma, eps=1e-6)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(h.astype(np.float64)), (K,),
                                       torch.from_numpy(gamma.astype(np.float64)), eps=1e-6).numpy()
    assert np.max(np.abs(x - ref) / np.maximum(np.abs(ref), 1e-30)) < 2.0 ** -20
    rref = 1.0 / np.sqrt((h.astype(np.float64) ** 2).mean(axis=1) + 1e-6)
    assert np.max(np.abs(rstd - rref) / rref) < 2.0 ** -22


def test_rmsnorm_modulation_closed_forms():
    rng = np.random.default_rng(3)
    K = 256
    h = rng.standard_normal((8, K)).astype(np.float32)
    scale = rng.uniform(-0.5, 0.5, K).astype(np.float32)
    shift = rng.uniform(-2.0, 2.0, K).astype(np.float32)
    plain, _ = P.rmsnorm_modulate32(h, eps=1e-6)
    mod, _ = P.rmsnorm_modulate32(h, scale=scale, shift=shift, eps=1e-6)
    ref = plain.astype(np.float64) * (1.0 + scale.astype(np.float64)) + shift
    assert np.max(np.abs(mod - ref)) < 1e-5
    # a row of equal values c normalises to sign(c) exactly when eps = 0
    row = np.full((2, K), 3.0, dtype=np.float32)
    row[1] = -0.25
    x, rstd = P.rmsnorm_modulate32(row, eps=0.0)
    assert np.all(x[0] == 1.0) and np.all(x[1] == -1.0)
    assert rstd[0] == np.float32(1.0 / 3.0) and rstd[1] == 4.0


def test_produce_rounds_once_to_the_16bit_type():
    x = np.array([[1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -11, 65504.0]], dtype=np.float32)
    assert P.to16(x, "bf16").tolist() == [[0x3F80, 0x3F82, 0x3F80, 0x4780]]   # ties to even
    assert P.to16(x, "f16").tolist() == [[0x3C04, 0x3C0C, 0x3C00, 0x7BFF]]    # 1 + 2^-11 is a tie: even
    bits = o.round_to_bf16(np.array([[1.5, -2.0]]))
    assert np.array_equal(P.produce(bits, "bf16", "none"), bits)


def test_fused_linear_reduces_to_the_plain_linear_and_adds_bias():
    rng = np.random.default_rng(11)
    M, K, N = 16, 64, 24
    h = rng.standard_normal((M, K)).astype(np.float32)
    h[3, 5] = 9.0
    hb = o.round_to_bf16(h)
    wq, sw = o.quantize_weight_int8(rng.standard_normal((N, K)).astype(np.float32) * 0.02)
    plain = o.int8_mixed_linear(hb, "bf16", wq, sw, 6.0, "f32")
    none = P.fused_int8_linear(hb, "bf16", "none", wq, sw, 6.0, None, "f32")
    assert np.array_equal(none["Y"], plain["Y"]) and np.array_equal(none["q"], plain["q"])
    bias = rng.standard_normal(N).astype(np.float32)
    with_bias = P.fused_int8_linear(hb, "bf16", "none", wq, sw, 6.0, bias, "f32")
    assert np.array_equal(with_bias["y"], plain["y"] + bias.astype(np.float64)[None, :])
    assert np.array_equal(with_bias["Y"], o.round_output(plain["y"] + bias.astype(np.float64)[None, :], "f32"))


def test_fused_gelu_feeds_its_output_to_the_linear():
    """The producer's 16-bit X, not H, decides outliers, scales and codes."""
    rng = np.random.default_rng(12)
    M, K, N = 8, 32, 16
    h = rng.standard_normal((M, K)).astype(np.float32)
    h[2, 7] = 7.0            # GELU(7) = 7: an outlier column after the producer
    h[4, 9] = -7.0           # GELU(-7) ~ 0: no outlier although |h| > 6
    hb = o.round_to_bf16(h)
    wq, sw = o.quantize_weight_int8(rng.standard_normal((N, K)).astype(np.float32) * 0.02)
    ref = P.fused_int8_linear(hb, "bf16", "gelu", wq, sw, 6.0, None, "f32")
    assert ref["O"].tolist() == [7]
    x = o.decode16(ref["x_bits"], "bf16")
    assert x[2, 7] == 7.0 and abs(x[4, 9]) < 1e-6
    # GELU is monotone increasing for h >= 0 and below the identity: the row
    # scale of each row is the largest |X| outside the outlier column
    keep = np.ones(K, bool)
    keep[7] = False
    assert np.array_equal(ref["sx"], np.abs(x[:, keep]).max(axis=1))


def test_rstd_alternatives_cover_every_summation_order():
    """A float64 sum of the squares in numpy's pairwise order, in row order,
    in reverse and sorted ascending all give one of the two rstd readings;
    the exactly rounded sum's rstd is one of them."""
    rng = np.random.default_rng(9)
    K = 4096
    h = (rng.standard_normal((64, K)) * rng.uniform(0.01, 50.0, size=(64, 1))).astype(np.float32)
    h = o.decode16(o.round_to_bf16(h), "bf16")
    a, b = P.rstd_alternatives(h, 1e-6)
    _, exact = P.rmsnorm_modulate32(h, eps=1e-6)
    assert np.all((exact == a) | (exact == b))
    sq = h.astype(np.float64) ** 2
    orders = [sq.sum(axis=1), np.array([sum(r.tolist()) for r in sq]), np.array([sum(r[::-1].tolist()) for r in sq]),
              np.array([sum(np.sort(r).tolist()) for r in sq])]
    for ss in orders:
        r = P._rstd_of_ss(ss, K, 1e-6)
        assert np.all((r == a) | (r == b))
    # a reading applied through the override gives the same X as the default
    x1, _ = P.rmsnorm_modulate32(h, eps=1e-6)
    x2, _ = P.rmsnorm_modulate32(h, eps=1e-6, rstd=exact)
    assert np.array_equal(x1, x2)
