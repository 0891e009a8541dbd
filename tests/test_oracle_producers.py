"""Pins of the producer oracle (oracle/producers.py) against references that
do not share its arithmetic: float64 library routines (numpy exp, torch's
tanh-form GELU and RMSNorm), closed forms and special values."""
import math

import numpy as np
import pytest
import torch

from oracle import producers as P
from oracle import w8ref as o


def test_exp32_is_accurate_and_exact_at_zero():
    x = np.linspace(-87.0, 88.0, 400001).astype(np.float32)
    got = P.exp32(x).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    assert np.max(np.abs(got - ref) / ref) < 2.0 ** -21          # about 2 ulp of float32
    assert P.exp32(np.float32(0.0)) == 1.0
    assert P.exp32(np.float32(1.0)) == np.float32(math.e)        # e rounded to float32
    assert P.exp32(np.float32(89.0)) == np.inf                   # past FLT_MAX
    assert P.exp32(np.float32(-110.0)) == 0.0                    # below the subnormals


def test_gelu32_matches_float64_reference():
    h = np.linspace(-12.0, 12.0, 200001).astype(np.float32)
    got = P.gelu32(h).astype(np.float64)
    ref = torch.nn.functional.gelu(torch.from_numpy(h.astype(np.float64)), approximate="tanh").numpy()
    assert np.max(np.abs(got - ref)) < 2e-6
    big = np.abs(ref) > 1e-3
    assert np.max(np.abs(got - ref)[big] / np.abs(ref[big])) < 4e-6
    # the same function as 0.5 h (1 + tanh u), written independently in float64
    u = math.sqrt(2.0 / math.pi) * (h.astype(np.float64) + 0.044715 * h.astype(np.float64) ** 3)
    assert np.max(np.abs(got - 0.5 * h * (1.0 + np.tanh(u)))) < 2e-6


def test_gelu32_special_values():
    g = P.gelu32(np.array([0.0, 20.0, -20.0, 1.0, -1.0], dtype=np.float32))
    assert g[0] == 0.0
    assert g[1] == 20.0                                          # exp(-2u) vanishes
    assert g[2] == 0.0 and np.signbit(g[2])                      # -20 / inf
    assert abs(g[3] - 0.8411919906082768) < 1e-6                 # tanh-form GELU(1)
    assert abs(g[4] + 0.15880800939172324) < 1e-6


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
