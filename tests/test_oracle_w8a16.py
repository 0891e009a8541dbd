"""Pins of the FP8 weight-only (W8A16) oracle (oracle/w8ref.py) against
references that do not share its arithmetic: torch's own float8_e4m3fn type
evaluating the card's loader expression (weight.to(bf16) * weight_scale),
closed forms, and brute force on tiny inputs."""
import numpy as np
import pytest
import torch

from oracle import w8ref as o


def _bf16_values(rng, n):
    """bf16-representable positive scales of weight-like magnitude."""
    return o.decode16(o.round_to_bf16(rng.uniform(1e-4, 3e-2, n)), "bf16")


def test_dequant_matches_torch_fp8_loader_expression():
    rng = np.random.default_rng(0)
    N = 64
    codes = np.tile(np.arange(256, dtype=np.uint8), (N, 1))
    codes[:, 0x7F] = 0x00          # NaN codes are outside the contract
    codes[:, 0xFF] = 0x80
    sw = _bf16_values(rng, N)
    got = o.dequantize_weight_fp8_bf16(codes, sw)
    w8 = torch.from_numpy(codes).view(torch.float8_e4m3fn)
    scale = torch.from_numpy(sw.astype(np.float32)).to(torch.bfloat16)[:, None]
    ref = (w8.to(torch.bfloat16) * scale).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_dequant_closed_forms():
    # 0x38 = 1.0, 0x40 = 2.0, 0xC4 = -3.0, 0x7E = 448, 0x01 = 2^-9 (smallest subnormal)
    codes = np.array([[0x38, 0x40, 0xC4, 0x7E, 0x01, 0x00, 0x80]], dtype=np.uint8)
    vals = o.decode16(o.dequantize_weight_fp8_bf16(codes, np.array([1.0], np.float32)), "bf16")
    assert vals.tolist() == [[1.0, 2.0, -3.0, 448.0, 2.0 ** -9, 0.0, -0.0]]
    assert np.signbit(vals[0, 6])
    # scale 0.75 (bf16-exact): 448 * 0.75 = 336 is exact in bf16; 1.125 * 0.75 = 0.84375
    # needs 5 significant bits, also exact
    codes = np.array([[0x7E, 0x39]], dtype=np.uint8)          # 448, 1.125
    vals = o.decode16(o.dequantize_weight_fp8_bf16(codes, np.array([0.75], np.float32)), "bf16")
    assert vals.tolist() == [[336.0, 0.84375]]
    # rounding: 1.875 (0x3F) * (1 + 2^-7) = 1.889648... needs 11 bits -> bf16 rounds to 1.890625
    s = np.array([1.0 + 2.0 ** -7], np.float32)
    v = o.decode16(o.dequantize_weight_fp8_bf16(np.array([[0x3F]], np.uint8), s), "bf16")[0, 0]
    assert v == 1.890625


def test_linear_brute_force_tiny():
    rng = np.random.default_rng(1)
    M, K, N = 3, 5, 4
    x_bits = o.round_to_bf16(rng.standard_normal((M, K)))
    codes = rng.integers(0, 256, (N, K)).astype(np.uint8)
    codes[codes == 0x7F] = 0x7E
    codes[codes == 0xFF] = 0xFE
    sw = _bf16_values(rng, N)
    ref = o.fp8_w8a16_linear(x_bits, "bf16", codes, sw, "f32")
    x = o.decode16(x_bits, "bf16")
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                wv = float(o.e4m3_decode(codes[n, k])) * float(sw[n])
                wb = float(o.decode16(o.round_to_bf16(np.array([wv])), "bf16")[0])
                acc += float(x[m, k]) * wb
            assert abs(ref["y"][m, n] - acc) <= 1e-12 * max(1.0, abs(acc))


def test_one_hot_rows_read_back_the_dequantised_weights():
    """X = I gives Y = W_deq^T exactly (one product per output)."""
    rng = np.random.default_rng(2)
    K, N = 48, 40
    codes = rng.integers(0, 0x7F, (N, K)).astype(np.uint8) | (rng.integers(0, 2, (N, K)) << 7).astype(np.uint8)
    sw = _bf16_values(rng, N)
    x_bits = o.round_to_bf16(np.eye(K))
    ref = o.fp8_w8a16_linear(x_bits, "bf16", codes, sw, "f32")
    assert np.array_equal(ref["Y"].T.astype(np.float64), o.decode16(ref["w_bits"], "bf16").astype(np.float64))


def test_unit_scale_small_integers_are_exact():
    rng = np.random.default_rng(3)
    M, K, N = 8, 64, 16
    ints = rng.integers(-8, 9, (N, K)).astype(np.float32)
    codes = o.e4m3_encode(ints)                           # integers up to 8 are E4M3 values
    assert np.array_equal(o.e4m3_decode(codes), ints)
    xi = rng.integers(-4, 5, (M, K)).astype(np.float64)
    ref = o.fp8_w8a16_linear(o.round_to_bf16(xi), "bf16", codes, np.ones(N, np.float32), "f32")
    assert np.array_equal(ref["y"], xi @ ints.T.astype(np.float64))


@pytest.mark.parametrize("out_dtype", ["bf16", "f16", "f32"])
def test_rows_subset_and_output_rounding(out_dtype):
    rng = np.random.default_rng(4)
    M, K, N = 20, 128, 24
    x_bits = o.round_to_bf16(rng.standard_normal((M, K)))
    codes, sw = o.quantize_weight_fp8(rng.standard_normal((N, K)).astype(np.float32) * 0.02)
    full = o.fp8_w8a16_linear(x_bits, "bf16", codes, sw, out_dtype)
    part = o.fp8_w8a16_linear(x_bits, "bf16", codes, sw, out_dtype, rows=[3, 17])
    assert np.array_equal(part["Y"], full["Y"][[3, 17]])
    assert np.array_equal(full["Y"], o.round_output(full["y"], out_dtype))



def test_weight_only_is_closer_to_the_float_linear_than_w8a8():
    """The card measures weight-only above W8A8 on the same weights (section
    "How it was tested"): without activation quantisation the error to the
    unquantised linear is smaller."""
    rng = np.random.default_rng(5)
    M, K, N = 64, 512, 96
    x_bits = o.round_to_bf16(rng.standard_normal((M, K)))
    w = rng.standard_normal((N, K)).astype(np.float32) * 0.02
    codes, sw = o.quantize_weight_fp8(w)
    exact = o.decode16(x_bits, "bf16").astype(np.float64) @ w.astype(np.float64).T
    e16 = o.relative_l2(o.fp8_w8a16_linear(x_bits, "bf16", codes, sw, "f32")["y"], exact)
    e8 = o.relative_l2(o.fp8_w8a8_linear(x_bits, "bf16", codes, sw, None, "f32")["y"], exact)
    assert e16 < e8
    assert e16 < 0.06                   # E4M3 weights: about 3 bits of mantissa
