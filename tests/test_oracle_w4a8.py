"""Pins of the W4A8 oracle (oracle/w4a8.py): hand examples of the int4 group
codes and the packed layout, round trips, brute force on tiny inputs, and the
grouped sum against a dequantise-then-multiply evaluation in exact rationals."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import w4a8 as o4
from oracle import w8ref as o


def test_group_codes_hand_example():
    # one row, two groups of 8: absmax 3.5 -> step 0.5; absmax 0 -> all zero
    w = np.array([[3.5, -3.5, 0.25, 0.75, -1.0, 1.25, 0.0, 2.0] + [0.0] * 8], dtype=np.float32)
    q, s = o4.quantize_groups_int4(w, group=8)
    assert s.tolist() == [[3.5, 0.0]]
    # 0.25 / 0.5 = 0.5 -> 0 (tie to even); 0.75 / 0.5 = 1.5 -> 2; 1.25 / 0.5 = 2.5 -> 2
    assert q[0, :8].tolist() == [7, -7, 0, 2, -2, 2, 0, 4]
    assert np.all(q[0, 8:] == 0)


def test_group_codes_error_bound_and_symmetry():
    rng = np.random.default_rng(1)
    w = rng.standard_normal((16, 512)).astype(np.float32)
    q, s = o4.quantize_groups_int4(w)
    assert q.min() >= -7 and q.max() <= 7
    deq = q.astype(np.float64).reshape(16, 4, 128) * (s.astype(np.float64) / 7.0)[:, :, None]
    err = np.abs(deq.reshape(16, 512) - w)
    step = np.repeat(s.astype(np.float64) / 7.0, 128, axis=1)
    assert np.all(err <= 0.5 * step * (1 + 1e-6))
    q2, s2 = o4.quantize_groups_int4(-w)
    assert np.array_equal(q2, -q) and np.array_equal(s2, s)
    # every group reaches +-7 at its absmax
    assert np.all(np.abs(q).reshape(16, 4, 128).max(axis=2) == 7)


def test_pack_layout_hand_example():
    q = np.array([[1, 2, 3, -1, -8, 7, 0, -2]], dtype=np.int8)
    p = o4.pack_int4(q)
    # byte b: low nibble k = b, high nibble k = b + 4
    assert p.tolist() == [[0x81, 0x72, 0x03, 0xEF]]
    assert np.array_equal(o4.unpack_int4(p), q)
    # the high nibble of a byte, read as int8, is 16 x its code; the low one after a 4-bit shift
    b = p.view(np.int8)
    assert (b & np.int8(-16)).tolist()[0] == [16 * v for v in (-8, 7, 0, -2)]
    assert ((p << 4).view(np.int8)).tolist()[0] == [16 * v for v in (1, 2, 3, -1)]


def test_pack_round_trip_random():
    rng = np.random.default_rng(2)
    q = rng.integers(-8, 8, (7, 256)).astype(np.int8)
    assert np.array_equal(o4.unpack_int4(o4.pack_int4(q)), q)


def test_linear_brute_force_tiny():
    rng = np.random.default_rng(3)
    M, K, N, G = 3, 16, 2, 8
    x_bits = o.round_to_bf16(rng.standard_normal((M, K)))
    packed, sw = o4.quantize_weight_int4(rng.standard_normal((N, K)).astype(np.float32), group=G)
    ref = o4.w4a8_linear(x_bits, "bf16", packed, sw, "f32", group=G)
    x = o.decode16(x_bits, "bf16")
    qw = o4.unpack_int4(packed)
    for m in range(M):
        sxm = float(np.abs(x[m]).max())
        r = np.float32(127.0) / np.float32(sxm)
        qx = [int(np.clip(np.rint(np.float32(v) * r), -127, 127)) for v in x[m]]
        for n in range(N):
            tot = 0.0
            for g in range(K // G):
                a = sum(qx[k] * int(qw[n, k]) for k in range(g * G, (g + 1) * G))
                tot += a * float(sw[g, n]) / 7.0
            want = tot * sxm / 127.0
            assert abs(ref["y"][m, n] - want) <= 1e-12 * max(1.0, abs(want))


def test_grouped_sum_equals_dequantised_product_exactly():
    """sum_g (sw/7) sum_k qx qw == sum_k qx (qw sw/7), evaluated in exact
    rationals on the dequantised weights (a different order of operations)."""
    rng = np.random.default_rng(4)
    M, K, N = 2, 256, 3
    x_bits = o.round_to_bf16(rng.standard_normal((M, K)))
    w = rng.standard_normal((N, K)).astype(np.float32)
    w[:, :128] *= 100.0                             # groups with very different scales
    packed, sw = o4.quantize_weight_int4(w)
    ref = o4.w4a8_linear(x_bits, "bf16", packed, sw, "f32")
    qw = o4.unpack_int4(packed)
    for m in range(M):
        for n in range(N):
            exact = Fraction(0)
            for k in range(K):
                exact += Fraction(int(ref["qx"][m, k])) * Fraction(int(qw[n, k])) * Fraction(float(sw[k // 128, n])) / 7
            exact *= Fraction(float(ref["sx"][m])) / 127
            assert abs(ref["y"][m, n] - float(exact)) <= 1e-12 * max(1.0, abs(float(exact)))


def test_zero_rows_and_groups():
    x_bits = o.round_to_bf16(np.zeros((2, 128)))
    packed, sw = o4.quantize_weight_int4(np.zeros((3, 128), np.float32))
    ref = o4.w4a8_linear(x_bits, "bf16", packed, sw, "f16")
    assert np.all(ref["y"] == 0.0) and np.all(sw == 0.0)


@pytest.mark.parametrize("out_dtype", ["f16", "f32"])
def test_close_to_the_float_linear(out_dtype):
    rng = np.random.default_rng(5)
    M, K, N = 32, 1024, 48
    x_bits = o.round_to_bf16(rng.standard_normal((M, K)))
    w = rng.standard_normal((N, K)).astype(np.float32) * 0.02
    packed, sw = o4.quantize_weight_int4(w)
    ref = o4.w4a8_linear(x_bits, "bf16", packed, sw, out_dtype)
    exact = o.decode16(x_bits, "bf16").astype(np.float64) @ w.astype(np.float64).T
    e = o.relative_l2(ref["y"], exact)
    assert 0.02 < e < 0.15          # int4 weights: about 3 bits; int8 activations add little
