"""Pins for the oracle's 16-bit decoders and final roundings.

Each check compares the oracle with something outside it: Python's own
binary16 packing (struct 'e'), exact rational rounding, or torch's bfloat16.
"""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import w8ref as o
from tests.exact import to_bf16, to_f16


def test_decode_f16_all_patterns_match_struct():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = o.decode16(bits, "f16")
    for b in range(0, 65536, 7):
        (ref,) = struct.unpack("<e", struct.pack("<H", b))
        g = float(got[b])
        if math.isnan(ref):
            assert math.isnan(g)
        else:
            assert g == ref and math.copysign(1, g) == math.copysign(1, ref), hex(b)


def test_decode_bf16_all_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = o.decode16(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    both_nan = np.isnan(got) & np.isnan(ref)
    assert np.array_equal(got.view(np.uint32)[~both_nan], ref.view(np.uint32)[~both_nan])


def _f16_probe_values(rng):
    vals = list(rng.standard_normal(2000) * 10.0 ** rng.integers(-8, 5, 2000))
    # exact halfway points between neighbouring binary16 values, both parities
    for b in list(range(0x0001, 0x7BFF, 97)) + [0x03FF, 0x0400, 0x7BFE]:
        lo = struct.unpack("<e", struct.pack("<H", b))[0]
        hi = struct.unpack("<e", struct.pack("<H", b + 1))[0]
        vals += [(lo + hi) / 2, -(lo + hi) / 2, np.nextafter((lo + hi) / 2, 0)]
    vals += [65504.0, 65519.99, 65520.0, 1e6, -1e6, 2.0 ** -25, 2.0 ** -26, 0.0, -0.0]
    return vals


def test_round_to_f16_matches_struct_pack():
    rng = np.random.default_rng(7)
    vals = _f16_probe_values(rng)
    got = o.round_to_f16(np.array(vals))
    for v, g in zip(vals, got):
        try:
            ref = struct.unpack("<H", struct.pack("<e", v))[0]
        except OverflowError:  # struct refuses values that round to inf
            ref = 0x7C00 if v > 0 else 0xFC00
        assert int(g) == ref, (v, hex(int(g)), hex(ref))


def test_round_to_f16_matches_exact_rationals():
    rng = np.random.default_rng(8)
    vals = _f16_probe_values(rng)[::3]
    got = o.decode16(o.round_to_f16(np.array(vals)), "f16")
    for v, g in zip(vals, got):
        ref = to_f16(Fraction(v))
        assert (float(ref) == float(g)), (v, g, ref)


def test_round_to_bf16_matches_exact_rationals():
    rng = np.random.default_rng(9)
    vals = list(rng.standard_normal(3000) * 10.0 ** rng.integers(-40, 39, 3000))
    # exact ties (odd and even lower neighbour), values one ulp off a tie,
    # the subnormal range, and overflow
    for b in list(range(0x0001, 0x7F7F, 251)) + [0x007F, 0x0080, 0x7F7E]:
        lo = float(o.decode16(np.array([b], np.uint16), "bf16")[0])
        hi = float(o.decode16(np.array([b + 1], np.uint16), "bf16")[0])
        mid = (lo + hi) / 2
        vals += [mid, -mid, np.nextafter(mid, 0.0), np.nextafter(mid, math.inf)]
    vals += [3.4e38, 3.39e38, -3.4e38, 1e-45, 0.0, -0.0]
    got = o.decode16(o.round_to_bf16(np.array(vals)), "bf16")
    for v, g in zip(vals, got):
        ref = to_bf16(Fraction(v))
        assert float(ref) == float(g), (v, g, ref)
        if v == 0:
            assert math.copysign(1, float(g)) == math.copysign(1, v)


def test_round_to_bf16_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(10)
    f = (rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000)).astype(np.float32)
    got = o.round_to_bf16(f.astype(np.float64))
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
def test_round_output_is_identity_on_representable(dt):
    rng = np.random.default_rng(11)
    x = rng.standard_normal(1000)
    once = o.stored_to_f64(o.round_output(x, dt), dt)
    twice = o.stored_to_f64(o.round_output(once, dt), dt)
    assert np.array_equal(once, twice)
