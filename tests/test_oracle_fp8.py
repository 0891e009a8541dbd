"""Pins for the FP8-E4M3 part of the oracle.

The E4M3 table and encoder are checked against torch's float8_e4m3fn (an
independent implementation of the same OCP format) and against hand values;
the quantisers against the FP8 card's own claim that dequantisation error is
quantisation noise; the linear against closed forms.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import w8ref as o


def bf16(a):
    return synth.encode16(np.asarray(a, np.float32), "bf16")


def torch_e4m3(v):
    t = torch.from_numpy(np.asarray(v, np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_table_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = o.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])


def test_encode_matches_torch_below_saturation():
    rng = np.random.default_rng(20)
    v = (rng.standard_normal(200000) * 10.0 ** rng.uniform(-4, 2.6, 200000)).astype(np.float32)
    v = v[np.abs(v) < 448]
    # every exact midpoint between neighbouring codes, and its float32 neighbours
    pos = o.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    extra = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(500)),
                            pos.astype(np.float32)])
    v = np.concatenate([v, extra, -extra]).astype(np.float32)
    v = v[np.abs(v) < 448]
    assert np.array_equal(o.e4m3_encode(v), torch_e4m3(v))


def test_encode_saturates_and_keeps_sign_of_zero():
    v = np.array([448, 449, 463.9, 464, 500, 1e30, -448, -1e9, 0.0, -0.0, -2.0 ** -11, -2.0 ** -12, 2.0 ** -11,
                  np.inf, -np.inf], np.float32)
    got = o.e4m3_encode(v).tolist()
    assert got == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x00, 0x80, 0x80, 0x80, 0x00, 0x7E, 0xFE]
    # torch agrees once the input is clamped to the finite range
    assert np.array_equal(o.e4m3_encode(v), torch_e4m3(np.clip(v, -448, 448)))


def test_hand_values():
    # ties go to the even code; subnormal spacing is 2^-9
    cases = {1.0625: 0x38, 1.1875: 0x3A, 2.0 ** -9: 0x01, 2.0 ** -10: 0x00, 3 * 2.0 ** -10: 0x02,
             460.0: 0x7E, 500.0: 0x7E, -0.3: 0xAA}
    got = o.e4m3_encode(np.array(list(cases), np.float32)).tolist()
    assert got == list(cases.values())
    codes, sx = o.quantize_activations_fp8(np.array([[448.0, 1.0, -0.3, 0.0]], np.float32))
    assert sx.tolist() == [1.0] and codes.tolist() == [[0x7E, 0x38, 0xAA, 0x00]]


def test_encode_decode_roundtrip_on_every_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = o.e4m3_decode(codes).astype(np.float32)
    back = o.e4m3_encode(vals)
    assert np.array_equal(back, codes)


def _dequant_bound(w, sw):
    """Half a unit in the last place of E4M3 at |w/sw|, times sw: 2^-4 of the
    binade for normals, 2^-10 below 2^-6; plus float32 slack."""
    a = np.abs(w.astype(np.float64)) / np.where(sw == 0, 1, sw)[:, None]
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    half_ulp = np.where(a < 2.0 ** -6, 2.0 ** -10, 2.0 ** (e - 4))
    return sw[:, None].astype(np.float64) * (half_ulp * (1 + 2.0 ** -20) + a * 2.0 ** -23)


def test_weight_quantisation_error_is_quantisation_noise():
    """The ModelOpt FP8 card reports dequantised weights match the bf16
    originals up to FP8 quantisation noise: |w - dec(q) sw| is at most half
    an E4M3 step (the saturated top value included)."""
    rng = np.random.default_rng(21)
    w = o.decode16(bf16(rng.standard_normal((64, 300)) * 0.02), "bf16")
    w[3] = 0.0
    codes, sw = o.quantize_weight_fp8(w)
    assert np.array_equal(sw, o.decode16(bf16(sw), "bf16"))            # scales are bf16 values
    assert sw[3] == 0 and not codes[3].any()
    assert np.all(np.isfinite(sw)) and np.all(sw[np.arange(64) != 3] > 0)
    err = np.abs(w.astype(np.float64) - o.e4m3_decode(codes) * sw[:, None])
    bound = _dequant_bound(w, sw)
    # The bf16-rounded scale may put the top element slightly above 448,
    # where it saturates: allow the saturation gap for those elements.
    sat = np.abs(w.astype(np.float64)) / np.where(sw == 0, 1, sw)[:, None] > 448
    gap = np.abs(w.astype(np.float64)) - 448 * sw[:, None]
    assert np.all(np.where(sat, err <= gap + bound, err <= bound))


def test_dynamic_scale_maps_row_max_to_448():
    rng = np.random.default_rng(22)
    x = o.decode16(bf16(rng.standard_normal((16, 128))), "bf16")
    codes, sx = o.quantize_activations_fp8(x)
    assert np.array_equal(sx, (np.abs(x).max(axis=1) / np.float32(448)).astype(np.float32))
    am = np.abs(x).argmax(axis=1)
    top = codes[np.arange(16), am] & 0x7F
    # fl32(x / fl32(amax/448)) lies within 2 ulp of 448, which rounds to 448
    assert np.all(top == 0x7E)


def test_static_scale_exact_operands_give_exact_gemm():
    """With static scale 1 and operands that are E4M3 values, the codes
    are exact, so Y = sw * X . (dec(Wq8))^T  with no quantisation error."""
    rng = np.random.default_rng(23)
    grid = o.e4m3_decode(np.arange(0, 0x70, dtype=np.uint8))          # up to 2^7
    x = (rng.choice(grid, size=(9, 64)) * rng.choice([-1, 1], size=(9, 64))).astype(np.float32)
    wc = rng.integers(0, 0x70, size=(7, 64)).astype(np.uint8) | (rng.integers(0, 2, size=(7, 64)) * 0x80).astype(np.uint8)
    sw = np.array([0.5, 1.0, 2.0 ** -3, 3.0, 1.25, 0.75, 2.0], np.float32)
    r = o.fp8_w8a8_linear(bf16(x), "bf16", wc, sw, act_scale=1.0, out_dtype="f32")
    ref = x.astype(np.float64) @ (o.e4m3_decode(wc) * sw[:, None]).T
    assert np.array_equal(r["y"], ref)
    assert np.array_equal(o.e4m3_decode(r["xq"]), x.astype(np.float64))


def test_static_scale_saturates_massive_activations():
    """A per-tensor scale from "max" calibration on ordinary activations
    saturates a massive activation (13000 in channel 2276) at 448 * s."""
    c = synth.fp8_text_encoder("q", massive=True)
    x = o.decode16(c.x_bits, "bf16")
    cal = o.decode16(c.extra["x_cal_bits"], "bf16")
    s = np.float32(np.abs(cal).max() / np.float32(448))
    codes, sx = o.quantize_activations_fp8(x, act_scale=s)
    assert codes[0, 2276] == 0x7E and codes[1, 2276] == 0x7E
    dyn_codes, dyn_sx = o.quantize_activations_fp8(x)
    assert x[0, 2276] == 12992.0                   # 13000 in bf16
    assert dyn_sx[0] == np.float32(np.float32(12992) / np.float32(448))


@pytest.mark.parametrize("seed", [24, 25])
def test_fp8_linear_error_bound_against_float_gemm(seed):
    """|Y - X W^T| is bounded by the per-element coding errors of both
    operands; a swapped operand, sign or index would exceed it."""
    rng = np.random.default_rng(seed)
    x = o.decode16(bf16(rng.standard_normal((12, 256))), "bf16").astype(np.float64)
    w = o.decode16(bf16(rng.standard_normal((10, 256)) * 0.02), "bf16").astype(np.float64)
    wc, sw = o.quantize_weight_fp8(w.astype(np.float32))
    r = o.fp8_w8a8_linear(bf16(x), "bf16", wc, sw, None, "f32")
    xd = o.e4m3_decode(r["xq"]) * r["sx"][:, None]
    wd = o.e4m3_decode(wc) * sw[:, None]
    assert np.allclose(r["y"], xd @ wd.T, rtol=1e-12, atol=1e-15)
    ex = np.abs(x - xd)
    ew = np.abs(w - wd)
    bound = ex @ np.abs(w).T + np.abs(x) @ ew.T + ex @ ew.T
    assert np.all(np.abs(r["y"] - x @ w.T) <= bound * (1 + 1e-9) + 1e-12)
    # the per-element errors themselves are at most half an E4M3 step
    assert np.all(ex <= _dequant_bound(x.astype(np.float32), r["sx"]))


def test_error_metric_definitions():
    a = np.array([[1.0, 0.0], [0.0, 2.0]])
    assert o.relative_l2(a, a) == 0.0
    assert math.isclose(o.relative_l2(2 * a, a), 1.0)
    assert math.isclose(o.mean_token_cosine(a, 3 * a), 1.0)
    assert math.isclose(o.mean_token_cosine(a, -a), -1.0)


def test_weight_scale_is_rounded_to_nearest_even_bf16():
    """The per-channel scale is stored as bf16 ("Qwen-Image-2.1 Text Encoder:
    FP8" card, section "Format"): sw = bf16(fl32(amax / 448)), round to
    nearest even, and the codes use that rounded scale.

    amax = 65/64 gives fl32(amax/448) = 0x3B149249, whose low half is above
    the bf16 midpoint: round to nearest gives 0x3B15 (0.0022735595703125),
    truncation would give 0x3B14. A row of amax = 1.0 has fl32(1/448) =
    0x3B12_4925 (below the midpoint, rounds down either way). The expected
    scales come from exact rationals and from torch's own fp32 -> bf16 cast;
    the expected codes from torch's float8_e4m3fn cast of fl32(w / sw)."""
    from fractions import Fraction
    from tests.exact import to_bf16, to_f32

    w_rows = np.array([[65 / 64, 0.002197265625, 0.002685546875, -0.00439453125, 0.0087890625, 0.0],
                       [1.0, 0.5, -0.25, 0.125, -0.0625, 2.0 ** -12]], np.float32)
    codes, sw = o.quantize_weight_fp8(w_rows)
    want = []
    for row in w_rows:
        amax = Fraction(float(np.abs(row).max()))
        want.append(float(to_bf16(to_f32(amax / 448))))
    assert sw.tolist() == want
    assert sw[0] == np.float32(0.0022735595703125)               # 0x3B15, not the truncated 0x3B14
    s32 = (np.abs(w_rows).max(axis=1) / np.float32(448)).astype(np.float32)
    tb = torch.from_numpy(s32).to(torch.bfloat16).float().numpy()
    assert np.array_equal(sw, tb)
    ratio = (w_rows / sw[:, None]).astype(np.float32)
    assert np.array_equal(codes, torch_e4m3(ratio))
    # with the rounded scale these weights take the codes below; a truncated
    # scale would move each of the four non-top entries up by one code
    assert codes[0, :5].tolist() == [0x7E, 0x37, 0x39, 0xBF, 0x47]
