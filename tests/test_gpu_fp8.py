"""GPU parity of the FP8-E4M3 W8A8 path against the CPU oracle.

Bit-exact: E4M3 weight codes, bf16-valued weight scales, activation codes and
scales (dynamic and static). Outputs: relative Frobenius error <= 1e-2 for
16-bit outputs, <= 2e-3 for fp32 (the int8 path's bounds; FP8 accumulation is
fp32 on both sides of the comparison's error budget), globally and per row,
and element by element within half an output ulp plus the float32
accumulation's own error (tests/bounds.py).
"""
import numpy as np
import pytest
import torch

import synth
import w8a8_mixed_precision_amd as w8
from oracle import w8ref as o
from tests import bounds
from tests.gpu_util import OUT, announce, dev16, host_stored, rel_fro, row_rel_fro

pytestmark = pytest.mark.gpu

TOL = {"f16": 1e-2, "bf16": 1e-2, "f32": 2e-3}


def _weights(case):
    wf = o.decode16(case.w_bits, case.w_dtype)
    wq_ref, sw_ref = o.quantize_weight_fp8(wf)
    wq, sw = w8.quantize_weight_rowwise(dev16(case.w_bits, case.w_dtype), "fp8")
    torch.cuda.synchronize()
    return wq, sw, wq_ref, sw_ref


def _static_scale(case):
    cal = o.decode16(case.extra["x_cal_bits"], case.x_dtype) if "x_cal_bits" in case.extra else \
        o.decode16(case.x_bits, case.x_dtype)
    return np.float32(np.abs(cal).max() / np.float32(448.0))


SMALL = [
    synth.random_linear(300, 272, 520, seed=51, x_dtype="bf16", name="ragged_bf16"),
    synth.random_linear(129, 48, 77, seed=52, x_dtype="f16", name="ragged_f16"),
    synth.random_linear(64, 1040, 256, seed=53, x_dtype="bf16", outlier_cols=3, outlier_lo=100, outlier_hi=2000,
                        name="wide_range"),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: c.name)
def test_fp8_weight_quantisation_bit_exact(case):
    announce("fp8 weight quant", case.name)
    wq, sw, wq_ref, sw_ref = _weights(case)
    assert np.array_equal(sw.cpu().numpy(), sw_ref)
    assert np.array_equal(wq.cpu().numpy(), wq_ref)


@pytest.mark.parametrize("case", SMALL, ids=lambda c: c.name)
@pytest.mark.parametrize("static", [False, True])
def test_fp8_activation_quantisation_bit_exact(case, static):
    xf = o.decode16(case.x_bits, case.x_dtype)
    s = _static_scale(case) if static else None
    xq_ref, sx_ref = o.quantize_activations_fp8(xf, s)
    announce("fp8 act quant", case.name, static)
    sp = torch.tensor([s], dtype=torch.float32, device="cuda") if static else None
    xq, sx = w8.debug_fp8_quantize_activations(dev16(case.x_bits, case.x_dtype), sp)
    assert np.array_equal(sx.cpu().numpy(), sx_ref)
    assert np.array_equal(xq.cpu().numpy(), xq_ref)


@pytest.mark.parametrize("scale", [1.0, 0.125, 3.0, 2.0 ** -20])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_every_16bit_value_encodes_like_the_oracle(scale, dtype):
    """All finite patterns of the format through the static-scale E4M3
    encoder (covers saturation, subnormals, ties and the sign of zero)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    fin = bits[np.isfinite(o.decode16(bits, dtype))]
    rows = np.concatenate([fin, np.zeros((-fin.size) % 256, np.uint16)]).reshape(-1, 256)
    xf = o.decode16(rows, dtype)
    xq_ref, sx_ref = o.quantize_activations_fp8(xf, np.float32(scale))
    announce("fp8 exhaustive encode", dtype, scale)
    xq, sx = w8.debug_fp8_quantize_activations(dev16(rows, dtype),
                                               torch.tensor([scale], dtype=torch.float32, device="cuda"))
    assert np.array_equal(xq.cpu().numpy(), xq_ref)


def _check(y, ref, out_dtype, label, wq_ref=None, sw_ref=None):
    """ref: the oracle's result dict; with the oracle's weights, element by
    element too."""
    stored = host_stored(y, out_dtype)
    got = o.stored_to_f64(stored, out_dtype)
    want = o.stored_to_f64(ref["Y"], out_dtype)
    assert np.all(np.isfinite(got)) and np.std(got) > 0, label
    e, er = rel_fro(got, want), row_rel_fro(got, want).max()
    assert e <= TOL[out_dtype] and er <= TOL[out_dtype], (label, e, er)
    if wq_ref is not None:
        err = bounds.fp8_err32(ref, wq_ref, sw_ref, ref["xq"].shape[1])
        bounds.assert_elementwise(stored, out_dtype, ref["y"], err, label)


@pytest.mark.parametrize("case", SMALL, ids=lambda c: c.name)
@pytest.mark.parametrize("out_dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("static", [False, True])
def test_fp8_linear_matches_oracle(case, out_dtype, static):
    wq, sw, wq_ref, sw_ref = _weights(case)
    s = _static_scale(case) if static else None
    ref = o.fp8_w8a8_linear(case.x_bits, case.x_dtype, wq_ref, sw_ref, s, out_dtype)
    announce("fp8_w8a8_linear", case.name, out_dtype, static)
    sp = torch.tensor([s], dtype=torch.float32, device="cuda") if static else None
    y = w8.fp8_w8a8_linear(dev16(case.x_bits, case.x_dtype), wq, sw, sp, OUT[out_dtype])
    torch.cuda.synchronize()
    _check(y, ref, out_dtype, (case.name, static), wq_ref, sw_ref)


@pytest.mark.parametrize("layer", list(synth.FP8_TEXT_LAYERS))
@pytest.mark.parametrize("static", [False, True])
def test_fp8_text_encoder_full_size(layer, static):
    c = synth.fp8_text_encoder(layer, massive=(layer == "q"))
    wq, sw, wq_ref, sw_ref = _weights(c)
    assert np.array_equal(sw.cpu().numpy(), sw_ref) and np.array_equal(wq.cpu().numpy(), wq_ref)
    s = _static_scale(c) if static else None
    xf = o.decode16(c.x_bits, "bf16")
    xq_ref, sx_ref = o.quantize_activations_fp8(xf, s)
    announce("fp8 text encoder", c.name, static)
    sp = torch.tensor([s], dtype=torch.float32, device="cuda") if static else None
    x = dev16(c.x_bits, "bf16")
    xq, sx = w8.debug_fp8_quantize_activations(x, sp)
    assert np.array_equal(xq.cpu().numpy(), xq_ref) and np.array_equal(sx.cpu().numpy(), sx_ref)
    ref = o.fp8_w8a8_linear(c.x_bits, "bf16", wq_ref, sw_ref, s, "bf16")
    y = w8.fp8_w8a8_linear(x, wq, sw, sp, torch.bfloat16)
    _check(y, ref, "bf16", c.name, wq_ref, sw_ref)


@pytest.mark.parametrize("part", ["qkv", "up"])
@pytest.mark.parametrize("static", [True, False])
def test_fp8_dit_1024_full_size(part, static):
    """FP8 W8A8 at the DiT 1024^2 shapes (4352 tokens, K = 4096, N = 12288 /
    16384), the static per-tensor input scale of the ModelOpt FP8 card
    ("max" calibration on an independent draw) and the dynamic per-token one:
    codes and scales on every row bit-exact, outputs on sampled rows (every
    injected row, the ragged last 256-row strip) within the bounds."""
    c = synth.dit_qkv_1024() if part == "qkv" else synth.dit_mlp_1024("up")
    wq, sw, wq_ref, sw_ref = _weights(c)
    assert np.array_equal(sw.cpu().numpy(), sw_ref) and np.array_equal(wq.cpu().numpy(), wq_ref)
    cal = synth.calibration_draw(c.M, c.K, seed=3001 + (part == "up"))
    s = np.float32(np.abs(o.decode16(cal, "bf16")).max() / np.float32(448.0)) if static else None
    xf = o.decode16(c.x_bits, "bf16")
    xq_ref, sx_ref = o.quantize_activations_fp8(xf, s)
    announce("fp8 dit 1024", c.name, static)
    sp = torch.tensor([s], dtype=torch.float32, device="cuda") if static else None
    x = dev16(c.x_bits, "bf16")
    xq, sx = w8.debug_fp8_quantize_activations(x, sp)
    assert np.array_equal(xq.cpu().numpy(), xq_ref) and np.array_equal(sx.cpu().numpy(), sx_ref)
    rng = np.random.default_rng(46)
    rows = np.unique(np.concatenate([rng.choice(c.M, 64, replace=False), np.array(c.injected_rows, int),
                                     [0], np.arange((c.M - 1) // 256 * 256, c.M)])).astype(int)
    y = w8.fp8_w8a8_linear(x, wq, sw, sp, torch.bfloat16)
    xs = c.x_bits[rows]
    ref = o.fp8_w8a8_linear(xs, "bf16", wq_ref, sw_ref, s, "bf16")
    if not static:
        assert np.array_equal(ref["sx"], sx_ref[rows])
    _check(y[torch.from_numpy(rows).cuda()], ref, "bf16", (c.name, static), wq_ref, sw_ref)


def _random_codes(rng, shape):
    """E4M3 codes without the two NaN patterns (0x7F, 0xFF)."""
    c = rng.integers(0, 254, size=shape, dtype=np.int64)
    c = np.where(c >= 0x7F, c + 1, c)                       # skip 0x7F
    return c.astype(np.uint8)


# (M, K, N): K % 64 == 0 takes the pipelined kernel; ragged M and N, a single
# row, one tile, and grids of 1..6 tiles that the K-slicing spreads over.
GEMM_SHAPES = [(300, 4096, 520), (77, 2048, 300), (512, 1024, 256), (1, 640, 16), (257, 4160, 513),
               (512, 12288, 1024)]


@pytest.mark.parametrize("shape", GEMM_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("tile,split", [(0, 0), (256, 1), (256, 2), (256, 3), (256, 5), (256, 8),
                                        (128, 1), (128, 2), (128, 3), (128, 8),
                                        (129, 1), (129, 2), (129, 5), (192, 1), (192, 2), (192, 3), (192, 8)])
@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_fp8_gemm_tiling_and_k_slicing_match_oracle(shape, tile, split, out_dtype):
    """The FP8 GEMM for every block shape (256x256, 128x128 on 64-byte K steps;
    128x128 = tile 129 and 128x192 on 128-byte K steps) and several K-slicings
    against the exact contraction; the sliced result is bitwise the same on a
    repeated call (fixed summation order) and the bookkeeping counters are left
    zero."""
    M, K, N = shape
    step = 128 if tile in (129, 192) else 64
    if tile in (129, 192) and K % 128:
        pytest.skip("128-byte K steps need K % 128 == 0")
    if split > K // step:
        pytest.skip("more slices than K steps")
    rng = np.random.default_rng(7000 + M + K + N + split + tile)
    xq, wq = _random_codes(rng, (M, K)), _random_codes(rng, (N, K))
    sx = rng.uniform(0.5, 2.0, size=M).astype(np.float32) / np.float32(448.0)
    sw = rng.uniform(0.5, 2.0, size=N).astype(np.float32) / np.float32(448.0)
    acc = o.fp8_contract(xq, wq)
    want = o.stored_to_f64(o.round_output(sx[:, None].astype(np.float64) * sw[None, :] * acc, out_dtype), out_dtype)
    announce("fp8 gemm", shape, "tile", tile, "split", split, out_dtype)
    t = [torch.from_numpy(a).cuda() for a in (xq, sx, wq, sw)]
    n_ws = w8.debug_fp8_gemm_workspace_size(M, N, K, split, tile)
    ws = w8.new_workspace(max(n_ws, 256))
    y1 = w8.debug_fp8_gemm(*t, split=split, tile=tile, out_dtype=OUT[out_dtype], workspace=ws)
    y2 = w8.debug_fp8_gemm(*t, split=split, tile=tile, out_dtype=OUT[out_dtype], workspace=ws)
    torch.cuda.synchronize()
    got = o.stored_to_f64(host_stored(y1, out_dtype), out_dtype)
    e, er = rel_fro(got, want), row_rel_fro(got, want).max()
    assert e <= TOL[out_dtype] and er <= TOL[out_dtype], (e, er)
    assert torch.equal(y1.view(torch.uint8), y2.view(torch.uint8))
    if n_ws:
        assert int(ws[:256].view(torch.int32).abs().sum().item()) == 0     # counters left zero


def test_fp8_linear_workspace_reuse_is_bitwise_stable():
    """Two text-encoder calls (K-sliced on this grid) through one workspace give
    identical bits, and the split-K counters are zero again after each."""
    c = synth.fp8_text_encoder("q")
    wq, sw = w8.quantize_weight_rowwise(dev16(c.w_bits, "bf16"), "fp8")
    x = dev16(c.x_bits, "bf16")
    n = w8.fp8_w8a8_linear_workspace_size(c.M, c.N, c.K)
    ws = w8.new_workspace(n)
    announce("fp8 workspace reuse", c.name)
    y1 = w8.fp8_w8a8_linear(x, wq, sw, None, torch.bfloat16, workspace=ws).clone()
    y2 = w8.fp8_w8a8_linear(x, wq, sw, None, torch.bfloat16, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert not ws[:4 * 4096].any()                             # the front's split-K counters


def test_packed_f16_conversion_equals_the_scalar_one_on_every_float():
    """The epilogues' fp16 outputs come from v_cvt_pk_f16_f32 (two values per
    instruction); on every float32 bit pattern it gives the bits of the scalar
    round-to-nearest-even conversion, NaN inputs included."""
    announce("packed fp16 conversion, all 2^32 float32 patterns")
    r = w8.debug_cvt_f16_pair_check()
    assert r["mismatch"] == 0, r
    assert r["mismatch_nan"] == 0, r
