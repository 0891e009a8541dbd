"""GPU parity of the producer-fused int8 linear (int8_mixed_linear_fused)
against the CPU oracle (oracle/producers.py on top of oracle/w8ref.py).

Bit-exact: X = producer(H) (the fp32 producer sequences are reproduced
exactly), and with it the outlier set, row scales and int8 codes.
Outputs: relative Frobenius error <= 1e-2 (fp16) / 2e-3 (fp32), globally and
per row, as for int8_mixed_linear; the bias goes into the same epilogue.
"""
import numpy as np
import pytest
import torch

import synth
import w8a8_mixed_precision_amd as w8
from oracle import producers as P
from oracle import w8ref as o
from tests.gpu_util import OUT, announce, dev16, host_stored, rel_fro, row_rel_fro

pytestmark = pytest.mark.gpu

TOL = {"f16": 1e-2, "f32": 2e-3}


def _producer(c, gamma=True, scale=True, shift=True):
    if c.kind == "gelu":
        return w8.Producer("gelu"), {}
    t = lambda v, on: torch.from_numpy(v).cuda() if (on and v is not None) else None
    kw = dict(gamma=c.gamma if gamma else None, scale=c.scale if scale else None, shift=c.shift if shift else None)
    return w8.Producer("rmsnorm", t(c.gamma, gamma), t(c.scale, scale), t(c.shift, shift), c.eps), \
        dict(kw, eps=c.eps)


SMALL = [
    synth.fused_case("rmsnorm", 300, 1024, 520, 61, name="rms_ragged_bf16"),
    synth.fused_case("rmsnorm", 129, 4096, 200, 62, dtype="f16", name="rms_f16"),
    synth.fused_case("rmsnorm", 77, 8192, 64, 63, name="rms_two_waves_per_row"),
    synth.fused_case("rmsnorm", 40, 16384, 130, 64, name="rms_four_waves_per_row"),
    synth.fused_case("gelu", 300, 2048, 520, 65, name="gelu_ragged_bf16"),
    synth.fused_case("gelu", 64, 16384, 256, 66, dtype="f16", name="gelu_f16_long"),
    synth.fused_case("gelu", 33, 48, 40, 67, outlier_cols=2, name="gelu_tiny"),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: c.name)
def test_producer_output_bit_exact(case):
    prod, kw = _producer(case)
    want = P.produce(case.h_bits, case.h_dtype, case.kind, **kw)
    announce("produce", case.name)
    x = w8.debug_produce(dev16(case.h_bits, case.h_dtype), prod)
    got = x.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want), int((got != want).sum())


@pytest.mark.parametrize("parts", [(True, False, False), (False, True, True), (False, False, False)],
                         ids=["gamma", "scale_shift", "plain"])
def test_rmsnorm_optional_vectors_bit_exact(parts):
    c = SMALL[0]
    prod, kw = _producer(c, *parts)
    want = P.produce(c.h_bits, c.h_dtype, "rmsnorm", **kw)
    announce("produce rmsnorm parts", parts)
    got = w8.debug_produce(dev16(c.h_bits, c.h_dtype), prod).cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("case", SMALL, ids=lambda c: c.name)
@pytest.mark.parametrize("t", [6.0, 0.5])
def test_fused_quantisation_bit_exact(case, t):
    prod, kw = _producer(case)
    x_bits = P.produce(case.h_bits, case.h_dtype, case.kind, **kw)
    O_ref, sx_ref, q_ref = o.quantize_activations_int8(o.decode16(x_bits, case.h_dtype), t)
    announce("fused quantisation", case.name, t)
    q, sx, O = w8.debug_int8_quantize_activations(dev16(case.h_bits, case.h_dtype), t, prod)
    assert np.array_equal(O.cpu().numpy(), O_ref)
    assert np.array_equal(sx.cpu().numpy(), sx_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)


def _weights(c):
    wf = o.decode16(c.w_bits, c.w_dtype)
    wq_ref, sw_ref = o.quantize_weight_int8(wf)
    wq, sw = w8.quantize_weight_rowwise(dev16(c.w_bits, c.w_dtype), "int8")
    return wq, sw, wq_ref, sw_ref


def _check(y, ref_stored, out_dtype, label):
    got = o.stored_to_f64(host_stored(y, out_dtype), out_dtype)
    want = o.stored_to_f64(ref_stored, out_dtype)
    assert np.all(np.isfinite(got)) and np.std(got) > 0, label
    e, er = rel_fro(got, want), row_rel_fro(got, want).max()
    assert e <= TOL[out_dtype] and er <= TOL[out_dtype], (label, e, er)


@pytest.mark.parametrize("case", SMALL, ids=lambda c: c.name)
@pytest.mark.parametrize("out_dtype", ["f16", "f32"])
@pytest.mark.parametrize("with_bias", [True, False])
def test_fused_linear_matches_oracle(case, out_dtype, with_bias):
    wq, sw, wq_ref, sw_ref = _weights(case)
    prod, kw = _producer(case)
    bias = case.bias if with_bias else None
    ref = P.fused_int8_linear(case.h_bits, case.h_dtype, case.kind, wq_ref, sw_ref, case.threshold, bias,
                              out_dtype, **kw)
    announce("fused linear", case.name, out_dtype, with_bias)
    y = w8.int8_mixed_linear(dev16(case.h_bits, case.h_dtype), wq, sw, case.threshold, OUT[out_dtype],
                             bias=torch.from_numpy(bias).cuda() if with_bias else None, producer=prod)
    torch.cuda.synchronize()
    _check(y, ref["Y"], out_dtype, case.name)


def test_bias_without_producer_is_the_plain_linear_plus_bias():
    c = synth.random_linear(300, 1024, 520, seed=68, outlier_cols=3)
    wq, sw, wq_ref, sw_ref = _weights(c)
    bias = np.random.default_rng(69).standard_normal(c.N).astype(np.float32)
    x = dev16(c.x_bits, c.x_dtype)
    announce("bias only", c.name)
    plain = w8.int8_mixed_linear(x, wq, sw, 6.0, torch.float32)
    with_bias = w8.int8_mixed_linear(x, wq, sw, 6.0, torch.float32, bias=torch.from_numpy(bias).cuda())
    torch.cuda.synchronize()
    diff = (with_bias - plain).cpu().numpy().astype(np.float64)
    # one fp32 rounding apart: the bias is added to the same fp32 value
    assert np.max(np.abs(diff - bias[None, :]) / np.maximum(np.abs(plain.cpu().numpy()), 1.0)) < 2e-6
    ref = P.fused_int8_linear(c.x_bits, c.x_dtype, "none", wq_ref, sw_ref, 6.0, bias, "f32")
    _check(with_bias, ref["Y"], "f32", c.name)


@pytest.mark.parametrize("idx", [0, 1], ids=["up_rmsnorm", "down_gelu"])
def test_dit_mlp_fused_full_size(idx):
    """The DiT 1024^2 MLP pair with its producers at full size: exact codes,
    scales and outlier set on every row, outputs on sampled rows (massive
    rows and the last 256-row strip included)."""
    c = synth.dit_mlp_fused_1024()[idx]
    wq, sw, wq_ref, sw_ref = _weights(c)
    prod, kw = _producer(c)
    x_bits = P.produce(c.h_bits, c.h_dtype, c.kind, **kw)
    O_ref, sx_ref, q_ref = o.quantize_activations_int8(o.decode16(x_bits, c.h_dtype), c.threshold)
    announce("fused full size", c.name)
    h = dev16(c.h_bits, c.h_dtype)
    q, sx, O = w8.debug_int8_quantize_activations(h, c.threshold, prod)
    assert np.array_equal(O.cpu().numpy(), O_ref)
    assert np.array_equal(sx.cpu().numpy(), sx_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    del q
    rng = np.random.default_rng(45)
    rows = np.unique(np.concatenate([rng.choice(c.M, 64, replace=False), [0, c.M - 1],
                                     np.arange(4096, c.M, 32), np.arange((c.M - 1) // 256 * 256, c.M, 7)]))
    y = w8.int8_mixed_linear(h, wq, sw, c.threshold, torch.float16, bias=torch.from_numpy(c.bias).cuda(),
                             producer=prod)
    ref = P.fused_int8_linear(c.h_bits, c.h_dtype, c.kind, wq_ref, sw_ref, c.threshold, c.bias, "f16",
                              rows=rows, x_bits=x_bits, **kw)
    _check(y[torch.from_numpy(rows).cuda()], ref["Y"], "f16", c.name)
