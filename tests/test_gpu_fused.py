"""GPU parity of the producer-fused int8 linear (int8_mixed_linear_fused)
against the CPU oracle (oracle/producers.py on top of oracle/w8ref.py).

Bit-exact: X = producer(H), and with it the outlier set, row scales and int8
codes. GELU: X is the correctly rounded GELU of each 16-bit pattern, checked
on every pattern of both formats. RMSNorm: the kernel adds the float64 squares
of a row in its own order; the test takes the kernel's rstd, checks that it is
one of the readings the definition allows (oracle.producers.rstd_alternatives;
the exactly rounded sum's on almost every row), then requires X, codes,
scales and outliers bit-exact for it.
Outputs: relative Frobenius error <= 1e-2 (fp16) / 2e-3 (fp32), globally and
per row, and element by element (tests/bounds.py); the bias goes into the same
epilogue.
"""
import numpy as np
import pytest
import torch

import synth
import w8a8_mixed_precision_amd as w8
from oracle import producers as P
from oracle import w8ref as o
from tests import bounds
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


def _gpu_rstd(case, prod, t=6.0):
    """The row pass's rstd for H (the same kernel the fused linear runs)."""
    *_, rstd = w8.debug_int8_quantize_activations(dev16(case.h_bits, case.h_dtype), t, prod, with_rstd=True)
    return rstd.cpu().numpy()


def _checked_rstd(case, kw, rstd_gpu):
    """rstd_gpu must be one of the two readings of every row, and the exact
    sum's reading except on rows where the two differ."""
    h = o.decode16(case.h_bits, case.h_dtype)
    a, b = P.rstd_alternatives(h, kw.get("eps", 1e-6))
    assert np.all((rstd_gpu == a) | (rstd_gpu == b)), int(((rstd_gpu != a) & (rstd_gpu != b)).sum())
    _, exact = P.rmsnorm_modulate32(h, eps=kw.get("eps", 1e-6))
    moved = np.flatnonzero(rstd_gpu != exact)
    assert np.all(a[moved] != b[moved])
    return rstd_gpu


def _x_ref(case, kw, prod=None):
    """The oracle's X for the case; RMSNorm with the kernel's (checked) rstd."""
    if case.kind == "rmsnorm":
        rstd = _checked_rstd(case, kw, _gpu_rstd(case, prod))
        return P.produce(case.h_bits, case.h_dtype, "rmsnorm", rstd=rstd, **kw)
    return P.produce(case.h_bits, case.h_dtype, case.kind, **kw)


@pytest.mark.parametrize("case", SMALL, ids=lambda c: c.name)
def test_producer_output_bit_exact(case):
    """The separate producer kernel (its own summation order for RMSNorm):
    every row equals the oracle's X under one of the allowed rstd readings."""
    prod, kw = _producer(case)
    announce("produce", case.name)
    x = w8.debug_produce(dev16(case.h_bits, case.h_dtype), prod)
    got = x.cpu().view(torch.int16).numpy().view(np.uint16)
    if case.kind == "gelu":
        want = P.produce(case.h_bits, case.h_dtype, "gelu")
        assert np.array_equal(got, want), int((got != want).sum())
        return
    h = o.decode16(case.h_bits, case.h_dtype)
    a, b = P.rstd_alternatives(h, case.eps)
    xa = P.produce(case.h_bits, case.h_dtype, "rmsnorm", rstd=a, **kw)
    xb = P.produce(case.h_bits, case.h_dtype, "rmsnorm", rstd=b, **kw)
    ok = np.all(got == xa, axis=1) | np.all(got == xb, axis=1)
    assert ok.all(), np.flatnonzero(~ok)[:10]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_gelu_of_every_16bit_pattern(dtype):
    """GELU of every finite pattern of the format, through the three kernels
    that make it: the elementwise producer (LDS table), the fused row pass
    (LDS table; seen through its codes and scales at t = inf) and the outlier
    fix-up (global table; seen in the staged outlier columns XO at t = 0, where
    every column of these 256-wide rows is an outlier column)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    fin = bits[np.isfinite(o.decode16(bits, dtype))]
    rows = np.concatenate([fin, np.zeros((-fin.size) % 256, np.uint16)]).reshape(-1, 256)
    want = P.gelu16(rows, dtype)
    h = dev16(rows, dtype)
    prod = w8.Producer("gelu")
    announce("gelu every pattern", dtype)
    got = w8.debug_produce(h, prod).cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want), int((got != want).sum())
    # fused row pass: codes and scales of X at t = inf
    _, sx_ref, q_ref = o.quantize_activations_int8(o.decode16(want, dtype), np.inf)
    q, sx, O = w8.debug_int8_quantize_activations(h, np.inf, prod)
    assert O.numel() == 0
    assert np.array_equal(sx.cpu().numpy(), sx_ref) and np.array_equal(q.cpu().numpy(), q_ref)
    # fix-up: X of every outlier column gathered into XO
    M, K, N = rows.shape[0], 256, 64
    O_ref = o.outlier_columns(o.decode16(want, dtype), 0.0)
    assert O_ref.size == K
    wq = torch.ones((N, K), dtype=torch.int8, device="cuda")
    sw = torch.full((N,), 127.0, dtype=torch.float32, device="cuda")
    ws = w8.new_workspace(w8.int8_mixed_linear_workspace_size(M, N, K))
    w8.int8_mixed_linear(h, wq, sw, 0.0, torch.float32, workspace=ws, producer=prod)
    lay = w8.int8_workspace_layout(M, N, K)
    xo = ws[lay["XO"]:lay["XO"] + 2 * M * K].view(torch.int16).cpu().numpy().view(np.uint16).reshape(M, K)
    assert np.array_equal(xo, want), int((xo != want).sum())


@pytest.mark.parametrize("parts", [(True, False, False), (False, True, True), (False, False, False)],
                         ids=["gamma", "scale_shift", "plain"])
def test_rmsnorm_optional_vectors_bit_exact(parts):
    c = SMALL[0]
    prod, kw = _producer(c, *parts)
    h = o.decode16(c.h_bits, c.h_dtype)
    a, b = P.rstd_alternatives(h, c.eps)
    announce("produce rmsnorm parts", parts)
    got = w8.debug_produce(dev16(c.h_bits, c.h_dtype), prod).cpu().view(torch.int16).numpy().view(np.uint16)
    xa = P.produce(c.h_bits, c.h_dtype, "rmsnorm", rstd=a, **kw)
    xb = P.produce(c.h_bits, c.h_dtype, "rmsnorm", rstd=b, **kw)
    assert np.all(np.all(got == xa, axis=1) | np.all(got == xb, axis=1))


@pytest.mark.parametrize("case", SMALL, ids=lambda c: c.name)
@pytest.mark.parametrize("t", [6.0, 0.5])
def test_fused_quantisation_bit_exact(case, t):
    prod, kw = _producer(case)
    announce("fused quantisation", case.name, t)
    x_bits = _x_ref(case, kw, prod)
    O_ref, sx_ref, q_ref = o.quantize_activations_int8(o.decode16(x_bits, case.h_dtype), t)
    q, sx, O = w8.debug_int8_quantize_activations(dev16(case.h_bits, case.h_dtype), t, prod)
    assert np.array_equal(O.cpu().numpy(), O_ref)
    assert np.array_equal(sx.cpu().numpy(), sx_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)


def _weights(c):
    wf = o.decode16(c.w_bits, c.w_dtype)
    wq_ref, sw_ref = o.quantize_weight_int8(wf)
    wq, sw = w8.quantize_weight_rowwise(dev16(c.w_bits, c.w_dtype), "int8")
    return wq, sw, wq_ref, sw_ref


def _check(y, ref, out_dtype, label, dtype=None, wq=None, sw=None, bias=None, rows=None):
    """ref: the oracle's result dict (with x_bits); with the oracle's weights,
    element by element too."""
    stored = host_stored(y, out_dtype)
    got = o.stored_to_f64(stored, out_dtype)
    want = o.stored_to_f64(ref["Y"], out_dtype)
    assert np.all(np.isfinite(got)) and np.std(got) > 0, label
    e, er = rel_fro(got, want), row_rel_fro(got, want).max()
    assert e <= TOL[out_dtype] and er <= TOL[out_dtype], (label, e, er)
    if wq is not None:
        x_bits = ref["x_bits"] if rows is None else ref["x_bits"][np.asarray(rows)]
        err = bounds.int8_err32(ref, x_bits, dtype, wq, sw, bias=bias)
        bounds.assert_elementwise(stored, out_dtype, ref["y"], err, label)


@pytest.mark.parametrize("case", SMALL, ids=lambda c: c.name)
@pytest.mark.parametrize("out_dtype", ["f16", "f32"])
@pytest.mark.parametrize("with_bias", [True, False])
def test_fused_linear_matches_oracle(case, out_dtype, with_bias):
    wq, sw, wq_ref, sw_ref = _weights(case)
    prod, kw = _producer(case)
    bias = case.bias if with_bias else None
    announce("fused linear", case.name, out_dtype, with_bias)
    x_bits = _x_ref(case, kw, prod)
    ref = P.fused_int8_linear(case.h_bits, case.h_dtype, case.kind, wq_ref, sw_ref, case.threshold, bias,
                              out_dtype, x_bits=x_bits, **kw)
    y = w8.int8_mixed_linear(dev16(case.h_bits, case.h_dtype), wq, sw, case.threshold, OUT[out_dtype],
                             bias=torch.from_numpy(bias).cuda() if with_bias else None, producer=prod)
    torch.cuda.synchronize()
    _check(y, ref, out_dtype, case.name, case.h_dtype, wq_ref, sw_ref, bias)


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
    _check(with_bias, ref, "f32", c.name, c.x_dtype, wq_ref, sw_ref, bias)


@pytest.mark.parametrize("idx", [0, 1], ids=["up_rmsnorm", "down_gelu"])
def test_dit_mlp_fused_full_size(idx):
    """The DiT 1024^2 MLP pair with its producers at full size: exact codes,
    scales and outlier set on every row, outputs on sampled rows (massive
    rows and the last 256-row strip included)."""
    c = synth.dit_mlp_fused_1024()[idx]
    wq, sw, wq_ref, sw_ref = _weights(c)
    prod, kw = _producer(c)
    announce("fused full size", c.name)
    x_bits = _x_ref(c, kw, prod)
    O_ref, sx_ref, q_ref = o.quantize_activations_int8(o.decode16(x_bits, c.h_dtype), c.threshold)
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
    _check(y[torch.from_numpy(rows).cuda()], ref, "f16", c.name, c.h_dtype, wq_ref, sw_ref, c.bias, rows)


@pytest.mark.parametrize("kind,t", [("gelu", 0.25), ("rmsnorm", 0.5)])
@pytest.mark.parametrize("K", [640, 528])
def test_fused_linear_with_gathered_outlier_columns(kind, t, K):
    """A low threshold makes more than 256 outlier columns: the GEMM epilogue
    gathers them from H through the producer (RMSNorm with the row pass's
    rstd, GELU from the global table). K = 528 takes the GEMM for K % 64 != 0."""
    c = synth.fused_case(kind, 300, K, 520, 91 + K, name=f"{kind}_gathered_{K}")
    wq, sw, wq_ref, sw_ref = _weights(c)
    prod, kw = _producer(c)
    announce("fused gathered", c.name, t)
    x_bits = _x_ref(c, kw, prod)
    ref = P.fused_int8_linear(c.h_bits, c.h_dtype, kind, wq_ref, sw_ref, t, c.bias, "f32", x_bits=x_bits, **kw)
    assert len(ref["O"]) > 256
    y = w8.int8_mixed_linear(dev16(c.h_bits, c.h_dtype), wq, sw, t, torch.float32,
                             bias=torch.from_numpy(c.bias).cuda(), producer=prod)
    torch.cuda.synchronize()
    _check(y, ref, "f32", c.name, c.h_dtype, wq_ref, sw_ref, c.bias)
