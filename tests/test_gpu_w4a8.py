"""GPU parity of the W4A8 linear (int4 per-group weights, int8 per-token
activations) against the CPU oracle (oracle/w4a8.py).

Bit-exact: the packed int4 codes and group scales of quantize_weight_rowwise
(fmt "int4"), and the whole contraction on inputs whose result is exact in
fp32 (integer codes, power-of-two scales). Outputs otherwise: relative
Frobenius error, globally and per row, <= 1e-2 for 16-bit outputs and
<= 2e-3 for fp32 (the stated output bounds of the linear), fp32 also within 1e-5.
"""
import numpy as np
import pytest
import torch

import synth
import w8a8_mixed_precision_amd as w8
from oracle import w4a8 as o4
from oracle import w8ref as o
from tests import bounds
from tests.gpu_util import OUT, announce, dev16, host_stored, rel_fro, row_rel_fro

pytestmark = pytest.mark.gpu

TOL = {"f16": 1e-2, "bf16": 1e-2, "f32": 2e-3}


@pytest.mark.parametrize("N,K,dtype", [(77, 128, "bf16"), (300, 1024, "f16"), (513, 4096, "bf16")])
def test_int4_weight_quantisation_bit_exact(N, K, dtype):
    rng = np.random.default_rng(N + K)
    w = rng.standard_normal((N, K)).astype(np.float32) * rng.uniform(1e-3, 1.0, (N, 1)).astype(np.float32)
    w[1, 128:] = 0.0 if K > 128 else w[1, 128:]        # an all-zero group (when there are two)
    w[2, :] = 0.0                                      # an all-zero row
    bits = o.round_to_bf16(w) if dtype == "bf16" else o.round_to_f16(w)
    packed_ref, sw_ref = o4.quantize_weight_int4(o.decode16(bits, dtype))
    announce("int4 weights", N, K, dtype)
    packed, sw = w8.quantize_weight_rowwise(dev16(bits, dtype), "int4")
    torch.cuda.synchronize()
    assert np.array_equal(sw.cpu().numpy(), sw_ref)
    assert np.array_equal(packed.cpu().numpy(), packed_ref)


@pytest.mark.parametrize("split", [0, 1, 2, 3])
def test_exact_contraction(split):
    """Integer activations with a +-127 in every row and int4 codes with a +-7
    in every group at power-of-two scales: every code and scale is exact and
    the fp32 result equals the oracle's float64 value."""
    rng = np.random.default_rng(80 + split)
    M, K, N = 130, 512, 200
    v = rng.integers(-127, 128, (M, K)).astype(np.float64)
    v[:, 5] = 127.0
    c = 2.0 ** rng.integers(-6, 2, (M, 1))
    q = rng.integers(-7, 8, (N, K)).astype(np.float64)
    q[:, ::128] = 7.0
    d = 2.0 ** rng.integers(-9, -3, (N, K // 128))
    w = q * np.repeat(d, 128, axis=1)
    x_bits = o.round_to_bf16(v * c)
    w_bits = o.round_to_bf16(w)
    assert np.array_equal(o.decode16(w_bits, "bf16"), w.astype(np.float32))
    packed, sw = o4.quantize_weight_int4(o.decode16(w_bits, "bf16"))
    ref = o4.w4a8_linear(x_bits, "bf16", packed, sw, "f32")
    assert np.array_equal(ref["qx"].astype(np.float64), v)
    announce("w4a8 exact", split)
    y = w8.w4a8_linear(dev16(x_bits, "bf16"), torch.from_numpy(packed).cuda(), torch.from_numpy(sw).cuda(),
                       torch.float32, split=split)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().astype(np.float64), ref["y"])


SMALL = [
    (300, 1024, 520, 81),        # ragged M and N over several 128 tiles
    (64, 256, 96, 82),
    (1, 128, 1, 83),             # one group, one output
    (257, 2048, 129, 84),
]


@pytest.mark.parametrize("M,K,N,seed", SMALL, ids=lambda v: str(v))
@pytest.mark.parametrize("out_dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("split", [0, 1, 2])
def test_w4a8_linear_matches_oracle(M, K, N, seed, out_dtype, split):
    if split > K // 128:
        pytest.skip("more slices than groups")
    rng = np.random.default_rng(seed)
    x_dtype = "f16" if seed % 2 else "bf16"
    xf = rng.standard_normal((M, K))
    x_bits = o.round_to_f16(xf) if x_dtype == "f16" else o.round_to_bf16(xf)
    packed, sw = o4.quantize_weight_int4(rng.standard_normal((N, K)).astype(np.float32) * 0.02)
    ref = o4.w4a8_linear(x_bits, x_dtype, packed, sw, out_dtype)
    announce("w4a8 linear", M, K, N, out_dtype, split)
    y = w8.w4a8_linear(dev16(x_bits, x_dtype), torch.from_numpy(packed).cuda(), torch.from_numpy(sw).cuda(),
                       OUT[out_dtype], split=split)
    torch.cuda.synchronize()
    stored = host_stored(y, out_dtype)
    got = o.stored_to_f64(stored, out_dtype)
    e, er = rel_fro(got, ref["y"]), row_rel_fro(got, ref["y"]).max()
    assert np.all(np.isfinite(got))
    assert e <= TOL[out_dtype] and er <= TOL[out_dtype], (e, er)
    if out_dtype == "f32":
        assert e <= 1e-5, e
    bounds.assert_elementwise(stored, out_dtype, ref["y"], bounds.w4a8_err32(ref, sw), (M, K, N, split))


def test_workspace_reuse_and_determinism():
    rng = np.random.default_rng(85)
    M, K, N = 128, 4096, 384
    x = dev16(o.round_to_bf16(rng.standard_normal((M, K))), "bf16")
    packed, sw = o4.quantize_weight_int4(rng.standard_normal((N, K)).astype(np.float32) * 0.02)
    wq, swd = torch.from_numpy(packed).cuda(), torch.from_numpy(sw).cuda()
    ws = w8.new_workspace(int(w8._abi.lib().w8dbg_w4a8_linear_workspace_size(M, N, K, 8)))
    announce("w4a8 workspace reuse")
    ys = [w8.w4a8_linear(x, wq, swd, torch.float32, workspace=ws, split=8) for _ in range(3)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(y, ys[0])


@pytest.mark.parametrize("layer", ["q", "k", "gate", "down"])
def test_text_encoder_layers_full_size(layer):
    """512-token text-encoder shapes in the linear's own launch configuration,
    checked on sampled rows."""
    c = synth.fp8_text_encoder(layer)
    packed, sw = o4.quantize_weight_int4(o.decode16(c.w_bits, c.w_dtype))
    rows = np.unique(np.concatenate([np.arange(0, c.M, 128), np.arange(127, c.M, 128),
                                     np.random.default_rng(86).choice(c.M, 24, replace=False)]))
    ref = o4.w4a8_linear(c.x_bits, c.x_dtype, packed, sw, "f16", rows=rows)
    announce("w4a8 full size", c.name)
    y = w8.w4a8_linear(dev16(c.x_bits, c.x_dtype), torch.from_numpy(packed).cuda(), torch.from_numpy(sw).cuda())
    torch.cuda.synchronize()
    stored = host_stored(y[torch.from_numpy(rows).cuda()], "f16")
    got = o.stored_to_f64(stored, "f16")
    e, er = rel_fro(got, ref["y"]), row_rel_fro(got, ref["y"]).max()
    assert e <= TOL["f16"] and er <= TOL["f16"], (e, er)
    bounds.assert_elementwise(stored, "f16", ref["y"], bounds.w4a8_err32(ref, sw), c.name)
