"""GPU parity of the FP8 weight-only (W8A16) linear against the CPU oracle
(oracle/w8ref.py: dequantize_weight_fp8_bf16, fp8_w8a16_linear).

Bit-exact: the dequantised bf16 weight of every finite E4M3 code (read back
through one-hot activation rows, where each output is a single product).
Outputs: relative Frobenius error, globally and per row, <= 1e-2 for 16-bit
outputs (their rounding alone is 2^-9 relative per element for bf16) and
<= 2e-3 for fp32 (the stated output bounds of the linear); fp32 outputs additionally within 1e-5,
the size of fp32 accumulation error over these K.
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

# (split, tile): the linear's own plan, then forced tilings that cover both
# block sizes, whole tiles and K-slicing
CONFIGS = [(0, 0), (1, 256), (1, 128), (2, 256), (3, 128), (4, 128)]


def _finite_codes(rng, shape):
    c = rng.integers(0, 256, shape).astype(np.uint8)
    c[c == 0x7F] = 0x7E
    c[c == 0xFF] = 0xFE
    return c


def _bf16_scales(rng, n, lo=1e-4, hi=3e-2):
    return o.decode16(o.round_to_bf16(rng.uniform(lo, hi, n)), "bf16")


@pytest.mark.parametrize("split,tile", CONFIGS)
def test_dequantised_weights_bit_exact(split, tile):
    """X = I: Y[m, n] = W_deq[n, m], one exact product per output, so every
    widened weight is compared bit for bit (all 254 finite codes occur)."""
    rng = np.random.default_rng(70)
    K, N = 256, 320
    codes = _finite_codes(rng, (N, K))
    codes[0, :254] = [c for c in range(256) if c not in (0x7F, 0xFF)]
    sw = _bf16_scales(rng, N)
    sw[1] = 1.0                                        # unit scale: the codes' own values
    x_bits = o.round_to_bf16(np.eye(K))
    ref = o.fp8_w8a16_linear(x_bits, "bf16", codes, sw, "f32")
    announce("w8a16 one-hot", split, tile)
    y = w8.debug_fp8_w8a16_linear(dev16(x_bits, "bf16"), torch.from_numpy(codes).cuda(),
                                  torch.from_numpy(sw).cuda(), split, tile, torch.float32)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    want = o.decode16(ref["w_bits"], "bf16").T
    assert np.array_equal(got, want), int((got != want).sum())


SMALL = [
    (300, 1024, 520, 71),       # ragged M and N over several 256 and 128 tiles
    (64, 256, 96, 72),
    (1, 64, 1, 73),             # one K step, one output
    (257, 2048, 129, 74),
]


@pytest.mark.parametrize("M,K,N,seed", SMALL, ids=lambda v: str(v))
@pytest.mark.parametrize("out_dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("split,tile", CONFIGS)
def test_w8a16_linear_matches_oracle(M, K, N, seed, out_dtype, split, tile):
    if split > K // 64:
        pytest.skip("more slices than K steps")
    rng = np.random.default_rng(seed)
    x_bits = o.round_to_bf16(rng.standard_normal((M, K)))
    codes, sw = o.quantize_weight_fp8(rng.standard_normal((N, K)).astype(np.float32) * 0.02)
    ref = o.fp8_w8a16_linear(x_bits, "bf16", codes, sw, out_dtype)
    announce("w8a16 linear", M, K, N, out_dtype, split, tile)
    y = w8.debug_fp8_w8a16_linear(dev16(x_bits, "bf16"), torch.from_numpy(codes).cuda(),
                                  torch.from_numpy(sw).cuda(), split, tile, OUT[out_dtype])
    torch.cuda.synchronize()
    stored = host_stored(y, out_dtype)
    got = o.stored_to_f64(stored, out_dtype)
    want = ref["y"]
    assert np.all(np.isfinite(got))
    e, er = rel_fro(got, want), row_rel_fro(got, want).max()
    assert e <= TOL[out_dtype] and er <= TOL[out_dtype], (e, er)
    if out_dtype == "f32":
        assert e <= 1e-5, e
    err = bounds.dense_err32(np.abs(o.decode16(x_bits, "bf16").astype(np.float64)),
                             np.abs(o.decode16(ref["w_bits"], "bf16").astype(np.float64)), want, K)
    bounds.assert_elementwise(stored, out_dtype, want, err, (M, K, N, split, tile))


def test_workspace_reuse_and_determinism():
    """Split-K counters are left zero, so a workspace is reused without
    clearing, and the ordered partial sums repeat bit for bit."""
    rng = np.random.default_rng(75)
    M, K, N = 128, 4096, 384
    x_bits = o.round_to_bf16(rng.standard_normal((M, K)))
    codes, sw = o.quantize_weight_fp8(rng.standard_normal((N, K)).astype(np.float32) * 0.02)
    x, wq, swd = dev16(x_bits, "bf16"), torch.from_numpy(codes).cuda(), torch.from_numpy(sw).cuda()
    ws = w8.new_workspace(int(w8._abi.lib().w8dbg_fp8_w8a16_linear_workspace_size(M, N, K, 8, 128)))
    announce("w8a16 workspace reuse")
    ys = [w8.debug_fp8_w8a16_linear(x, wq, swd, 8, 128, torch.float32, workspace=ws) for _ in range(3)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(y, ys[0])
    want = o.fp8_w8a16_linear(x_bits, "bf16", codes, sw, "f32")["y"]
    assert rel_fro(ys[0].cpu().numpy(), want) <= 1e-5


@pytest.mark.parametrize("layer", list(synth.FP8_TEXT_LAYERS))
def test_text_encoder_layers_full_size(layer):
    """The 512-token text-encoder linears at full size in the linear's own
    launch configuration; outputs checked on sampled rows (the first and
    last rows of every 128-row block among them)."""
    c = synth.fp8_text_encoder(layer)
    codes, sw = o.quantize_weight_fp8(o.decode16(c.w_bits, c.w_dtype))
    rows = np.unique(np.concatenate([np.arange(0, c.M, 128), np.arange(127, c.M, 128),
                                     np.random.default_rng(76).choice(c.M, 24, replace=False)]))
    ref = o.fp8_w8a16_linear(c.x_bits, c.x_dtype, codes, sw, "bf16", rows=rows)
    announce("w8a16 full size", c.name)
    y = w8.fp8_w8a16_linear(dev16(c.x_bits, c.x_dtype), torch.from_numpy(codes).cuda(), torch.from_numpy(sw).cuda())
    torch.cuda.synchronize()
    stored = host_stored(y[torch.from_numpy(rows).cuda()], "bf16")
    got = o.stored_to_f64(stored, "bf16")
    e, er = rel_fro(got, ref["y"]), row_rel_fro(got, ref["y"]).max()
    assert e <= TOL["bf16"] and er <= TOL["bf16"], (e, er)
    err = bounds.dense_err32(np.abs(o.decode16(c.x_bits[rows], c.x_dtype).astype(np.float64)),
                             np.abs(o.decode16(ref["w_bits"], "bf16").astype(np.float64)), ref["y"], c.K)
    bounds.assert_elementwise(stored, "bf16", ref["y"], err, c.name)
