"""The int8 linear's output does not depend on the GEMM grid that computes it.

Every output element is the exact int32 sum (in any split of K) followed by
the same float32 epilogue and one rounding to the output type, whichever
block computes it: a whole 256x256 tile (64- or 128-byte K steps), a K-slice
of one, or a 128x128 quarter. The grids of devices with other compute-unit
counts are reached through w8dbg_int8_mixed_linear_plan; every result must
equal the device's own bit for bit (fp16 and fp32 outputs, with and without
outlier columns, past the LDS staging of outliers, bias and producers).
"""
import numpy as np
import pytest
import torch

import synth
import w8a8_mixed_precision_amd as w8
from tests.gpu_util import announce, dev16

pytestmark = pytest.mark.gpu

CUS = [3, 5, 8, 12, 40]

# (M, K, N, x dtype, outlier columns, threshold)
CASES = [
    (700, 1024, 1500, "bf16", 3, 6.0),        # 128-byte K steps; side product over 32 staged columns
    (1000, 576, 1300, "f16", 0, float("inf")),  # 64-byte K steps (K % 128 == 64), no side product
    (600, 2048, 777, "bf16", 40, 6.0),        # 33..256 outlier columns: XO / WO from the workspace
    (520, 384, 1024, "f16", 384, 0.0),        # every column an outlier (> 256): gathered in the epilogue
    (300, 336, 900, "bf16", 2, 6.0),          # K % 64 != 0: the general kernel (one grid)
]


def _ids(c):
    return f"{c[0]}x{c[1]}x{c[2]}_{c[3]}_o{c[4]}_t{c[5]}"


@pytest.mark.parametrize("out_dtype", [torch.float16, torch.float32], ids=["f16", "f32"])
@pytest.mark.parametrize("c", CASES, ids=_ids)
def test_every_grid_gives_the_same_output(c, out_dtype):
    M, K, N, xd, n_out, t = c
    case = synth.random_linear(M, K, N, seed=700 + M % 89, x_dtype=xd, outlier_cols=n_out)
    wq, sw = w8.quantize_weight_rowwise(dev16(case.w_bits, xd), "int8")
    x = dev16(case.x_bits, xd)
    announce("int8 grids", _ids(c), out_dtype)
    ref = w8.int8_mixed_linear(x, wq, sw, t, out_dtype)
    for cus in CUS:
        y = torch.full((M, N), float("nan"), dtype=out_dtype, device="cuda")
        w8.debug_int8_mixed_linear_plan(x, wq, sw, t, cus, y)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16) if out_dtype == torch.float16 else y.view(torch.int32),
                           ref.view(torch.int16) if out_dtype == torch.float16 else ref.view(torch.int32)), (c, cus)


@pytest.mark.parametrize("kind", ["bias", "rmsnorm", "gelu"])
def test_every_grid_gives_the_same_output_with_bias_and_producers(kind):
    M, K, N = 700, 1024, 1500
    case = synth.random_linear(M, K, N, seed=733, x_dtype="bf16", outlier_cols=3)
    wq, sw = w8.quantize_weight_rowwise(dev16(case.w_bits, "bf16"), "int8")
    x = dev16(case.x_bits, "bf16")
    rng = np.random.default_rng(734)
    bias = torch.from_numpy(rng.normal(0, 0.1, N).astype(np.float32)).cuda()
    prod = None
    if kind == "rmsnorm":
        vec = [torch.from_numpy(rng.uniform(lo, hi, K).astype(np.float32)).cuda()
               for lo, hi in ((0.8, 1.2), (-0.2, 0.2), (-0.2, 0.2))]
        prod = w8.Producer("rmsnorm", *vec, eps=1e-6)
    elif kind == "gelu":
        prod = w8.Producer("gelu")
    announce("int8 grids", kind)
    ref = w8.int8_mixed_linear(x, wq, sw, 6.0, torch.float16, bias=bias, producer=prod)
    for cus in CUS:
        y = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
        w8.debug_int8_mixed_linear_plan(x, wq, sw, 6.0, cus, y, bias=bias, producer=prod)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), (kind, cus)
