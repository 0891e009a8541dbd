"""The no-allocation entry point int8_mixed_linear_noalloc, called through the
C ABI, against int8_mixed_linear with a workspace: bit-identical outputs (the
same kernels on the same data), two calls in a row with the second smaller,
then the first shape again; the outputs are also within the oracle's bounds."""
import ctypes

import numpy as np
import pytest
import torch

import synth
import w8a8_mixed_precision_amd as w8
from oracle import w8ref as o
from tests import bounds
from tests.gpu_util import announce, dev16, host_stored

pytestmark = pytest.mark.gpu


def _noalloc(x, wq, sw, t, y):
    lib = w8._abi.lib()
    M, K = x.shape
    N = wq.shape[0]
    st = lib.int8_mixed_linear_noalloc(x.data_ptr(), w8._abi.W8_DT_BF16 if x.dtype == torch.bfloat16 else
                                       w8._abi.W8_DT_F16, M, K, wq.data_ptr(), sw.data_ptr(), N, ctypes.c_float(t),
                                       y.data_ptr(), w8._abi.W8_DT_F16 if y.dtype == torch.float16 else
                                       w8._abi.W8_DT_F32, torch.cuda.current_stream().cuda_stream)
    w8._abi.check(st)
    return y


def test_noalloc_matches_the_workspace_entry_point():
    big = synth.random_linear(300, 8192, 520, seed=301, x_dtype="bf16", outlier_cols=5)   # K-split GEMM
    small = synth.random_linear(70, 256, 96, seed=302, x_dtype="bf16", outlier_cols=2)
    mid = synth.random_linear(513, 1040, 777, seed=303, x_dtype="bf16", outlier_cols=300)   # gathered outliers
    for c in (big, small, big, mid, small):
        wf = o.decode16(c.w_bits, "bf16")
        wq_ref, sw_ref = o.quantize_weight_int8(wf)
        wq, sw = w8.quantize_weight_rowwise(dev16(c.w_bits, "bf16"), "int8")
        x = dev16(c.x_bits, "bf16")
        announce("noalloc", c.name)
        y = _noalloc(x, wq, sw, 6.0, torch.empty((c.M, c.N), dtype=torch.float16, device="cuda"))
        ref_y = w8.int8_mixed_linear(x, wq, sw, 6.0, torch.float16)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref_y.view(torch.int16)), c.name
        ref = o.int8_mixed_linear(c.x_bits, "bf16", wq_ref, sw_ref, 6.0, "f16")
        err = bounds.int8_err32(ref, c.x_bits, "bf16", wq_ref, sw_ref)
        bounds.assert_elementwise(host_stored(y, "f16"), "f16", ref["y"], err, c.name)
