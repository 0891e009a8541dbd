"""CPU oracle for one DiT block's linears chained by the block driver, with
the fp16 exclusion policy for a massive-activation writer.

TEST INFRASTRUCTURE, like ``w8ref``: only the test suite, ``smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; it shares no code with the
HIP path.

Sources: the "Image21-INT8" card (section "Quantization": LLM.int8 on the
block's linears at threshold 6.0) and the "Image21-Turbo-OrbitQuant-W4A4" card
(section "What 4-bit breaks here and what stays in fp16": the transformer's
text tokens carry values near 9000 written by the MLP output projections of
some blocks, and those projections are kept in fp16). The attention between
QKV and the output projection is not part of the quantized path; the driver
stands in a stub for it: each token's attention output is its own value
vector (the value rows of QKV), as if every token attended only to itself.

The block (activations fp16 [M, D], weights as stored by the library):
  qkv = Linear8(RMSNorm1(X))               [M, 3D]   LLM.int8, bias, RMSNorm producer
  a   = qkv[:, 2D:3D]                                 attention stub
  o   = Linear8(a)                          [M, D]
  h   = X + o                                         residual, one rounding to fp16
  u   = Linear8(RMSNorm2(h))                [M, F]
  d   = Linear8(GELU(u))                    [M, D]    or, for a massive-activation
        GELU(u) W16^T + b (fp16 weights, no quantisation; fp32 result)
  Y   = h + d                                         one rounding to fp16
Every Linear8 output is rounded to fp16 (the type the next step reads).
"""
from __future__ import annotations

import numpy as np

from . import producers as P
from . import w8ref


def linear16(x_bits, x_dtype, w_bits, w_dtype, out_dtype="f32", bias=None):
    """Plain 16-bit linear: Y = X W^T (+ bias), the 16-bit values multiplied
    and summed in float64, rounded once to the output type."""
    x = w8ref.decode16(x_bits, x_dtype).astype(np.float64)
    w = w8ref.decode16(w_bits, w_dtype).astype(np.float64)
    y = x @ w.T
    if bias is not None:
        y = y + np.asarray(bias, np.float32).astype(np.float64)[None, :]
    return {"y": y, "Y": w8ref.round_output(y, out_dtype)}


def residual16(a_bits, b_values):
    """fp16 bits of a + b: a fp16 bits, b float64 values; one rounding."""
    return w8ref.round_to_f16(w8ref.decode16(a_bits, "f16").astype(np.float64) + b_values)


def dit_block(x_bits, blk: dict, threshold: float = 6.0):
    """The block above on fp16 X. ``blk`` holds, per linear L in (qkv, o, up,
    down): ``wq_L`` int8 [N, K], ``sw_L`` fp32 [N], ``b_L`` fp32 [N] or None;
    ``norm1`` / ``norm2`` dicts of RMSNorm gamma/scale/shift/eps; and
    ``w16_down`` (fp16 bits [D, F]) for the exclusion policy, or None.
    Returns every intermediate (fp16 bits) and Y."""
    D = blk["wq_o"].shape[0]
    out = {}
    r = P.fused_int8_linear(x_bits, "f16", "rmsnorm", blk["wq_qkv"], blk["sw_qkv"], threshold, blk["b_qkv"], "f16",
                            **blk["norm1"])
    out["qkv"] = r["Y"]
    out["a"] = np.ascontiguousarray(out["qkv"][:, 2 * D:3 * D])
    r = P.fused_int8_linear(out["a"], "f16", "none", blk["wq_o"], blk["sw_o"], threshold, blk["b_o"], "f16")
    out["o"] = r["Y"]
    out["h"] = residual16(x_bits, w8ref.decode16(out["o"], "f16").astype(np.float64))
    r = P.fused_int8_linear(out["h"], "f16", "rmsnorm", blk["wq_up"], blk["sw_up"], threshold, blk["b_up"], "f16",
                            **blk["norm2"])
    out["u"] = r["Y"]
    if blk.get("w16_down") is not None:
        out["g"] = P.produce(out["u"], "f16", "gelu")
        d = linear16(out["g"], "f16", blk["w16_down"], "f16", "f32", blk["b_down"])["y"]
        out["Y"] = residual16(out["h"], d)
    else:
        r = P.fused_int8_linear(out["u"], "f16", "gelu", blk["wq_down"], blk["sw_down"], threshold, blk["b_down"],
                                "f16")
        out["d"] = r["Y"]
        out["Y"] = residual16(out["h"], w8ref.decode16(out["d"], "f16").astype(np.float64))
    return out
