"""CPU oracle for the W4A8 linear: int4 weights with one fp32 scale per
group of K values, int8 activations with one scale per token.

TEST INFRASTRUCTURE, like ``w8ref``: only the test suite, ``smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; it shares no code with the
HIP path.

Source: the "Qwen-Image-fni8" card, section "Format": int4 per-group weights,
int8 activations, fp32 scales (its dp4a kernels and resident layout are prior
art and not followed). Where the card is silent these readings apply (each is
listed with its reason in the project's design notes):
  * groups are G = 128 consecutive values of K within one weight row;
  * int4 codes are symmetric, like the int8 codes of LLM.int8: a group's scale
    is its absmax s (fp32), r = fl32(7 / s), q = rne(fl32(w * r)) clamped to
    [-7, 7]; s == 0 or w == 0 gives 0; the weight is dequantised as q * s / 7;
  * activations are coded per token exactly as the int8 path codes a row with
    no outlier columns (threshold +inf): sx = absmax, q = rne(fl32(x * fl32(127 / sx)));
  * the product sums each group's int8 x int4 products exactly, scales the
    group sum by sw[g, n] / 7, and the whole row by sx[m] / 127 (float64 here,
    one final rounding).
Storage (this library's resident form): codes packed two per byte, 8 values
per 32-bit little-endian word: word c of row n holds k = 8c .. 8c + 7, byte b
(b = 0..3) has k = 8c + b in its low nibble and k = 8c + b + 4 in its high
nibble, each nibble the 4-bit two's complement code. Scales are stored
group-major, sw[g, n] ([K / G, N] fp32).
"""
from __future__ import annotations

import numpy as np

from . import w8ref

F32 = np.float32
GROUP = 128


def quantize_groups_int4(w: np.ndarray, group: int = GROUP):
    """w float32 [N, K] (K a multiple of group) -> (q int8 [N, K] in [-7, 7],
    s float32 [N, K // group] group absmax)."""
    w = np.asarray(w, dtype=F32)
    N, K = w.shape
    assert K % group == 0
    wg = w.reshape(N, K // group, group)
    s = np.abs(wg).max(axis=2).astype(F32)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        r = F32(7.0) / s                              # one IEEE fp32 division per group
        p = wg * r[:, :, None]                        # IEEE fp32 product
        q = np.clip(np.rint(p), -7.0, 7.0)            # ties to even
    zero = (s == 0)[:, :, None] | (wg == 0)
    q = np.where(zero, 0.0, q).astype(np.int8)
    return q.reshape(N, K), s


def pack_int4(q: np.ndarray) -> np.ndarray:
    """int8 codes [N, K] in [-8, 7] (K % 8 == 0) -> packed uint8 [N, K // 2]."""
    q = np.asarray(q, dtype=np.int8)
    N, K = q.shape
    assert K % 8 == 0
    nib = (q.astype(np.int16) & 0xF).astype(np.uint8).reshape(N, K // 8, 8)
    out = nib[:, :, 0:4] | (nib[:, :, 4:8] << np.uint8(4))      # byte b: k = 8c+b, 8c+b+4
    return out.reshape(N, K // 2).astype(np.uint8)


def unpack_int4(p: np.ndarray) -> np.ndarray:
    """Inverse of pack_int4: packed uint8 [N, K // 2] -> int8 codes [N, K]."""
    p = np.asarray(p, dtype=np.uint8)
    N, H = p.shape
    b = p.reshape(N, H // 4, 4)
    lo = (b & 0xF).astype(np.int16)
    hi = (b >> 4).astype(np.int16)
    both = np.concatenate([lo, hi], axis=2)                      # k order 8c .. 8c+7
    both = np.where(both >= 8, both - 16, both)
    return both.reshape(N, H * 2).astype(np.int8)


def quantize_weight_int4(w: np.ndarray, group: int = GROUP):
    """Stored W4A8 weight: (packed uint8 [N, K // 2], sw float32 [K // group, N])."""
    q, s = quantize_groups_int4(w, group)
    return pack_int4(q), np.ascontiguousarray(s.T)


def w4a8_linear(x_bits, x_dtype, packed, sw, out_dtype="f16", group: int = GROUP, rows=None):
    """Y = X W^T with int8 per-token activations and int4 per-group weights.

    sw: [K // group, N] group absmax. Returns the codes, the exact integer
    group sums and the float64 result before and after the final rounding."""
    xf = w8ref.decode16(x_bits, x_dtype)
    _, sx, qx = w8ref.quantize_activations_int8(xf, np.inf, rows=rows)
    qw = unpack_int4(packed)
    N, K = qw.shape
    G = K // group
    acc = np.einsum("mgk,ngk->mng", qx.astype(np.int64).reshape(-1, G, group),
                    qw.astype(np.int64).reshape(N, G, group))    # exact int64 group sums
    sw64 = np.asarray(sw, dtype=F32).astype(np.float64).T        # [N, G]
    y = (acc.astype(np.float64) * (sw64 / 7.0)[None, :, :]).sum(axis=2) * (sx.astype(np.float64) / 127.0)[:, None]
    return {"qx": qx, "sx": sx, "acc": acc, "y": y, "Y": w8ref.round_output(y, out_dtype)}
