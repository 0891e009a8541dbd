"""Pins of the block oracle (oracle/block.py): the plain 16-bit linear
against brute force and exact small-integer products; the block's wiring
(stub, residuals, exclusion) against closed forms."""
import numpy as np

from oracle import block as B
from oracle import producers as P
from oracle import w8ref as o


def test_linear16_brute_force_and_exact_integers():
    rng = np.random.default_rng(0)
    x_bits = o.round_to_f16(rng.standard_normal((3, 5)))
    w_bits = o.round_to_f16(rng.standard_normal((4, 5)))
    bias = rng.standard_normal(4).astype(np.float32)
    ref = B.linear16(x_bits, "f16", w_bits, "f16", "f32", bias)
    x, w = o.decode16(x_bits, "f16"), o.decode16(w_bits, "f16")
    for m in range(3):
        for n in range(4):
            want = sum(float(x[m, k]) * float(w[n, k]) for k in range(5)) + float(bias[n])
            assert abs(ref["y"][m, n] - want) < 1e-12
    xi = rng.integers(-9, 10, (6, 64)).astype(np.float64)
    wi = rng.integers(-9, 10, (7, 64)).astype(np.float64)
    r = B.linear16(o.round_to_bf16(xi), "bf16", o.round_to_bf16(wi), "bf16", "f32")
    assert np.array_equal(r["y"], xi @ wi.T)


def _tiny_block(rng, D=32, F=64, with16=False):
    def lin(n, k):
        wq, sw = o.quantize_weight_int8(rng.standard_normal((n, k)).astype(np.float32) * 0.05)
        return wq, sw, (rng.standard_normal(n) * 0.1).astype(np.float32)
    blk = {}
    for name, (n, k) in {"qkv": (3 * D, D), "o": (D, D), "up": (F, D), "down": (D, F)}.items():
        blk[f"wq_{name}"], blk[f"sw_{name}"], blk[f"b_{name}"] = lin(n, k)
    norm = dict(gamma=rng.uniform(0.8, 1.2, D).astype(np.float32), scale=None, shift=None, eps=1e-6)
    blk["norm1"], blk["norm2"] = norm, dict(norm)
    blk["w16_down"] = o.round_to_f16(rng.standard_normal((D, F)) * 0.05) if with16 else None
    return blk


def test_block_wiring():
    rng = np.random.default_rng(1)
    D = 32
    blk = _tiny_block(rng, D)
    x_bits = o.round_to_f16(rng.standard_normal((5, D)))
    out = B.dit_block(x_bits, blk)
    assert np.array_equal(out["a"], out["qkv"][:, 2 * D:])                 # the stub is V
    h = o.decode16(x_bits, "f16").astype(np.float64) + o.decode16(out["o"], "f16")
    assert np.array_equal(out["h"], o.round_to_f16(h))                      # residual, one rounding
    y = o.decode16(out["h"], "f16").astype(np.float64) + o.decode16(out["d"], "f16")
    assert np.array_equal(out["Y"], o.round_to_f16(y))


def test_exclusion_runs_the_writer_in_16_bit():
    rng = np.random.default_rng(2)
    D, F = 32, 64
    blk = _tiny_block(rng, D, F, with16=True)
    x_bits = o.round_to_f16(rng.standard_normal((4, D)))
    out = B.dit_block(x_bits, blk)
    assert "d" not in out
    g = P.produce(out["u"], "f16", "gelu")
    assert np.array_equal(out["g"], g)
    d = o.decode16(g, "f16").astype(np.float64) @ o.decode16(blk["w16_down"], "f16").astype(np.float64).T
    d = d + blk["b_down"].astype(np.float64)[None, :]
    assert np.array_equal(out["Y"], o.round_to_f16(o.decode16(out["h"], "f16").astype(np.float64) + d))
