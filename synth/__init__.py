"""Seeded synthetic workloads for the quantized linear layers.

This module only draws inputs. It holds none of the quantisation or GEMM
arithmetic, so both the CPU oracle (through the tests) and the HIP path can be
fed the very same arrays.

Inputs are returned as raw 16-bit patterns (``uint16``) together with a dtype
tag (``"bf16"`` or ``"f16"``), so no library conversion sits between the
generator and either consumer.

Structure follows the model cards the method comes from:
  * activations ~N(0,1), weights ~N(0,0.02), as for a randomly initialised
    linear layer;
  * a few whole input columns carrying |x| in 6..60 -- the regime the LLM.int8
    outlier threshold of 6.0 is about (Image21-INT8 card, "Quantization");
  * "massive activations": single channels of a few text tokens near 9000 and
    13000, in channel 2276 (Image21-Turbo-OrbitQuant-W4A4 card, "What 4-bit
    breaks here and what stays in fp16");
  * token counts of the 1024^2 and 2048^2 DiT (4096 / 16384 image tokens plus
    256 text tokens) and a 512-token text-encoder batch.

bf16 values are produced by round-to-nearest-even of float32 draws; fp16 values
by numpy's float16 cast (also round-to-nearest-even).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

THRESHOLD = 6.0  # outlier threshold named on the Image21-INT8 card


def _bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _f16_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def encode16(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 samples to the 16-bit storage type and return the bits."""
    if dtype == "bf16":
        return _bf16_bits(a)
    if dtype == "f16":
        return _f16_bits(a)
    raise ValueError(dtype)


def _normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _signed_uniform(rng, n, lo, hi) -> np.ndarray:
    mag = rng.uniform(lo, hi, size=n).astype(np.float32)
    sign = np.where(rng.random(n) < 0.5, -1.0, 1.0).astype(np.float32)
    return mag * sign


@dataclass
class LinearCase:
    """One quantized-linear call: X [M,K] and W [N,K] as 16-bit patterns."""

    name: str
    M: int
    K: int
    N: int
    x_bits: np.ndarray
    x_dtype: str
    w_bits: np.ndarray
    w_dtype: str
    threshold: float = THRESHOLD
    out_dtype: str = "f16"
    injected_cols: tuple = ()
    injected_rows: tuple = ()
    extra: dict = field(default_factory=dict)

    @property
    def ops(self) -> int:
        return 2 * self.M * self.N * self.K


def random_linear(M, K, N, seed, x_dtype="bf16", w_dtype=None, w_std=0.02,
                  outlier_cols=0, outlier_lo=6.0, outlier_hi=60.0,
                  outlier_rows=None, name=None, threshold=THRESHOLD,
                  out_dtype="f16") -> LinearCase:
    """Generic seeded case (used for ragged / edge parity shapes).

    ``outlier_cols`` whole columns (or only ``outlier_rows`` of them) get
    values +-U(outlier_lo, outlier_hi).
    """
    rng = np.random.default_rng(seed)
    x = _normal(rng, (M, K))
    cols = ()
    if outlier_cols:
        cols = tuple(sorted(int(c) for c in rng.choice(K, size=min(outlier_cols, K), replace=False)))
        rows = np.arange(M) if outlier_rows is None else np.asarray(outlier_rows)
        for c in cols:
            x[rows, c] = _signed_uniform(rng, len(rows), outlier_lo, outlier_hi)
    wrng = np.random.default_rng(seed + 1)
    w = _normal(wrng, (N, K), w_std)
    w_dtype = w_dtype or x_dtype
    return LinearCase(name or f"random_{M}x{K}x{N}_s{seed}", M, K, N,
                      encode16(x, x_dtype), x_dtype, encode16(w, w_dtype), w_dtype,
                      threshold=threshold, out_dtype=out_dtype, injected_cols=cols)


# ---------------------------------------------------------------------------
# The five workload families.  Seeds: X = 1000*i+1, W = 1000*i+2,
# calibration = 1000*i+3 for family i; sub-layers add 10*j.
# ---------------------------------------------------------------------------

def tiny_int8() -> LinearCase:
    """Tiny LLM.int8 linear: X fp16 [64,256], 2 columns x 4 rows of +-U(8,20)."""
    i = 0
    rng = np.random.default_rng(1000 * i + 1)
    M, K, N = 64, 256, 512
    x = _normal(rng, (M, K))
    cols, rows = (37, 201), (3, 18, 41, 60)
    for c in cols:
        x[list(rows), c] = _signed_uniform(rng, len(rows), 8.0, 20.0)
    w = _normal(np.random.default_rng(1000 * i + 2), (N, K), 0.02)
    return LinearCase("tiny_64x256x512", M, K, N, encode16(x, "f16"), "f16",
                      encode16(w, "f16"), "f16", out_dtype="f16",
                      injected_cols=cols, injected_rows=rows)


def _dit_x(rng, M, K, n_cols=None, massive=False):
    x = _normal(rng, (M, K))
    cols, rows = (), ()
    if n_cols:
        cols = tuple(sorted(int(c) for c in rng.choice(K, size=n_cols, replace=False)))
        for c in cols:
            x[:, c] = _signed_uniform(rng, M, 6.0, 60.0)
    if massive:
        # 8 text-token rows (text tokens are the last 256 rows) carry a
        # massive activation near 9000 in channel 2276.
        rows = tuple(4096 + 32 * r for r in range(8) if 4096 + 32 * r < M)
        x[list(rows), 2276] = rng.uniform(8500.0, 9500.0, size=len(rows)).astype(np.float32)
        cols = (2276,)
    return x, cols, rows


def dit_qkv_1024() -> LinearCase:
    """DiT attention QKV at 1024^2: X [4352,4096], W [12288,4096], 4 outlier columns."""
    i = 1
    M, K, N = 4352, 4096, 12288
    x, cols, _ = _dit_x(np.random.default_rng(1000 * i + 1), M, K, n_cols=round(0.001 * K))
    w = _normal(np.random.default_rng(1000 * i + 2), (N, K), 0.02)
    return LinearCase("dit1024_qkv_4352x4096x12288", M, K, N, encode16(x, "bf16"), "bf16",
                      encode16(w, "bf16"), "bf16", injected_cols=cols)


def dit_mlp_1024(part: str) -> LinearCase:
    """DiT MLP at 1024^2: up X[4352,4096] W[16384,4096]; down X[4352,16384] W[4096,16384]."""
    i = 2
    j = {"up": 0, "down": 1}[part]
    M = 4352
    K, N = (4096, 16384) if part == "up" else (16384, 4096)
    x, cols, rows = _dit_x(np.random.default_rng(1000 * i + 1 + 10 * j), M, K, massive=True)
    w = _normal(np.random.default_rng(1000 * i + 2 + 10 * j), (N, K), 0.02)
    return LinearCase(f"dit1024_mlp_{part}_{M}x{K}x{N}", M, K, N, encode16(x, "bf16"), "bf16",
                      encode16(w, "bf16"), "bf16", injected_cols=cols, injected_rows=rows)


FP8_TEXT_LAYERS = {  # (K, N) of the text-encoder linears, hidden 4096
    "q": (4096, 4096), "k": (4096, 1024), "v": (4096, 1024),
    "gate": (4096, 12288), "up": (4096, 12288), "down": (12288, 4096),
}


def fp8_text_encoder(layer: str, massive: bool = False) -> LinearCase:
    """FP8 W8A8 text-encoder linear at 512 tokens.

    ``massive=True`` plants 13000 (row 0) and 9000 (row 1) in channel 2276,
    the values and channel the OrbitQuant card reports for the Qwen3-VL
    text encoder.  ``extra["x_cal_bits"]`` is an independent N(0,1) draw
    that a per-tensor "max" calibration can be run on.
    """
    i = 3
    j = list(FP8_TEXT_LAYERS).index(layer)
    K, N = FP8_TEXT_LAYERS[layer]
    M = 512
    x = _normal(np.random.default_rng(1000 * i + 1 + 10 * j), (M, K))
    rows = ()
    if massive and K > 2276:
        x[0, 2276] = 13000.0
        x[1, 2276] = 9000.0
        rows = (0, 1)
    w = _normal(np.random.default_rng(1000 * i + 2 + 10 * j), (N, K), 0.02)
    x_cal = _normal(np.random.default_rng(1000 * i + 3 + 10 * j), (M, K))
    name = f"fp8te_{layer}_{M}x{K}x{N}" + ("_massive" if massive else "")
    return LinearCase(name, M, K, N, encode16(x, "bf16"), "bf16", encode16(w, "bf16"), "bf16",
                      out_dtype="bf16", injected_cols=(2276,) if rows else (), injected_rows=rows,
                      extra={"x_cal_bits": encode16(x_cal, "bf16")})


def calibration_draw(M: int, K: int, seed: int) -> np.ndarray:
    """An independent N(0,1) bf16 draw [M, K]: the data a per-tensor "max"
    calibration of a static input scale runs on."""
    return encode16(_normal(np.random.default_rng(seed), (M, K)), "bf16")


def dit_2048(part: str, m_rows: int | None = None) -> LinearCase:
    """DiT at 2048^2: M = 16640 tokens; QKV, MLP up and MLP down; ~0.1% outlier columns.

    ``m_rows`` keeps only the first rows (a single GPU's share of the tokens).
    """
    i = 4
    j = {"qkv": 0, "up": 1, "down": 2}[part]
    K, N = {"qkv": (4096, 12288), "up": (4096, 16384), "down": (16384, 4096)}[part]
    M = 16640 if m_rows is None else m_rows
    x, cols, _ = _dit_x(np.random.default_rng(1000 * i + 1 + 10 * j), M, K, n_cols=round(0.001 * K))
    w = _normal(np.random.default_rng(1000 * i + 2 + 10 * j), (N, K), 0.02)
    return LinearCase(f"dit2048_{part}_{M}x{K}x{N}", M, K, N, encode16(x, "bf16"), "bf16",
                      encode16(w, "bf16"), "bf16", injected_cols=cols)


def dit_1024_block() -> list[LinearCase]:
    """The three quantized linears of one DiT block at 1024^2."""
    return [dit_qkv_1024(), dit_mlp_1024("up"), dit_mlp_1024("down")]


@dataclass
class FusedCase:
    """One producer-fused linear: H [M,K] (16-bit patterns) is the producer's
    input, X = producer(H) the linear's. RMSNorm cases carry float32 gain,
    modulation scale and shift vectors [K]; every case a float32 bias [N]."""

    name: str
    kind: str                # "rmsnorm" or "gelu"
    M: int
    K: int
    N: int
    h_bits: np.ndarray
    h_dtype: str
    w_bits: np.ndarray
    w_dtype: str
    bias: np.ndarray
    gamma: np.ndarray | None = None
    scale: np.ndarray | None = None
    shift: np.ndarray | None = None
    eps: float = 1e-6
    threshold: float = THRESHOLD

    @property
    def ops(self) -> int:
        return 2 * self.M * self.N * self.K


def fused_case(kind: str, M: int, K: int, N: int, seed: int, dtype: str = "bf16", name: str | None = None,
               outlier_cols: int = 4, massive: bool = False) -> FusedCase:
    """Seeded producer-fused linear.

    rmsnorm: H is a residual stream ~N(0,1) whose ``outlier_cols`` channels run
    at +-U(20,60) (they stay above the threshold after normalisation), with
    optional massive activations (~9000 in channel 2276 of 8 text-token rows,
    as in ``_dit_x``); gain ~U(0.8,1.2), modulation scale ~U(-0.2,0.2), shift
    ~U(-0.2,0.2), so the normalised bulk stays far below the threshold and the
    outlier columns are the planted ones (about 0.1%, the regime the threshold
    is about). gelu: H is an MLP hidden state ~N(0,1) whose ``outlier_cols``
    channels run at +-U(6,60) (GELU keeps the positive ones, zeroes the
    negative ones). Weights ~N(0,0.02), bias ~N(0,0.1)."""
    rng = np.random.default_rng(seed)
    h = _normal(rng, (M, K))
    lo, hi = (20.0, 60.0) if kind == "rmsnorm" else (6.0, 60.0)
    if outlier_cols:
        for c in rng.choice(K, size=min(outlier_cols, K), replace=False):
            h[:, int(c)] = _signed_uniform(rng, M, lo, hi)
    if massive and K > 2276:
        rows = [4096 + 32 * r for r in range(8) if 4096 + 32 * r < M]
        h[rows, 2276] = rng.uniform(8500.0, 9500.0, size=len(rows)).astype(np.float32)
    w = _normal(np.random.default_rng(seed + 1), (N, K), 0.02)
    prng = np.random.default_rng(seed + 2)
    bias = (prng.standard_normal(N) * 0.1).astype(np.float32)
    gamma = scale = shift = None
    if kind == "rmsnorm":
        gamma = prng.uniform(0.8, 1.2, K).astype(np.float32)
        scale = prng.uniform(-0.2, 0.2, K).astype(np.float32)
        shift = prng.uniform(-0.2, 0.2, K).astype(np.float32)
    return FusedCase(name or f"{kind}_{M}x{K}x{N}_s{seed}", kind, M, K, N, encode16(h, dtype), dtype,
                     encode16(w, dtype), dtype, bias, gamma, scale, shift)


def dit_mlp_fused_1024() -> list[FusedCase]:
    """The DiT 1024^2 MLP with its producers: up = (RMSNorm + modulation of the
    residual stream) -> 4096 x 16384, down = GELU(hidden) -> 16384 x 4096."""
    i = 5
    return [fused_case("rmsnorm", 4352, 4096, 16384, 1000 * i + 1, name="dit1024_mlp_up_rmsnorm_4352x4096x16384",
                       massive=True),
            fused_case("gelu", 4352, 16384, 4096, 1000 * i + 11, name="dit1024_mlp_down_gelu_4352x16384x4096",
                       outlier_cols=16)]
