"""GPU parity of the LLM.int8 path against the CPU oracle (through the C ABI).

Bit-exact: int8 weight codes and scales, activation codes, row scales, the
outlier-column set, int32 accumulators. Outputs: relative Frobenius error
<= 1e-2 for fp16 output and <= 2e-3 for fp32 output, globally and per row,
and element by element within half an output ulp plus the float32 epilogue's
own error (tests/bounds.py).
"""
import math

import numpy as np
import pytest
import torch

import synth
import w8a8_mixed_precision_amd as w8
from oracle import w8ref as o
from tests import bounds
from tests.gpu_util import announce, dev16, host_stored, rel_fro, row_rel_fro

pytestmark = pytest.mark.gpu

TOL = {"f16": 1e-2, "f32": 2e-3}


def _quant_weights_both(case):
    wf = o.decode16(case.w_bits, case.w_dtype)
    wq_ref, sw_ref = o.quantize_weight_int8(wf)
    wq, sw = w8.quantize_weight_rowwise(dev16(case.w_bits, case.w_dtype), "int8")
    torch.cuda.synchronize()
    return wq, sw, wq_ref, sw_ref


def _check_outputs(y_gpu, ref, out_dtype, label, x_bits=None, x_dtype="bf16", wq=None, sw=None, rows=None):
    """ref: the oracle's result dict. With x_bits, wq and sw (the oracle's
    operands) the element-wise bound is checked too."""
    stored = host_stored(y_gpu, out_dtype)
    got = o.stored_to_f64(stored, out_dtype)
    want = o.stored_to_f64(ref["Y"], out_dtype)
    assert np.all(np.isfinite(got)), label
    assert np.std(got) > 0, label          # finite and non-constant
    e = rel_fro(got, want)
    er = row_rel_fro(got, want).max()
    assert e <= TOL[out_dtype] and er <= TOL[out_dtype], (label, e, er)
    if x_bits is not None:
        err = bounds.int8_err32(ref, x_bits, x_dtype, wq, sw, rows=rows)
        bounds.assert_elementwise(stored, out_dtype, ref["y"], err, label)
    return e, er


# ----------------------------------------------------------------------------
# small and ragged cases (oracle runs on all of them in full)
# ----------------------------------------------------------------------------

def _cases():
    yield synth.tiny_int8()
    yield synth.random_linear(300, 272, 520, seed=31, x_dtype="bf16", outlier_cols=5, name="ragged_bf16")
    yield synth.random_linear(257, 48, 130, seed=32, x_dtype="f16", outlier_cols=2, outlier_rows=[0, 100, 256],
                              name="ragged_f16_rows")
    yield synth.random_linear(513, 1040, 777, seed=33, x_dtype="bf16", outlier_cols=40, name="many_outliers")
    yield synth.random_linear(70, 16, 33, seed=34, x_dtype="bf16", outlier_cols=0, name="k16_no_outliers")
    yield synth.random_linear(333, 640, 300, seed=35, x_dtype="bf16", outlier_cols=3, name="ragged_mn_k64")
    # few tiles, long K: on 256 CUs the GEMM splits them along K (3 slices of
    # 128 K-steps; 4 uneven slices of 193 K-steps)
    yield synth.random_linear(300, 8192, 520, seed=36, x_dtype="bf16", outlier_cols=4, name="split_k_bf16")
    yield synth.random_linear(200, 12352, 300, seed=37, x_dtype="f16", outlier_cols=6, name="split_k_f16_uneven")


CASES = list(_cases())


@pytest.mark.parametrize("case", CASES, ids=lambda c: c.name)
def test_weight_quantisation_bit_exact(case):
    announce("int8 weight quant", case.name)
    wq, sw, wq_ref, sw_ref = _quant_weights_both(case)
    assert np.array_equal(wq.cpu().numpy(), wq_ref)
    assert np.array_equal(sw.cpu().numpy(), sw_ref)


@pytest.mark.parametrize("case", CASES, ids=lambda c: c.name)
# 6.001 and 1e-6 fall between representable values of both 16-bit formats;
# 7e4 is above the largest finite f16
@pytest.mark.parametrize("t", [6.0, math.inf, 0.0, 2.0, 6.001, 1e-6, 7e4])
def test_activation_quantisation_bit_exact(case, t):
    announce("int8 act quant", case.name, t)
    xf = o.decode16(case.x_bits, case.x_dtype)
    O_ref, sx_ref, q_ref = o.quantize_activations_int8(xf, t)
    q, sx, O = w8.debug_int8_quantize_activations(dev16(case.x_bits, case.x_dtype), t)
    assert np.array_equal(O.cpu().numpy(), O_ref)
    assert np.array_equal(sx.cpu().numpy(), sx_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)


def test_activation_quantisation_fixup_rows():
    """A row's scale ignores a column that another row makes an outlier
    column, even when that column holds the row's largest |x| <= t."""
    rng = np.random.default_rng(40)
    x = rng.standard_normal((96, 512)).astype(np.float32)
    x[5, 100] = 7.5                   # column 100 becomes an outlier column
    x[6, 100] = 5.5                   # ...and is row 6's provisional absmax
    x[7, 100] = -6.0                  # exactly t: not an outlier, but its column is
    x[8, 300] = 9.0
    x[8, 301] = 5.9                   # row 8: max in a clean column
    x[9, :] = 0.0
    x[9, 100] = 3.0                   # row 9: all clean columns zero -> sx = 0
    bits = synth.encode16(x, "bf16")
    xf = o.decode16(bits, "bf16")
    O_ref, sx_ref, q_ref = o.quantize_activations_int8(xf, 6.0)
    assert 100 in O_ref and sx_ref[9] == 0
    announce("int8 fixup rows")
    q, sx, O = w8.debug_int8_quantize_activations(dev16(bits, "bf16"), 6.0)
    assert np.array_equal(O.cpu().numpy(), O_ref)
    assert np.array_equal(sx.cpu().numpy(), sx_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)


@pytest.mark.parametrize("K", [16400, 20480])
def test_activation_quantisation_long_rows(K):
    """K above 16384 takes the two-pass (streaming) row kernel."""
    c = synth.random_linear(40, K, 16, seed=41, x_dtype="bf16", outlier_cols=3)
    xf = o.decode16(c.x_bits, "bf16")
    O_ref, sx_ref, q_ref = o.quantize_activations_int8(xf, 6.0)
    announce("int8 act quant long rows", K)
    q, sx, O = w8.debug_int8_quantize_activations(dev16(c.x_bits, "bf16"), 6.0)
    assert np.array_equal(O.cpu().numpy(), O_ref)
    assert np.array_equal(sx.cpu().numpy(), sx_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)


def test_outlier_set_larger_than_the_lds_list():
    """t = 0 makes every non-zero column an outlier: 8191 of them, more than
    the code kernel lists in LDS, so its per-row gather fallback runs."""
    c = synth.random_linear(40, 8192, 24, seed=45, x_dtype="bf16")
    x = c.x_bits.copy()
    x[:, 77] = 0                                   # one all-zero column stays int8
    xf = o.decode16(x, "bf16")
    O_ref, sx_ref, q_ref = o.quantize_activations_int8(xf, 0.0)
    assert O_ref.size == 8191
    announce("int8 act quant unlisted outliers")
    q, sx, O = w8.debug_int8_quantize_activations(dev16(x, "bf16"), 0.0)
    assert np.array_equal(O.cpu().numpy(), O_ref)
    assert np.array_equal(sx.cpu().numpy(), sx_ref) and np.array_equal(q.cpu().numpy(), q_ref)
    wq, sw, wq_ref, sw_ref = _quant_weights_both(c)
    ref = o.int8_mixed_linear(x, "bf16", wq_ref, sw_ref, 0.0, "f32")
    y = w8.int8_mixed_linear(dev16(x, "bf16"), wq, sw, 0.0, torch.float32)
    torch.cuda.synchronize()
    _check_outputs(y, ref, "f32", "unlisted", x, "bf16", wq_ref, sw_ref)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_every_16bit_value_encodes_like_the_oracle(dtype):
    """All finite patterns of the format, 256 per row, each row with its own
    scale (the last row padded with zeros)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = o.decode16(bits, dtype)
    fin = bits[np.isfinite(vals)]
    pad = (-fin.size) % 256
    rows = np.concatenate([fin, np.zeros(pad, np.uint16)]).reshape(-1, 256)
    xf = o.decode16(rows, dtype)
    O_ref, sx_ref, q_ref = o.quantize_activations_int8(xf, math.inf)
    announce("int8 exhaustive encode", dtype)
    q, sx, O = w8.debug_int8_quantize_activations(dev16(rows, dtype), math.inf)
    assert O.numel() == 0
    assert np.array_equal(sx.cpu().numpy(), sx_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)


@pytest.mark.parametrize("M,N,K", [(300, 520, 272), (257, 130, 48), (600, 700, 320), (64, 512, 256), (1, 1, 16),
                                   (256, 256, 16384), (300, 200, 64), (77, 300, 128), (256, 512, 192),
                                   (520, 260, 320),
                                   # K-split of the last wave of tiles (even, uneven, many tiles, ragged)
                                   (300, 520, 16384), (77, 300, 12352), (600, 700, 8192), (513, 1040, 16384)])
def test_int8_gemm_accumulators_bit_exact(M, N, K):
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    q = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    w = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    if M > 2 and N > 2:
        q[0, :] = 127
        w[0, :] = 127      # largest positive sum: 127^2 K
        w[1, :] = -127     # largest negative sum
    ref = o.int8_contract(q, w)
    announce("int8 gemm i32", M, N, K)
    acc = w8.debug_int8_gemm_i32(torch.from_numpy(q).cuda(), torch.from_numpy(w).cuda())
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), ref)


@pytest.mark.parametrize("M,N,K", [(300, 520, 4096), (77, 300, 2048), (513, 1040, 1024), (256, 512, 192),
                                   (1, 16, 640), (4352, 4352, 128), (4352, 12288, 128)])
@pytest.mark.parametrize("tail,split", [(1, 1), (1, 2), (1, 3), (2, 1), (2, 2), (2, 5), (3, 1)])
def test_int8_gemm_tail_treatments_bit_exact(M, N, K, tail, split):
    """Every treatment of the leftover tiles of a partial wave (all tiles
    when there are fewer tiles than compute units): whole 256x256 tiles,
    K-sliced 256x256 tiles, 128x128 quarters whole or K-sliced (quarters
    outside [M, N) included), and stream-K (tail 3): one block per compute
    unit over the last full wave and the leftover tiles: from 32
    blocks sharing one tile (6 tiles of 64 K steps) to pieces of 3 steps that
    cross tile boundaries (289 tiles of 2 steps; 816 tiles of 2 steps: two
    rounds of whole tiles, then stream-K over 304). Repeated calls through
    one workspace stay exact and leave the counters zero."""
    if split > K // 64:
        pytest.skip("more slices than K steps")
    rng = np.random.default_rng(M * 5 + N + K + 10 * tail + split)
    q = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    w = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    if M > 2 and N > 2:
        q[0, :] = 127
        w[0, :] = 127
        w[1, :] = -127
    ref = o.int8_contract(q, w)
    announce("int8 gemm i32 tail", M, N, K, tail, split)
    n_ws = w8.debug_int8_gemm_i32_workspace_size(M, N, K, tail, split)
    ws = w8.new_workspace(max(n_ws, 256))
    tq, tw = torch.from_numpy(q).cuda(), torch.from_numpy(w).cuda()
    for _ in range(2):
        acc = w8.debug_int8_gemm_i32(tq, tw, tail, split, workspace=ws)
        assert np.array_equal(acc.cpu().numpy().astype(np.int64), ref)
    if n_ws:
        assert int(ws[:256].view(torch.int32).abs().sum().item()) == 0     # counters left zero


@pytest.mark.parametrize("case", CASES, ids=lambda c: c.name)
@pytest.mark.parametrize("out_dtype", ["f16", "f32"])
@pytest.mark.parametrize("t", [6.0, math.inf, 0.0])
def test_int8_mixed_linear_matches_oracle(case, out_dtype, t):
    wq, sw, wq_ref, sw_ref = _quant_weights_both(case)
    ref = o.int8_mixed_linear(case.x_bits, case.x_dtype, wq_ref, sw_ref, t, out_dtype)
    announce("int8_mixed_linear", case.name, out_dtype, t)
    y = w8.int8_mixed_linear(dev16(case.x_bits, case.x_dtype), wq, sw, t, {"f16": torch.float16,
                                                                          "f32": torch.float32}[out_dtype])
    torch.cuda.synchronize()
    _check_outputs(y, ref, out_dtype, (case.name, t), case.x_bits, case.x_dtype, wq_ref, sw_ref)


def test_workspace_reuse_leaves_bookkeeping_clean():
    """The outlier flags and split-K counters live in the workspace's fixed
    front: reusing one workspace across calls with different outlier sets (and
    a K-split GEMM) gives each call its own exact result, and the counters are
    zero again after every call."""
    a = synth.random_linear(300, 8192, 520, seed=46, x_dtype="bf16", outlier_cols=5)
    b = synth.random_linear(300, 8192, 520, seed=47, x_dtype="bf16", outlier_cols=2)
    wq, sw, wq_ref, sw_ref = _quant_weights_both(a)
    ws = w8.new_workspace(w8.int8_mixed_linear_workspace_size(300, 520, 8192))
    lay = w8.int8_workspace_layout(300, 520, 8192)
    announce("int8 workspace reuse")
    for c in (a, b, a, b):
        y = w8.int8_mixed_linear(dev16(c.x_bits, "bf16"), wq, sw, 6.0, torch.float32, workspace=ws)
        ref = o.int8_mixed_linear(c.x_bits, "bf16", wq_ref, sw_ref, 6.0, "f32")
        _check_outputs(y, ref, "f32", c.name, c.x_bits, "bf16", wq_ref, sw_ref)
        torch.cuda.synchronize()
        assert not ws[lay["cnt"]:lay["flags"]].any()          # every split-K counter zero
    # the flags carry the last call's stamp on exactly its outlier columns
    flags = ws[lay["flags"]:lay["flags"] + 4 * 8192].view(torch.int32).cpu().numpy().view(np.uint32)
    O_b = o.quantize_activations_int8(o.decode16(b.x_bits, "bf16"), 6.0)[0]
    stamped = np.flatnonzero(flags == flags[O_b[0]])
    assert np.array_equal(stamped, O_b)


def test_one_workspace_serves_shapes_of_both_kinds():
    """One zero-filled workspace, large enough for both, runs a K = 4096 linear,
    a K = 16384 linear (whose flags and codes span what the first used for
    other regions), the first again and an FP8 linear, each with the result
    of a fresh workspace."""
    up = synth.random_linear(520, 4096, 700, seed=48, x_dtype="bf16", outlier_cols=4)
    down = synth.random_linear(520, 16384, 300, seed=49, x_dtype="bf16", outlier_cols=3)
    sizes = [w8.int8_mixed_linear_workspace_size(520, 700, 4096), w8.int8_mixed_linear_workspace_size(520, 300, 16384),
             w8.fp8_w8a8_linear_workspace_size(520, 700, 4096)]
    ws = w8.new_workspace(max(sizes))
    wu, su, wu_ref, su_ref = _quant_weights_both(up)
    wd, sd, wd_ref, sd_ref = _quant_weights_both(down)
    w8q, s8 = w8.quantize_weight_rowwise(dev16(up.w_bits, "bf16"), "fp8")
    announce("int8 one workspace, two shapes")
    xu, xd = dev16(up.x_bits, "bf16"), dev16(down.x_bits, "bf16")
    for c, x, wq, sw, wq_ref, sw_ref in ((up, xu, wu, su, wu_ref, su_ref), (down, xd, wd, sd, wd_ref, sd_ref),
                                         (up, xu, wu, su, wu_ref, su_ref)):
        y = w8.int8_mixed_linear(x, wq, sw, 6.0, torch.float16, workspace=ws)
        fresh = w8.int8_mixed_linear(x, wq, sw, 6.0, torch.float16)
        assert torch.equal(y, fresh), c.name
        ref = o.int8_mixed_linear(c.x_bits, "bf16", wq_ref, sw_ref, 6.0, "f16")
        _check_outputs(y, ref, "f16", c.name, c.x_bits, "bf16", wq_ref, sw_ref)
    y8 = w8.fp8_w8a8_linear(xu, w8q, s8, None, torch.bfloat16, workspace=ws)
    assert torch.equal(y8, w8.fp8_w8a8_linear(xu, w8q, s8, None, torch.bfloat16))
    y = w8.int8_mixed_linear(xd, wd, sd, 6.0, torch.float16, workspace=ws)
    assert torch.equal(y, w8.int8_mixed_linear(xd, wd, sd, 6.0, torch.float16))


@pytest.mark.parametrize("n_out,t", [(40, 6.0), (300, 6.0), (600, 0.0), (528, 0.0)],
                         ids=["staged_global", "gathered", "all_gathered", "all_gathered_k528"])
@pytest.mark.parametrize("x_dtype", ["bf16", "f16"])
def test_outlier_counts_past_the_lds_staging(n_out, t, x_dtype):
    """More than 32 outlier columns: the epilogue reads the staged XO/WO from
    global memory (up to 256 columns), or, past that, gathers the outlier
    columns from X and Wq itself; t = 0 makes every column an outlier."""
    K = {40: 640, 300: 640, 600: 608, 528: 528}[n_out]     # 528: the GEMM for K % 64 != 0
    c = synth.random_linear(300, K, 520, seed=50 + n_out, x_dtype=x_dtype, outlier_cols=min(n_out, K))
    wq, sw, wq_ref, sw_ref = _quant_weights_both(c)
    ref = o.int8_mixed_linear(c.x_bits, x_dtype, wq_ref, sw_ref, t, "f32")
    if t > 0:
        assert len(ref["O"]) >= n_out - 2
    announce("int8 outlier count", n_out, t, x_dtype, len(ref["O"]))
    y = w8.int8_mixed_linear(dev16(c.x_bits, x_dtype), wq, sw, t, torch.float32)
    torch.cuda.synchronize()
    _check_outputs(y, ref, "f32", ("outliers", n_out, t), c.x_bits, x_dtype, wq_ref, sw_ref)


def test_zero_row_gives_zero_output_row():
    c = synth.random_linear(40, 128, 64, seed=42, x_dtype="bf16", outlier_cols=2)
    x = c.x_bits.copy()
    x[17] = 0
    wq, sw, _, _ = _quant_weights_both(c)
    announce("int8 zero row")
    y = w8.int8_mixed_linear(dev16(x, "bf16"), wq, sw, 6.0, torch.float32).cpu().numpy()
    assert not y[17].any() and y[16].any()


def test_deterministic_non_default_stream_and_no_out_of_bounds_writes():
    c = synth.random_linear(333, 528, 270, seed=43, x_dtype="bf16", outlier_cols=3)
    wq, sw, wq_ref, sw_ref = _quant_weights_both(c)
    x = dev16(c.x_bits, "bf16")
    M, N = c.M, c.N
    guard = 4096
    buf = torch.full((M * N + 2 * guard,), 12345.0, dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    announce("int8 determinism/stream/guard")
    with torch.cuda.stream(s):
        y1 = w8.int8_mixed_linear(x, wq, sw, 6.0, torch.float32, out=buf[guard:guard + M * N].view(M, N))
        y1c = y1.clone()
        y2 = w8.int8_mixed_linear(x, wq, sw, 6.0, torch.float32)
    s.synchronize()
    assert torch.equal(y1c, y2)
    b = buf.cpu().numpy()
    assert np.all(b[:guard] == 12345.0) and np.all(b[guard + M * N:] == 12345.0)
    ref = o.int8_mixed_linear(c.x_bits, "bf16", wq_ref, sw_ref, 6.0, "f32")
    _check_outputs(y2, ref, "f32", "stream", c.x_bits, "bf16", wq_ref, sw_ref)


def test_gemm_timeline_export_is_ordered_and_output_unchanged():
    """The timeline export runs the same launch as int8_mixed_linear (the same
    output bits) and every block's stamps are ordered: it starts, fills the
    ring, runs the K loop and finishes in order (stream-K blocks: for their
    last piece); 128x128 tail blocks write their start and end only."""
    announce("int8 gemm timeline")
    for M, K, N in [(4100, 256, 4352), (600, 512, 1100)]:
        c = synth.random_linear(M, K, N, seed=44, x_dtype="bf16", outlier_cols=3)
        wq, sw, _, _ = _quant_weights_both(c)
        x = dev16(c.x_bits, "bf16")
        ws = w8.new_workspace(w8.int8_mixed_linear_workspace_size(c.M, c.N, c.K))
        y_ref = w8.int8_mixed_linear(x, wq, sw, 6.0, torch.float16, workspace=ws)
        y = torch.empty_like(y_ref)
        r = w8.debug_int8_gemm_timeline(x, wq, sw, 6.0, y, ws)
        assert torch.equal(y, y_ref)
        st, dp = r["stamps"], r["dp_tiles"]
        assert st.shape == (r["grid"], 8) and 0 <= dp <= r["grid"]
        loop = st[:dp] if r["rest"] == "small" else st
        ran = loop[:, 1] >= 0                     # stream-K blocks past the last K step do nothing
        assert np.all(loop[ran, 0] > 0)
        assert np.all(loop[ran, 0] <= loop[ran, 1]) and np.all(loop[ran, 1] <= loop[ran, 2])
        assert np.all(loop[ran, 4] < loop[ran, 5])
        done = ran & (loop[:, 3] >= 0)
        assert np.all(loop[done, 2] <= loop[done, 3])
        if r["rest"] == "small":
            tail = st[dp:]
            assert np.all(tail[:, 0] > 0) and np.all(tail[:, 3] >= tail[:, 0]) and np.all(tail[:, 1] == -1)


# ----------------------------------------------------------------------------
# the DiT workloads at full size: 1024^2 in the configuration bench.py times,
# and 2048^2 (16640 tokens)
# ----------------------------------------------------------------------------

FULL = {
    "dit1024_qkv": synth.dit_qkv_1024,
    "dit1024_mlp_up": lambda: synth.dit_mlp_1024("up"),
    "dit1024_mlp_down": lambda: synth.dit_mlp_1024("down"),
    "dit2048_qkv": lambda: synth.dit_2048("qkv"),
    "dit2048_mlp_up": lambda: synth.dit_2048("up"),
    "dit2048_mlp_down": lambda: synth.dit_2048("down"),
}


@pytest.mark.parametrize("name", list(FULL))
def test_dit_full_size(name):
    c = FULL[name]()
    announce("full-size", c.name)
    xf = o.decode16(c.x_bits, "bf16")
    wq, sw, wq_ref, sw_ref = _quant_weights_both(c)
    assert np.array_equal(wq.cpu().numpy(), wq_ref) and np.array_equal(sw.cpu().numpy(), sw_ref)
    x = dev16(c.x_bits, "bf16")
    # codes, scales and outlier set on every row
    O_ref, sx_ref, q_ref = o.quantize_activations_int8(xf, 6.0)
    q, sx, O = w8.debug_int8_quantize_activations(x, 6.0)
    assert np.array_equal(O.cpu().numpy(), O_ref)
    assert set(c.injected_cols) <= set(O_ref.tolist())
    assert np.array_equal(sx.cpu().numpy(), sx_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    # accumulators and outputs on sampled rows (every injected row included)
    # and on the whole last 256-row strip, whose tiles the GEMM splits along K
    rng = np.random.default_rng(44)
    last_strip = np.arange((c.M - 1) // 256 * 256, c.M)
    rows = np.unique(np.concatenate([rng.choice(c.M, 96, replace=False), np.array(c.injected_rows, int),
                                     [0, c.M - 1], last_strip])).astype(int)
    acc = w8.debug_int8_gemm_i32(q, wq)
    acc_rows = acc[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.int64)
    assert np.array_equal(acc_rows, o.int8_contract(q_ref[rows], wq_ref))
    del acc
    y = w8.int8_mixed_linear(x, wq, sw, 6.0, torch.float16)
    ref = o.int8_mixed_linear(c.x_bits, "bf16", wq_ref, sw_ref, 6.0, "f16", rows=rows)
    _check_outputs(y[torch.from_numpy(rows).cuda()], ref, "f16", c.name, c.x_bits, "bf16", wq_ref, sw_ref, rows)
