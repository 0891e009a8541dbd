"""The C ABI on the CPU: the library loads, exports every declared symbol,
and rejects bad arguments on the host before any HIP call (no GPU needed:
none of these calls reaches a kernel launch)."""
import ctypes
import math
import os
import re

import pytest

from w8a8_mixed_precision_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w8mp.h")

# Fake, 256-byte aligned addresses: validation must reject the call before
# anything dereferences them.
A = 0x10000
WS_BIG = 1 << 40
# the region every workspace starts with: 4096 split-K counters, then one
# outlier-flag word per column up to the largest int8 K (256-byte aligned)
FRONT = 4 * 4096 + (4 * _abi.W8_INT8_MAX_K + 255) // 256 * 256


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"if", "sizeof"})


def test_library_exports_every_declared_symbol():
    lib = _abi.lib()
    names = declared_functions()
    assert "int8_mixed_linear" in names and "fp8_w8a8_linear" in names and "quantize_weight_rowwise" in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_abi.SIGNATURES), "binding and header disagree"


def test_status_strings():
    assert _abi.status_string(0) == "W8_OK"
    assert _abi.status_string(3) == "W8_ERR_WORKSPACE"
    assert _abi.status_string(99) == "W8_UNKNOWN_STATUS"


def _int8(**kw):
    a = dict(X=A, x_dt=_abi.W8_DT_BF16, M=64, K=256, Wq=A, sw=A, N=32, t=6.0, Y=A, y_dt=_abi.W8_DT_F16,
             ws=A, ws_bytes=WS_BIG, stream=None)
    a.update(kw)
    return _abi.lib().int8_mixed_linear(a["X"], a["x_dt"], a["M"], a["K"], a["Wq"], a["sw"], a["N"], a["t"], a["Y"],
                                        a["y_dt"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), _abi.W8_ERR_INVALID_ARGUMENT),
    (dict(Wq=None), _abi.W8_ERR_INVALID_ARGUMENT),
    (dict(Y=None), _abi.W8_ERR_INVALID_ARGUMENT),
    (dict(M=0), _abi.W8_ERR_INVALID_ARGUMENT),
    (dict(N=0), _abi.W8_ERR_INVALID_ARGUMENT),
    (dict(K=0), _abi.W8_ERR_INVALID_ARGUMENT),
    (dict(K=24), _abi.W8_ERR_INVALID_ARGUMENT),
    (dict(K=8), _abi.W8_ERR_INVALID_ARGUMENT),
    (dict(K=133152), _abi.W8_ERR_UNSUPPORTED),
    (dict(t=-1.0), _abi.W8_ERR_INVALID_ARGUMENT),
    (dict(t=math.nan), _abi.W8_ERR_INVALID_ARGUMENT),
    (dict(x_dt=_abi.W8_DT_F32), _abi.W8_ERR_UNSUPPORTED),
    (dict(y_dt=_abi.W8_DT_BF16), _abi.W8_ERR_UNSUPPORTED),
    (dict(X=A + 8), _abi.W8_ERR_INVALID_ARGUMENT),
    (dict(ws=None), _abi.W8_ERR_WORKSPACE),
    (dict(ws=A + 16), _abi.W8_ERR_WORKSPACE),
    (dict(ws_bytes=1024), _abi.W8_ERR_WORKSPACE),
])
def test_int8_mixed_linear_rejects(kw, status):
    assert _int8(**kw) == status
    assert _abi.lib().w8_last_error().decode() != ""


def _fused(prod=None, **kw):
    a = dict(X=A, x_dt=_abi.W8_DT_BF16, M=64, K=256, Wq=A, sw=A, bias=None, N=32, t=6.0, Y=A,
             y_dt=_abi.W8_DT_F16, ws=A, ws_bytes=WS_BIG, stream=None)
    a.update(kw)
    p = ctypes.byref(prod) if prod is not None else None
    return _abi.lib().int8_mixed_linear_fused(a["X"], a["x_dt"], a["M"], a["K"], p, a["Wq"], a["sw"], a["bias"],
                                              a["N"], a["t"], a["Y"], a["y_dt"], a["ws"], a["ws_bytes"],
                                              a["stream"])


@pytest.mark.parametrize("prod,kw,status", [
    (_abi.Producer(7, None, None, None, 0.0), {}, _abi.W8_ERR_INVALID_ARGUMENT),            # unknown kind
    (_abi.Producer(_abi.W8_PRODUCER_RMSNORM, None, None, None, -1.0), {}, _abi.W8_ERR_INVALID_ARGUMENT),
    (_abi.Producer(_abi.W8_PRODUCER_RMSNORM, None, None, None, math.nan), {}, _abi.W8_ERR_INVALID_ARGUMENT),
    (_abi.Producer(_abi.W8_PRODUCER_GELU_TANH, None, None, None, 0.0), dict(K=16400), _abi.W8_ERR_UNSUPPORTED),
    (None, dict(X=None), _abi.W8_ERR_INVALID_ARGUMENT),
    (None, dict(ws_bytes=1024), _abi.W8_ERR_WORKSPACE),
])
def test_int8_fused_linear_rejects(prod, kw, status):
    assert _fused(prod, **kw) == status
    assert _abi.lib().w8_last_error().decode() != ""


def test_debug_produce_rejects():
    lib = _abi.lib()
    gelu = _abi.Producer(_abi.W8_PRODUCER_GELU_TANH, None, None, None, 0.0)
    assert lib.w8dbg_produce(None, _abi.W8_DT_BF16, 4, 64, ctypes.byref(gelu), A, None) == \
        _abi.W8_ERR_INVALID_ARGUMENT
    assert lib.w8dbg_produce(A, _abi.W8_DT_BF16, 4, 32768, ctypes.byref(gelu), A, None) == _abi.W8_ERR_UNSUPPORTED


def test_workspace_size_is_exact_boundary():
    lib = _abi.lib()
    need = lib.int8_mixed_linear_workspace_size(64, 32, 256)
    assert need >= FRONT + 64 * 256 + 2 * (64 + 32) * 256
    assert _int8(ws_bytes=need - 1) == _abi.W8_ERR_WORKSPACE
    assert lib.int8_mixed_linear_workspace_size(0, 32, 256) == 0
    # grows with every dimension
    assert lib.int8_mixed_linear_workspace_size(65, 32, 256) > need
    assert lib.int8_mixed_linear_workspace_size(64, 33, 256) > need
    assert lib.int8_mixed_linear_workspace_size(64, 32, 272) > need
    assert lib.fp8_w8a8_linear_workspace_size(512, 4096, 4096) >= 512 * 4096 + 4 * 512


def _fp8(**kw):
    a = dict(X=A, x_dt=_abi.W8_DT_BF16, M=512, K=4096, Wq=A, sw=A, N=1024, s=None, Y=A, y_dt=_abi.W8_DT_BF16,
             ws=A, ws_bytes=WS_BIG, stream=None)
    a.update(kw)
    return _abi.lib().fp8_w8a8_linear(a["X"], a["x_dt"], a["M"], a["K"], a["Wq"], a["sw"], a["N"], a["s"], a["Y"],
                                      a["y_dt"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), _abi.W8_ERR_INVALID_ARGUMENT),
    (dict(K=100), _abi.W8_ERR_INVALID_ARGUMENT),
    (dict(K=65552), _abi.W8_ERR_UNSUPPORTED),
    (dict(y_dt=7), _abi.W8_ERR_UNSUPPORTED),
    (dict(x_dt=_abi.W8_DT_F32), _abi.W8_ERR_UNSUPPORTED),
    (dict(ws_bytes=16), _abi.W8_ERR_WORKSPACE),
    (dict(Y=A + 2), _abi.W8_ERR_INVALID_ARGUMENT),
])
def test_fp8_linear_rejects(kw, status):
    assert _fp8(**kw) == status


def _w16(**kw):
    a = dict(X=A, x_dt=_abi.W8_DT_BF16, M=512, K=4096, Wq=A, sw=A, N=1024, Y=A, y_dt=_abi.W8_DT_BF16,
             ws=A, ws_bytes=WS_BIG, stream=None)
    a.update(kw)
    return _abi.lib().fp8_w8a16_linear(a["X"], a["x_dt"], a["M"], a["K"], a["Wq"], a["sw"], a["N"], a["Y"],
                                       a["y_dt"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), _abi.W8_ERR_INVALID_ARGUMENT),
    (dict(sw=None), _abi.W8_ERR_INVALID_ARGUMENT),
    (dict(M=0), _abi.W8_ERR_INVALID_ARGUMENT),
    (dict(K=100), _abi.W8_ERR_INVALID_ARGUMENT),                 # K % 16 != 0
    (dict(K=4112), _abi.W8_ERR_UNSUPPORTED),                     # K % 64 != 0
    (dict(K=65600), _abi.W8_ERR_UNSUPPORTED),
    (dict(x_dt=_abi.W8_DT_F16), _abi.W8_ERR_UNSUPPORTED),        # bf16 activations only
    (dict(y_dt=7), _abi.W8_ERR_UNSUPPORTED),
    (dict(Wq=A + 8), _abi.W8_ERR_INVALID_ARGUMENT),
    (dict(ws=None), _abi.W8_ERR_WORKSPACE),
    (dict(ws_bytes=16), _abi.W8_ERR_WORKSPACE),
])
def test_w8a16_linear_rejects(kw, status):
    assert _w16(**kw) == status


def _w4(**kw):
    a = dict(X=A, x_dt=_abi.W8_DT_BF16, M=512, K=4096, Wq=A, sw=A, N=1024, Y=A, y_dt=_abi.W8_DT_F16,
             ws=A, ws_bytes=WS_BIG, stream=None)
    a.update(kw)
    return _abi.lib().w4a8_linear(a["X"], a["x_dt"], a["M"], a["K"], a["Wq"], a["sw"], a["N"], a["Y"], a["y_dt"],
                                  a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), _abi.W8_ERR_INVALID_ARGUMENT),
    (dict(Wq=None), _abi.W8_ERR_INVALID_ARGUMENT),
    (dict(N=0), _abi.W8_ERR_INVALID_ARGUMENT),
    (dict(K=4160), _abi.W8_ERR_UNSUPPORTED),                     # K % 128 != 0
    (dict(K=100), _abi.W8_ERR_INVALID_ARGUMENT),
    (dict(x_dt=_abi.W8_DT_F32), _abi.W8_ERR_UNSUPPORTED),
    (dict(y_dt=9), _abi.W8_ERR_UNSUPPORTED),
    (dict(M=1 << 21, K=4096), _abi.W8_ERR_UNSUPPORTED),          # codes above 4 GiB
    (dict(sw=A + 4), _abi.W8_ERR_INVALID_ARGUMENT),
    (dict(ws_bytes=1024), _abi.W8_ERR_WORKSPACE),
])
def test_w4a8_linear_rejects(kw, status):
    assert _w4(**kw) == status


def test_w4a8_weight_format_and_debug_rejects():
    lib = _abi.lib()
    q = lib.quantize_weight_rowwise
    assert q(A, _abi.W8_DT_BF16, 16, 192, _abi.W8_Q_INT4_G128, A, A, None) == _abi.W8_ERR_UNSUPPORTED  # K % 128
    assert q(A, _abi.W8_DT_BF16, 16, 192, 3, A, A, None) == _abi.W8_ERR_UNSUPPORTED
    need = lib.w4a8_linear_workspace_size(512, 1024, 4096)
    assert need >= 512 * 4096 + 4 * 512
    assert _w4(ws_bytes=need - 1) == _abi.W8_ERR_WORKSPACE
    g = lib.w8dbg_w4a8_linear
    bf, f16 = _abi.W8_DT_BF16, _abi.W8_DT_F16
    assert g(A, bf, 4, 256, A, A, 4, -1, A, f16, A, WS_BIG, None) == _abi.W8_ERR_INVALID_ARGUMENT
    assert g(A, bf, 4, 256, A, A, 4, 3, A, f16, A, WS_BIG, None) == _abi.W8_ERR_UNSUPPORTED          # > K/128
    assert lib.w8dbg_w4a8_linear_workspace_size(4, 4, 256, 2) >= 2 * 128 * 128 * 4


def test_dit_block_and_linear16_reject():
    lib = _abi.lib()
    blk = _abi.DitBlock(256, 1024, 6.0, *([A] * 12), None, _abi.Producer(), _abi.Producer())
    fwd = lambda b, X=A, M=64, Y=A, ws=A, n=WS_BIG: lib.w8_dit_block_forward(
        ctypes.byref(b) if b is not None else None, X, M, Y, ws, n, None)
    assert fwd(None) == _abi.W8_ERR_INVALID_ARGUMENT
    assert fwd(blk, X=None) == _abi.W8_ERR_INVALID_ARGUMENT
    assert fwd(blk, M=0) == _abi.W8_ERR_INVALID_ARGUMENT
    assert fwd(blk, Y=A + 2) == _abi.W8_ERR_INVALID_ARGUMENT
    need = lib.w8_dit_block_workspace_size(64, 256, 1024)
    assert need > 64 * 256 * 2 * 8
    assert fwd(blk, n=need - 1) == _abi.W8_ERR_WORKSPACE
    bad = _abi.DitBlock(200, 1024, 6.0, *([A] * 12), None, _abi.Producer(), _abi.Producer())
    assert fwd(bad) == _abi.W8_ERR_INVALID_ARGUMENT                    # D % 64 != 0
    nodown = _abi.DitBlock(256, 1024, 6.0, *([A] * 9), None, None, A, None, _abi.Producer(), _abi.Producer())
    assert fwd(nodown) == _abi.W8_ERR_INVALID_ARGUMENT                 # neither int8 nor fp16 down weights
    assert "down projection" in _abi.lib().w8_last_error().decode()
    f16, f32 = _abi.W8_DT_F16, _abi.W8_DT_F32
    l16 = lib.w8dbg_linear16
    assert l16(A, f16, 4, 96, A, 4, 0, 0, A, f32, A, WS_BIG, None) == _abi.W8_ERR_UNSUPPORTED        # K % 64
    assert l16(A, f32, 4, 128, A, 4, 0, 0, A, f32, A, WS_BIG, None) == _abi.W8_ERR_UNSUPPORTED       # X type
    assert l16(A, f16, 4, 128, A, 4, 3, 128, A, f32, A, WS_BIG, None) == _abi.W8_ERR_UNSUPPORTED     # split > K/64
    assert l16(A, f16, 4, 128, A, 4, 1, 64, A, f32, A, WS_BIG, None) == _abi.W8_ERR_INVALID_ARGUMENT  # tile
    assert l16(None, f16, 4, 128, A, 4, 0, 0, A, f32, A, WS_BIG, None) == _abi.W8_ERR_INVALID_ARGUMENT
    assert l16(A, f16, 4, 128, A, 4, 2, 128, A, f32, A, 256, None) == _abi.W8_ERR_WORKSPACE
    assert l16(A, f16, 4, 128, A, 4, 2, 256, A, f32, A, 128, None) == _abi.W8_ERR_WORKSPACE     # < 256 bytes
    assert lib.w8dbg_linear16_workspace_size(4, 4, 128, 2, 128) >= 2 * 128 * 128 * 4


def test_w8a16_workspace_and_debug_rejects():
    lib = _abi.lib()
    assert lib.fp8_w8a16_linear_workspace_size(512, 4096, 4096) >= 256
    assert lib.fp8_w8a16_linear_workspace_size(0, 4096, 4096) == 0
    assert lib.w8dbg_fp8_w8a16_linear_workspace_size(4, 4, 128, 2, 256) >= 2 * 256 * 256 * 4
    assert lib.w8dbg_fp8_w8a16_linear_workspace_size(4, 4, 128, 1, 0) == FRONT    # the common front only
    g = lib.w8dbg_fp8_w8a16_linear
    bf = _abi.W8_DT_BF16
    assert g(A, bf, 4, 128, A, A, 4, -1, 0, A, bf, A, WS_BIG, None) == _abi.W8_ERR_INVALID_ARGUMENT
    assert g(A, bf, 4, 128, A, A, 4, 1, 64, A, bf, A, WS_BIG, None) == _abi.W8_ERR_INVALID_ARGUMENT   # tile
    assert g(A, bf, 4, 128, A, A, 4, 3, 0, A, bf, A, WS_BIG, None) == _abi.W8_ERR_UNSUPPORTED         # > K/64
    need = lib.w8dbg_fp8_w8a16_linear_workspace_size(4, 4, 128, 2, 128)
    assert g(A, bf, 4, 128, A, A, 4, 2, 128, A, bf, A, need - 256, None) == _abi.W8_ERR_WORKSPACE


@pytest.mark.parametrize("args,status", [
    ((None, _abi.W8_DT_BF16, 16, 64, _abi.W8_Q_INT8, A, A, None), _abi.W8_ERR_INVALID_ARGUMENT),
    ((A, _abi.W8_DT_F32, 16, 64, _abi.W8_Q_INT8, A, A, None), _abi.W8_ERR_UNSUPPORTED),
    ((A, _abi.W8_DT_BF16, 16, 64, 5, A, A, None), _abi.W8_ERR_UNSUPPORTED),
    ((A, _abi.W8_DT_BF16, 16, 60, _abi.W8_Q_INT8, A, A, None), _abi.W8_ERR_INVALID_ARGUMENT),
    ((A, _abi.W8_DT_BF16, 0, 64, _abi.W8_Q_FP8_E4M3, A, A, None), _abi.W8_ERR_INVALID_ARGUMENT),
])
def test_weight_quantisation_rejects(args, status):
    assert _abi.lib().quantize_weight_rowwise(*args) == status


def test_debug_exports_reject():
    lib = _abi.lib()
    assert lib.w8dbg_int8_gemm_i32(A, A, 4, 4, 20, 0, 1, A, None, 0, None) == _abi.W8_ERR_INVALID_ARGUMENT
    assert lib.w8dbg_int8_gemm_i32(None, A, 4, 4, 32, 0, 1, A, None, 0, None) == _abi.W8_ERR_INVALID_ARGUMENT
    assert lib.w8dbg_int8_gemm_i32(A, A, 4, 4, 64, 4, 1, A, None, 0, None) == _abi.W8_ERR_INVALID_ARGUMENT
    assert lib.w8dbg_int8_gemm_i32(A, A, 4, 4, 64, 3, 2, A, None, 0, None) == _abi.W8_ERR_INVALID_ARGUMENT  # stream-K
    assert lib.w8dbg_int8_gemm_i32(A, A, 4, 4, 80, 3, 1, A, None, 0, None) == _abi.W8_ERR_UNSUPPORTED
    assert lib.w8dbg_int8_gemm_i32(A, A, 4, 4, 64, 2, 0, A, None, 0, None) == _abi.W8_ERR_INVALID_ARGUMENT
    assert lib.w8dbg_int8_gemm_i32(A, A, 4, 4, 80, 2, 1, A, None, 0, None) == _abi.W8_ERR_UNSUPPORTED
    assert lib.w8dbg_int8_gemm_i32(A, A, 4, 4, 128, 1, 3, A, None, 0, None) == _abi.W8_ERR_UNSUPPORTED
    assert lib.w8dbg_int8_gemm_i32_workspace_size(4, 4, 128, 2, 2) >= 4 * 2 * 128 * 128 * 4
    assert lib.w8dbg_int8_gemm_i32_workspace_size(4, 4, 128, 1, 2) >= 2 * 256 * 256 * 4
    assert lib.w8dbg_int8_gemm_i32(A, A, 4, 4, 128, 2, 2, A, A, 1024, None) == _abi.W8_ERR_WORKSPACE
    assert lib.w8dbg_fp8_quantize_activations(A, _abi.W8_DT_BF16, 4, 20, None, A, A, None) == \
        _abi.W8_ERR_INVALID_ARGUMENT
    assert lib.w8dbg_int8_quantize_activations(A, _abi.W8_DT_BF16, 4, 32, None, 6.0, A, A, A, A, A, 1,
                                               None) == _abi.W8_ERR_WORKSPACE
    f8 = lib.w8dbg_fp8_gemm
    bf = _abi.W8_DT_BF16
    assert f8(None, A, A, A, 4, 4, 64, 1, 0, A, bf, None, 0, None) == _abi.W8_ERR_INVALID_ARGUMENT
    assert f8(A, A, A, A, 4, 4, 64, -1, 0, A, bf, None, 0, None) == _abi.W8_ERR_INVALID_ARGUMENT
    assert f8(A, A, A, A, 4, 4, 64, 1, 64, A, bf, None, 0, None) == _abi.W8_ERR_INVALID_ARGUMENT   # tile
    assert f8(A, A, A, A, 4, 4, 80, 2, 0, A, bf, None, 0, None) == _abi.W8_ERR_UNSUPPORTED     # K % 64 != 0
    assert f8(A, A, A, A, 4, 4, 80, 1, 128, A, bf, None, 0, None) == _abi.W8_ERR_UNSUPPORTED   # K % 64 != 0
    assert f8(A, A, A, A, 4, 4, 128, 3, 0, A, bf, None, 0, None) == _abi.W8_ERR_UNSUPPORTED    # > K / 64 slices
    assert f8(A, A, A, A, 4, 4, 64, 1, 0, A, 9, None, 0, None) == _abi.W8_ERR_UNSUPPORTED
    need = lib.w8dbg_fp8_gemm_workspace_size(4, 4, 128, 2, 256)
    assert need >= 2 * 256 * 256 * 4                                                        # two fp32 partials
    assert lib.w8dbg_fp8_gemm_workspace_size(4, 4, 128, 2, 128) >= 2 * 128 * 128 * 4
    assert f8(A, A, A, A, 4, 4, 128, 2, 256, A, bf, A, need - 256, None) == _abi.W8_ERR_WORKSPACE
    assert lib.w8dbg_fp8_gemm_workspace_size(4, 4, 128, 1, 0) == FRONT


def test_binding_refuses_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_abi, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_abi, "_lib", None)
    with pytest.raises(ImportError):
        _abi.lib()


def test_workspace_layout_has_a_fixed_front():
    """The split-K counters and the outlier flags sit at the same offsets for
    every shape (so one workspace serves calls of different shapes), before
    every shape-dependent region; XO/WO hold a bounded number of outlier
    columns (not K), so WO of a large weight no longer dwarfs the codes."""
    lib = _abi.lib()
    shapes = [(64, 32, 256), (4352, 12288, 4096), (4352, 4096, 16384), (1, 1, 16), (16640, 16384, 4096)]
    lays = []
    for M, N, K in shapes:
        v = (ctypes.c_size_t * 11)()
        assert lib.w8dbg_int8_workspace_layout(M, N, K, v) == _abi.W8_OK
        lays.append(list(v))
    for (M, N, K), (cnt, flags, nO, O, q, sx, rstd, XO, WO, part, cap) in zip(shapes, lays):
        assert cnt == 0 and flags == 4 * 4096 and nO == FRONT
        assert flags + 4 * _abi.W8_INT8_MAX_K <= nO
        assert O >= nO + 4 and q >= O + 4 * K and sx >= q + M * K and rstd >= sx + 4 * M
        assert XO >= rstd + 4 * M and WO >= XO + 2 * M * cap and part >= WO + 2 * N * cap
        assert cap == 256
        assert all(x % 256 == 0 for x in (cnt, flags, nO, O, q, sx, rstd, XO, WO, part))
        assert lib.int8_mixed_linear_workspace_size(M, N, K) >= part
    # the 1024^2 MLP-up workspace: about the codes plus 10 MB, not 2 (M + N) K bytes
    M, N, K = 4352, 16384, 4096
    assert lib.int8_mixed_linear_workspace_size(M, N, K) < M * K + FRONT + 2 * (M + N) * 256 + 40 * 2 ** 20
    assert lib.w8dbg_int8_workspace_layout(0, 1, 16, (ctypes.c_size_t * 11)()) == _abi.W8_ERR_INVALID_ARGUMENT


def test_workspace_sizes_are_shape_functions():
    """Size queries depend on (M, N, K) only: they answer without a device
    (here there is none) and cover the shape's own regions."""
    lib = _abi.lib()
    M, N, K = 512, 4096, 4096
    assert lib.int8_mixed_linear_workspace_size(M, N, K) >= FRONT + M * K + 2 * (M + N) * 256
    assert lib.fp8_w8a8_linear_workspace_size(M, N, K) >= FRONT + M * K + 4 * M
    assert lib.fp8_w8a16_linear_workspace_size(M, N, K) >= FRONT
    assert lib.w4a8_linear_workspace_size(M, N, K) >= FRONT + M * K + 4 * M
    assert lib.w8_dit_block_workspace_size(4352, 4096, 16384) > lib.int8_mixed_linear_workspace_size(4352, 4096, 16384)


def test_events_exports_validate_like_the_linears():
    lib = _abi.lib()
    ev = (ctypes.c_void_p * 4)()
    bf, f16 = _abi.W8_DT_BF16, _abi.W8_DT_F16
    assert lib.w8dbg_int8_mixed_linear_events(None, bf, 4, 64, None, A, A, None, 4, 6.0, A, f16, A, WS_BIG, ev,
                                              None) == _abi.W8_ERR_INVALID_ARGUMENT
    assert lib.w8dbg_int8_mixed_linear_events(A, bf, 4, 64, None, A, A, None, 4, 6.0, A, f16, A, 256, ev,
                                              None) == _abi.W8_ERR_WORKSPACE
    assert lib.w8dbg_fp8_w8a8_linear_events(A, bf, 4, 64, A, A, 4, None, A, bf, A, 256, ev, None) == \
        _abi.W8_ERR_WORKSPACE
    v = (ctypes.c_size_t * 7)()
    assert lib.w8dbg_dit_block_layout(4352, 4096, 16384, v) == _abi.W8_OK
    qkv, a, o, h, u, g, d = list(v)
    M, D, F = 4352, 4096, 16384
    assert qkv >= lib.int8_mixed_linear_workspace_size(M, D, F)
    assert a >= qkv + 2 * M * 3 * D and o >= a + 2 * M * D and h >= o + 2 * M * D and u >= h + 2 * M * D
    assert g >= u + 2 * M * F and d >= g + 2 * M * F


def test_noalloc_rejects_shapes_beyond_its_scratch():
    """int8_mixed_linear_noalloc validates on the host like int8_mixed_linear
    and rejects a shape whose workspace exceeds its 96 MiB scratch before
    touching the device (the DiT 2048^2 MLP down projection: 16640 x 16384
    codes alone are 272 MB)."""
    lib = _abi.lib()
    f = lib.int8_mixed_linear_noalloc
    bf, f16 = _abi.W8_DT_BF16, _abi.W8_DT_F16
    assert f(A, bf, 16640, 16384, A, A, 4096, 6.0, A, f16, None) == _abi.W8_ERR_UNSUPPORTED
    assert "scratch" in lib.w8_last_error().decode()
    assert f(None, bf, 64, 256, A, A, 32, 6.0, A, f16, None) == _abi.W8_ERR_INVALID_ARGUMENT
    assert f(A, bf, 64, 24, A, A, 32, 6.0, A, f16, None) == _abi.W8_ERR_INVALID_ARGUMENT
    assert f(A, bf, 64, 256, A, A, 32, float("nan"), A, f16, None) == _abi.W8_ERR_INVALID_ARGUMENT
    assert f(A, bf, 64, 256, A, A, 0, 6.0, A, f16, None) == _abi.W8_ERR_INVALID_ARGUMENT
    assert f(A, bf, 64, 256, None, A, 32, 6.0, A, f16, None) == _abi.W8_ERR_INVALID_ARGUMENT
    assert f(A, bf, 64, 256, A, A, 32, 6.0, None, f16, None) == _abi.W8_ERR_INVALID_ARGUMENT
    assert f(A, bf, 64, 256, A, A, 32, 6.0, A, _abi.W8_DT_BF16, None) == _abi.W8_ERR_UNSUPPORTED


def test_gemm_timeline_query_and_rejects():
    """With stamps NULL the timeline export reports the launch's grid without
    running anything. For the DiT 1024^2 QKV linear that is 816 whole tiles
    with no device to plan for (here), or on a 256-CU device 768 whole tiles
    and the 48 leftover ones as 128x128 quarters; a short stamps buffer is
    rejected."""
    lib = _abi.lib()
    bf, f16 = _abi.W8_DT_BF16, _abi.W8_DT_F16
    M, N, K = 4352, 12288, 4096
    ws = lib.int8_mixed_linear_workspace_size(M, N, K)
    g = (ctypes.c_int * 4)()
    assert lib.w8dbg_int8_gemm_timeline(A, bf, M, K, A, A, N, 6.0, A, f16, A, ws, None, 0, g, None) == _abi.W8_OK
    assert list(g) in ([816, 816, 1, 0], [768 + 4 * 48, 768, 1, 1])
    assert lib.w8dbg_int8_gemm_timeline(A, bf, M, K, A, A, N, 6.0, A, f16, A, ws, A, 8 * g[0] - 1, g,
                                        None) == _abi.W8_ERR_INVALID_ARGUMENT
    assert lib.w8dbg_int8_gemm_timeline(A, bf, 64, 48, A, A, 32, 6.0, A, f16, A, WS_BIG, A, 1 << 20, g,
                                        None) == _abi.W8_ERR_UNSUPPORTED
    assert g[2] == 0
    assert lib.w8dbg_int8_gemm_timeline(A, bf, M, K, A, A, N, 6.0, A, f16, A, ws, None, 0, None,
                                        None) == _abi.W8_ERR_INVALID_ARGUMENT


def test_lds_stream_rejects():
    lib = _abi.lib()
    f = lib.w8dbg_lds_stream
    d = ctypes.c_double()
    big = 256 * 4096 * 4
    assert f(A, big, 4096, 96, 256, 4, 10, A, ctypes.byref(d), None) == _abi.W8_ERR_INVALID_ARGUMENT    # seg
    assert f(A, big, 4100, 64, 256, 4, 10, A, ctypes.byref(d), None) == _abi.W8_ERR_INVALID_ARGUMENT    # K % seg
    assert f(A, big - 1, 4096, 64, 256, 4, 10, A, ctypes.byref(d), None) == _abi.W8_ERR_INVALID_ARGUMENT  # buf
    assert f(None, big, 4096, 64, 256, 4, 10, A, ctypes.byref(d), None) == _abi.W8_ERR_INVALID_ARGUMENT
    assert f(A, 1 << 40, 1 << 23, 64, 256, 1, 10, A, ctypes.byref(d), None) == _abi.W8_ERR_INVALID_ARGUMENT  # 256 K
    assert f(A, big, 4096, 64, 0, 4, 10, A, ctypes.byref(d), None) == _abi.W8_ERR_INVALID_ARGUMENT


def test_mfma_peak_rejects():
    lib = _abi.lib()
    d = ctypes.c_double()
    assert lib.w8dbg_mfma_peak(5, 4, 10, A, ctypes.byref(d), None) == _abi.W8_ERR_INVALID_ARGUMENT
    assert lib.w8dbg_mfma_peak(-1, 4, 10, A, ctypes.byref(d), None) == _abi.W8_ERR_INVALID_ARGUMENT
    assert lib.w8dbg_mfma_peak(3, 0, 10, A, ctypes.byref(d), None) == _abi.W8_ERR_INVALID_ARGUMENT
    assert lib.w8dbg_mfma_peak(4, 4, 10, None, ctypes.byref(d), None) == _abi.W8_ERR_INVALID_ARGUMENT
