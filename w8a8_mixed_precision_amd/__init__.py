"""MI355X (gfx950) quantized linear layers: LLM.int8 mixed precision and FP8-E4M3 W8A8.

Thin binding over libw8mp.so. Every step of the computation runs in the
library's HIP kernels; this module only allocates outputs and workspaces with
torch and passes device pointers and the current HIP stream.
"""
from __future__ import annotations

import torch

from . import _abi
from ._abi import W8Error, lib  # noqa: F401

_DT = {torch.float16: _abi.W8_DT_F16, torch.bfloat16: _abi.W8_DT_BF16, torch.float32: _abi.W8_DT_F32}

__all__ = [
    "quantize_weight_rowwise", "int8_mixed_linear", "fp8_w8a8_linear", "fp8_w8a16_linear", "Producer",
    "debug_produce", "debug_fp8_w8a16_linear", "fp8_w8a16_linear_workspace_size", "w4a8_linear",
    "w4a8_linear_workspace_size", "DitBlock", "debug_linear16",
    "debug_int8_quantize_activations", "debug_int8_gemm_i32", "debug_fp8_quantize_activations", "debug_fp8_gemm",
    "int8_mixed_linear_workspace_size", "fp8_w8a8_linear_workspace_size", "new_workspace", "W8Error",
    "int8_workspace_layout", "debug_int8_mixed_linear_events", "debug_fp8_w8a8_linear_events",
    "int8_mixed_linear_noalloc",
]


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _dt(t: torch.Tensor) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise ValueError(f"unsupported dtype {t.dtype}") from None


def _workspace(nbytes: int, device) -> torch.Tensor:
    # torch's allocator returns 256-byte aligned blocks; the library needs the
    # workspace zero-filled before first use (it leaves its bookkeeping zero)
    return torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)


def new_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A workspace of `nbytes` for repeated calls (zero-filled, as required).
    One workspace may serve calls of any shapes and entry points in turn, as
    long as it is as large as each call's size query (calls on different
    streams that may overlap need distinct workspaces)."""
    return _workspace(nbytes, device)


def int8_workspace_layout(M: int, N: int, K: int) -> dict:
    """Byte offsets of the regions of an int8_mixed_linear workspace (parity
    export): cnt, flags, nO, O, q, sx, rstd, XO, WO, part, and out_cap (the
    outlier columns XO/WO hold)."""
    import ctypes

    v = (ctypes.c_size_t * 11)()
    _abi.check(lib().w8dbg_int8_workspace_layout(M, N, K, v))
    names = ["cnt", "flags", "nO", "O", "q", "sx", "rstd", "XO", "WO", "part", "out_cap"]
    return {k: int(v[i]) for i, k in enumerate(names)}


def int8_mixed_linear_workspace_size(M: int, N: int, K: int) -> int:
    return int(lib().int8_mixed_linear_workspace_size(M, N, K))


def fp8_w8a8_linear_workspace_size(M: int, N: int, K: int) -> int:
    return int(lib().fp8_w8a8_linear_workspace_size(M, N, K))


def fp8_w8a16_linear_workspace_size(M: int, N: int, K: int) -> int:
    return int(lib().fp8_w8a16_linear_workspace_size(M, N, K))


def quantize_weight_rowwise(w: torch.Tensor, fmt: str = "int8"):
    """W [N,K] f16/bf16 -> (Wq, sw): "int8" gives int8 codes [N,K] and sw [N];
    "fp8" E4M3 codes [N,K] (uint8) and sw [N]; "int4" packed int4 codes
    [N,K/2] (uint8) and group scales [K/128, N] (see include/w8mp.h)."""
    _dev(w, "w")
    N, K = w.shape
    if fmt == "int8":
        wq = torch.empty((N, K), dtype=torch.int8, device=w.device)
        f = _abi.W8_Q_INT8
    elif fmt == "fp8":
        wq = torch.empty((N, K), dtype=torch.uint8, device=w.device)
        f = _abi.W8_Q_FP8_E4M3
    elif fmt == "int4":
        wq = torch.empty((N, K // 2), dtype=torch.uint8, device=w.device)
        f = _abi.W8_Q_INT4_G128
    else:
        raise ValueError(fmt)
    sw = torch.empty((K // 128, N) if fmt == "int4" else (N,), dtype=torch.float32, device=w.device)
    _abi.check(lib().quantize_weight_rowwise(w.data_ptr(), _dt(w), N, K, f, wq.data_ptr(), sw.data_ptr(),
                                             _stream(w)))
    return wq, sw


class Producer:
    """The op that produces X from H, fused into the int8 quantisation pass
    (struct w8_producer in include/w8mp.h): kind "rmsnorm" (RMSNorm with the
    optional gain gamma, modulation scale and shift, fp32 [K] GPU tensors, and
    eps) or "gelu" (tanh form)."""

    KINDS = {"none": _abi.W8_PRODUCER_NONE, "rmsnorm": _abi.W8_PRODUCER_RMSNORM, "gelu": _abi.W8_PRODUCER_GELU_TANH}

    def __init__(self, kind: str, gamma: torch.Tensor | None = None, scale: torch.Tensor | None = None,
                 shift: torch.Tensor | None = None, eps: float = 1e-6):
        if kind not in self.KINDS:
            raise ValueError(f"producer kind {kind!r}")
        for name, v in (("gamma", gamma), ("scale", scale), ("shift", shift)):
            if v is not None:
                _dev(v, name)
                if v.dtype != torch.float32 or v.dim() != 1:
                    raise ValueError(f"{name} must be a 1-D fp32 tensor")
        self.kind, self.gamma, self.scale, self.shift, self.eps = kind, gamma, scale, shift, float(eps)

    def struct(self, K: int) -> "_abi.Producer":
        for name, v in (("gamma", self.gamma), ("scale", self.scale), ("shift", self.shift)):
            if v is not None and v.numel() != K:
                raise ValueError(f"{name} must have K = {K} entries")
        ptr = lambda v: v.data_ptr() if v is not None else None
        return _abi.Producer(self.KINDS[self.kind], ptr(self.gamma), ptr(self.scale), ptr(self.shift), self.eps)


def _producer_arg(producer: "Producer | None", K: int):
    import ctypes

    return None if producer is None else ctypes.byref(producer.struct(K))


def int8_mixed_linear(x: torch.Tensor, wq: torch.Tensor, sw: torch.Tensor, threshold: float = 6.0,
                      out_dtype: torch.dtype = torch.float16, out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None, bias: torch.Tensor | None = None,
                      producer: Producer | None = None) -> torch.Tensor:
    """Y = X W^T (+ bias) under the LLM.int8 decomposition (see include/w8mp.h).
    With `producer`, x is the producer's input H and X = producer(H) is made in
    the quantisation pass (int8_mixed_linear_fused)."""
    _dev(x, "x"), _dev(wq, "wq"), _dev(sw, "sw")
    M, K = x.shape
    N = wq.shape[0]
    if wq.shape[1] != K or wq.dtype != torch.int8 or sw.shape != (N,) or sw.dtype != torch.float32:
        raise ValueError("wq must be int8 [N,K] and sw fp32 [N]")
    if bias is not None:
        _dev(bias, "bias")
        if bias.shape != (N,) or bias.dtype != torch.float32:
            raise ValueError("bias must be fp32 [N]")
    y = out if out is not None else torch.empty((M, N), dtype=out_dtype, device=x.device)
    need = int8_mixed_linear_workspace_size(M, N, K)
    ws = workspace if workspace is not None else _workspace(need, x.device)
    if bias is None and producer is None:
        _abi.check(lib().int8_mixed_linear(x.data_ptr(), _dt(x), M, K, wq.data_ptr(), sw.data_ptr(), N,
                                           float(threshold), y.data_ptr(), _dt(y), ws.data_ptr(), ws.numel(),
                                           _stream(x)))
    else:
        _abi.check(lib().int8_mixed_linear_fused(x.data_ptr(), _dt(x), M, K, _producer_arg(producer, K),
                                                 wq.data_ptr(), sw.data_ptr(),
                                                 bias.data_ptr() if bias is not None else None, N,
                                                 float(threshold), y.data_ptr(), _dt(y), ws.data_ptr(), ws.numel(),
                                                 _stream(x)))
    return y


def int8_mixed_linear_noalloc(x: torch.Tensor, wq: torch.Tensor, sw: torch.Tensor, threshold: float = 6.0,
                              out_dtype: torch.dtype = torch.float16, out: torch.Tensor | None = None) -> torch.Tensor:
    """int8_mixed_linear on the library's static device scratch: no workspace
    argument and no allocation inside the call (pass `out` to allocate nothing
    here either). Calls that may overlap on one device race (include/w8mp.h)."""
    _dev(x, "x"), _dev(wq, "wq"), _dev(sw, "sw")
    M, K = x.shape
    N = wq.shape[0]
    if wq.shape[1] != K or wq.dtype != torch.int8 or sw.shape != (N,) or sw.dtype != torch.float32:
        raise ValueError("wq must be int8 [N,K] and sw fp32 [N]")
    y = out if out is not None else torch.empty((M, N), dtype=out_dtype, device=x.device)
    _abi.check(lib().int8_mixed_linear_noalloc(x.data_ptr(), _dt(x), M, K, wq.data_ptr(), sw.data_ptr(), N,
                                               float(threshold), y.data_ptr(), _dt(y), _stream(x)))
    return y


def _events_arg(events):
    import ctypes

    if events is None:
        return None
    arr = (ctypes.c_void_p * 4)(*[int(e) if e else None for e in events])
    return arr


def debug_int8_gemm_timeline(x: torch.Tensor, wq: torch.Tensor, sw: torch.Tensor, threshold: float,
                             out: torch.Tensor, workspace: torch.Tensor) -> dict:
    """int8_mixed_linear with its GEMM launch's per-block timeline (see
    w8dbg_int8_gemm_timeline in include/w8mp.h). Returns {"stamps": int64
    [blocks, 8] on the host (unwritten words -1), "grid": blocks, "dp_tiles":
    blocks that own whole 256x256 tiles, "rest": what the other blocks are
    ("split", "small" or "streamk")}."""
    import ctypes

    M, K = x.shape
    N = wq.shape[0]
    g = (ctypes.c_int * 4)()
    args = (x.data_ptr(), _dt(x), M, K, wq.data_ptr(), sw.data_ptr(), N, float(threshold), out.data_ptr(), _dt(out),
            workspace.data_ptr(), workspace.numel())
    _abi.check(lib().w8dbg_int8_gemm_timeline(*args, None, 0, g, _stream(x)))
    if g[2] != 1:
        raise W8Error(_abi.W8_ERR_UNSUPPORTED, "the timeline needs K % 64 == 0")
    stamps = torch.full((g[0], 8), -1, dtype=torch.int64, device=x.device)
    _abi.check(lib().w8dbg_int8_gemm_timeline(*args, stamps.data_ptr(), stamps.numel(), g, _stream(x)))
    return {"stamps": stamps.cpu().numpy(), "grid": int(g[0]), "dp_tiles": int(g[1]),
            "rest": ("split", "small", "streamk")[g[3]]}


def debug_int8_mixed_linear_events(x: torch.Tensor, wq: torch.Tensor, sw: torch.Tensor, threshold: float, events,
                                   out: torch.Tensor, workspace: torch.Tensor, bias: torch.Tensor | None = None,
                                   producer: Producer | None = None) -> torch.Tensor:
    """int8_mixed_linear_fused that also records the four HIP events `events`
    (raw hipEvent_t handles) on its stream: before the row pass and after the
    row pass, the fix-up and the GEMM."""
    M, K = x.shape
    N = wq.shape[0]
    _abi.check(lib().w8dbg_int8_mixed_linear_events(
        x.data_ptr(), _dt(x), M, K, _producer_arg(producer, K), wq.data_ptr(), sw.data_ptr(),
        bias.data_ptr() if bias is not None else None, N, float(threshold), out.data_ptr(), _dt(out),
        workspace.data_ptr(), workspace.numel(), _events_arg(events), _stream(x)))
    return out


def debug_int8_mixed_linear_plan(x: torch.Tensor, wq: torch.Tensor, sw: torch.Tensor, threshold: float, cus: int,
                                 out: torch.Tensor, bias: torch.Tensor | None = None,
                                 producer: Producer | None = None) -> torch.Tensor:
    """int8_mixed_linear_fused with the GEMM grid planned for `cus` compute
    units (w8dbg_int8_mixed_linear_plan in include/w8mp.h); a fresh zeroed
    workspace."""
    M, K = x.shape
    N = wq.shape[0]
    ws = new_workspace(lib().w8dbg_int8_mixed_linear_plan_workspace_size(M, N, K, int(cus)), x.device)
    _abi.check(lib().w8dbg_int8_mixed_linear_plan(
        x.data_ptr(), _dt(x), M, K, _producer_arg(producer, K), wq.data_ptr(), sw.data_ptr(),
        bias.data_ptr() if bias is not None else None, N, float(threshold), out.data_ptr(), _dt(out),
        ws.data_ptr(), ws.numel(), int(cus), _stream(x)))
    return out


def debug_fp8_w8a8_linear_events(x: torch.Tensor, wq8: torch.Tensor, sw: torch.Tensor, act_scale, events,
                                 out: torch.Tensor, workspace: torch.Tensor) -> torch.Tensor:
    """fp8_w8a8_linear that records `events` (before the activation pass, after
    it twice, after the GEMM)."""
    M, K = x.shape
    N = wq8.shape[0]
    sp = 0 if act_scale is None else act_scale.data_ptr()
    _abi.check(lib().w8dbg_fp8_w8a8_linear_events(x.data_ptr(), _dt(x), M, K, wq8.data_ptr(), sw.data_ptr(), N, sp,
                                                  out.data_ptr(), _dt(out), workspace.data_ptr(), workspace.numel(),
                                                  _events_arg(events), _stream(x)))
    return out


def fp8_w8a8_linear(x: torch.Tensor, wq8: torch.Tensor, sw: torch.Tensor, act_scale: torch.Tensor | None = None,
                    out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
                    workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Y = X W^T with E4M3 weights and activations (see include/w8mp.h).
    act_scale: None (dynamic per token) or a one-element fp32 GPU tensor."""
    _dev(x, "x"), _dev(wq8, "wq8"), _dev(sw, "sw")
    M, K = x.shape
    N = wq8.shape[0]
    y = out if out is not None else torch.empty((M, N), dtype=out_dtype, device=x.device)
    need = fp8_w8a8_linear_workspace_size(M, N, K)
    ws = workspace if workspace is not None else _workspace(need, x.device)
    sp = 0 if act_scale is None else _dev(act_scale, "act_scale").data_ptr()
    _abi.check(lib().fp8_w8a8_linear(x.data_ptr(), _dt(x), M, K, wq8.data_ptr(), sw.data_ptr(), N, sp,
                                     y.data_ptr(), _dt(y), ws.data_ptr(), ws.numel(), _stream(x)))
    return y


def fp8_w8a16_linear(x: torch.Tensor, wq8: torch.Tensor, sw: torch.Tensor, out_dtype: torch.dtype = torch.bfloat16,
                     out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Y = X W_deq^T, W_deq = bf16(E4M3 value * channel scale), bf16 compute
    (weight-only FP8; see include/w8mp.h). x must be bf16."""
    _dev(x, "x"), _dev(wq8, "wq8"), _dev(sw, "sw")
    M, K = x.shape
    N = wq8.shape[0]
    y = out if out is not None else torch.empty((M, N), dtype=out_dtype, device=x.device)
    ws = workspace if workspace is not None else _workspace(fp8_w8a16_linear_workspace_size(M, N, K), x.device)
    _abi.check(lib().fp8_w8a16_linear(x.data_ptr(), _dt(x), M, K, wq8.data_ptr(), sw.data_ptr(), N, y.data_ptr(),
                                      _dt(y), ws.data_ptr(), ws.numel(), _stream(x)))
    return y


def w4a8_linear_workspace_size(M: int, N: int, K: int) -> int:
    return int(lib().w4a8_linear_workspace_size(M, N, K))


def w4a8_linear(x: torch.Tensor, wq4: torch.Tensor, sw4: torch.Tensor, out_dtype: torch.dtype = torch.float16,
                out: torch.Tensor | None = None, workspace: torch.Tensor | None = None, split: int | None = None
                ) -> torch.Tensor:
    """Y = X W^T with int4 per-group weights (quantize_weight_rowwise(w,
    "int4")) and int8 per-token activations. `split`: force the number of
    K-slices (parity export), None for the library's choice."""
    _dev(x, "x"), _dev(wq4, "wq4"), _dev(sw4, "sw4")
    M, K = x.shape
    N = wq4.shape[0]
    y = out if out is not None else torch.empty((M, N), dtype=out_dtype, device=x.device)
    if split is None:
        ws = workspace if workspace is not None else _workspace(w4a8_linear_workspace_size(M, N, K), x.device)
        _abi.check(lib().w4a8_linear(x.data_ptr(), _dt(x), M, K, wq4.data_ptr(), sw4.data_ptr(), N, y.data_ptr(),
                                     _dt(y), ws.data_ptr(), ws.numel(), _stream(x)))
    else:
        n_ws = int(lib().w8dbg_w4a8_linear_workspace_size(M, N, K, int(split)))
        ws = workspace if workspace is not None else _workspace(n_ws, x.device)
        _abi.check(lib().w8dbg_w4a8_linear(x.data_ptr(), _dt(x), M, K, wq4.data_ptr(), sw4.data_ptr(), N,
                                           int(split), y.data_ptr(), _dt(y), ws.data_ptr(), ws.numel(), _stream(x)))
    return y


class DitBlock:
    """One DiT block's quantized linears chained by the library's driver
    (w8_dit_block_forward in include/w8mp.h): QKV after RMSNorm1, an attention
    stub (each token's value vector), the output projection, residual, MLP up
    after RMSNorm2, GELU, MLP down (int8, or fp16 with `w_down16` for a
    massive-activation writer), residual. fp16 activations; int8 weights and
    scales from quantize_weight_rowwise; biases fp32 or None; norms are
    Producer("rmsnorm", ...) or None."""

    def __init__(self, D: int, F: int, w_qkv, s_qkv, w_o, s_o, w_up, s_up, w_down=None, s_down=None, b_qkv=None,
                 b_o=None, b_up=None, b_down=None, norm1: Producer | None = None, norm2: Producer | None = None,
                 w_down16: torch.Tensor | None = None, threshold: float = 6.0):
        self.D, self.F = int(D), int(F)
        self.t = dict(qkv=(w_qkv, s_qkv, b_qkv), o=(w_o, s_o, b_o), up=(w_up, s_up, b_up), down=(w_down, s_down, b_down))
        for name, trio in self.t.items():
            for v in trio:
                if v is not None:
                    _dev(v, name)
        if w_down16 is not None:
            _dev(w_down16, "w_down16")
            if w_down16.dtype != torch.float16 or tuple(w_down16.shape) != (self.D, self.F):
                raise ValueError("w_down16 must be fp16 [D, F]")
        self.w_down16 = w_down16
        self.norm1, self.norm2, self.threshold = norm1, norm2, float(threshold)
        ptr = lambda v: v.data_ptr() if v is not None else None
        none = Producer("none")
        self._s = _abi.DitBlock(self.D, self.F, self.threshold,
                                *[ptr(v) for n in ("qkv", "o", "up", "down") for v in self.t[n]],
                                ptr(w_down16), (norm1 or none).struct(self.D), (norm2 or none).struct(self.D))

    def workspace_size(self, M: int) -> int:
        return int(lib().w8_dit_block_workspace_size(M, self.D, self.F))

    def intermediates(self, workspace: torch.Tensor, M: int) -> dict:
        """Views of the block's intermediates in `workspace` after forward()
        (parity export): qkv, a, o, h, u as fp16 [M, .]; d as fp16 [M, D], or
        fp32 with the 16-bit down-projection, which also writes g = GELU(u)."""
        import ctypes

        v = (ctypes.c_size_t * 7)()
        _abi.check(lib().w8dbg_dit_block_layout(M, self.D, self.F, v))
        off = dict(zip(["qkv", "a", "o", "h", "u", "g", "d"], [int(x) for x in v]))
        D, F = self.D, self.F
        cols = dict(qkv=3 * D, a=D, o=D, h=D, u=F, g=F)

        def view(name, n, dtype, esize):
            b = workspace[off[name]: off[name] + M * n * esize]
            return b.view(dtype).view(M, n)

        out = {k: view(k, n, torch.float16, 2) for k, n in cols.items()}
        out["d"] = view("d", D, torch.float32, 4) if self.w_down16 is not None else view("d", D, torch.float16, 2)
        return out

    def forward(self, x: torch.Tensor, out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None) -> torch.Tensor:
        import ctypes

        _dev(x, "x")
        if x.dtype != torch.float16 or x.dim() != 2 or x.shape[1] != self.D:
            raise ValueError("x must be fp16 [M, D]")
        M = x.shape[0]
        y = out if out is not None else torch.empty_like(x)
        ws = workspace if workspace is not None else _workspace(self.workspace_size(M), x.device)
        _abi.check(lib().w8_dit_block_forward(ctypes.byref(self._s), x.data_ptr(), M, y.data_ptr(), ws.data_ptr(),
                                              ws.numel(), _stream(x)))
        return y


def debug_linear16(x: torch.Tensor, w: torch.Tensor, split: int = 0, out_dtype: torch.dtype = torch.float32,
                   workspace: torch.Tensor | None = None, tile: int = 128) -> torch.Tensor:
    """The block driver's plain 16-bit linear: Y = X W^T (x and w both fp16
    or both bf16). split 0: the driver's own tiling; else tile 128: 128x128
    blocks each in `split` K-slices; tile 256: 256x256 blocks with the last
    partial wave's tiles in `split` K-slices."""
    _dev(x, "x"), _dev(w, "w")
    M, K = x.shape
    N = w.shape[0]
    if w.dtype != x.dtype or w.shape[1] != K:
        raise ValueError("w must be [N, K] of x's dtype")
    y = torch.empty((M, N), dtype=out_dtype, device=x.device)
    n_ws = int(lib().w8dbg_linear16_workspace_size(M, N, K, int(split), int(tile)))
    ws = workspace if workspace is not None else _workspace(n_ws, x.device)
    _abi.check(lib().w8dbg_linear16(x.data_ptr(), _dt(x), M, K, w.data_ptr(), N, int(split), int(tile), y.data_ptr(),
                                    _dt(y),
                                    ws.data_ptr(), ws.numel(), _stream(x)))
    return y


def debug_fp8_w8a16_linear(x: torch.Tensor, wq8: torch.Tensor, sw: torch.Tensor, split: int = 0, tile: int = 0,
                           out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
                           workspace: torch.Tensor | None = None) -> torch.Tensor:
    """fp8_w8a16_linear with `tile` x `tile` output blocks and `split`
    K-slices (split 0: the linear's own choice)."""
    _dev(x, "x"), _dev(wq8, "wq8"), _dev(sw, "sw")
    M, K = x.shape
    N = wq8.shape[0]
    y = out if out is not None else torch.empty((M, N), dtype=out_dtype, device=x.device)
    n_ws = int(lib().w8dbg_fp8_w8a16_linear_workspace_size(M, N, K, int(split), int(tile)))
    ws = workspace if workspace is not None else _workspace(n_ws, x.device)
    _abi.check(lib().w8dbg_fp8_w8a16_linear(x.data_ptr(), _dt(x), M, K, wq8.data_ptr(), sw.data_ptr(), N, int(split),
                                            int(tile), y.data_ptr(), _dt(y), ws.data_ptr(), ws.numel(), _stream(x)))
    return y


def debug_int8_quantize_activations(x: torch.Tensor, threshold: float = 6.0, producer: Producer | None = None,
                                    with_rstd: bool = False):
    """(q int8 [M,K], sx fp32 [M], outlier column indices int32 [nO]) of X, or of
    X = producer(x); with_rstd adds the RMSNorm producer's per-row rstd [M]."""
    _dev(x, "x")
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.int8, device=x.device)
    sx = torch.empty((M,), dtype=torch.float32, device=x.device)
    idx = torch.empty((K,), dtype=torch.int32, device=x.device)
    n = torch.empty((1,), dtype=torch.int32, device=x.device)
    ws = _workspace(int(lib().w8dbg_int8_quantize_activations_workspace_size(M, K)), x.device)
    _abi.check(lib().w8dbg_int8_quantize_activations(x.data_ptr(), _dt(x), M, K, _producer_arg(producer, K),
                                                     float(threshold), q.data_ptr(), sx.data_ptr(), idx.data_ptr(),
                                                     n.data_ptr(), ws.data_ptr(), ws.numel(), _stream(x)))
    if with_rstd:
        # the rstd region follows the workspace's common front (counters, flags)
        front = int8_workspace_layout(M, 1, K)["nO"]
        rstd = ws[front: front + 4 * M].view(torch.float32).clone()
        return q, sx, idx[: int(n.item())], rstd
    return q, sx, idx[: int(n.item())]


def debug_produce(h: torch.Tensor, producer: Producer) -> torch.Tensor:
    """X = producer(H), [M,K] in H's 16-bit type."""
    _dev(h, "h")
    M, K = h.shape
    x = torch.empty_like(h)
    _abi.check(lib().w8dbg_produce(h.data_ptr(), _dt(h), M, K, _producer_arg(producer, K), x.data_ptr(),
                                   _stream(h)))
    return x


def debug_int8_gemm_i32(q: torch.Tensor, wq: torch.Tensor, tail: int = 0, split: int = 1,
                        workspace: torch.Tensor | None = None) -> torch.Tensor:
    """acc [M,N] int32 = q . wq^T on the int8 MFMA kernel. tail 0: the linear's
    own grid; 1: leftover tiles as `split` 256x256 K-slices (1: all whole);
    2: as `split` K-slices of 128x128 quarters; 3: stream-K over the last full
    wave and the leftover tiles (see include/w8mp.h)."""
    _dev(q, "q"), _dev(wq, "wq")
    M, K = q.shape
    N = wq.shape[0]
    acc = torch.empty((M, N), dtype=torch.int32, device=q.device)
    n_ws = debug_int8_gemm_i32_workspace_size(M, N, K, tail, split)
    ws = workspace if workspace is not None else (_workspace(n_ws, q.device) if n_ws else None)
    _abi.check(lib().w8dbg_int8_gemm_i32(q.data_ptr(), wq.data_ptr(), M, N, K, int(tail), int(split), acc.data_ptr(),
                                         ws.data_ptr() if ws is not None else None,
                                         ws.numel() if ws is not None else 0, _stream(q)))
    return acc


def debug_int8_gemm_i32_workspace_size(M: int, N: int, K: int, tail: int = 0, split: int = 1) -> int:
    return int(lib().w8dbg_int8_gemm_i32_workspace_size(M, N, K, int(tail), int(split)))


def debug_mfma_peak(kind: str, blocks: int, iters: int, device="cuda"):
    """Launch the measured-peak MFMA kernel ("int8", "fp8" or "bf16" on
    constant operands; "int8_random", "fp8_random" on operands that change
    every round) on the current stream; returns (checksum tensor, operations
    launched). The caller times it."""
    import ctypes

    k = {"int8": 0, "fp8": 1, "bf16": 2, "int8_random": 3, "fp8_random": 4}[kind]
    out = torch.empty(blocks * 256, dtype=torch.int32, device=device)
    ops = ctypes.c_double()
    _abi.check(lib().w8dbg_mfma_peak(k, int(blocks), int(iters), out.data_ptr(), ctypes.byref(ops),
                                     torch.cuda.current_stream(out.device).cuda_stream))
    return out, ops.value


def debug_cvt_f16_pair_check(device="cuda") -> dict:
    """The packed float32 -> fp16 conversion against the scalar one over every
    float32 bit pattern (w8dbg_cvt_f16_pair_check in include/w8mp.h)."""
    out = torch.tensor([0, 0, -1], dtype=torch.int32, device=device)
    _abi.check(lib().w8dbg_cvt_f16_pair_check(out.data_ptr(), _stream(out)))
    o = [v & 0xFFFFFFFF for v in out.cpu().tolist()]
    return {"mismatch": o[0], "mismatch_nan": o[1], "first": o[2]}


def debug_lds_stream(buf: torch.Tensor, K: int, seg: int, blocks: int, panels: int, iters: int):
    """Launch the operand-streaming kernel (w8dbg_lds_stream in include/w8mp.h)
    over the device buffer `buf` on the current stream; returns (checksum
    tensor, bytes moved). The caller times it."""
    import ctypes

    out = torch.empty(blocks, dtype=torch.int32, device=buf.device)
    nbytes = ctypes.c_double()
    _abi.check(lib().w8dbg_lds_stream(buf.data_ptr(), buf.numel() * buf.element_size(), int(K), int(seg),
                                      int(blocks), int(panels), int(iters), out.data_ptr(), ctypes.byref(nbytes),
                                      torch.cuda.current_stream(buf.device).cuda_stream))
    return out, nbytes.value


def debug_fp8_quantize_activations(x: torch.Tensor, act_scale: torch.Tensor | None = None):
    """(E4M3 codes uint8 [M,K], sx fp32 [M])."""
    _dev(x, "x")
    M, K = x.shape
    xq = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    sx = torch.empty((M,), dtype=torch.float32, device=x.device)
    sp = 0 if act_scale is None else _dev(act_scale, "act_scale").data_ptr()
    _abi.check(lib().w8dbg_fp8_quantize_activations(x.data_ptr(), _dt(x), M, K, sp, xq.data_ptr(), sx.data_ptr(),
                                                    _stream(x)))
    return xq, sx


def debug_fp8_gemm(xq: torch.Tensor, sx: torch.Tensor, wq8: torch.Tensor, sw: torch.Tensor, split: int = 0,
                   tile: int = 0, out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Y [M,N] = sx[m] sw[n] (xq . wq8^T) on the FP8 MFMA kernel: `tile` x
    `tile` output blocks with `split` K-slices each (split 0: the linear's own
    choice of both)."""
    _dev(xq, "xq"), _dev(sx, "sx"), _dev(wq8, "wq8"), _dev(sw, "sw")
    M, K = xq.shape
    N = wq8.shape[0]
    y = out if out is not None else torch.empty((M, N), dtype=out_dtype, device=xq.device)
    n_ws = debug_fp8_gemm_workspace_size(M, N, K, split, tile)
    ws = workspace if workspace is not None else (_workspace(n_ws, xq.device) if n_ws else None)
    _abi.check(lib().w8dbg_fp8_gemm(xq.data_ptr(), sx.data_ptr(), wq8.data_ptr(), sw.data_ptr(), M, N, K,
                                    int(split), int(tile), y.data_ptr(), _dt(y),
                                    ws.data_ptr() if ws is not None else None,
                                    ws.numel() if ws is not None else 0, _stream(xq)))
    return y


def debug_fp8_gemm_workspace_size(M: int, N: int, K: int, split: int = 0, tile: int = 0) -> int:
    return int(lib().w8dbg_fp8_gemm_workspace_size(M, N, K, int(split), int(tile)))
