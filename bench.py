"""Throughput of the LLM.int8 mixed-precision linear on one MI355X.

One step = the three quantized linears of one DiT block at 1024^2
(4096 image + 256 text tokens): attention QKV 4352x4096 -> 12288, MLP up
4352x4096 -> 16384, MLP down 4352x16384 -> 4096, each a full
int8_mixed_linear call (outlier detection, row scales, int8 codes, outlier
fix-up and gather, int8 MFMA GEMM with the fused 16-bit outlier product and
dequant epilogue), threshold 6.0, bf16 in, fp16 out. Weights are quantized
once before timing (the model cards store INT8 weights and never re-quantise
them). Inputs are seeded synthetic activations with the massive-activation
and outlier-column structure of the pages, resident in HBM before timing.

Prints one JSON line. `value` is TOPS = sum(2 M N K) / time.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "int8 mixed-precision linear TOPS at 1024^2 DiT shapes; % of MFMA peak"
PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA, published
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense fp8 MFMA, published
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, published
THRESHOLD = 6.0


class HipEvents:
    """A pool of HIP events (host objects made with hipEventCreate through
    ctypes) for the library's event-recording exports, which record them on
    the stream their kernels run on."""

    def __init__(self, n: int):
        import ctypes

        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(e.value)

    def group(self, i: int, k: int = 4):
        return self.ev[k * i: k * i + k]

    def ms(self, a, b) -> float:
        t = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(t), self.ct.c_void_p(a), self.ct.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(t.value)

    def sync(self, e) -> None:
        self.hip.hipEventSynchronize(self.ct.c_void_p(e))

    def close(self) -> None:
        for e in self.ev:
            self.hip.hipEventDestroy(self.ct.c_void_p(e))
        self.ev = []


def staged_int8(w8, ev, args_list, steps: int):
    """`steps` rounds over the calls in args_list (x, wq, sw, y, ws), each call
    recording 4 events (start, after the row pass, after the fix-up, after the
    GEMM). Returns per call index a list of [row, fixup, gemm] ms per round."""
    n = len(args_list)
    for r in range(steps):
        for i, (x, wq, sw, y, ws) in enumerate(args_list):
            w8.debug_int8_mixed_linear_events(x, wq, sw, THRESHOLD, ev.group(r * n + i), y, ws)
    ev.sync(ev.ev[4 * steps * n - 1])
    out = [[] for _ in range(n)]
    for r in range(steps):
        for i in range(n):
            e = ev.group(r * n + i)
            out[i].append([ev.ms(e[0], e[1]), ev.ms(e[1], e[2]), ev.ms(e[2], e[3])])
    return out


def _median(v):
    import numpy as np

    return float(np.median(np.asarray(v, dtype=np.float64)))


def _call_ms(torch, fn, steps: int):
    """Per-call GPU time (ms) of `steps` calls of fn, each bracketed by events
    on torch's current stream (where the library launches)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    ev[-1][1].synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def _dev16(bits, torch):
    import numpy as np

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def gemm_algorithmic_ops(cases) -> float:
    return float(sum(c.ops for c in cases))


def cpu_baseline(cases, rows: int):
    """The oracle, as it stands, on the first `rows` token rows of each shape
    (the outlier set is still taken over all rows)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import w8ref as o

    prepared = []
    for c in cases:
        wq, sw = o.quantize_weight_int8(o.decode16(c.w_bits, "bf16"))   # offline, not timed
        prepared.append((c, wq, sw))
    sel = np.arange(rows)
    t0 = time.perf_counter()
    ops = 0
    for c, wq, sw in prepared:
        o.int8_mixed_linear(c.x_bits, "bf16", wq, sw, THRESHOLD, "f16", rows=sel)
        ops += 2 * rows * c.N * c.K
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": int(threads), "kind": "oracle",
            "sample": f"token rows 0..{rows - 1} of each of the 3 shapes (outlier set over all 4352 rows); "
                      f"{ops / 1e9:.1f} G ops in {dt:.1f} s"}


def fp8_layers(torch, w8, steps: int) -> dict:
    """FP8-E4M3 W8A8 linears, per layer and activation-scale mode: medians over
    `steps` calls of the whole call, the activation pass and the GEMM, from
    HIP events the library records between its kernels; GEMM TFLOP/s and the
    GEMM's fraction of its roofline max(2MNK / 5.0 PFLOP/s, bytes / 8 TB/s),
    bytes = M K + N K + 2 M N. The 512-token text-encoder layers, and the DiT
    1024^2 QKV and MLP-up shapes (4352 tokens) under a static per-tensor scale
    (the ModelOpt FP8 card's DiT recipe)."""
    import synth

    res = {}
    cases = [(synth.fp8_text_encoder(layer), ("dynamic", "static")) for layer in synth.FP8_TEXT_LAYERS]
    cases += [(synth.dit_qkv_1024(), ("static",)), (synth.dit_mlp_1024("up"), ("static",))]
    ev = HipEvents(4 * steps)
    for c, modes in cases:
        x = _dev16(c.x_bits, torch)
        wq, sw = w8.quantize_weight_rowwise(_dev16(c.w_bits, torch), "fp8")
        y = torch.empty((c.M, c.N), dtype=torch.bfloat16, device="cuda")
        ws = w8.new_workspace(w8.fp8_w8a8_linear_workspace_size(c.M, c.N, c.K))
        # static per-tensor input scale: "max" calibration on an independent draw
        cal = c.extra["x_cal_bits"] if "x_cal_bits" in c.extra else synth.calibration_draw(c.M, c.K, seed=3001)
        xcal = _dev16(cal, torch).float()
        scale = (xcal.abs().max() / 448.0).reshape(1).contiguous()
        del xcal
        for mode in modes:
            act = scale if mode == "static" else None
            for _ in range(3):
                w8.fp8_w8a8_linear(x, wq, sw, act, out=y, workspace=ws)
            for i in range(steps):
                w8.debug_fp8_w8a8_linear_events(x, wq, sw, act, ev.group(i), y, ws)
            ev.sync(ev.ev[4 * steps - 1])
            st = [[ev.ms(e[0], e[1]), ev.ms(e[2], e[3])] for e in (ev.group(i) for i in range(steps))]
            rows_us = _median([a for a, _ in st]) * 1e3
            gemm_us = _median([b for _, b in st]) * 1e3
            gbytes = c.M * c.K + c.N * c.K + 2 * c.M * c.N
            t_roof = max(c.ops / (PEAK_FP8_TFLOPS * 1e12), gbytes / (PEAK_HBM_GBS * 1e9)) * 1e6
            key = f"{c.name}_{mode}"
            res[key] = {
                "call_us": round(_median([a + b for a, b in st]) * 1e3, 2),
                "act_quant_us": round(rows_us, 2),
                "act_quant_GBs": round(3 * c.M * c.K / (rows_us * 1e-6) / 1e9, 1),
                "gemm_us": round(gemm_us, 2),
                "gemm_tflops": round(c.ops / (gemm_us * 1e-6) / 1e12, 1),
                "gemm_pct_fp8_peak": round(100 * c.ops / (gemm_us * 1e-6) / 1e12 / PEAK_FP8_TFLOPS, 2),
                "gemm_roofline_us": round(t_roof, 2),
                "gemm_roofline_frac": round(t_roof / gemm_us, 3),
            }
            print(f"[bench] fp8 {key}: {res[key]}", file=sys.stderr, flush=True)
        del x, wq, y, ws
    ev.close()
    return res


def w8a16_layers(torch, w8, steps: int) -> dict:
    """FP8 weight-only (W8A16) text-encoder linears at 512 tokens: median GEMM
    time from events around each call (the call is the one GEMM kernel), TFLOP/s
    and the fraction of its roofline max(2MNK / 2.5 PFLOP/s bf16,
    bytes / 8 TB/s), bytes = 2 M K + N K + 2 M N (bf16 X, E4M3 W, bf16 Y)."""
    import synth

    res = {}
    for layer in synth.FP8_TEXT_LAYERS:
        c = synth.fp8_text_encoder(layer)
        x = _dev16(c.x_bits, torch)
        wq, sw = w8.quantize_weight_rowwise(_dev16(c.w_bits, torch), "fp8")
        y = torch.empty((c.M, c.N), dtype=torch.bfloat16, device="cuda")
        ws = w8.new_workspace(w8.fp8_w8a16_linear_workspace_size(c.M, c.N, c.K))
        for _ in range(3):
            w8.fp8_w8a16_linear(x, wq, sw, out=y, workspace=ws)
        gemm_us = _median(_call_ms(torch, lambda: w8.fp8_w8a16_linear(x, wq, sw, out=y, workspace=ws), steps)) * 1e3
        gbytes = 2 * c.M * c.K + c.N * c.K + 2 * c.M * c.N
        t_roof = max(c.ops / (PEAK_BF16_TFLOPS * 1e12), gbytes / (PEAK_HBM_GBS * 1e9)) * 1e6
        key = f"{layer}_{c.M}x{c.K}x{c.N}"
        res[key] = {
            "gemm_us": round(gemm_us, 2),
            "gemm_tflops": round(c.ops / (gemm_us * 1e-6) / 1e12, 1),
            "gemm_roofline_us": round(t_roof, 2),
            "gemm_roofline_frac": round(t_roof / gemm_us, 3),
        }
        print(f"[bench] w8a16 {layer}: {res[key]}", file=sys.stderr, flush=True)
    return res


def w4a8_layers(torch, w8, steps: int) -> dict:
    """W4A8 (int4 per-group weights, int8 per-token activations) on the
    512-token text-encoder shapes: median whole-call time (activation pass and
    GEMM) from events around each call, TOPS and its fraction of the roofline
    max(2MNK / 5.0 POPS int8, bytes / 8 TB/s), bytes = M K + N K / 2 + 2 M N
    + 4 N K / 128 (codes, packed weights, fp16 Y, group scales)."""
    import synth

    res = {}
    for layer in synth.FP8_TEXT_LAYERS:
        c = synth.fp8_text_encoder(layer)
        x = _dev16(c.x_bits, torch)
        wq, sw = w8.quantize_weight_rowwise(_dev16(c.w_bits, torch), "int4")
        y = torch.empty((c.M, c.N), dtype=torch.float16, device="cuda")
        ws = w8.new_workspace(w8.w4a8_linear_workspace_size(c.M, c.N, c.K))
        for _ in range(3):
            w8.w4a8_linear(x, wq, sw, out=y, workspace=ws)
        call_us = _median(_call_ms(torch, lambda: w8.w4a8_linear(x, wq, sw, out=y, workspace=ws), steps)) * 1e3
        gbytes = c.M * c.K + c.N * c.K // 2 + 2 * c.M * c.N + 4 * c.N * c.K // 128
        t_roof = max(c.ops / (PEAK_INT8_TOPS * 1e12), gbytes / (PEAK_HBM_GBS * 1e9)) * 1e6
        key = f"{layer}_{c.M}x{c.K}x{c.N}"
        res[key] = {
            "call_us": round(call_us, 2),
            "call_tops": round(c.ops / (call_us * 1e-6) / 1e12, 1),
            "roofline_us": round(t_roof, 2),
            "call_roofline_frac": round(t_roof / call_us, 3),
        }
        print(f"[bench] w4a8 {layer}: {res[key]}", file=sys.stderr, flush=True)
    return res


def dit_block(torch, w8, steps: int) -> dict:
    """One DiT 1024^2 block through the library's driver (M = 4352 tokens,
    D = 4096, F = 16384: QKV, attention stub, output projection, residual, MLP
    up after RMSNorm, GELU, MLP down, residual), with the MLP down-projection
    int8 or kept in fp16 as a massive-activation writer. Time per block from
    events on the launch stream, and the block's linears' ops per second."""
    g = torch.Generator(device="cuda").manual_seed(11)
    M, D, F = 4352, 4096, 16384
    x = torch.randn(M, D, device="cuda", generator=g)
    x[4096::32, 2276] = 9000.0
    x = x.to(torch.float16)

    def lin(n, k):
        w = (torch.randn(n, k, device="cuda", generator=g) * 0.02).to(torch.float16)
        b = torch.randn(n, device="cuda", generator=g) * 0.1
        wq, sw = w8.quantize_weight_rowwise(w, "int8")
        return wq, sw, b, w

    qkv, o_, up, down = lin(3 * D, D), lin(D, D), lin(F, D), lin(D, F)
    norm = lambda: w8.Producer("rmsnorm", torch.rand(D, device="cuda", generator=g) * 0.4 + 0.8)
    ops = 2.0 * M * D * (3 * D + D + F) + 2.0 * M * F * D
    res = {}
    for name, with16 in (("int8_down", False), ("fp16_down", True)):
        blk = w8.DitBlock(D, F, qkv[0], qkv[1], o_[0], o_[1], up[0], up[1],
                          w_down=None if with16 else down[0], s_down=None if with16 else down[1],
                          b_qkv=qkv[2], b_o=o_[2], b_up=up[2], b_down=down[2], norm1=norm(), norm2=norm(),
                          w_down16=down[3] if with16 else None)
        y = torch.empty_like(x)
        ws = w8.new_workspace(blk.workspace_size(M))
        for _ in range(2):
            blk.forward(x, out=y, workspace=ws)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            blk.forward(x, out=y, workspace=ws)
        e1.record()
        e1.synchronize()
        us = e0.elapsed_time(e1) / steps * 1e3
        res[name] = {"us_per_block": round(us, 1), "linear_tops": round(ops / (us * 1e-6) / 1e12, 1)}
        print(f"[bench] dit block {name}: {res[name]}", file=sys.stderr, flush=True)
        del ws, blk
    return res


def weight_quant(torch, w8, cases, steps: int) -> dict:
    """Offline weight quantisation (int8 rowwise and FP8 per-channel) on the
    step's weights: time per call from events on the stream the kernels run on
    (torch's current stream), and HBM GB/s against 3 N K bytes (read 16-bit W,
    write 8-bit codes)."""
    res = {}
    for c in cases:
        w = _dev16(c.w_bits, torch)
        for fmt in ("int8", "fp8"):
            w8.quantize_weight_rowwise(w, fmt)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                w8.quantize_weight_rowwise(w, fmt)
            e1.record()
            e1.synchronize()
            us = e0.elapsed_time(e1) / steps * 1e3
            gbs = 3 * c.N * c.K / (us * 1e-6) / 1e9
            res[f"{fmt}_{c.N}x{c.K}"] = {"us": round(us, 2), "GBs": round(gbs, 1),
                                         "hbm_frac": round(gbs / PEAK_HBM_GBS, 3)}
        del w
    print(f"[bench] weight quantisation: {res}", file=sys.stderr, flush=True)
    return res


def fused_mlp(torch, w8, steps: int) -> dict:
    """DiT 1024^2 MLP pair with its producers (up after RMSNorm+modulation,
    down after tanh-GELU), bias in the epilogue. Fused: one
    int8_mixed_linear_fused call per layer. Unfused: the library's one-pass
    producer kernel writes X, then the linear reads it. Both timed with events
    on the launch stream over `steps` calls, alternating, best of 3 rounds; the
    fused call's stages (medians) from HIP events the library records between
    its kernels."""
    import synth

    res = {}
    for c in synth.dit_mlp_fused_1024():
        h = _dev16(c.h_bits, torch)
        wq, sw = w8.quantize_weight_rowwise(_dev16(c.w_bits, torch), "int8")
        bias = torch.from_numpy(c.bias).cuda()
        if c.kind == "rmsnorm":
            t = lambda v: torch.from_numpy(v).cuda()
            prod = w8.Producer("rmsnorm", t(c.gamma), t(c.scale), t(c.shift), c.eps)
        else:
            prod = w8.Producer("gelu")
        y = torch.empty((c.M, c.N), dtype=torch.float16, device="cuda")
        ws = w8.new_workspace(w8.int8_mixed_linear_workspace_size(c.M, c.N, c.K))

        def fused():
            w8.int8_mixed_linear(h, wq, sw, THRESHOLD, out=y, workspace=ws, bias=bias, producer=prod)

        def unfused():
            w8.int8_mixed_linear(w8.debug_produce(h, prod), wq, sw, THRESHOLD, out=y, workspace=ws, bias=bias)

        out = {}
        for fn in (fused, unfused):
            for _ in range(3):
                fn()
        # the two variants alternate over 3 rounds (the clock drifts under a
        # long GEMM run); each keeps its fastest round
        for _ in range(3):
            for name, fn in (("fused", fused), ("unfused", unfused)):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(steps):
                    fn()
                e1.record()
                e1.synchronize()
                us = round(e0.elapsed_time(e1) / steps * 1e3, 2)
                out[f"{name}_us"] = min(us, out.get(f"{name}_us", us))
        ev = HipEvents(4 * steps)
        for i in range(steps):
            w8.debug_int8_mixed_linear_events(h, wq, sw, THRESHOLD, ev.group(i), y, ws, bias=bias, producer=prod)
        ev.sync(ev.ev[-1])
        st = [[ev.ms(e[0], e[1]), ev.ms(e[1], e[2]), ev.ms(e[2], e[3])] for e in (ev.group(i) for i in range(steps))]
        ev.close()
        out["fused_quant_us"] = round(_median([a for a, _, _ in st]) * 1e3, 2)
        out["fused_fixup_us"] = round(_median([b for _, b, _ in st]) * 1e3, 2)
        out["fused_gemm_us"] = round(_median([g for _, _, g in st]) * 1e3, 2)
        out["fused_quant_GBs"] = round(3 * c.M * c.K / (out["fused_quant_us"] * 1e-6) / 1e9, 1)
        # HBM bytes of the quantisation stage: fused reads H and writes codes;
        # unfused also writes X and reads it back
        out["quant_bytes_fused"] = 3 * c.M * c.K
        out["quant_bytes_unfused"] = 7 * c.M * c.K
        out["saved_us"] = round(out["unfused_us"] - out["fused_us"], 2)
        out["fused_tops"] = round(c.ops / (out["fused_us"] * 1e-6) / 1e12, 1)
        res[c.name] = out
        print(f"[bench] fused {c.name}: {out}", file=sys.stderr, flush=True)
        del h, y, ws, wq
    return res


def counter_workload(torch, w8, cases, steps: int, copy_mib: int) -> None:
    """Minimal run for hardware-counter collection: `steps` int8 steps (after
    one warm-up step), then three plain device copies of `copy_mib` MiB, the
    calibration for the byte counters (a copy reads and writes exactly that
    many bytes)."""
    xs, wqs, sws, ys, wss = _prepare(torch, w8, cases)
    for _ in range(1 + steps):
        for i in range(len(cases)):
            w8.int8_mixed_linear(xs[i], wqs[i], sws[i], THRESHOLD, out=ys[i], workspace=wss[i])
    torch.cuda.synchronize()
    n = copy_mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[bench] counter workload done: {steps} steps, 3 copies of {copy_mib} MiB", file=sys.stderr, flush=True)


def counter_workload_fp8(torch, w8, steps: int) -> None:
    """Minimal run for hardware-counter collection on the FP8 W8A8 linears: one
    warm-up call and `steps` calls per layer; the text-encoder linears at 512
    tokens (q, k, v, gate, up, down) with the dynamic per-token scale, then the
    DiT 1024^2 QKV and MLP-up shapes with a static per-tensor scale."""
    import synth

    cases = [(synth.fp8_text_encoder(layer), False) for layer in synth.FP8_TEXT_LAYERS]
    cases += [(synth.dit_qkv_1024(), True), (synth.dit_mlp_1024("up"), True)]
    for c, static in cases:
        x = _dev16(c.x_bits, torch)
        wq, sw = w8.quantize_weight_rowwise(_dev16(c.w_bits, torch), "fp8")
        y = torch.empty((c.M, c.N), dtype=torch.bfloat16, device="cuda")
        ws = w8.new_workspace(w8.fp8_w8a8_linear_workspace_size(c.M, c.N, c.K))
        act = None
        if static:
            act = (x.float().abs().max() / 448.0).reshape(1).contiguous()
        for _ in range(1 + steps):
            w8.fp8_w8a8_linear(x, wq, sw, act, out=y, workspace=ws)
        torch.cuda.synchronize()
        del x, wq, y, ws
    print(f"[bench] fp8 counter workload done: {steps} calls per layer", file=sys.stderr, flush=True)


def vendor_reference(torch, steps: int) -> dict:
    """The ROCm libraries behind torch on the same shapes, for context: plain
    int8 x int8 -> int32 products (torch._int_mm) on the DiT 1024^2 linears and
    FP8-E4M3 products with per-tensor scales and bf16 output (torch._scaled_mm)
    on the text-encoder linears at 512 tokens and the DiT 1024^2 linears. They
    compute less than the library's linears (no outlier decomposition, no row
    scales, no activation quantisation). Medians of `steps` calls, each timed
    with events on torch's stream; random operands (timing only)."""
    out = {"int8_mm": {}, "fp8_scaled_mm": {}}
    g = torch.Generator(device="cuda").manual_seed(7)

    def med(fn):
        for _ in range(3):
            fn()
        ts = []
        for _ in range(steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        return _median(ts)

    for M, K, N in [(4352, 4096, 12288), (4352, 4096, 16384), (4352, 16384, 4096)]:
        a = torch.randint(-127, 128, (M, K), dtype=torch.int8, device="cuda", generator=g)
        b = torch.randint(-127, 128, (N, K), dtype=torch.int8, device="cuda", generator=g)
        us = med(lambda: torch._int_mm(a, b.t()))
        out["int8_mm"][f"{M}x{K}x{N}"] = {"us": round(us, 2), "tops": round(2 * M * N * K / us / 1e6, 1)}
        print(f"[bench] vendor int8 {M}x{K}x{N}: {out['int8_mm'][f'{M}x{K}x{N}']}", file=sys.stderr, flush=True)
        del a, b
    one = torch.ones((), device="cuda")
    for M, K, N in [(512, 4096, 4096), (512, 4096, 1024), (512, 4096, 12288), (512, 12288, 4096),
                    (4352, 4096, 12288), (4352, 4096, 16384)]:
        x = torch.randn(M, K, device="cuda", generator=g).to(torch.float8_e4m3fn)
        w = torch.randn(N, K, device="cuda", generator=g).to(torch.float8_e4m3fn)
        us = med(lambda: torch._scaled_mm(x, w.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16))
        out["fp8_scaled_mm"][f"{M}x{K}x{N}"] = {"us": round(us, 2), "tflops": round(2 * M * N * K / us / 1e6, 1)}
        print(f"[bench] vendor fp8 {M}x{K}x{N}: {out['fp8_scaled_mm'][f'{M}x{K}x{N}']}", file=sys.stderr, flush=True)
        del x, w
    return out


def _prepare(torch, w8, cases):
    """Inputs resident in HBM, weights quantized once (untimed)."""
    xs, wqs, sws, ys, wss = [], [], [], [], []
    for c in cases:
        xs.append(_dev16(c.x_bits, torch))
        wq, sw = w8.quantize_weight_rowwise(_dev16(c.w_bits, torch), "int8")
        wqs.append(wq)
        sws.append(sw)
        ys.append(torch.empty((c.M, c.N), dtype=torch.float16, device="cuda"))
        wss.append(w8.new_workspace(w8.int8_mixed_linear_workspace_size(c.M, c.N, c.K)))
    torch.cuda.synchronize()
    return xs, wqs, sws, ys, wss


def recorded_traffic(w8) -> float | None:
    """HBM bytes per launch of the int8 GEMM from the committed counter record
    (profiles/k_int8_gemm_dit1024_traffic.md), or None when there is none or
    the GEMM sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "k_int8_gemm_dit1024_traffic.md")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if line.startswith("traffic_bytes_per_launch:") or line.startswith("sources_sha256:"):
            k, v = line.split(":", 1)
            rec[k] = v.strip()
    if "traffic_bytes_per_launch" not in rec or "sources_sha256" not in rec:
        return None
    if rec["sources_sha256"] != gemm_sources_sha256():
        return None
    return float(rec["traffic_bytes_per_launch"])


def gemm_sources_sha256() -> str:
    """Digest of the sources the int8 GEMM kernel is built from (its file, the
    headers it includes and the generator of the GELU table they embed)."""
    import hashlib

    h = hashlib.sha256()
    for f in ("gemm_int8.hip", "tile.h", "common.h", "launch.h", "produce.h", "producer.h", "gelu_table_gen.cpp"):
        with open(os.path.join(ROOT, "w8a8_mixed_precision_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def shape_timing(torch, w8, c, call, step_stages, steps: int) -> dict:
    """One shape: stage medians inside the step (the three shapes in turn, so
    each call finds the last-level cache (MALL, 256 MB) holding the other
    shapes' data); then the call alone, repeated on the same buffers ("hot")
    and rotated over three copies of X, Wq and Y whose combined size exceeds
    the MALL ("cold"), medians of events around each call."""
    x, wq, sw, y, ws = call
    rows_bytes = 3 * c.M * c.K            # read X (2 B) + write codes (1 B)

    def med(stages, k):
        return _median([r[k] for r in stages]) * 1e3

    call_us = _median([sum(r) for r in step_stages]) * 1e3
    out = {
        "call_us": round(call_us, 2),
        "tops": round(c.ops / (call_us * 1e-6) / 1e12, 1),
        "pct_of_mfma_peak": round(100 * c.ops / (call_us * 1e-6) / 1e12 / PEAK_INT8_TOPS, 2),
        "row_pass_us": round(med(step_stages, 0), 2),
        "row_pass_GBs": round(rows_bytes / (med(step_stages, 0) * 1e-6) / 1e9, 1),
        "fixup_us": round(med(step_stages, 1), 2),
        "gemm_us": round(med(step_stages, 2), 2),
        "gemm_tops": round(c.ops / (med(step_stages, 2) * 1e-6) / 1e12, 1),
    }
    ev = HipEvents(4 * steps)
    hot = staged_int8(w8, ev, [call], steps)[0]
    copies = [(x.clone(), wq.clone(), sw, torch.empty_like(y), ws) for _ in range(3)]
    cold = []
    for r in range(0, steps, 3):
        n = min(3, steps - r)
        cold += [v[0] for v in staged_int8(w8, ev, copies[:n], 1)]
    ev.close()
    del copies
    for name, stages in (("hot", hot), ("cold", cold)):
        t = _median([sum(r) for r in stages]) * 1e3
        out[f"{name}_call_us"] = round(t, 2)
        out[f"{name}_pct_of_mfma_peak"] = round(100 * c.ops / (t * 1e-6) / 1e12 / PEAK_INT8_TOPS, 2)
        out[f"{name}_gemm_us"] = round(med(stages, 2), 2)
    return out


def extra_shapes(torch, w8, steps: int) -> dict:
    """The other int8 workloads, each call timed alone (medians of events
    around the stages): the DiT 2048^2 linears (16640 tokens) and the tiny
    64 x 256 -> 512 fp16 linear, which is bound by launch latency."""
    import synth

    res = {}
    for c in [synth.dit_2048("qkv"), synth.dit_2048("up"), synth.dit_2048("down"), synth.tiny_int8()]:
        enc = torch.float16 if c.x_dtype == "f16" else torch.bfloat16
        import numpy as np

        x = torch.from_numpy(np.ascontiguousarray(c.x_bits).view(np.int16)).view(enc).cuda()
        w = torch.from_numpy(np.ascontiguousarray(c.w_bits).view(np.int16)).view(enc).cuda()
        wq, sw = w8.quantize_weight_rowwise(w, "int8")
        del w
        y = torch.empty((c.M, c.N), dtype=torch.float16, device="cuda")
        ws = w8.new_workspace(w8.int8_mixed_linear_workspace_size(c.M, c.N, c.K))
        ev = HipEvents(4 * steps)
        staged_int8(w8, ev, [(x, wq, sw, y, ws)], 2)
        st = staged_int8(w8, ev, [(x, wq, sw, y, ws)], steps)[0]
        ev.close()
        t = _median([sum(r) for r in st]) * 1e3
        g = _median([r[2] for r in st]) * 1e3
        res[c.name] = {"call_us": round(t, 2), "tops": round(c.ops / (t * 1e-6) / 1e12, 2),
                       "pct_of_mfma_peak": round(100 * c.ops / (t * 1e-6) / 1e12 / PEAK_INT8_TOPS, 2),
                       "gemm_us": round(g, 2), "row_pass_us": round(_median([r[0] for r in st]) * 1e3, 2),
                       "fixup_us": round(_median([r[1] for r in st]) * 1e3, 2)}
        print(f"[bench] {c.name}: {res[c.name]}", file=sys.stderr, flush=True)
        del x, wq, y, ws
    return res


def tile_timeline(w8, c, call) -> dict:
    """One GEMM launch of the shape with its per-block timeline (the
    library's timeline export; a second call, after one warm-up): medians over
    the blocks that own whole 256x256 tiles of the stretch before the K loop
    (operand ring fill), the K loop and the epilogue; the K loop in shader-clock
    cycles per 64-byte K step (1024 is the MFMA issue floor: 32 MFMAs of 32
    cycles per wave) and that clock's rate; the start of each round of whole
    tiles; the 128x128 tail's start and length. Times in us from the first
    block's start (constant 100 MHz clock)."""
    import numpy as np

    x, wq, sw, y, ws = call
    w8.debug_int8_gemm_timeline(x, wq, sw, THRESHOLD, y, ws)
    r = w8.debug_int8_gemm_timeline(x, wq, sw, THRESHOLD, y, ws)
    st = r["stamps"].astype(np.float64)
    dp = r["dp_tiles"]
    t0 = st[:, 0].min()
    big = st[:dp]
    nk = c.K // 64
    done = big[:, 3] >= 0
    loop_us = (big[:, 2] - big[:, 1]) * 0.01
    cyc = big[:, 5] - big[:, 4]
    starts = np.sort(big[:, 0] - t0) * 0.01
    cus = 256
    out = {
        "blocks": r["grid"],
        "whole_tiles": dp,
        "span_us": round(float((st[:, 3].max() - t0) * 0.01), 2),
        "ring_fill_us": round(float(np.median(big[:, 1] - big[:, 0]) * 0.01), 2),
        "k_loop_us": round(float(np.median(loop_us)), 2),
        "epilogue_us": round(float(np.median(big[done, 3] - big[done, 2]) * 0.01), 2),
        "k_step_cycles": round(float(np.median(cyc) / nk), 1),
        "clock64_mhz": round(float(np.median(cyc / loop_us)), 1),
        "round_starts_us": [round(float(starts[i]), 2) for i in range(0, dp, cus)],
    }
    if r["grid"] > dp:
        tail = st[dp:]
        out["tail_start_us"] = round(float((tail[:, 0].min() - t0) * 0.01), 2)
        out["tail_us"] = round(float((tail[:, 3].max() - tail[:, 0].min()) * 0.01), 2)
        out["tail_block_us"] = round(float(np.median(tail[:, 3] - tail[:, 0]) * 0.01), 2)
    return out


def measured_peaks(torch, w8) -> dict:
    """The chip's attainable rates, measured here: dense MFMA issue (int8,
    fp8, bf16) with every SIMD busy (the library's peak kernel, median of 5
    launches), the same with operands that change every round (random bits, as
    a GEMM's: the chip holds a lower clock), a device-to-device copy of 2 GiB
    (median of 5), and the rate at which one block per CU streams operand rows
    into LDS (the library's streaming kernel), per CU."""
    res = {}
    blocks = 4 * max(torch.cuda.get_device_properties(0).multi_processor_count, 1)
    for kind, iters in (("int8", 20000), ("fp8", 10000), ("bf16", 20000), ("int8_random", 20000),
                        ("fp8_random", 10000)):
        w8.debug_mfma_peak(kind, blocks, 100)
        ts = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            _, ops = w8.debug_mfma_peak(kind, blocks, iters)
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        res[f"{kind}_mfma_tops"] = round(ops / _median(ts) / 1e12, 1)
    n = 2 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    ts = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        e1.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    res["copy_GBs"] = round(2 * n / _median(ts) / 1e9, 1)
    del src, dst
    # the GEMMs' operand path: 256-row panels streamed into LDS by one block
    # per CU, 64-byte (the GEMMs' K step) or 128-byte row segments, from
    # panels that stay in L2 (4 MiB in all) or that do not (96 MiB)
    cus = max(torch.cuda.get_device_properties(0).multi_processor_count, 1)
    K = 4096
    panel_buf = torch.ones(96 * 256 * K, dtype=torch.uint8, device="cuda")
    for panels, where in ((4, "l2"), (96, "mall")):
        for seg in (64, 128):
            w8.debug_lds_stream(panel_buf, K, seg, cus, panels, 64)
            ts = []
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                _, nbytes = w8.debug_lds_stream(panel_buf, K, seg, cus, panels, 2048)
                e1.record()
                e1.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e-3)
            res[f"lds_stream_{where}_seg{seg}_GBs_per_cu"] = round(nbytes / _median(ts) / 1e9 / cus, 1)
    del panel_buf
    print(f"[bench] measured peaks: {res}", file=sys.stderr, flush=True)
    return res


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-rows", type=int, default=4352, help="token rows per shape for the oracle baseline (4352 = the whole step)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp8", action="store_true", help="skip the text-encoder layer timings (FP8 W8A8, FP8 weight-only, W4A8)")
    ap.add_argument("--no-fused", action="store_true", help="skip the producer-fused DiT MLP timings")
    ap.add_argument("--no-block", action="store_true", help="skip the DiT block driver timings")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the measured peaks and the DiT 2048^2 and tiny int8 shapes")
    ap.add_argument("--vendor", action="store_true",
                    help="only time the ROCm libraries behind torch (torch._int_mm, torch._scaled_mm) on the same "
                         "shapes, for context; prints one JSON line")
    ap.add_argument("--counters", type=int, default=0, metavar="MIB",
                    help="counter-collection mode: a few int8 steps, then plain copies of MIB MiB; no JSON line")
    ap.add_argument("--counters-fp8", action="store_true",
                    help="counter-collection mode: --steps calls of each FP8 W8A8 linear (text encoder, DiT 1024^2); "
                         "no JSON line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported: the library has no "
              "multi-GPU path (the linear would shard along N with no exchange).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import synth
    import w8a8_mixed_precision_amd as w8

    assert torch.cuda.is_available(), "needs a GPU"
    cases = synth.dit_1024_block()
    print(f"[bench] workload: {[c.name for c in cases]}", file=sys.stderr, flush=True)

    if args.vendor:
        print(json.dumps({"vendor_reference": vendor_reference(torch, max(5, args.steps // 2))}), flush=True)
        return 0
    if args.counters:
        counter_workload(torch, w8, cases, args.steps, args.counters)
        return 0
    if args.counters_fp8:
        counter_workload_fp8(torch, w8, args.steps)
        return 0

    # inputs resident in HBM, weights quantized once (untimed)
    xs, wqs, sws, ys, wss = _prepare(torch, w8, cases)

    def step():
        for i in range(len(cases)):
            w8.int8_mixed_linear(xs[i], wqs[i], sws[i], THRESHOLD, out=ys[i], workspace=wss[i])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)

    # timed region: exactly K steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ops_step = gemm_algorithmic_ops(cases)
    tops = ops_step * args.steps / dt / 1e12
    print(f"[bench] timed {args.steps} steps in {dt * 1e3:.2f} ms", file=sys.stderr, flush=True)

    # Second pass over the same K steps, every call recording HIP events
    # between its kernels on the stream they run on: per-stage GPU times.
    ev = HipEvents(4 * args.steps * len(cases))
    calls = [(xs[i], wqs[i], sws[i], ys[i], wss[i]) for i in range(len(cases))]
    st = staged_int8(w8, ev, calls, args.steps)
    ev.close()
    gemm_all = [r[2] for per in st for r in per]
    gemm_avg_ms = sum(gemm_all) / len(gemm_all)
    gemm_tops = (ops_step / len(cases)) / (gemm_avg_ms * 1e-3) / 1e12
    per_shape = {}
    for i, c in enumerate(cases):
        per_shape[c.name] = shape_timing(torch, w8, c, calls[i], st[i], args.steps)
        per_shape[c.name]["tile_timeline"] = tile_timeline(w8, c, calls[i])
        print(f"[bench] {c.name}: {per_shape[c.name]}", file=sys.stderr, flush=True)
    del st

    out = {
        "metric": METRIC,
        "value": round(tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dt / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": "DiT block linears at 1024^2: QKV 4352x4096x12288 + MLP up 4352x4096x16384 + "
                        "MLP down 4352x16384x4096 (MxKxN), int8_mixed_linear, threshold 6.0, bf16 in, fp16 out",
            "tokens": 4352,
            "threshold": THRESHOLD,
            "parallelism": "single GPU",
        },
        "pct_of_mfma_peak": round(100.0 * tops / PEAK_INT8_TOPS, 2),
        "roofline": {
            "bound": "mfma",
            "kernel": "k_int8_gemm (int8 MFMA GEMM + outlier MFMA + dequant epilogue)",
            "achieved": round(gemm_tops, 2),
            "peak": PEAK_INT8_TOPS,
            "unit": "TFLOP/s",
            "frac": round(gemm_tops / PEAK_INT8_TOPS, 4),
            "traffic": recorded_traffic(w8),
            "avg_launch_us": round(gemm_avg_ms * 1e3, 2),
        },
        "per_shape": per_shape,
    }
    if not args.no_extra:
        out["measured_peak"] = measured_peaks(torch, w8)
        out["roofline"]["frac_of_measured_peak"] = round(gemm_tops / out["measured_peak"]["int8_mfma_tops"], 4)
        out["roofline"]["frac_of_measured_random_operand_peak"] = round(
            gemm_tops / out["measured_peak"]["int8_random_mfma_tops"], 4)
        out["pct_of_measured_mfma_peak"] = round(100.0 * tops / out["measured_peak"]["int8_mfma_tops"], 2)
        out["other_int8_shapes"] = extra_shapes(torch, w8, max(5, args.steps // 2))
    if not args.no_fp8:
        out["weight_quant"] = weight_quant(torch, w8, cases, max(1, args.steps // 4))
        out["fp8_w8a8"] = {
            "workload": "FP8-E4M3 W8A8 text-encoder linears, 512 tokens, hidden 4096, bf16 in/out, "
                        "per-channel weight scale; dynamic per-token and static per-tensor activation scale",
            "layers": fp8_layers(torch, w8, args.steps),
        }
        out["fp8_w8a16"] = {
            "workload": "FP8-E4M3 weight-only text-encoder linears, 512 tokens, hidden 4096: bf16 X, E4M3 weights "
                        "widened to bf16 (value x channel scale) in the GEMM, bf16 MFMA, bf16 out",
            "layers": w8a16_layers(torch, w8, args.steps),
        }
        out["w4a8"] = {
            "workload": "W4A8 text-encoder linears, 512 tokens, hidden 4096: int4 weights with one fp32 scale per "
                        "128 inputs, int8 per-token activations, int8 MFMA, fp16 out",
            "layers": w4a8_layers(torch, w8, args.steps),
        }
    if not args.no_fused:
        out["fused_mlp"] = {
            "workload": "DiT 1024^2 MLP with producers: up = RMSNorm+modulation(H [4352,4096]) x W [16384,4096], "
                        "down = GELU(H [4352,16384]) x W [4096,16384]; bias, threshold 6.0, bf16 in, fp16 out",
            "layers": fused_mlp(torch, w8, args.steps),
        }
    if not args.no_block:
        out["dit_block"] = {
            "workload": "DiT 1024^2 block through the driver: X fp16 [4352,4096], QKV [12288,4096], O [4096,4096], "
                        "up [16384,4096], down [4096,16384] int8 (LLM.int8, t = 6.0) or fp16 (exclusion policy); "
                        "RMSNorm and GELU producers, biases, residuals, attention stub",
            "modes": dit_block(torch, w8, max(1, args.steps // 2)),
        }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cases, args.cpu_rows)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
