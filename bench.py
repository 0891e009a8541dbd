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
    """FP8-E4M3 W8A8 text-encoder linears at 512 tokens, per layer and
    activation-scale mode: whole-call, row-pass and GEMM time from the HIP-event
    hook, GEMM TFLOP/s and the GEMM's fraction of its roofline
    max(2MNK / 5.0 PFLOP/s, bytes / 8 TB/s), bytes = M K + N K + 2 M N."""
    import synth

    res = {}
    for layer in synth.FP8_TEXT_LAYERS:
        c = synth.fp8_text_encoder(layer)
        x = _dev16(c.x_bits, torch)
        wq, sw = w8.quantize_weight_rowwise(_dev16(c.w_bits, torch), "fp8")
        y = torch.empty((c.M, c.N), dtype=torch.bfloat16, device="cuda")
        ws = w8.new_workspace(w8.fp8_w8a8_linear_workspace_size(c.M, c.N, c.K))
        # static per-tensor input scale: "max" calibration on an independent draw
        xcal = _dev16(c.extra["x_cal_bits"], torch).float()
        scale = (xcal.abs().max() / 448.0).reshape(1).contiguous()
        for mode, act in (("dynamic", None), ("static", scale)):
            for _ in range(3):
                w8.fp8_w8a8_linear(x, wq, sw, act, out=y, workspace=ws)
            w8.profile_start(steps)
            for _ in range(steps):
                w8.fp8_w8a8_linear(x, wq, sw, act, out=y, workspace=ws)
            ms, n = w8.profile_stop()
            gemm_us = ms[2] / n * 1e3
            rows_us = ms[0] / n * 1e3
            gbytes = c.M * c.K + c.N * c.K + 2 * c.M * c.N
            t_roof = max(c.ops / (PEAK_FP8_TFLOPS * 1e12), gbytes / (PEAK_HBM_GBS * 1e9)) * 1e6
            res[f"{layer}_{c.M}x{c.K}x{c.N}_{mode}"] = {
                "call_us": round(sum(ms) / n * 1e3, 2),
                "act_quant_us": round(rows_us, 2),
                "act_quant_GBs": round(3 * c.M * c.K / (rows_us * 1e-6) / 1e9, 1),
                "gemm_us": round(gemm_us, 2),
                "gemm_tflops": round(c.ops / (gemm_us * 1e-6) / 1e12, 1),
                "gemm_roofline_us": round(t_roof, 2),
                "gemm_roofline_frac": round(t_roof / gemm_us, 3),
            }
            print(f"[bench] fp8 {layer} {mode}: {res[f'{layer}_{c.M}x{c.K}x{c.N}_{mode}']}", file=sys.stderr, flush=True)
    return res


def w8a16_layers(torch, w8, steps: int) -> dict:
    """FP8 weight-only (W8A16) text-encoder linears at 512 tokens: GEMM time
    from the HIP-event hook (the whole call is the one GEMM kernel), TFLOP/s
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
        w8.profile_start(steps)
        for _ in range(steps):
            w8.fp8_w8a16_linear(x, wq, sw, out=y, workspace=ws)
        ms, n = w8.profile_stop()
        gemm_us = ms[2] / n * 1e3
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
    512-token text-encoder shapes: whole-call, activation-pass and GEMM time
    from the HIP-event hook, GEMM TOPS and its fraction of the roofline
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
        w8.profile_start(steps)
        for _ in range(steps):
            w8.w4a8_linear(x, wq, sw, out=y, workspace=ws)
        ms, n = w8.profile_stop()
        gemm_us = ms[2] / n * 1e3
        gbytes = c.M * c.K + c.N * c.K // 2 + 2 * c.M * c.N + 4 * c.N * c.K // 128
        t_roof = max(c.ops / (PEAK_INT8_TOPS * 1e12), gbytes / (PEAK_HBM_GBS * 1e9)) * 1e6
        key = f"{layer}_{c.M}x{c.K}x{c.N}"
        res[key] = {
            "call_us": round(sum(ms) / n * 1e3, 2),
            "act_quant_us": round(ms[0] / n * 1e3, 2),
            "gemm_us": round(gemm_us, 2),
            "gemm_tops": round(c.ops / (gemm_us * 1e-6) / 1e12, 1),
            "gemm_roofline_us": round(t_roof, 2),
            "gemm_roofline_frac": round(t_roof / gemm_us, 3),
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
    row pass (quantisation) and GEMM stages from the library's HIP-event hook."""
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
        for name, fn in (("fused", fused), ("unfused", unfused)):
            w8.profile_start(steps)
            for _ in range(steps):
                fn()
            ms, n = w8.profile_stop()
            out[f"{name}_quant_us"] = round(ms[0] / n * 1e3, 2)
            out[f"{name}_fixup_us"] = round(ms[1] / n * 1e3, 2)
            out[f"{name}_gemm_us"] = round(ms[2] / n * 1e3, 2)
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
    """Digest of the sources the int8 GEMM kernel is built from."""
    import hashlib

    h = hashlib.sha256()
    for f in ("gemm_int8.hip", "tile.h", "common.h"):
        with open(os.path.join(ROOT, "w8a8_mixed_precision_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


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
    ap.add_argument("--counters", type=int, default=0, metavar="MIB",
                    help="counter-collection mode: a few int8 steps, then plain copies of MIB MiB; no JSON line")
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

    if args.counters:
        counter_workload(torch, w8, cases, args.steps, args.counters)
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

    # Second pass over the same K steps with the library's HIP-event hook on:
    # per-stage GPU time of every call, on the stream the kernels run on.
    w8.profile_start(args.steps * len(cases))
    for _ in range(args.steps):
        step()
    stage_ms, ncalls = w8.profile_stop()
    gemm_avg_ms = stage_ms[2] / ncalls
    gemm_tops = (ops_step / len(cases)) / (gemm_avg_ms * 1e-3) / 1e12
    per_shape = {}
    for i, c in enumerate(cases):
        w8.profile_start(args.steps)
        for _ in range(args.steps):
            w8.int8_mixed_linear(xs[i], wqs[i], sws[i], THRESHOLD, out=ys[i], workspace=wss[i])
        ms, n = w8.profile_stop()
        call_us = sum(ms) / n * 1e3
        rows_bytes = 3 * c.M * c.K            # read X (2 B) + write codes (1 B)
        per_shape[c.name] = {
            "call_us": round(call_us, 2),
            "tops": round(c.ops / (call_us * 1e-6) / 1e12, 1),
            "row_pass_us": round(ms[0] / n * 1e3, 2),
            "row_pass_GBs": round(rows_bytes / (ms[0] / n * 1e-3) / 1e9, 1),
            "fixup_us": round(ms[1] / n * 1e3, 2),
            "gemm_us": round(ms[2] / n * 1e3, 2),
            "gemm_tops": round(c.ops / (ms[2] / n * 1e-3) / 1e12, 1),
        }
        print(f"[bench] {c.name}: {per_shape[c.name]}", file=sys.stderr, flush=True)

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
