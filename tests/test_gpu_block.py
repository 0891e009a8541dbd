"""GPU parity of the block driver (w8_dit_block_forward) and its plain 16-bit
linear against the CPU oracle (oracle/block.py).

The 16-bit linear: relative Frobenius error <= 1e-5 for fp32 output (fp32
sums against float64) and <= 1e-2 for 16-bit output. The block: Y within
1e-2 relative Frobenius, globally and per row, at small sizes and at the full
DiT 1024^2 size; and step by step: every intermediate the driver leaves in its
workspace (qkv, a, o, h, u, GELU(u) or d) against the oracle's step applied to
the driver's own input of that step, element by element (tests/bounds.py),
the attention stub bit-exact. The full size with the library's own weight
quantisation is also checked to be finite and not constant (the
"Qwen-Image-fni8" card's sanity test).
"""
import numpy as np
import pytest
import torch

import w8a8_mixed_precision_amd as w8
from oracle import block as B
from oracle import producers as P
from oracle import w8ref as o
from tests import bounds
from tests.gpu_util import OUT, announce, dev16, host_stored, rel_fro, row_rel_fro

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K,N,dtype,split,tile", [(300, 1024, 520, "f16", 0, 0), (300, 1024, 520, "bf16", 2, 128),
                                                    (64, 256, 96, "f16", 4, 128), (1, 64, 1, "bf16", 1, 128),
                                                    (257, 4096, 129, "f16", 8, 128),
                                                    (300, 1024, 520, "bf16", 1, 256), (300, 1024, 520, "f16", 3, 256),
                                                    (1, 64, 1, "f16", 1, 256), (513, 2048, 777, "bf16", 16, 256)])
@pytest.mark.parametrize("out_dtype", ["f32", "f16"])
def test_linear16_matches_oracle(M, K, N, dtype, split, tile, out_dtype):
    rng = np.random.default_rng(M + K + N)
    enc = o.round_to_f16 if dtype == "f16" else o.round_to_bf16
    x_bits, w_bits = enc(rng.standard_normal((M, K))), enc(rng.standard_normal((N, K)) * 0.05)
    ref = B.linear16(x_bits, dtype, w_bits, dtype, out_dtype)
    announce("linear16", M, K, N, dtype, split, tile, out_dtype)
    y = w8.debug_linear16(dev16(x_bits, dtype), dev16(w_bits, dtype), split, OUT[out_dtype], tile=tile)
    torch.cuda.synchronize()
    got = o.stored_to_f64(host_stored(y, out_dtype), out_dtype)
    e, er = rel_fro(got, ref["y"]), row_rel_fro(got, ref["y"]).max()
    tol = 1e-5 if out_dtype == "f32" else 1e-2
    assert e <= tol and er <= tol, (e, er)


def _block(rng, D, F, with16, massive_rows=()):
    blk, dev = {}, {}
    for name, (n, k) in {"qkv": (3 * D, D), "o": (D, D), "up": (F, D), "down": (D, F)}.items():
        w = rng.standard_normal((n, k)).astype(np.float32) * 0.02
        w_bits = o.round_to_f16(w)
        wq, sw = o.quantize_weight_int8(o.decode16(w_bits, "f16"))
        b = (rng.standard_normal(n) * 0.1).astype(np.float32)
        blk[f"wq_{name}"], blk[f"sw_{name}"], blk[f"b_{name}"] = wq, sw, b
        dev[name] = (torch.from_numpy(wq).cuda(), torch.from_numpy(sw).cuda(), torch.from_numpy(b).cuda())
    norms = []
    for _ in range(2):
        g = rng.uniform(0.8, 1.2, D).astype(np.float32)
        sc = rng.uniform(-0.2, 0.2, D).astype(np.float32)
        sh = rng.uniform(-0.2, 0.2, D).astype(np.float32)
        norms.append((dict(gamma=g, scale=sc, shift=sh, eps=1e-6),
                      w8.Producer("rmsnorm", torch.from_numpy(g).cuda(), torch.from_numpy(sc).cuda(),
                                  torch.from_numpy(sh).cuda(), 1e-6)))
    blk["norm1"], blk["norm2"] = norms[0][0], norms[1][0]
    w16 = o.round_to_f16(rng.standard_normal((D, F)) * 0.02) if with16 else None
    blk["w16_down"] = w16
    gpu = w8.DitBlock(D, F, *dev["qkv"][:2], *dev["o"][:2], *dev["up"][:2],
                      w_down=None if with16 else dev["down"][0], s_down=None if with16 else dev["down"][1],
                      b_qkv=dev["qkv"][2], b_o=dev["o"][2], b_up=dev["up"][2], b_down=dev["down"][2],
                      norm1=norms[0][1], norm2=norms[1][1],
                      w_down16=dev16(w16, "f16") if with16 else None)
    return blk, gpu


@pytest.mark.parametrize("split", [0, 2, 8])
def test_linear16_whole_waves_and_sliced_tail(split):
    """More 256x256 tiles than compute units: the full waves' tiles whole and
    the leftover tiles in K-slices (split 0: the driver's own plan), at the
    DiT 1024^2 output shape with a short K; every output checked."""
    rng = np.random.default_rng(97 + split)
    M, K, N = 4352, 1024, 4096
    x_bits, w_bits = o.round_to_f16(rng.standard_normal((M, K))), o.round_to_f16(rng.standard_normal((N, K)) * 0.05)
    ref = B.linear16(x_bits, "f16", w_bits, "f16", "f32")
    announce("linear16 tail", M, K, N, split)
    y = w8.debug_linear16(dev16(x_bits, "f16"), dev16(w_bits, "f16"), split, torch.float32, tile=256)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    e, er = rel_fro(got, ref["y"]), row_rel_fro(got, ref["y"]).max()
    assert e <= 1e-5 and er <= 1e-5, (e, er)


@pytest.mark.parametrize("with16", [False, True], ids=["int8_down", "fp16_down"])
@pytest.mark.parametrize("M", [300, 64])
def test_block_matches_oracle(with16, M):
    rng = np.random.default_rng(90 + M + with16)
    D, F = 256, 1024
    x = rng.standard_normal((M, D))
    x[M - 8:, 37] = rng.uniform(8500, 9500, 8)     # massive activations in a few text rows
    x[:, 101] *= 20.0                              # an outlier channel
    x_bits = o.round_to_f16(x)
    blk, gpu = _block(rng, D, F, with16)
    ref = B.dit_block(x_bits, blk)
    announce("block", M, D, F, with16)
    y = gpu.forward(dev16(x_bits, "f16"))
    torch.cuda.synchronize()
    got = o.stored_to_f64(host_stored(y, "f16"), "f16")
    want = o.stored_to_f64(ref["Y"], "f16")
    e, er = rel_fro(got, want), row_rel_fro(got, want).max()
    assert e <= 1e-2 and er <= 1e-2, (e, er)
    # the workspace is reused without clearing: a second call repeats bit for bit
    ws = w8.new_workspace(gpu.workspace_size(M))
    y1 = gpu.forward(dev16(x_bits, "f16"), workspace=ws)
    y2 = gpu.forward(dev16(x_bits, "f16"), workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(y1, y)


@pytest.mark.parametrize("with16", [False, True], ids=["int8_down", "fp16_down"])
def test_block_full_size_matches_oracle(with16):
    """The DiT 1024^2 block (M = 4352 tokens, D = 4096, F = 16384) in the
    driver's own launch configuration against the oracle's whole chain
    (about 20 s of host work): the massive activations of the text-token rows
    in channel 2276, one outlier channel, Y within 1e-2 globally and per row."""
    rng = np.random.default_rng(95 + with16)
    M, D, F = 4352, 4096, 16384
    x = rng.standard_normal((M, D))
    x[4096::32, 2276] = rng.uniform(8500, 9500, 8)
    x[:, 101] *= 20.0
    x_bits = o.round_to_f16(x)
    blk, gpu = _block(rng, D, F, with16)
    announce("block full size vs oracle", M, D, F, with16)
    y = gpu.forward(dev16(x_bits, "f16"))
    torch.cuda.synchronize()
    got = o.stored_to_f64(host_stored(y, "f16"), "f16")
    del y, gpu
    want = o.stored_to_f64(B.dit_block(x_bits, blk)["Y"], "f16")
    e, er = rel_fro(got, want), row_rel_fro(got, want).max()
    assert e <= 1e-2 and er <= 1e-2, (e, er)


@pytest.mark.parametrize("with16", [False, True], ids=["int8_down", "fp16_down"])
def test_block_full_size_is_finite_and_not_constant(with16):
    """The DiT 1024^2 block (M = 4352, D = 4096, F = 16384) with random
    weights and the massive text-token activations of the MLP workload."""
    g = torch.Generator(device="cuda").manual_seed(7)
    M, D, F = 4352, 4096, 16384
    x = torch.randn(M, D, device="cuda", generator=g)
    x[4096::32, 2276] = 9000.0
    x = x.to(torch.float16)

    def lin(n, k):
        w = (torch.randn(n, k, device="cuda", generator=g) * 0.02).to(torch.float16)
        wq, sw = w8.quantize_weight_rowwise(w, "int8")
        return wq, sw, w

    qkv, o_, up, down = lin(3 * D, D), lin(D, D), lin(F, D), lin(D, F)
    blk = w8.DitBlock(D, F, qkv[0], qkv[1], o_[0], o_[1], up[0], up[1],
                      w_down=None if with16 else down[0], s_down=None if with16 else down[1],
                      norm1=w8.Producer("rmsnorm"), norm2=w8.Producer("rmsnorm"),
                      w_down16=down[2] if with16 else None)
    announce("block full size", with16)
    y = blk.forward(x)
    torch.cuda.synchronize()
    yf = y.float()
    assert torch.isfinite(yf).all() and float(yf.std()) > 0
    # the massive channel survives the block (residual stream)
    assert float(yf[4096, 2276]) > 4000


def _f16(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _check_linear_step(got_bits, h_bits, kind, blk, name, norm, label, rows, rstd=None):
    """One int8 linear of the block: the oracle's fused linear on the
    driver's own input h_bits, element by element on `rows`. RMSNorm: with
    the given rstd (checked against the allowed readings), or with each
    reading when a row has two."""
    kw = dict(norm) if norm else {}
    wq, sw, b = blk[f"wq_{name}"], blk[f"sw_{name}"], blk[f"b_{name}"]
    cands = [None]
    if kind == "rmsnorm":
        h = o.decode16(h_bits, "f16")
        a, bb = P.rstd_alternatives(h, kw.get("eps", 1e-6))
        if rstd is not None:
            assert np.all((rstd == a) | (rstd == bb))
            cands = [rstd]
        else:
            cands = [a] if np.array_equal(a, bb) else [a, bb]
    ok = np.zeros(len(rows), bool)
    errs = []
    for r in cands:
        x_bits = P.produce(h_bits, "f16", kind, rstd=r, **kw) if kind != "none" else h_bits
        ref = P.fused_int8_linear(h_bits, "f16", kind, wq, sw, 6.0, b, "f16", rows=rows, x_bits=x_bits, **kw)
        err = bounds.int8_err32(ref, x_bits[rows], "f16", wq, sw, bias=b)
        g = o.stored_to_f64(got_bits[rows], "f16")
        big = np.maximum(np.abs(g), np.abs(ref["y"]))
        bound = bounds.half_ulp(big, "f16") + 2 * err + 1e-12 * big
        ok |= np.all(np.abs(g - ref["y"]) <= bound, axis=1)
        errs.append(float(np.max(np.abs(g - ref["y"]) / bound)))
    assert ok.all(), (label, np.flatnonzero(~ok)[:10], errs)


def _check_residual(got_bits, a_bits, d_values, label):
    """y = rne16(fl32(a + fl32(d))), d itself the float32 sum of the linear's
    output and the bias when the bias is added here: within half an fp16 ulp
    plus a float32 rounding of d and one of the sum."""
    s = o.decode16(a_bits, "f16").astype(np.float64) + d_values
    bounds.assert_elementwise(got_bits, "f16", s, bounds.U * (np.abs(s) + np.abs(d_values)), label)


def _check_block_steps(x_bits, blk, gpu, ws, M, rows):
    D, F = gpu.D, gpu.F
    it = gpu.intermediates(ws, M)
    qkv, a, o_, h, u = (_f16(it[k]) for k in ("qkv", "a", "o", "h", "u"))
    _check_linear_step(qkv, x_bits, "rmsnorm", blk, "qkv", blk["norm1"], "qkv", rows)
    assert np.array_equal(a, qkv[:, 2 * D:3 * D])                       # the attention stub
    _check_linear_step(o_, a, "none", blk, "o", None, "o", rows)
    _check_residual(h, x_bits, o.decode16(o_, "f16").astype(np.float64), "h")
    # with the 16-bit down-projection, the up projection is the last int8
    # call in the shared workspace, which still holds its rstd (an int8 down
    # projection overwrites it with its codes)
    rstd2 = None
    if blk.get("w16_down") is not None:
        lay = w8.int8_workspace_layout(M, F, D)
        rstd2 = ws[lay["rstd"]:lay["rstd"] + 4 * M].view(torch.float32).cpu().numpy()
    _check_linear_step(u, h, "rmsnorm", blk, "up", blk["norm2"], "u", rows, rstd=rstd2)
    if blk.get("w16_down") is not None:
        g = _f16(it["g"])
        assert np.array_equal(g, P.gelu16(u, "f16"))
        d = it["d"].cpu().numpy().astype(np.float64)
        ref = B.linear16(g[rows], "f16", blk["w16_down"], "f16", "f32")
        err = bounds.dense_err32(np.abs(o.decode16(g[rows], "f16").astype(np.float64)),
                                 np.abs(o.decode16(blk["w16_down"], "f16").astype(np.float64)), ref["y"], F)
        bounds.assert_elementwise(d[rows].astype(np.float32), "f32", ref["y"], err, "d16")
        dv = d + blk["b_down"].astype(np.float64)[None, :]
    else:
        d = _f16(it["d"])
        _check_linear_step(d, u, "gelu", blk, "down", None, "d", rows)
        dv = o.decode16(d, "f16").astype(np.float64)
    return h, dv


@pytest.mark.parametrize("with16", [False, True], ids=["int8_down", "fp16_down"])
def test_block_every_step_matches_oracle(with16):
    """Every intermediate of a small block, each against the oracle's step on
    the driver's own input of that step, and Y against the residual of the
    driver's h and d."""
    M = 300
    rng = np.random.default_rng(190 + with16)
    D, F = 256, 1024
    x = rng.standard_normal((M, D))
    x[M - 8:, 37] = rng.uniform(8500, 9500, 8)
    x[:, 101] *= 20.0
    x_bits = o.round_to_f16(x)
    blk, gpu = _block(rng, D, F, with16)
    ws = w8.new_workspace(gpu.workspace_size(M))
    announce("block steps", M, D, F, with16)
    y = gpu.forward(dev16(x_bits, "f16"), workspace=ws)
    torch.cuda.synchronize()
    h, dv = _check_block_steps(x_bits, blk, gpu, ws, M, np.arange(M))
    _check_residual(_f16(y), h, dv, "Y")


@pytest.mark.parametrize("with16", [False, True], ids=["int8_down", "fp16_down"])
def test_block_full_size_every_step(with16):
    """The DiT 1024^2 block, every intermediate on sampled rows (the massive
    text-token rows and the ragged last strip among them)."""
    rng = np.random.default_rng(195 + with16)
    M, D, F = 4352, 4096, 16384
    x = rng.standard_normal((M, D))
    x[4096::32, 2276] = rng.uniform(8500, 9500, 8)
    x[:, 101] *= 20.0
    x_bits = o.round_to_f16(x)
    blk, gpu = _block(rng, D, F, with16)
    ws = w8.new_workspace(gpu.workspace_size(M))
    announce("block full size steps", with16)
    y = gpu.forward(dev16(x_bits, "f16"), workspace=ws)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.random.default_rng(196).choice(M, 40, replace=False),
                                     np.arange(4096, M, 32), np.arange(4352 - 12, M)]))
    h, dv = _check_block_steps(x_bits, blk, gpu, ws, M, rows)
    _check_residual(_f16(y)[rows], h[rows], dv[rows], "Y")
