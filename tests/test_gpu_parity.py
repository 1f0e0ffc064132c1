"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bit-exact for packed indices, block constants, double-quantisation codes,
scales, mean and dequantised values; within the stated tolerance for the
layer's outputs and gradients (bf16: max |d| / max(max|ref|, rms ref) <=
2e-2 against the fp64 oracle; fp16: the same measure <= 2.5e-3; fp32:
|d| <= 1e-5 + 1e-5 |ref|).
"""
import numpy as np
import pytest
import torch

import qlora_fine_tuning_quantize_amd as q
import synth_inputs as si
from tests.helpers import (BF16_TOL, F16_TOL, U_BF16, U_F16, assert_f32_close,
                           assert_layer_within16, host, layer_bounds16,
                           rel_err)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
# a 16-bit forward of up to this many tokens computes u in workgroups of its
# own launch and sums the slices of x W^^T with the bypass in a second one
FUSED_MAX_M = 128


def _say(*a):
    print(*a, flush=True)


# ---------------------------------------------------------------------------
# quantisation / double quantisation / dequantisation: bit-exact
# ---------------------------------------------------------------------------
def _check_quant(orc, w_cpu: torch.Tensor, dq: bool, block: int = 64):
    Wq = q.nf4_quantize(w_cpu.to(DEV).contiguous(), double_quant=dq, block=block)
    torch.cuda.synchronize()
    st = orc.quantize_nf4(host(w_cpu).reshape(-1), double_quant=dq, block=block)
    np.testing.assert_array_equal(host(Wq.packed)[:st["packed"].size], st["packed"])
    if dq:
        np.testing.assert_array_equal(host(Wq.absmax_q)[:st["absmax_q"].size], st["absmax_q"])
        np.testing.assert_array_equal(host(Wq.absmax_scale)[:st["absmax_scale"].size].view(np.uint32),
                                      st["absmax_scale"].view(np.uint32))
        assert host(Wq.absmax_mean)[:1].view(np.uint32)[0] == np.float32(st["absmax_mean"]).view(np.uint32)
    else:
        np.testing.assert_array_equal(host(Wq.absmax)[:st["absmax"].size].view(np.uint32),
                                      st["absmax"].view(np.uint32))
    ref32 = orc.dequantize(st)
    got32 = host(q.nf4_dequantize(Wq, torch.float32)).reshape(-1)
    np.testing.assert_array_equal(got32.view(np.uint32), ref32.view(np.uint32))
    got16 = host(q.nf4_dequantize(Wq, torch.bfloat16)).reshape(-1)
    np.testing.assert_array_equal(got16, orc.round_bf16(ref32))
    goth = host(q.nf4_dequantize(Wq, torch.float16)).reshape(-1)
    np.testing.assert_array_equal(goth.view(np.uint16), orc.round_f16(ref32).view(np.uint16))
    return Wq, st


@pytest.mark.parametrize("rows,cols", [(1, 1), (1, 7), (3, 5), (1, 63), (1, 64), (1, 65), (7, 129),
                                       (64, 64), (256, 256), (300, 1000), (33, 64 * 257)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("dq", [False, True])
def test_quant_dequant_bit_exact(orc, rows, cols, dtype, dq):
    _say(f"quant rows={rows} cols={cols} dtype={dtype} dq={dq}")
    w = si.normal((rows, cols), 0.02, seed=rows * 131 + cols, dtype=dtype)
    flat = w.view(-1)
    if flat.numel() >= 256:
        flat[64:128] = 0                       # an all-zero block
        flat[5] = 0.4                          # 20-sigma outliers
        flat[200] = -0.4
    _check_quant(orc, w, dq)


@pytest.mark.parametrize("rows,cols", [(1, 1), (1, 127), (1, 128), (1, 129), (3, 5), (7, 129),
                                       (64, 256), (300, 1000), (33, 128 * 257)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("dq", [False, True])
def test_quant_dequant_bit_exact_block128(orc, rows, cols, dtype, dq):
    """Blocks of 128 weights (one constant per 128)."""
    _say(f"quant block 128 rows={rows} cols={cols} dtype={dtype} dq={dq}")
    w = si.normal((rows, cols), 0.02, seed=rows * 137 + cols, dtype=dtype)
    flat = w.view(-1)
    if flat.numel() >= 512:
        flat[128:256] = 0                      # an all-zero block
        flat[5] = 0.4                          # 20-sigma outliers
        flat[300] = -0.4
    _check_quant(orc, w, dq, block=128)


def test_quant_subnormal_and_signed_zero_blocks(orc):
    w = torch.zeros(4 * 64, dtype=torch.float32)
    w[0:64] = torch.linspace(-1e-39, 1e-39, 64)        # fp32 subnormals only
    w[64:128] = -0.0
    w[128:192] = torch.linspace(-3.0, 3.0, 64)
    w[192] = 1e-30
    for dq in (False, True):
        _check_quant(orc, w.view(4, 64), dq)
        _check_quant(orc, w.to(torch.bfloat16).view(4, 64), dq)


def test_quant_block_maxima_at_the_reciprocal_limits(orc):
    """fp32 blocks whose maximum lies at or beyond 2^-125 / 2^125 (the
    quantiser then divides instead of multiplying by a reciprocal), at the
    normal minimum, near the fp32 maximum, and blocks with elements planted
    exactly on the codepoint midpoints times the block maximum."""
    rng = np.random.default_rng(11)
    maxima = [2.0 ** -126, 2.0 ** -125, 2.0 ** -124, 1.5 * 2.0 ** -125, 2.0 ** 124, 2.0 ** 125,
              1.5 * 2.0 ** 125, 2.0 ** 126, 3.0e38, 1.0, 0.02, 7.0]
    blocks = []
    for a in maxima:
        b = (rng.uniform(-1, 1, 64) * a).astype(np.float32)
        b[rng.integers(64)] = np.float32(a) * (1 if rng.integers(2) else -1)
        blocks.append(b)
    cb = np.array(orc.codebook(), dtype=np.float64)
    mids = (cb[:-1] + cb[1:]) / 2
    for a in (0.02, 1.0, 3.0, 2.0 ** -100):
        b = np.zeros(64, np.float32)
        b[0] = a
        b[1:16] = (mids * a).astype(np.float32)
        b[16:31] = np.nextafter(b[1:16], np.float32(np.inf))
        b[31:46] = np.nextafter(b[1:16], np.float32(-np.inf))
        blocks.append(b)
    w = torch.from_numpy(np.concatenate(blocks).reshape(len(blocks), 64))
    _check_quant(orc, w, False)
    _check_quant(orc, w, True)  # the mean of maxima 2^250 apart is still the exact one


def test_quant_dq_mean_exact_sum_decides_a_tie(orc):
    """Block maxima 2^60, 2^36, 2^7, 2^-100: the mean is 2^58 + 2^35 only if
    the sum of the constants is exact (an fp64 running sum gives 2^58)."""
    rng = np.random.default_rng(5)
    blocks = []
    for a in (2.0 ** 60, 2.0 ** 36, 2.0 ** 7, 2.0 ** -100):
        b = (rng.uniform(-1, 1, 64) * a).astype(np.float32)
        b[3] = np.float32(a)
        blocks.append(b)
    w = torch.from_numpy(np.concatenate(blocks).reshape(4, 64))
    Wq, _ = _check_quant(orc, w, True)
    assert host(Wq.absmax_mean)[0] == np.float32(2.0 ** 58 + 2.0 ** 35)


@pytest.mark.parametrize("nblocks", [40000, 131072 + 77])
def test_quant_dq_wide_range_constants(orc, nblocks):
    """Block maxima spread over 2^-140 .. 2^120 (a range far beyond 2^30),
    with a few subnormal and zero blocks, over enough blocks that many
    workgroups contribute partial sums (the larger case also walks several
    grid-stride steps per wave)."""
    _say(f"quant dq wide range nblocks={nblocks}")
    rng = np.random.default_rng(nblocks)
    e = rng.integers(-140, 120, nblocks).astype(np.float64)
    amax = (rng.uniform(1, 2, nblocks) * np.exp2(e)).astype(np.float32)
    amax[7] = np.float32(3 * 2.0 ** -149)
    amax[11] = 0
    w = rng.uniform(-1, 1, (nblocks, 64)).astype(np.float32) * amax[:, None]
    w[np.arange(nblocks), rng.integers(0, 64, nblocks)] = amax
    _check_quant(orc, torch.from_numpy(w), True)


def _bf16_sweep_weights(a_scale_exp: int) -> torch.Tensor:
    """Blocks of 64 bf16 values: element 0 is the block maximum a (128 bf16
    mantissas times 2**a_scale_exp), the other 63 run through every finite
    bf16 value w with |w| <= a, both signs.  Covers every (w, a) ratio class
    of bf16 inputs."""
    bits = np.arange(0, 0x7F80, dtype=np.uint32)  # all finite non-negative bf16 patterns
    vals = (bits << 16).view(np.float32)
    blocks = []
    for m in range(128):
        a = np.float32((1 + m / 128) * 2.0 ** a_scale_exp)
        ws = vals[vals <= a]
        ws = np.concatenate([ws, -ws[ws > 0]])
        n_blk = (ws.size + 62) // 63
        pad = np.zeros(n_blk * 63, dtype=np.float32)
        pad[:ws.size] = ws
        blk = np.concatenate([np.full((n_blk, 1), a, dtype=np.float32), pad.reshape(n_blk, 63)], 1)
        blocks.append(blk)
    allw = np.concatenate(blocks).reshape(-1)
    return torch.from_numpy(allw).to(torch.bfloat16)


@pytest.mark.parametrize("a_exp", [0, -20, 7])
def test_quant_exhaustive_bf16_ratios(orc, a_exp):
    w = _bf16_sweep_weights(a_exp)
    _say(f"bf16 sweep a_exp={a_exp}: {w.numel()} elements")
    Wq = q.nf4_quantize(w.to(DEV).view(1, -1), double_quant=False)
    torch.cuda.synchronize()
    packed, absmax = orc.quantize(host(w))
    np.testing.assert_array_equal(host(Wq.packed)[:packed.size], packed)
    np.testing.assert_array_equal(host(Wq.absmax)[:absmax.size], absmax)


# ---------------------------------------------------------------------------
# the layer: forward and backward
# ---------------------------------------------------------------------------
def _layer_case(orc, M, N, K, r, dq, act, lora, alpha=32.0, seed_cfg=90, dy_ones=False,
                rows=None, block=64):
    t = si.linear_inputs(seed_cfg, M, N, K, r, act_dtype=act, w_dtype=act, lora_dtype=lora,
                         sub=M + N + K + r)
    if dy_ones:
        t["dy"] = torch.ones((M, N), dtype=act)
    d = {k: v.to(DEV) for k, v in t.items()}
    W = q.nf4_quantize(d["W"], double_quant=dq, block=block)
    u = torch.empty((M, r), dtype=torch.float32, device=DEV)
    y = q.qlora_linear_fwd(d["x"], W, d["A"], d["B"], alpha, u_save=u)
    dx, dA, dB = q.qlora_linear_bwd(d["dy"], d["x"], W, d["A"], d["B"], alpha)
    dx2, dA2, dB2 = q.qlora_linear_bwd(d["dy"], d["x"], W, d["A"], d["B"], alpha, u_saved=u)
    torch.cuda.synchronize()
    st = orc.quantize_nf4(host(t["W"]), double_quant=dq, block=block)
    w_hat = orc.dequantize(st).reshape(N, K)
    xs = host(t["x"]) if rows is None else host(t["x"])[rows]
    y_ref, u_ref = orc.linear_fwd(xs, w_hat, host(t["A"]), host(t["B"]), alpha, r)
    dx_ref, dA_ref, dB_ref = orc.linear_bwd(host(t["x"]), w_hat, host(t["A"]), host(t["B"]),
                                            host(t["dy"]), alpha, r, rows=rows)
    sel = slice(None) if rows is None else rows
    got = {"y": y.float().cpu().numpy()[sel], "u": u.cpu().numpy()[sel],
           "dx": dx.float().cpu().numpy()[sel], "dA": dA.cpu().numpy(), "dB": dB.cpu().numpy()}
    ref = {"y": y_ref, "u": u_ref, "dx": dx_ref, "dA": dA_ref, "dB": dB_ref}
    # the saved-u backward is the same computation.  A 16-bit forward of up
    # to 128 tokens (the decode forward, M <= 16, and the few-token forward)
    # computes u in workgroups of its own launch, in another fp32 summation
    # order than the backward's recomputation; the backward rounds u to 16
    # bits for its matrix ops, where the two orders can round to neighbouring
    # values: there the saved-u dA and dB are held to the oracle at the
    # layer's tolerance.  dx does not depend on u.
    if act != torch.float32 and M <= FUSED_MAX_M:
        tol = F16_TOL if act == torch.float16 else BF16_TOL
        assert rel_err(dA2.cpu().numpy(), dA_ref) <= tol
        assert rel_err(dB2.cpu().numpy(), dB_ref) <= tol
    else:
        np.testing.assert_array_equal(dA2.cpu().numpy(), got["dA"])
        np.testing.assert_array_equal(dB2.cpu().numpy(), got["dB"])
    np.testing.assert_array_equal(dx2.float().cpu().numpy()[sel], got["dx"])
    if act != torch.float32:  # every 16-bit output within its derived per-element bound
        s = float(np.float32(alpha) / np.float32(r))
        bounds = layer_bounds16(host(t["x"]), w_hat, host(t["A"]), host(t["B"]), s,
                                dy=host(t["dy"]), rows=rows)
        assert_layer_within16(got, ref, bounds, U_F16 if act == torch.float16 else U_BF16)
    return got, ref


def _assert_fwd_within16(t, w_hat, alpha, r, act, y, y_ref, u=None, u_ref=None):
    """The forward's 16-bit y (and fp32 u) within the derived per-element bound."""
    s = float(np.float32(alpha) / np.float32(r))
    b = layer_bounds16(host(t["x"]), w_hat, host(t["A"]), host(t["B"]), s)
    got, ref = {"y": y.float().cpu().numpy()}, {"y": y_ref}
    if u is not None:
        got["u"], ref["u"] = u.cpu().numpy(), u_ref
    assert_layer_within16(got, ref, b, U_F16 if act == torch.float16 else U_BF16)


@pytest.mark.parametrize("dy_ones", [False, True])
def test_layer_fp32_small_config(orc, dy_ones):
    """fp32 compute: W 256x256, x 4x256, r 8, alpha 16, no double quant."""
    c = si.SMALL_FP32
    got, ref = _layer_case(orc, c["M"], c["N"], c["K"], c["r"], False, torch.float32,
                           torch.float32, alpha=c["alpha"], seed_cfg=c["config"], dy_ones=dy_ones)
    for k in ("y", "u", "dx", "dA", "dB"):
        assert_f32_close(got[k], ref[k], k)
    if dy_ones:  # the pages' .sum().backward(): identical dx rows and dB rows
        assert np.all(got["dx"] == got["dx"][0:1])


BF16_CASES = [
    # M, N, K, r, dq, lora dtype         (path exercised)
    (1, 256, 256, 8, True, torch.bfloat16),     # decode GEMV
    (3, 200, 320, 16, False, torch.float32),    # GEMV, ragged N, fp32 LoRA
    (16, 384, 1024, 16, True, torch.bfloat16),  # GEMV at M = 16
    (1, 200, 4416, 16, True, torch.bfloat16),   # GEMV: second round of 5 blocks, ragged N
    (16, 96, 8192, 128, False, torch.float32),  # GEMV: two full rounds, r = 128, fp32 absmax
    (5, 64, 14336, 64, True, torch.bfloat16),   # GEMV: 3.5 rounds, r = 64
    (17, 128, 128, 16, True, torch.bfloat16),   # smallest matrix-core GEMM
    (300, 384, 384, 16, True, torch.bfloat16),  # ragged M over two token tiles
    (300, 200, 320, 8, False, torch.float32),   # ragged N: guarded fwd tile; dx ragged in N and K
    (512, 256, 640, 64, True, torch.bfloat16),  # r = 64
    (257, 128, 128, 128, True, torch.bfloat16), # r = 128
    (64, 64, 64, 5, True, torch.bfloat16),      # rank not a multiple of 8
    # split-K (few tiles, long contraction): fp32 partial tiles + fixed-order sum
    (300, 200, 1024, 16, False, torch.float32), # fwd 2 slices, ragged M and N
    (77, 1024, 2048, 16, True, torch.bfloat16), # fwd 4 slices, dx 2 slices
    (200, 512, 4096, 8, True, torch.bfloat16),  # fwd 8 slices
    (130, 4096, 512, 16, True, torch.bfloat16), # dx 8 slices
    (7, 64, 512, 16, True, torch.bfloat16),     # GEMV: a round of 8 blocks
    # matrix-core dx on ragged shapes (N % 64 != 0, K % 128 != 0)
    (77, 200, 1088, 16, True, torch.bfloat16),  # 64-token dx tiles, last step and column tile ragged
    (300, 456, 4416, 16, True, torch.bfloat16), # 256-token dx tiles, ragged N and K
    (130, 2120, 576, 16, True, torch.bfloat16), # ragged dx with split-K
    (1, 200, 2048, 5, False, torch.bfloat16),   # GEMV: ragged N, rank 5, fp32 absmax
    # 64-token forward tiles (17..64 tokens), 128-token tiles (65..128)
    (100, 200, 320, 8, False, torch.float32),   # ragged M and N, fp32 absmax and factors
    (48, 256, 512, 128, True, torch.bfloat16),  # r = 128 (8 rank chunks), split
    (128, 384, 4096, 16, True, torch.bfloat16), # one full 128-token tile, split
    (65, 256, 512, 16, True, torch.bfloat16),   # 128-token tiles with one row past 64
    (127, 200, 1088, 16, False, torch.float32), # 128-token tiles, ragged N, dx ragged in N and K
    (96, 1024, 4096, 64, True, torch.bfloat16), # 128-token tiles, r = 64, split-K forward and dx
]


@pytest.mark.parametrize("M,N,K,r,dq,lora", BF16_CASES)
def test_layer_bf16_parity(orc, M, N, K, r, dq, lora):
    _say(f"layer bf16 M={M} N={N} K={K} r={r} dq={dq} lora={lora}")
    got, ref = _layer_case(orc, M, N, K, r, dq, torch.bfloat16, lora)
    errs = {k: rel_err(got[k], ref[k]) for k in ("y", "u", "dx", "dA", "dB")}
    _say("  rel errors", {k: f"{v:.2e}" for k, v in errs.items()})
    for k, e in errs.items():
        assert e <= BF16_TOL, (k, e)


BLOCK128_CASES = [
    # M, N, K, r, dq, act                       (path exercised)
    (1, 256, 1024, 16, True, torch.bfloat16),   # decode GEMV
    (16, 200, 4352, 16, False, torch.bfloat16), # GEMV, second round, ragged N
    (64, 256, 512, 8, True, torch.bfloat16),    # 64-token forward tile, split
    (120, 256, 1024, 16, True, torch.bfloat16), # 128-token forward and dx tiles
    (300, 384, 768, 16, True, torch.bfloat16),  # 256-token GEMM, ragged M
    (77, 1024, 2048, 16, False, torch.bfloat16),# split-K forward and dx
    (300, 200, 384, 8, True, torch.bfloat16),   # ragged N: guarded tile, tiled dx
    (4, 256, 256, 8, False, torch.float32),     # fp32 path
]


@pytest.mark.parametrize("M,N,K,r,dq,act", BLOCK128_CASES)
def test_layer_parity_block128(orc, M, N, K, r, dq, act):
    """The layer with blocks of 128 weights, every kernel path."""
    _say(f"layer block 128 M={M} N={N} K={K} r={r} dq={dq} act={act}")
    got, ref = _layer_case(orc, M, N, K, r, dq, act, act, block=128)
    for k in ("y", "u", "dx", "dA", "dB"):
        if act == torch.float32:
            assert_f32_close(got[k], ref[k], k)
        else:
            assert rel_err(got[k], ref[k]) <= BF16_TOL, k


# Degenerate shapes: one or a few outputs (N < 8 sends g and dB to the
# element-wise rows/cols kernels and dx to the fp32-path kernel), rank 1,
# a single token, K of one block.
DEGENERATE_CASES = [
    # M, N, K, r
    (1, 1, 64, 1),
    (5, 3, 64, 2),
    (300, 7, 128, 1),
    (17, 1, 128, 16),
    (300, 1, 64, 128),
    (2, 9, 64, 3),
    (129, 5, 192, 7),
]


@pytest.mark.parametrize("act", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("M,N,K,r", DEGENERATE_CASES)
def test_layer_degenerate_shapes(orc, M, N, K, r, act):
    _say(f"degenerate M={M} N={N} K={K} r={r} act={act}")
    lora = torch.float32 if act == torch.float32 else act
    got, ref = _layer_case(orc, M, N, K, r, True, act, lora)
    if act == torch.float32:
        for k in ("y", "u", "dx", "dA", "dB"):
            assert_f32_close(got[k], ref[k], k)
        return
    tol = F16_TOL if act == torch.float16 else BF16_TOL
    errs = {k: rel_err(got[k], ref[k]) for k in ("y", "u", "dx", "dA", "dB")}
    _say("  rel errors", {k: f"{v:.2e}" for k, v in errs.items()})
    for k, e in errs.items():
        assert e <= tol, (k, e)


# fp16 compute (Gemma lesson 09, sec. 9.3: the dequantised weight and the
# products take the compute dtype; fp16 where bf16 is unavailable): every
# kernel path with fp16 activations, W^ dequantised to fp16 and fp16 (or
# fp32) LoRA factors.
F16_CASES = [
    # M, N, K, r, dq, lora dtype, block   (path exercised)
    (1, 256, 256, 8, True, torch.float16, 64),      # decode GEMV
    (3, 200, 320, 16, False, torch.float32, 64),    # GEMV, ragged N, fp32 factors
    (16, 384, 1024, 16, True, torch.float16, 64),   # GEMV at M = 16
    (5, 64, 14336, 64, True, torch.float16, 64),    # GEMV: 3.5 rounds, r = 64
    (100, 200, 320, 8, False, torch.float32, 64),   # 64-token forward, ragged M and N
    (64, 256, 1024, 16, True, torch.float16, 64),   # 64-token forward with split-K, 64-token dx
    (128, 384, 4096, 16, True, torch.float16, 64),  # one 128-token tile, split-K
    (90, 200, 1088, 8, False, torch.float32, 64),   # 128-token tiles, ragged N and K, fp32 factors
    (300, 384, 384, 16, True, torch.float16, 64),   # 256-token GEMM, ragged M
    (300, 200, 320, 8, False, torch.float32, 64),   # ragged N: guarded tile, fp32-path dx
    (512, 256, 640, 64, True, torch.float16, 64),   # r = 64
    (257, 128, 128, 128, True, torch.float16, 64),  # r = 128
    (64, 64, 64, 5, True, torch.float16, 64),       # rank not a multiple of 8
    (200, 512, 4096, 8, True, torch.float16, 64),   # forward 8 slices
    (130, 4096, 512, 16, True, torch.float16, 64),  # dx 8 slices
    (300, 384, 768, 16, True, torch.float16, 128),  # blocks of 128
    (16, 200, 4352, 16, False, torch.float16, 128), # GEMV, blocks of 128, ragged N
]


@pytest.mark.parametrize("M,N,K,r,dq,lora,block", F16_CASES)
def test_layer_fp16_parity(orc, M, N, K, r, dq, lora, block):
    _say(f"layer fp16 M={M} N={N} K={K} r={r} dq={dq} lora={lora} block={block}")
    got, ref = _layer_case(orc, M, N, K, r, dq, torch.float16, lora, block=block)
    errs = {k: rel_err(got[k], ref[k]) for k in ("y", "u", "dx", "dA", "dB")}
    _say("  rel errors", {k: f"{v:.2e}" for k, v in errs.items()})
    for k, e in errs.items():
        assert e <= F16_TOL, (k, e)


@pytest.mark.parametrize("proj", ["gate", "down"])
def test_mlp8b_config_fp16_sampled(orc, proj):
    """The 8B-shaped MLP projection (2048 tokens, r 16, alpha 32, NF4 +
    double quant) with fp16 compute: y and dx on 32 sampled token rows, dA
    and dB in full."""
    c = si.MLP_8B
    N, K = c["projs"][proj]
    M, r = c["M"], c["r"]
    rows = np.sort(np.random.default_rng(6).choice(M, 32, replace=False))
    rows[0], rows[-1] = 0, M - 1
    _say(f"mlp8b fp16 {proj}: M={M} N={N} K={K}")
    got, ref = _layer_case(orc, M, N, K, r, True, torch.float16, torch.float16,
                           alpha=c["alpha"], seed_cfg=c["config"], rows=rows)
    errs = {k: rel_err(got[k], ref[k]) for k in ("y", "u", "dx", "dA", "dB")}
    _say("  rel errors", {k: f"{v:.2e}" for k, v in errs.items()})
    for k, e in errs.items():
        assert e <= F16_TOL, (k, e)


def test_fp16_tiny_weights_dequantise_to_subnormals(orc):
    """Blocks whose constants are so small that the dequantised fp16 values
    are subnormal (below 2^-14) or round to zero: the fp16 output rounding
    matches the oracle's bit for bit."""
    w = si.normal((8, 256), 1.0, seed=23, dtype=torch.float32)
    w = w * torch.tensor([1e-3, 1e-5, 3e-7, 6e-8, 1e-8, 2.0 ** -24, 1.0, 0.02]).view(8, 1)
    for dq in (False, True):
        _check_quant(orc, w, dq)
        _check_quant(orc, w.to(torch.float16), dq)


@pytest.mark.parametrize("M,N,K,r,act,lora,fwd_splits", [
    (300, 384, 384, 16, torch.bfloat16, torch.bfloat16, False),  # ragged M, two token tiles
    (300, 200, 320, 8, torch.bfloat16, torch.float32, False),    # ragged N, guarded store path
    (257, 128, 128, 128, torch.bfloat16, torch.bfloat16, False), # r = 128 (8 rank chunks)
    (4, 256, 256, 8, torch.float32, torch.float32, False),       # fp32 path
    (16, 384, 1024, 16, torch.bfloat16, torch.bfloat16, False),  # M <= 16: forward took the GEMV
    (300, 384, 384, 16, torch.float16, torch.float16, False),    # fp16 compute
    (100, 200, 320, 8, torch.float16, torch.float32, False),     # fp16, 64-token tiles, fp32 factors
    (48, 200, 320, 8, torch.bfloat16, torch.float32, False),     # few-token forward: u slices + slice sum
    (200, 512, 4096, 8, torch.bfloat16, torch.bfloat16, True),   # the forward splits K, fwd_u does not
])
def test_forward_given_u(orc, M, N, K, r, act, lora, fwd_splits):
    """qlora_linear_fwd_u with the u_save of qlora_linear_fwd reproduces its y
    (bit for bit where both run the same unsplit kernel; within rounding where
    the forward splits the contraction or, up to 128 tokens, sums the slices
    of x W^^T and adds the bypass in a second launch) and the oracle's y."""
    _say(f"fwd_u M={M} N={N} K={K} r={r} act={act} lora={lora}")
    t = si.linear_inputs(91, M, N, K, r, act_dtype=act, w_dtype=act, lora_dtype=lora, sub=M + r)
    d = {k: v.to(DEV) for k, v in t.items()}
    W = q.nf4_quantize(d["W"], double_quant=True)
    u = torch.empty((M, r), dtype=torch.float32, device=DEV)
    y = q.qlora_linear_fwd(d["x"], W, d["A"], d["B"], 32.0, u_save=u)
    y_u = q.qlora_linear_fwd_u(d["x"], W, u, d["B"], 32.0)
    torch.cuda.synchronize()
    if (M > FUSED_MAX_M and not fwd_splits) or act == torch.float32:
        np.testing.assert_array_equal(y_u.float().cpu().numpy(), y.float().cpu().numpy())
    st = orc.quantize_nf4(host(t["W"]), double_quant=True)
    w_hat = orc.dequantize(st).reshape(N, K)
    y_ref, _ = orc.linear_fwd(host(t["x"]), w_hat, host(t["A"]), host(t["B"]), 32.0, r)
    if act == torch.float32:
        assert_f32_close(y_u.cpu().numpy(), y_ref, "y")
    else:
        tol = F16_TOL if act == torch.float16 else BF16_TOL
        assert rel_err(y_u.float().cpu().numpy(), y_ref) <= tol
        _assert_fwd_within16(t, w_hat, 32.0, r, act, y_u, y_ref)


@pytest.mark.parametrize("M", [1, 4, 16])
def test_decode_config_full_size(orc, M):
    """Llama-3-8B attention projection: W 4096x4096 NF4 + double quant,
    r 16, alpha 32, bf16; forward only, every output checked."""
    c = si.DECODE
    N, K, r = c["N"], c["K"], c["r"]
    t = si.linear_inputs(c["config"], M, N, K, r, with_dy=False)
    d = {k: v.to(DEV) for k, v in t.items()}
    W = q.nf4_quantize(d["W"], double_quant=True)
    y = q.qlora_linear_fwd(d["x"], W, d["A"], d["B"], c["alpha"])
    torch.cuda.synchronize()
    st = orc.quantize_nf4(host(t["W"]), double_quant=True)
    np.testing.assert_array_equal(host(W.packed)[:st["packed"].size], st["packed"])
    np.testing.assert_array_equal(host(W.absmax_q)[:st["absmax_q"].size], st["absmax_q"])
    w_hat = orc.dequantize(st).reshape(N, K)
    y_ref, _ = orc.linear_fwd(host(t["x"]), w_hat, host(t["A"]), host(t["B"]), c["alpha"], r)
    e = rel_err(y.float().cpu().numpy(), y_ref)
    _say(f"decode M={M}: rel err {e:.2e}")
    assert e <= BF16_TOL
    _assert_fwd_within16(t, w_hat, c["alpha"], r, torch.bfloat16, y, y_ref)


# Decode-sized forwards (M <= 16) on larger weights, every output and u.
# Every M <= 16 takes the decode path: a weight-streaming launch (64 rows x
# runs of 128-column chunks per workgroup, the contraction split into
# slices; double-quantised weights with K % 128 == 0 load each wave's block
# constants at once) whose first workgroups form u slices, then a launch
# that sums the slices and adds the bypass.  The cases cover one to 56
# slices, runs of 1 to 8 chunks, ragged row sets, fp32 and 16-bit factors,
# both storage forms and both compute formats.
DECODE_LARGE_CASES = [
    # M, N, K, r, act, lora dtype, double quant
    (1, 8192, 4096, 16, torch.bfloat16, torch.bfloat16, True),
    (3, 8192, 4096, 16, torch.bfloat16, torch.bfloat16, True),
    (8, 8192, 4096, 16, torch.bfloat16, torch.float32, False),
    (16, 8192, 4096, 32, torch.bfloat16, torch.bfloat16, True),
    (5, 8192, 4096, 32, torch.float16, torch.float32, True),
    (16, 8192, 4096, 64, torch.bfloat16, torch.bfloat16, True),
    (1, 14336, 4096, 16, torch.bfloat16, torch.bfloat16, True),
    (1, 14336, 4096, 32, torch.float16, torch.float16, False),
    (3, 14336, 4096, 16, torch.bfloat16, torch.bfloat16, True),
    (16, 14336, 4096, 16, torch.float16, torch.float16, True),
    (4, 4096, 14336, 16, torch.bfloat16, torch.bfloat16, True),
    (16, 4096, 14336, 16, torch.bfloat16, torch.bfloat16, True),
    (2, 2048, 28672, 16, torch.bfloat16, torch.bfloat16, True),
    (1, 1024, 14336, 32, torch.bfloat16, torch.float32, False),
    (16, 2048, 16384, 16, torch.float16, torch.float16, True),
    (1, 8192, 28672, 64, torch.bfloat16, torch.bfloat16, True),   # 70B down shape, one token
]


@pytest.mark.parametrize("M,N,K,r,act,lora,dq", DECODE_LARGE_CASES)
def test_decode_large_weights(orc, M, N, K, r, act, lora, dq):
    _say(f"decode-sized M={M} N={N} K={K} r={r} act={act} lora={lora} dq={dq}")
    t = si.linear_inputs(97, M, N, K, r, act_dtype=act, w_dtype=act, lora_dtype=lora,
                         with_dy=False, sub=M + r)
    d = {k: v.to(DEV) for k, v in t.items()}
    W = q.nf4_quantize(d["W"], double_quant=dq)
    u = torch.empty((M, r), dtype=torch.float32, device=DEV)
    y = q.qlora_linear_fwd(d["x"], W, d["A"], d["B"], 32.0, u_save=u)
    torch.cuda.synchronize()
    st = orc.quantize_nf4(host(t["W"]), double_quant=dq)
    np.testing.assert_array_equal(host(W.packed)[:st["packed"].size], st["packed"])
    w_hat = orc.dequantize(st).reshape(N, K)
    y_ref, u_ref = orc.linear_fwd(host(t["x"]), w_hat, host(t["A"]), host(t["B"]), 32.0, r)
    tol = F16_TOL if act == torch.float16 else BF16_TOL
    ey, eu = rel_err(y.float().cpu().numpy(), y_ref), rel_err(u.cpu().numpy(), u_ref)
    _say(f"  rel err y {ey:.2e} u {eu:.2e}")
    assert ey <= tol and eu <= tol
    _assert_fwd_within16(t, w_hat, 32.0, r, act, y, y_ref, u, u_ref)


# Decode-sized forwards with blocks of 128 (the per-element constant path of
# the streaming kernel) on long contractions.
DECODE_BLOCK128_CASES = [
    # M, N, K, r, act, lora dtype, double quant
    (2, 2048, 28672, 16, torch.bfloat16, torch.bfloat16, True),
    (16, 1024, 14336, 64, torch.float16, torch.float16, False),
    (1, 200, 8192, 5, torch.bfloat16, torch.float32, True),
]


@pytest.mark.parametrize("M,N,K,r,act,lora,dq", DECODE_BLOCK128_CASES)
def test_decode_block128_long_contraction(orc, M, N, K, r, act, lora, dq):
    _say(f"decode block 128 M={M} N={N} K={K} r={r} act={act} lora={lora} dq={dq}")
    t = si.linear_inputs(98, M, N, K, r, act_dtype=act, w_dtype=act, lora_dtype=lora,
                         with_dy=False, sub=M + r)
    d = {k: v.to(DEV) for k, v in t.items()}
    W = q.nf4_quantize(d["W"], double_quant=dq, block=128)
    u = torch.empty((M, r), dtype=torch.float32, device=DEV)
    y = q.qlora_linear_fwd(d["x"], W, d["A"], d["B"], 16.0, u_save=u)
    torch.cuda.synchronize()
    st = orc.quantize_nf4(host(t["W"]), double_quant=dq, block=128)
    np.testing.assert_array_equal(host(W.packed)[:st["packed"].size], st["packed"])
    w_hat = orc.dequantize(st).reshape(N, K)
    y_ref, u_ref = orc.linear_fwd(host(t["x"]), w_hat, host(t["A"]), host(t["B"]), 16.0, r)
    tol = F16_TOL if act == torch.float16 else BF16_TOL
    ey, eu = rel_err(y.float().cpu().numpy(), y_ref), rel_err(u.cpu().numpy(), u_ref)
    _say(f"  rel err y {ey:.2e} u {eu:.2e}")
    assert ey <= tol and eu <= tol
    _assert_fwd_within16(t, w_hat, 16.0, r, act, y, y_ref, u, u_ref)


@pytest.mark.parametrize("proj", ["gate", "down"])
def test_mlp8b_config_full_size_sampled(orc, proj):
    """8B-shaped MLP projection at M = 2048 tokens, r 16, alpha 32, NF4 +
    double quant: y and dx on 64 sampled token rows, dA and dB in full."""
    c = si.MLP_8B
    N, K = c["projs"][proj]
    M, r = c["M"], c["r"]
    rows = np.sort(np.random.default_rng(3).choice(M, 64, replace=False))
    rows[0], rows[-1] = 0, M - 1
    _say(f"mlp8b {proj}: M={M} N={N} K={K}")
    got, ref = _layer_case(orc, M, N, K, r, True, torch.bfloat16, torch.bfloat16,
                           alpha=c["alpha"], seed_cfg=c["config"], rows=rows)
    errs = {k: rel_err(got[k], ref[k]) for k in ("y", "u", "dx", "dA", "dB")}
    _say("  rel errors", {k: f"{v:.2e}" for k, v in errs.items()})
    for k, e in errs.items():
        assert e <= BF16_TOL, (k, e)


@pytest.mark.parametrize("M", [128, 512, 1024])
@pytest.mark.parametrize("proj", ["gate", "down"])
def test_mlp8b_shape_few_tokens_sampled(orc, proj, M):
    """8B-shaped MLP projection at 128, 512 and 1024 tokens (the split-K
    launches, and at 1024 the 256-wide tiles with and without split-K): y
    and dx on 32 sampled token rows, dA and dB in full."""
    c = si.MLP_8B
    N, K = c["projs"][proj]
    r = c["r"]
    rows = np.sort(np.random.default_rng(5).choice(M, 32, replace=False))
    rows[0], rows[-1] = 0, M - 1
    _say(f"mlp8b {proj}: M={M} N={N} K={K}")
    got, ref = _layer_case(orc, M, N, K, r, True, torch.bfloat16, torch.bfloat16,
                           alpha=c["alpha"], seed_cfg=c["config"], rows=rows)
    errs = {k: rel_err(got[k], ref[k]) for k in ("y", "u", "dx", "dA", "dB")}
    _say("  rel errors", {k: f"{v:.2e}" for k, v in errs.items()})
    for k, e in errs.items():
        assert e <= BF16_TOL, (k, e)


@pytest.mark.parametrize("proj", ["gate", "down"])
def test_mlp70b_config_full_size_sampled(orc, proj):
    """70B-shaped MLP projection at M = 4096 tokens, r 64, alpha 16 (s = 0.25),
    NF4 + double quant: y and dx on 32 sampled token rows, dA and dB in full."""
    c = si.MLP_70B
    N, K = c["projs"][proj]
    M, r = c["M"], c["r"]
    rows = np.sort(np.random.default_rng(4).choice(M, 32, replace=False))
    rows[0], rows[-1] = 0, M - 1
    _say(f"mlp70b {proj}: M={M} N={N} K={K}")
    got, ref = _layer_case(orc, M, N, K, r, True, torch.bfloat16, torch.bfloat16,
                           alpha=c["alpha"], seed_cfg=c["config"], rows=rows)
    errs = {k: rel_err(got[k], ref[k]) for k in ("y", "u", "dx", "dA", "dB")}
    _say("  rel errors", {k: f"{v:.2e}" for k, v in errs.items()})
    for k, e in errs.items():
        assert e <= BF16_TOL, (k, e)


@pytest.mark.parametrize("M,N,K,r", [
    (1000, 28608, 4096, 64),   # g: several factor chunks per workgroup, the last ragged;
                               # dB: several token runs per workgroup, the last ragged
    (1000, 4096, 28544, 64),   # u and dA: the same over the contraction K
    (900, 22000, 1024, 18),    # dB with r % 4 != 0 (one value per R load), two runs
])
def test_lora_products_multi_chunk_ragged(orc, M, N, K, r):
    """The LoRA products (u, g, dA, dB) where a workgroup covers several
    contraction chunks or token runs and the last one is cut short: y and dx
    on 32 sampled token rows, dA and dB in full, every output within its
    per-element bound."""
    rows = np.sort(np.random.default_rng(6).choice(M, 32, replace=False))
    rows[0], rows[-1] = 0, M - 1
    _say(f"lora multi-chunk M={M} N={N} K={K} r={r}")
    got, ref = _layer_case(orc, M, N, K, r, True, torch.bfloat16, torch.bfloat16,
                           alpha=16.0, rows=rows)
    errs = {k: rel_err(got[k], ref[k]) for k in ("y", "u", "dx", "dA", "dB")}
    _say("  rel errors", {k: f"{v:.2e}" for k, v in errs.items()})
    for k, e in errs.items():
        assert e <= BF16_TOL, (k, e)


@pytest.mark.parametrize("layer", [0, 31])
def test_weightset_layer_bit_exact(orc, layer):
    """8B-shaped weight set (N(0, 0.02) with 0.1% outliers at 20 sigma): every
    tensor of one layer quantised (+ double quant) and dequantised bit-exactly;
    bits/param as the pages' arithmetic says."""
    for name in si.WEIGHTSET_8B["shapes"]:
        w = si.weightset_tensor(layer, name, device=DEV)
        _say(f"weight set layer {layer} {name} {tuple(w.shape)}")
        Wq = q.nf4_quantize(w, double_quant=True)
        deq = q.nf4_dequantize(Wq, torch.bfloat16)
        torch.cuda.synchronize()
        st = orc.quantize_nf4(host(w).reshape(-1), double_quant=True)
        np.testing.assert_array_equal(host(Wq.packed)[:st["packed"].size], st["packed"])
        np.testing.assert_array_equal(host(Wq.absmax_q)[:st["absmax_q"].size], st["absmax_q"])
        np.testing.assert_array_equal(host(Wq.absmax_scale)[:st["absmax_scale"].size], st["absmax_scale"])
        assert host(Wq.absmax_mean)[0] == st["absmax_mean"]
        np.testing.assert_array_equal(host(deq).reshape(-1), orc.round_bf16(orc.dequantize(st)))
        assert abs(orc.bits_per_param(st) - (4 + 8 / 64 + 32 / 16384 + 32 / w.numel())) < 1e-12
