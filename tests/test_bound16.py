"""The derived 16-bit bound (helpers.bound16) admits an evaluation of the
layer with the kernels' roundings -- weights and rank-r operands rounded to
the 16-bit format, fp32 accumulation, one output rounding -- and rejects one
with a single term of a dot product left out (CPU; numpy's fp32 products
stand in for the fp32 accumulation, the oracle gives the exact values and
the 16-bit roundings)."""
import numpy as np
import pytest
import torch

import synth_inputs as si
from tests.helpers import (U_BF16, U_F16, assert_16bit_within, f64, host, layer_bounds16,
                           rel_err, BF16_TOL)

FMT = {"bf16": (torch.bfloat16, U_BF16), "f16": (torch.float16, U_F16)}


def _round16(orc, a, fmt):
    a = np.asarray(a, np.float32)
    return f64(orc.round_bf16(a)) if fmt == "bf16" else orc.round_f16(a).astype(np.float64)


def _case(orc, fmt, M, N, K, r, alpha=32.0):
    act, u16 = FMT[fmt]
    t = si.linear_inputs(77, M, N, K, r, act_dtype=act, w_dtype=act, lora_dtype=act)
    x, A, B, dy = (host(t[k]) for k in ("x", "A", "B", "dy"))
    st = orc.quantize_nf4(host(t["W"]).reshape(-1), double_quant=True)
    w = orc.dequantize(st).reshape(N, K)
    y_ref, u_ref = orc.linear_fwd(x, w, A, B, alpha, r)
    dx_ref, _, _ = orc.linear_bwd(x, w, A, B, dy, alpha, r)
    s = np.float32(alpha) / np.float32(r)
    f32 = lambda a: np.asarray(a, np.float32)
    xf, Af, Bf, dyf = f64(x), f64(A), f64(B), f64(dy)
    w16 = _round16(orc, w, fmt)
    # the kernels' arithmetic: 16-bit operands, fp32 accumulation, 16-bit output
    u32 = f32(xf) @ f32(Af).T
    y32 = f32(xf) @ f32(w16).T + f32(_round16(orc, s * u32, fmt)) @ f32(Bf).T
    g32 = np.float32(s) * (f32(dyf) @ f32(Bf))
    dx32 = f32(dyf) @ f32(w16) + f32(_round16(orc, g32, fmt)) @ f32(Af)
    emu = {"y": _round16(orc, y32, fmt), "dx": _round16(orc, dx32, fmt)}
    ref = {"y": y_ref, "dx": dx_ref}
    bounds = layer_bounds16(x, w, A, B, float(s), dy=dy)
    terms = {"y": (xf, w), "dx": (dyf, w.T)}  # y[m, n] = sum_k x[m, k] w[n, k]
    return emu, ref, bounds, terms, u16


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("M,N,K,r", [(48, 256, 4096, 16), (16, 96, 14336, 64)])
def test_bound16_admits_the_kernel_roundings(orc, fmt, M, N, K, r):
    emu, ref, bounds, _, u16 = _case(orc, fmt, M, N, K, r)
    for k in ("y", "dx"):
        sq, mag, n, lin = bounds[k]
        assert_16bit_within(emu[k], ref[k], sq, mag, n, u16, k, lin)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_bound16_rejects_one_dropped_term(orc, fmt):
    """Leave out of one output the term at the 90th percentile of |term| of
    its dot product (and, separately, the largest one): the bound fails,
    while for the 4096-long forward dot products the normalised measure of
    the same error stays inside 2e-2."""
    M, N, K, r = 48, 256, 4096, 16
    emu, ref, bounds, terms, u16 = _case(orc, fmt, M, N, K, r)
    for k in ("y", "dx"):
        sq, mag, n, lin = bounds[k]
        a, b = terms[k]
        for (m, j) in ((5, 7), (31, 200)):
            t = a[m] * b[j]
            order = np.argsort(np.abs(t))
            for q in (0.9, 1.0):
                kk = order[min(len(t) - 1, int(q * len(t)))]
                bad = emu[k].copy()
                bad[m, j] -= t[kk]
                with pytest.raises(AssertionError):
                    assert_16bit_within(bad, ref[k], sq, mag, n, u16, f"{k} without one term", lin)
                if q == 0.9 and k == "y":  # 4096-long dot products
                    assert rel_err(bad, ref[k]) < BF16_TOL  # the normalised measure passes it
