"""Small helpers shared by the tests (no arithmetic of the layer itself)."""
import math

import numpy as np
import torch


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bfloat16 tensor -> numpy uint16 bit patterns (host copy)."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    """Host numpy view of a tensor; bf16 becomes uint16 bit patterns (fp16
    stays numpy float16)."""
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    return t.contiguous().cpu().numpy()


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max(max |ref|, rms(ref)): the bf16 tolerance measure
    (plain relative error is ill-posed where ref cancels to ~0)."""
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    denom = max(float(np.max(np.abs(ref))), float(np.sqrt(np.mean(ref ** 2))), 1e-30)
    return float(np.max(np.abs(got - ref))) / denom


BF16_TOL = 2e-2        # bf16 activations: max rel error against the fp64 oracle
F16_TOL = 2.5e-3       # fp16 activations: BF16_TOL x 2^-11 / 2^-8 (the unit roundoff ratio)
F32_ATOL = 1e-5        # fp32 activations: |d| <= atol + rtol |ref| (allclose defaults)
F32_RTOL = 1e-5


def assert_f32_close(got: np.ndarray, ref: np.ndarray, what: str):
    excess = np.abs(np.asarray(got, np.float64) - ref) - (F32_ATOL + F32_RTOL * np.abs(ref))
    assert np.all(excess <= 0), f"{what}: max excess over atol+rtol|ref| = {excess.max():.3e}"


# fp32 compute at sizes where a fixed atol no longer fits the magnitudes:
# the probabilistic bound of Higham and Mary ("A new approach to
# probabilistic rounding error analysis", SIAM J. Sci. Comput. 41(5), 2019,
# Thm. 2.4) for a value computed by a chain of n fp32 roundings, any
# summation order (the inner-product bound, applied along the chain of
# roundings that reaches the output): |got - exact| <= g~_n(lam) * mag, where
# mag is the same expression evaluated on absolute values, g~_n(lam) =
# exp(lam sqrt(n) u + n u^2 / (1 - u)) - 1 and u = 2^-24.  Under that
# paper's model of independent mean-zero rounding errors an element fails
# with probability below 2 n exp(-lam^2 (1 - u)^2 / 2) (~1e-10 at lam = 8,
# n = 4000); the fp64 oracle's own error is below 2^-40 mag.
F32_LAMBDA = 8.0


def gamma_prob_f32(n: int, lam: float = F32_LAMBDA) -> float:
    u = 2.0 ** -24
    return math.expm1(lam * math.sqrt(n) * u + n * u * u / (1.0 - u))


def f32_chain(out, M, N, K, r):
    """Roundings on the longest path to each fp32 output of the layer (sums of
    n terms count n; scalings and the final additions one each; 4 spare for
    partial sums scaled before their reduction, such as the dropout's
    1/(1-p)): u = x A^T, y = x W^T + s u B^T, g = s dy B, dx = dy W + g A,
    dA = g^T x, dB = s dy^T u."""
    return {"u": K, "y": K + r + 2, "dx": N + r + 2, "dA": N + 1 + M,
            "dB": K + M + 1}[out] + 4


def assert_f32_within(got: np.ndarray, ref: np.ndarray, mag: np.ndarray, n: int, what: str):
    bound = gamma_prob_f32(n) * np.asarray(mag, np.float64) + 2.0 ** -40 * np.abs(ref)
    excess = np.abs(np.asarray(got, np.float64) - ref) - bound
    i = int(np.argmax(excess))
    assert np.all(excess <= 0), (f"{what}: |d| exceeds the fp32 bound (n = {n}) by "
                                 f"{excess.flat[i]:.3e} at flat index {i}")


# 16-bit compute (bf16, fp16): a per-element bound derived from the roundings
# the kernels make.  Products of 16-bit values are exact in fp32; what is
# rounded is (a) each weight operand to the 16-bit format (the dequantised
# value, or the codebook value of the unscaled table: relative error <= u16
# per element), (b) the fp32 rank-r operands s u and g (and fp32 factors) to
# the 16-bit format before their matrix steps (<= u16 each, both operands of
# a product: 2 u16), (c) the fp32 accumulation chains (the Higham-Mary fp32
# term above) and (d) the output, once, to 16 bits (<= u16 |y|).  The operand
# roundings enter an output as sum_k a_k b_k d_k with |d_k| <= u16 (2 u16);
# with the roundings modelled as independent and mean-zero (as for fp32),
# |sum| <= lam u16 sqrt(sum_k (a_k b_k)^2) except with probability below
# 2 exp(-lam^2 / 2) (Hoeffding; 5e-11 at lam = 7).  sq carries the sum of
# squared terms, with weight 4 on the rank-r ones.  Unlike the normalised 2e-2
# measure, this is per element: one dropped term larger than about one rms
# term of its dot product fails it (tests/test_bound16.py).
U_BF16 = 2.0 ** -9
U_F16 = 2.0 ** -11
LAM16 = 7.0


def f64(a) -> np.ndarray:
    """fp64 values of host data: bf16 bit patterns (uint16), fp16 or fp32."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def eta16(u16: float) -> float:
    """Half the smallest subnormal of the 16-bit format: the absolute error of
    a rounding into its subnormal range."""
    return 2.0 ** -25 if u16 == U_F16 else 2.0 ** -134


def bound16(ref, sq, mag, n: int, u16: float, lin=0.0, lam: float = LAM16) -> np.ndarray:
    """lin: 1 + the sum of the |other operand| over every rounded operand of
    the output (each rounding may be absolute, eta16, in the subnormal range)."""
    ref = np.abs(np.asarray(ref, np.float64))
    core = lam * u16 * np.sqrt(sq) + gamma_prob_f32(n) * np.asarray(mag, np.float64)
    return core + u16 * (ref + core) + eta16(u16) * (1.0 + np.asarray(lin)) + 2.0 ** -40 * ref


def assert_16bit_within(got, ref, sq, mag, n: int, u16: float, what: str, lin=0.0):
    excess = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64)) - bound16(
        ref, sq, mag, n, u16, lin)
    i = int(np.argmax(excess))
    assert np.all(excess <= 0), (f"{what}: |d| exceeds the 16-bit bound by {excess.flat[i]:.3e} "
                                 f"at flat index {i}")


def layer_bounds16(x, w_hat, A, B, s: float, dy=None, rows=None) -> dict:
    """(sq, mag, n) of y and u (on `rows`), dx (on `rows`), dA and dB of the
    layer y = x W^T + s (x A^T) B^T, from host inputs (bf16 patterns, fp16 or
    fp32) and the fp32 dequantised weight."""
    xf, wf, Af, Bf = f64(x), np.asarray(w_hat, np.float64), f64(A), f64(B)
    K, r = xf.shape[1], Af.shape[0]
    sel = slice(None) if rows is None else rows
    ax, aw, aA, aB = np.abs(xf), np.abs(wf), np.abs(Af), np.abs(Bf)
    u = xf @ Af.T
    # squared terms of u and g themselves: an fp32 factor rounded to 16 bits
    # inside them passes its error on to every output they feed
    uu = (xf ** 2) @ (Af ** 2).T
    sx = ax.sum(1, keepdims=True)
    out = {
        "y": ((xf[sel] ** 2) @ (wf ** 2).T
              + 4 * ((s * u[sel]) ** 2 + s * s * uu[sel]) @ (Bf ** 2).T,
              ax[sel] @ aw.T + abs(s) * (ax[sel] @ aA.T) @ aB.T, K + r,
              sx[sel] + aB.sum(1)[None, :] + abs(s) * sx[sel] * aB.sum(1)[None, :]),
        # u is an fp32 output; the factors may be rounded to 16 bits for it
        "u": (4 * (xf[sel] ** 2) @ (Af ** 2).T, ax[sel] @ aA.T, K, sx[sel]),
    }
    if dy is not None:
        dyf = f64(dy)
        N, M = dyf.shape[1], dyf.shape[0]
        g = s * (dyf @ Bf)
        gg = (dyf ** 2) @ (Bf ** 2)
        ady = np.abs(dyf)
        sdy = ady.sum(1, keepdims=True)
        out["dx"] = ((dyf[sel] ** 2) @ (wf ** 2) + 4 * (g[sel] ** 2 + s * s * gg[sel]) @ (Af ** 2),
                     ady[sel] @ aw + abs(s) * (ady[sel] @ aB) @ aA, N + r,
                     sdy[sel] + aA.sum(0)[None, :] + abs(s) * sdy[sel] * aA.sum(0)[None, :])
        out["dA"] = (4 * (g ** 2 + s * s * gg).T @ (xf ** 2), abs(s) * (ady @ aB).T @ ax, N + M,
                     ax.sum(0)[None, :] * (1 + abs(s) * sdy.sum()))
        out["dB"] = (4 * (dyf ** 2).T @ ((s * u) ** 2 + s * s * uu), abs(s) * ady.T @ (ax @ aA.T),
                     K + M, ady.sum(0)[:, None] * abs(s) * (1 + sx.sum()))
    return out


def assert_layer_within16(got: dict, ref: dict, bounds: dict, u16: float):
    """Every output of the layer present in got within bound16."""
    for k, (sq, mag, n, lin) in bounds.items():
        if k in got:
            assert_16bit_within(got[k], ref[k], sq, mag, n, u16, k, lin)
