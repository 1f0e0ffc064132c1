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


def assert_f32_within(got: np.ndarray, ref: np.ndarray, mag: np.ndarray, n: int, what: str):
    bound = gamma_prob_f32(n) * np.asarray(mag, np.float64) + 2.0 ** -40 * np.abs(ref)
    excess = np.abs(np.asarray(got, np.float64) - ref) - bound
    i = int(np.argmax(excess))
    assert np.all(excess <= 0), (f"{what}: |d| exceeds the fp32 bound (n = {n}) by "
                                 f"{excess.flat[i]:.3e} at flat index {i}")
