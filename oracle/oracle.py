"""CPU oracle for the QLoRA quantized linear layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  It shares nothing with the GPU library: the arithmetic
lives in ``nf4_oracle.c`` (plain C, fp64 accumulation) and in the few lines
below that say so.

Every function cites the passage of the pages it follows, by page title and
section:
  [ch26] "26. QLoRA and 4bit Quantization" (datawhalechina), Steps 2-4.
  [ch22] "22. QLoRA and 4bit Quantization" (datawhalechina), Steps 1-4 and
         the engineering notes.
  [L9]   Gemma tutorial lesson 09 "QLoRA 4-bit quantised fine-tuning"
         (agentupdate.ai), sections 9.2.1 and 9.2.2.
  [gc4]  gufacode fine-tuning chapter 4, "three core techniques of QLoRA".

bfloat16 tensors travel as numpy uint16 bit patterns, fp16 tensors as numpy
float16.

Parity pins live in tests/test_oracle_pins.py.  Double-quantisation bit
patterns and large-shape GEMM values have no printed value to compare with:
they are pinned by the definitions, invariants and brute force on small
shapes only.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_f32 = ctypes.c_float
_f64 = ctypes.c_double


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build  # noqa: WPS433 (test infrastructure)
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.orc_codebook.argtypes = [_p]
    lib.orc_nearest_index.argtypes = [_f32]
    lib.orc_nearest_index.restype = ctypes.c_int
    lib.orc_nf4_quantize.argtypes = [_p, _i64, _i32, _p, _p]
    lib.orc_dq_codes.argtypes = [_p, _i64, _f32, _i32, _p, _p]
    lib.orc_nf4_dequantize.argtypes = [_p, _i64, _i32, _p, _p, _p, _f32, _i32, _p]
    lib.orc_round_bf16.argtypes = [_p, _i64, _p]
    lib.orc_round_f16.argtypes = [_p, _i64, _p]
    lib.orc_linear_fwd.argtypes = [_i64, _i64, _i64, _i32, _f64, _p, _p, _p, _p, _p, _p, _p]
    lib.orc_linear_bwd.argtypes = [_i64, _i64, _i64, _i32, _f64, _p, _p, _p, _p, _p, _p,
                                   _p, _i64, _p, _p, _p, _p, _p]
    lib.orc_philox4x32_10.argtypes = [_p, _p, _p]
    lib.orc_dropout_keep.argtypes = [_i64, _i64, ctypes.c_uint32, ctypes.c_uint64, _p]
    lib.orc_adamw_step.argtypes = [_p, _p, _p, _p, _p, _i64, _f32, _f32, _f32, _f32, _f32, _f32,
                                   _f32, _f32]
    lib.orc_num_threads.restype = ctypes.c_int
    lib.orc_set_num_threads.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle needs contiguous arrays"
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_load().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Host threads of the oracle's parallel loops (for timing; results do
    not depend on it)."""
    _load().orc_set_num_threads(int(n))


# ---------------------------------------------------------------------------
# bf16 bit patterns <-> fp32 (exact widening; the rounding direction is the
# oracle's own RNE in C)
# ---------------------------------------------------------------------------
def bf16_to_f32(u16: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(u16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().orc_round_bf16(_ptr(x), x.size, _ptr(out))
    return out


def round_f16(x: np.ndarray) -> np.ndarray:
    """fp32 -> IEEE binary16 (numpy float16 values), round to nearest even;
    the rounding is the oracle's own, in C, written from the format's
    definition (Gemma lesson 09, sec. 9.3 names fp16 as a compute dtype)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().orc_round_f16(_ptr(x), x.size, _ptr(out))
    return out.view(np.float16)


def as_f32(w: np.ndarray) -> np.ndarray:
    """Weights/activations given as fp32, fp16 (numpy float16; widening is
    exact) or as bf16 bit patterns (uint16)."""
    if w.dtype == np.uint16:
        return bf16_to_f32(w)
    return np.ascontiguousarray(w, dtype=np.float32)


# ---------------------------------------------------------------------------
# NF4 format
# ---------------------------------------------------------------------------
def codebook() -> np.ndarray:
    """[ch26] Step 4 / [ch22] Step 4: the printed 16-entry NF4 table."""
    out = np.empty(16, dtype=np.float32)
    _load().orc_codebook(_ptr(out))
    return out


def nearest_index(v: float) -> int:
    """[ch26] Step 2: nearest codepoint of a normalised value, ties low."""
    return int(_load().orc_nearest_index(float(np.float32(v))))


def quantize(w: np.ndarray, block: int = 64):
    """[L9] 9.2.1 block-wise quantisation; [ch22] Step 4 two indices per byte.

    Returns (packed uint8[ceil(n/2)], absmax fp32[ceil(n/block)])."""
    assert block % 2 == 0
    wf = as_f32(w).reshape(-1)
    n = wf.size
    nb = (n + block - 1) // block
    packed = np.empty((n + 1) // 2, dtype=np.uint8)
    absmax = np.empty(nb, dtype=np.float32)
    _load().orc_nf4_quantize(_ptr(wf), n, block, _ptr(packed), _ptr(absmax))
    return packed, absmax


def unpack_indices(packed: np.ndarray, n: int) -> np.ndarray:
    """Inverse of the packing: element 2j is the high nibble of byte j."""
    hi = packed >> 4
    lo = packed & 15
    out = np.empty(2 * packed.size, dtype=np.uint8)
    out[0::2] = hi
    out[1::2] = lo
    return out[:n]


def dq_mean(absmax: np.ndarray) -> np.float32:
    """[L9] 9.2.2 double quantisation, centring term: the mean of the block
    constants, from their exact sum (math.fsum), divided in fp64 and rounded
    once to fp32."""
    a = np.ascontiguousarray(absmax, dtype=np.float32).astype(np.float64)
    if a.size == 0:
        return np.float32(0.0)
    return np.float32(math.fsum(a.tolist()) / a.size)


def dq_codes(absmax: np.ndarray, mu: np.float32, block2: int = 256):
    """[L9] 9.2.2: 8-bit integer codes of the centred constants, one fp32
    scale per block2 constants.  Returns (q int8[nb], sigma fp32[nb2])."""
    a = np.ascontiguousarray(absmax, dtype=np.float32)
    nb = a.size
    nb2 = (nb + block2 - 1) // block2
    q = np.empty(nb, dtype=np.int8)
    sigma = np.empty(nb2, dtype=np.float32)
    _load().orc_dq_codes(_ptr(a), nb, float(mu), block2, _ptr(q), _ptr(sigma))
    return q, sigma


def quantize_nf4(w: np.ndarray, double_quant: bool, block: int = 64, block2: int = 256) -> dict:
    """Full NF4 storage of a weight: indices + (absmax | q, sigma, mu)."""
    packed, absmax = quantize(w, block)
    out = {"packed": packed, "n": int(np.asarray(w).size), "block": block, "block2": block2,
           "double_quant": bool(double_quant)}
    if double_quant:
        mu = dq_mean(absmax)
        q, sigma = dq_codes(absmax, mu, block2)
        out.update(absmax_q=q, absmax_scale=sigma, absmax_mean=mu, absmax_raw=absmax)
    else:
        out.update(absmax=absmax)
    return out


def dequantize(st: dict) -> np.ndarray:
    """[ch26] Step 4 table[idx] * scale, with the scale rebuilt from its
    8-bit code as fmaf(q, sigma, mu) when double-quantised.  fp32 result."""
    lib = _load()
    n = st["n"]
    out = np.empty(n, dtype=np.float32)
    if st["double_quant"]:
        lib.orc_nf4_dequantize(_ptr(st["packed"]), n, st["block"], None, _ptr(st["absmax_q"]),
                               _ptr(st["absmax_scale"]), float(st["absmax_mean"]),
                               st["block2"], _ptr(out))
    else:
        lib.orc_nf4_dequantize(_ptr(st["packed"]), n, st["block"], _ptr(st["absmax"]), None,
                               None, 0.0, st["block2"], _ptr(out))
    return out


def bits_per_param(st: dict) -> float:
    """Storage bits per parameter of a quantised weight ([gc4])."""
    n = st["n"]
    b = st["packed"].size
    if st["double_quant"]:
        b += st["absmax_q"].size + 4 * st["absmax_scale"].size + 4
    else:
        b += 4 * st["absmax"].size
    return 8.0 * b / n


# ---------------------------------------------------------------------------
# The layer
# ---------------------------------------------------------------------------
def _as_f64(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(as_f32(a), dtype=np.float64)


def philox4x32_10(ctr, key) -> np.ndarray:
    """Philox4x32-10 (Salmon et al., SC'11) of one 4-word counter and 2-word key."""
    c = np.ascontiguousarray(ctr, dtype=np.uint32).reshape(4)
    k = np.ascontiguousarray(key, dtype=np.uint32).reshape(2)
    out = np.empty(4, dtype=np.uint32)
    _load().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def dropout_params(p: float):
    """LoRA dropout (the pages' LoraConfig lora_dropout) as the layer applies
    it: keep threshold floor(p 2^32) on a 32-bit draw, and the inverted
    scale fp32(1 / (1 - p)) of the kept inputs."""
    assert 0.0 <= p < 1.0
    return int(math.floor(p * 4294967296.0)), np.float32(1.0 / (1.0 - p))


def dropout_keep(M: int, K: int, p: float, seed: int) -> np.ndarray:
    """keep [M, K] (uint8 0/1) of the bypass input: element m K + k is kept
    when word (m K + k) % 4 of Philox4x32-10 at counter ((m K + k) / 4, 0, 0)
    with key = the 64-bit seed is >= floor(p 2^32)."""
    thr, _ = dropout_params(p)
    keep = np.empty((M, K), dtype=np.uint8)
    _load().orc_dropout_keep(M, K, thr, seed, _ptr(keep))
    return keep


def dropout_mult(M: int, K: int, p: float, seed: int) -> np.ndarray:
    """The dropout multipliers d [M, K] (fp64): 0 or fp32(1/(1-p))."""
    _, scale = dropout_params(p)
    return dropout_keep(M, K, p, seed).astype(np.float64) * float(scale)


def linear_fwd(x, w_hat: np.ndarray, A, B, alpha: float, r: int, drop=None):
    """[ch26] Step 3: y = x W^T + (alpha/r) (x A^T) B^T, fp64 accumulation.

    x [M,K], w_hat [N,K] fp32 (dequantised), A [r,K], B [N,r]; x/A/B may be
    fp32 or bf16 bit patterns.  drop: optional dropout multipliers d [M,K]
    of the bypass input (u = (d .* x) A^T).  Returns (y [M,N], u [M,r]) in
    fp64."""
    assert r <= 512
    xd = _as_f64(x)
    M, K = xd.shape
    wf = np.ascontiguousarray(w_hat, dtype=np.float32).reshape(-1, K)
    N = wf.shape[0]
    Ad = _as_f64(A).reshape(r, K)
    Bd = _as_f64(B).reshape(N, r)
    s = float(np.float32(alpha) / np.float32(r))
    y = np.empty((M, N), dtype=np.float64)
    u = np.empty((M, r), dtype=np.float64)
    dd = None if drop is None else np.ascontiguousarray(drop, dtype=np.float64).reshape(M, K)
    _load().orc_linear_fwd(M, N, K, r, s, _ptr(xd), _ptr(wf), _ptr(Ad), _ptr(Bd), _ptr(dd),
                           _ptr(y), _ptr(u))
    return y, u


def linear_bwd(x, w_hat: np.ndarray, A, B, dy, alpha: float, r: int, rows=None, want_dx=True,
               drop=None):
    """[ch22] Step 1 (gradients reach x, A, B; none for the frozen base):
    dB = s dy^T u, dA = g^T xd, dx = dy W + d .* (g A), with xd = d .* x the
    bypass input after dropout (xd = x without it), u = xd A^T, g = s dy B.

    rows: optional token-row indices for which dx is produced (dA and dB
    always use every row).  Returns (dx [len(rows) or M, K] | None, dA, dB)."""
    xd = _as_f64(x)
    M, K = xd.shape
    wf = np.ascontiguousarray(w_hat, dtype=np.float32).reshape(-1, K)
    N = wf.shape[0]
    Ad = _as_f64(A).reshape(r, K)
    Bd = _as_f64(B).reshape(N, r)
    dyd = _as_f64(dy).reshape(M, N)
    s = float(np.float32(alpha) / np.float32(r))
    rows_arr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nr = M if rows_arr is None else rows_arr.size
    dx = np.empty((nr, K), dtype=np.float64) if want_dx else None
    dA = np.empty((r, K), dtype=np.float64)
    dB = np.empty((N, r), dtype=np.float64)
    ub = np.empty((M, r), dtype=np.float64)
    gb = np.empty((M, r), dtype=np.float64)
    dd = None if drop is None else np.ascontiguousarray(drop, dtype=np.float64).reshape(M, K)
    _load().orc_linear_bwd(M, N, K, r, s, _ptr(xd), _ptr(wf), _ptr(Ad), _ptr(Bd), _ptr(dd), _ptr(dyd),
                           _ptr(rows_arr), nr, _ptr(dx), _ptr(dA), _ptr(dB), _ptr(ub), _ptr(gb))
    return dx, dA, dB


def adamw_scalars(lr: float, beta1: float, beta2: float, eps: float, weight_decay: float,
                  step: int) -> dict:
    """The fp32 scalars of one AdamW step, computed in fp64 and rounded once
    (the bias corrections 1 - beta^t at step t >= 1)."""
    if step < 1:
        raise ValueError("step counts from 1")
    f = np.float32
    return dict(decay=f(1.0 - lr * weight_decay), b1=f(beta1), omb1=f(1.0 - beta1), b2=f(beta2),
                omb2=f(1.0 - beta2), eps=f(eps), step_size=f(lr / (1.0 - beta1 ** step)),
                bc2_sqrt=f(math.sqrt(1.0 - beta2 ** step)))


def adamw_step(p, g, m, v, lr: float, beta1: float = 0.9, beta2: float = 0.999,
               eps: float = 1e-8, weight_decay: float = 0.01, step: int = 1, want_bf16=False):
    """[gc4] / [L9] 9.4: one AdamW step with fp32 moments, in fp32 arithmetic,
    on copies of p, m, v.  Returns (p, m, v, p_bf16 bits or None)."""
    p = np.array(p, dtype=np.float32, copy=True).reshape(-1)
    m = np.array(m, dtype=np.float32, copy=True).reshape(-1)
    v = np.array(v, dtype=np.float32, copy=True).reshape(-1)
    g = np.ascontiguousarray(g, dtype=np.float32).reshape(-1)
    sc = adamw_scalars(lr, beta1, beta2, eps, weight_decay, step)
    pb = np.empty(p.size, dtype=np.uint16) if want_bf16 else None
    _load().orc_adamw_step(_ptr(p), _ptr(g), _ptr(m), _ptr(v), _ptr(pb), p.size, sc["decay"],
                           sc["b1"], sc["omb1"], sc["b2"], sc["omb2"], sc["eps"],
                           sc["step_size"], sc["bc2_sqrt"])
    return p, m, v, pb
