"""Thin Python binding of libqlora.so (the C ABI in include/qlora.h).

Argument marshalling only: torch provides device memory and the current
stream; every step of the layer runs in the HIP kernels behind the C ABI.
The functions carry the same names as the C entry points.  There is no CPU
fallback: if the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqlora.so")

QL_OK, QL_EINVAL, QL_ESHAPE, QL_EALIGN, QL_EUNSUPPORTED, QL_EWORKSPACE, QL_EHIP = range(7)
QL_F32, QL_BF16, QL_F16 = 0, 1, 2
QL_OP_QUANTIZE, QL_OP_FWD, QL_OP_BWD = 0, 1, 2
NF4_BLOCK, NF4_BLOCK_LARGE, DQ_BLOCK = 64, 128, 256

# every extern "C" symbol declared in include/qlora.h
EXPORTED = ("ql_nf4_sizes", "ql_nf4_sizes_block", "ql_workspace_bytes", "nf4_quantize",
            "nf4_quantize_many", "nf4_dequantize",
            "qlora_linear_fwd", "qlora_linear_fwd_noalloc", "qlora_linear_fwd_u", "qlora_linear_bwd",
            "qlora_linear_bwd_acc",
            "qlora_linear_fwd_dropout", "qlora_linear_bwd_dropout", "ql_dropout_mask",
            "ql_adamw_step", "ql_strerror", "ql_abi_version")


class QlNf4(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("absmax", ctypes.c_void_p),
                ("absmax_q", ctypes.c_void_p), ("absmax_scale", ctypes.c_void_p),
                ("absmax_mean", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("block", ctypes.c_int32), ("block2", ctypes.c_int32),
                ("double_quant", ctypes.c_int32), ("reserved", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libqlora.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(LIB_PATH)
    p, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                            ctypes.c_size_t)
    sp = ctypes.POINTER(QlNf4)
    L.ql_nf4_sizes.argtypes = [i64, i64, i32, ctypes.POINTER(sz * 5)]
    L.ql_nf4_sizes.restype = ctypes.c_int
    L.ql_nf4_sizes_block.argtypes = [i64, i64, i32, i32, ctypes.POINTER(sz * 5)]
    L.ql_nf4_sizes_block.restype = ctypes.c_int
    L.ql_workspace_bytes.argtypes = [i32, i64, i64, i64, i32]
    L.ql_workspace_bytes.restype = sz
    L.nf4_quantize.argtypes = [p, i32, sp, p, sz, p]
    L.nf4_quantize.restype = ctypes.c_int
    L.nf4_quantize_many.argtypes = [i32, ctypes.POINTER(p), i32, sp, p, sz, p]
    L.nf4_quantize_many.restype = ctypes.c_int
    L.nf4_dequantize.argtypes = [sp, p, i32, p]
    L.nf4_dequantize.restype = ctypes.c_int
    L.qlora_linear_fwd.argtypes = [p, i32, i64, sp, p, p, i32, i32, f32, p, p, p, sz, p]
    L.qlora_linear_fwd.restype = ctypes.c_int
    L.qlora_linear_fwd_noalloc.argtypes = [p, i32, i64, sp, p, p, i32, i32, f32, p, p, p]
    L.qlora_linear_fwd_noalloc.restype = ctypes.c_int
    L.qlora_linear_fwd_u.argtypes = [p, i32, i64, sp, p, p, i32, i32, f32, p, p]
    L.qlora_linear_fwd_u.restype = ctypes.c_int
    L.qlora_linear_bwd.argtypes = [p, p, i32, i64, sp, p, p, i32, i32, f32, p, p, p, p, p, sz, p]
    L.qlora_linear_bwd.restype = ctypes.c_int
    L.qlora_linear_bwd_acc.argtypes = L.qlora_linear_bwd.argtypes
    L.qlora_linear_bwd_acc.restype = ctypes.c_int
    f64, u64 = ctypes.c_double, ctypes.c_uint64
    L.qlora_linear_fwd_dropout.argtypes = [p, i32, i64, sp, p, p, i32, i32, f32, f64, u64, p, p, p,
                                           sz, p]
    L.qlora_linear_fwd_dropout.restype = ctypes.c_int
    L.qlora_linear_bwd_dropout.argtypes = [p, p, i32, i64, sp, p, p, i32, i32, f32, f64, u64, p, p,
                                           p, p, i32, p, sz, p]
    L.qlora_linear_bwd_dropout.restype = ctypes.c_int
    L.ql_dropout_mask.argtypes = [i64, i64, f64, u64, p, p]
    L.ql_dropout_mask.restype = ctypes.c_int
    L.ql_adamw_step.argtypes = [p, p, p, p, p, i64, f64, f64, f64, f64, f64, i64, p]
    L.ql_adamw_step.restype = ctypes.c_int
    L.ql_strerror.argtypes = [ctypes.c_int]
    L.ql_strerror.restype = ctypes.c_char_p
    L.ql_abi_version.restype = ctypes.c_int
    _lib = L
    return L


class QLoRAError(RuntimeError):
    """A HIP runtime failure reported by the library."""


class QLoRAArgumentError(ValueError):
    """An argument check of the C ABI failed (nothing was enqueued)."""


def _check(status: int, what: str):
    if status == QL_OK:
        return
    msg = f"{what}: {lib().ql_strerror(status).decode()} (status {status})"
    if status == QL_EHIP:
        raise QLoRAError(msg)
    err = QLoRAArgumentError(msg)
    err.status = status
    raise err


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return QL_BF16
    if t == torch.float16:
        return QL_F16
    if t == torch.float32:
        return QL_F32
    raise ValueError(f"unsupported dtype {t}")


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def nf4_sizes(rows: int, cols: int, double_quant: bool, block: int = NF4_BLOCK) -> list[int]:
    out = (ctypes.c_size_t * 5)()
    if block == NF4_BLOCK:
        _check(lib().ql_nf4_sizes(rows, cols, int(double_quant), ctypes.byref(out)),
               "ql_nf4_sizes")
    else:
        _check(lib().ql_nf4_sizes_block(rows, cols, int(block), int(double_quant),
                                        ctypes.byref(out)), "ql_nf4_sizes_block")
    return list(out)


def workspace_bytes(op: int, M: int, N: int, K: int, r: int) -> int:
    return int(lib().ql_workspace_bytes(op, M, N, K, r))


def workspace(op: int, M: int, N: int, K: int, r: int, device) -> torch.Tensor:
    nbytes = max(workspace_bytes(op, M, N, K, r), 256)
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


@dataclass
class NF4Weight:
    """Device buffers of an NF4-quantised weight [rows = N, cols = K] with
    blocks of `block` (64 or 128) weights."""
    packed: torch.Tensor
    rows: int
    cols: int
    double_quant: bool
    absmax: torch.Tensor | None = None
    absmax_q: torch.Tensor | None = None
    absmax_scale: torch.Tensor | None = None
    absmax_mean: torch.Tensor | None = None
    block: int = NF4_BLOCK

    @staticmethod
    def empty(rows: int, cols: int, double_quant: bool, device,
              block: int = NF4_BLOCK) -> "NF4Weight":
        b = nf4_sizes(rows, cols, double_quant, block)
        # round each buffer up to 16 bytes so all vector loads stay in bounds
        mk = lambda n, dt, es: torch.empty(max(1, (n + 15) // 16 * 16 // es), dtype=dt,
                                           device=device)
        w = NF4Weight(packed=mk(b[0], torch.uint8, 1), rows=rows, cols=cols,
                      double_quant=double_quant, block=block)
        if double_quant:
            w.absmax_q = mk(b[2], torch.int8, 1)
            w.absmax_scale = mk(b[3], torch.float32, 4)
            w.absmax_mean = mk(b[4], torch.float32, 4)
        else:
            w.absmax = mk(b[1], torch.float32, 4)
        return w

    def struct(self) -> QlNf4:
        return QlNf4(self.packed.data_ptr(),
                     self.absmax.data_ptr() if self.absmax is not None else None,
                     self.absmax_q.data_ptr() if self.absmax_q is not None else None,
                     self.absmax_scale.data_ptr() if self.absmax_scale is not None else None,
                     self.absmax_mean.data_ptr() if self.absmax_mean is not None else None,
                     self.rows, self.cols, self.block, DQ_BLOCK, int(self.double_quant), 0)

    def storage_bytes(self) -> int:
        return sum(nf4_sizes(self.rows, self.cols, self.double_quant, self.block))


def nf4_quantize(w: torch.Tensor, double_quant: bool = True, out: NF4Weight | None = None,
                 ws: torch.Tensor | None = None, block: int = NF4_BLOCK) -> NF4Weight:
    """NF4-quantise a 2-D weight [N, K] (bf16, fp16 or fp32, on the GPU) with
    blocks of `block` (64 or 128) weights."""
    assert w.dim() == 2 and w.is_contiguous() and w.is_cuda
    N, K = w.shape
    q = out or NF4Weight.empty(N, K, double_quant, w.device, block)
    assert (q.rows, q.cols, q.double_quant, q.block) == (N, K, double_quant, block)
    if ws is None and double_quant:
        ws = workspace(QL_OP_QUANTIZE, 0, N, K, 0, w.device)
    st = q.struct()
    _check(lib().nf4_quantize(_ptr(w), _dtype_code(w.dtype), ctypes.byref(st), _ptr(ws),
                              0 if ws is None else ws.numel(), _stream(w.device)),
           "nf4_quantize")
    return q


def quantize_many_workspace_bytes(shapes) -> int:
    """Workspace of nf4_quantize_many with double quantisation: the sum of
    the per-weight quantisation workspaces, in order."""
    return sum(workspace_bytes(QL_OP_QUANTIZE, 0, N, K, 0) for N, K in shapes)


def nf4_quantize_many(ws_in: list, double_quant: bool = True, out: list | None = None,
                      ws: torch.Tensor | None = None, block: int = NF4_BLOCK) -> list:
    """NF4-quantise several 2-D weights of one dtype (on one GPU) in as few
    launches as the library can; each result equals nf4_quantize's."""
    n = len(ws_in)
    for w in ws_in:
        assert w.dim() == 2 and w.is_contiguous() and w.is_cuda and w.dtype == ws_in[0].dtype
    dev = ws_in[0].device if n else torch.device("cuda")
    outs = out or [NF4Weight.empty(w.shape[0], w.shape[1], double_quant, w.device, block)
                   for w in ws_in]
    assert len(outs) == n
    for w, o in zip(ws_in, outs):
        assert (o.rows, o.cols, o.double_quant, o.block) == (*w.shape, double_quant, block)
    if ws is None and double_quant and n:
        ws = torch.empty(max(256, quantize_many_workspace_bytes([w.shape for w in ws_in])),
                         dtype=torch.uint8, device=dev)
    structs = (QlNf4 * max(n, 1))(*[q.struct() for q in outs])
    ptrs = (ctypes.c_void_p * max(n, 1))(*[w.data_ptr() for w in ws_in])
    _check(lib().nf4_quantize_many(n, ptrs, _dtype_code(ws_in[0].dtype) if n else QL_BF16,
                                   structs, _ptr(ws), 0 if ws is None else ws.numel(),
                                   _stream(dev)), "nf4_quantize_many")
    return outs


def nf4_dequantize(q: NF4Weight, dtype=torch.bfloat16, out: torch.Tensor | None = None) -> torch.Tensor:
    if out is None:
        out = torch.empty((q.rows, q.cols), dtype=dtype, device=q.packed.device)
    st = q.struct()
    _check(lib().nf4_dequantize(ctypes.byref(st), _ptr(out), _dtype_code(out.dtype),
                                _stream(out.device)), "nf4_dequantize")
    return out


def qlora_linear_fwd(x: torch.Tensor, W: NF4Weight, A: torch.Tensor, B: torch.Tensor,
                     alpha: float, y: torch.Tensor | None = None,
                     u_save: torch.Tensor | None = None,
                     ws: torch.Tensor | None = None) -> torch.Tensor:
    """y = x W^T + (alpha/r) (x A^T) B^T  with x [M, K], A [r, K], B [N, r].
    The compute dtype is x's (bf16, fp16 or fp32); A and B are fp32 or of
    x's 16-bit dtype (bf16 factors also with fp32 x)."""
    assert x.dim() == 2 and x.is_contiguous() and A.is_contiguous() and B.is_contiguous()
    M, K = x.shape
    r = A.shape[0]
    assert K == W.cols and A.shape == (r, K) and B.shape == (W.rows, r) and A.dtype == B.dtype
    if y is None:
        y = torch.empty((M, W.rows), dtype=x.dtype, device=x.device)
    if ws is None:
        ws = workspace(QL_OP_FWD, M, W.rows, K, r, x.device)
    st = W.struct()
    _check(lib().qlora_linear_fwd(_ptr(x), _dtype_code(x.dtype), M, ctypes.byref(st), _ptr(A),
                                  _ptr(B), _dtype_code(A.dtype), r, float(alpha), _ptr(y),
                                  _ptr(u_save), _ptr(ws), ws.numel(), _stream(x.device)),
           "qlora_linear_fwd")
    return y


NOALLOC_WORKSPACE_BYTES = 32 << 20


def qlora_linear_fwd_noalloc(x: torch.Tensor, W: NF4Weight, A: torch.Tensor, B: torch.Tensor,
                             alpha: float, y: torch.Tensor | None = None,
                             u_save: torch.Tensor | None = None) -> torch.Tensor:
    """qlora_linear_fwd with the library's own fixed per-GPU workspace (no
    workspace argument, nothing allocated by the call or its kernels); raises
    for shapes whose workspace exceeds NOALLOC_WORKSPACE_BYTES.  Calls that
    overlap on one GPU race."""
    assert x.dim() == 2 and x.is_contiguous() and A.is_contiguous() and B.is_contiguous()
    M, K = x.shape
    r = A.shape[0]
    assert K == W.cols and A.shape == (r, K) and B.shape == (W.rows, r) and A.dtype == B.dtype
    if y is None:
        y = torch.empty((M, W.rows), dtype=x.dtype, device=x.device)
    st = W.struct()
    _check(lib().qlora_linear_fwd_noalloc(_ptr(x), _dtype_code(x.dtype), M, ctypes.byref(st),
                                          _ptr(A), _ptr(B), _dtype_code(A.dtype), r, float(alpha),
                                          _ptr(y), _ptr(u_save), _stream(x.device)),
           "qlora_linear_fwd_noalloc")
    return y


def qlora_linear_fwd_dropout(x: torch.Tensor, W: NF4Weight, A: torch.Tensor, B: torch.Tensor,
                             alpha: float, dropout_p: float, seed: int,
                             y: torch.Tensor | None = None, u_save: torch.Tensor | None = None,
                             ws: torch.Tensor | None = None) -> torch.Tensor:
    """The forward with LoRA dropout on the bypass input: u = (d .* x) A^T,
    y = x W^T + (alpha/r) u B^T, the mask drawn from (dropout_p, seed)."""
    assert x.dim() == 2 and x.is_contiguous() and A.is_contiguous() and B.is_contiguous()
    M, K = x.shape
    r = A.shape[0]
    assert K == W.cols and A.shape == (r, K) and B.shape == (W.rows, r) and A.dtype == B.dtype
    if y is None:
        y = torch.empty((M, W.rows), dtype=x.dtype, device=x.device)
    if ws is None:
        ws = workspace(QL_OP_FWD, M, W.rows, K, r, x.device)
    st = W.struct()
    _check(lib().qlora_linear_fwd_dropout(_ptr(x), _dtype_code(x.dtype), M, ctypes.byref(st),
                                          _ptr(A), _ptr(B), _dtype_code(A.dtype), r, float(alpha),
                                          float(dropout_p), int(seed) & (2**64 - 1), _ptr(y),
                                          _ptr(u_save), _ptr(ws), ws.numel(), _stream(x.device)),
           "qlora_linear_fwd_dropout")
    return y


def dropout_mask(M: int, K: int, dropout_p: float, seed: int, device) -> torch.Tensor:
    """The LoRA dropout keep mask [M, K] (uint8 0/1) the layer draws for
    (dropout_p, seed)."""
    keep = torch.empty((M, K), dtype=torch.uint8, device=device)
    _check(lib().ql_dropout_mask(M, K, float(dropout_p), int(seed) & (2**64 - 1), _ptr(keep),
                                 _stream(keep.device)), "ql_dropout_mask")
    return keep


def qlora_linear_fwd_u(x: torch.Tensor, W: NF4Weight, u: torch.Tensor, B: torch.Tensor,
                       alpha: float, y: torch.Tensor | None = None) -> torch.Tensor:
    """y = x W^T + (alpha/r) u B^T with u = x A^T given (fp32 [M, r])."""
    assert x.dim() == 2 and x.is_contiguous() and u.is_contiguous() and B.is_contiguous()
    M, K = x.shape
    r = u.shape[1]
    assert K == W.cols and u.shape == (M, r) and u.dtype == torch.float32
    assert B.shape == (W.rows, r)
    if y is None:
        y = torch.empty((M, W.rows), dtype=x.dtype, device=x.device)
    st = W.struct()
    _check(lib().qlora_linear_fwd_u(_ptr(x), _dtype_code(x.dtype), M, ctypes.byref(st), _ptr(u),
                                    _ptr(B), _dtype_code(B.dtype), r, float(alpha), _ptr(y),
                                    _stream(x.device)), "qlora_linear_fwd_u")
    return y


def qlora_linear_bwd(dy: torch.Tensor, x: torch.Tensor, W: NF4Weight, A: torch.Tensor,
                     B: torch.Tensor, alpha: float, u_saved: torch.Tensor | None = None,
                     need_dx: bool = True, dx: torch.Tensor | None = None,
                     dA: torch.Tensor | None = None, dB: torch.Tensor | None = None,
                     ws: torch.Tensor | None = None, accumulate: bool = False):
    """Returns (dx | None, dA fp32 [r, K], dB fp32 [N, r]); no base-weight gradient.
    accumulate: add into the given dA and dB (gradient accumulation) instead of
    overwriting them."""
    M, K = x.shape
    r = A.shape[0]
    N = W.rows
    assert dy.shape == (M, N) and dy.dtype == x.dtype and dy.is_contiguous() and x.is_contiguous()
    dev = x.device
    if need_dx and dx is None:
        dx = torch.empty((M, K), dtype=x.dtype, device=dev)
    if not need_dx:
        dx = None
    if accumulate and (dA is None or dB is None):
        raise ValueError("accumulate needs the dA and dB to add into")
    dA = dA if dA is not None else torch.empty((r, K), dtype=torch.float32, device=dev)
    dB = dB if dB is not None else torch.empty((N, r), dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(QL_OP_BWD, M, N, K, r, dev)
    st = W.struct()
    fn = lib().qlora_linear_bwd_acc if accumulate else lib().qlora_linear_bwd
    _check(fn(_ptr(dy), _ptr(x), _dtype_code(x.dtype), M, ctypes.byref(st), _ptr(A), _ptr(B),
              _dtype_code(A.dtype), r, float(alpha), _ptr(u_saved), _ptr(dx), _ptr(dA), _ptr(dB),
              _ptr(ws), ws.numel(), _stream(dev)),
           "qlora_linear_bwd_acc" if accumulate else "qlora_linear_bwd")
    return dx, dA, dB


def qlora_linear_bwd_dropout(dy: torch.Tensor, x: torch.Tensor, W: NF4Weight, A: torch.Tensor,
                             B: torch.Tensor, alpha: float, dropout_p: float, seed: int,
                             u_saved: torch.Tensor | None = None, need_dx: bool = True,
                             dx: torch.Tensor | None = None, dA: torch.Tensor | None = None,
                             dB: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                             accumulate: bool = False):
    """The backward with LoRA dropout (the forward's dropout_p and seed):
    returns (dx | None, dA, dB).  u_saved, if given, is the dropout forward's
    u_save."""
    M, K = x.shape
    r = A.shape[0]
    N = W.rows
    assert dy.shape == (M, N) and dy.dtype == x.dtype and dy.is_contiguous() and x.is_contiguous()
    dev = x.device
    if need_dx and dx is None:
        dx = torch.empty((M, K), dtype=x.dtype, device=dev)
    if not need_dx:
        dx = None
    if accumulate and (dA is None or dB is None):
        raise ValueError("accumulate needs the dA and dB to add into")
    dA = dA if dA is not None else torch.empty((r, K), dtype=torch.float32, device=dev)
    dB = dB if dB is not None else torch.empty((N, r), dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(QL_OP_BWD, M, N, K, r, dev)
    st = W.struct()
    _check(lib().qlora_linear_bwd_dropout(_ptr(dy), _ptr(x), _dtype_code(x.dtype), M,
                                          ctypes.byref(st), _ptr(A), _ptr(B), _dtype_code(A.dtype),
                                          r, float(alpha), float(dropout_p),
                                          int(seed) & (2**64 - 1), _ptr(u_saved), _ptr(dx),
                                          _ptr(dA), _ptr(dB), int(accumulate), _ptr(ws), ws.numel(),
                                          _stream(dev)), "qlora_linear_bwd_dropout")
    return dx, dA, dB


def adamw_step(param: torch.Tensor, grad: torch.Tensor, exp_avg: torch.Tensor,
               exp_avg_sq: torch.Tensor, lr: float, step: int, beta1: float = 0.9,
               beta2: float = 0.999, eps: float = 1e-8, weight_decay: float = 0.01,
               param_bf16: torch.Tensor | None = None) -> None:
    """One AdamW step in place on fp32 param / exp_avg / exp_avg_sq (contiguous,
    same length as grad); param_bf16, if given, receives the bf16 copy."""
    for t in (param, grad, exp_avg, exp_avg_sq):
        assert t.dtype == torch.float32 and t.is_contiguous() and t.numel() == param.numel()
    if param_bf16 is not None:
        assert param_bf16.dtype == torch.bfloat16 and param_bf16.numel() == param.numel()
    _check(lib().ql_adamw_step(_ptr(param), _ptr(grad), _ptr(exp_avg), _ptr(exp_avg_sq),
                               _ptr(param_bf16), param.numel(), float(lr), float(beta1),
                               float(beta2), float(eps), float(weight_decay), int(step),
                               _stream(param.device)), "ql_adamw_step")
