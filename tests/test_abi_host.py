"""The C-ABI library on the host (no GPU needed): it loads, exports every
symbol include/qlora.h declares, reports sizes, and rejects bad arguments
before anything is enqueued."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import qlora_fine_tuning_quantize_amd as q
from qlora_fine_tuning_quantize_amd import binding as b

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "qlora.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char \*)\s*\**(\w+)\s*\(", src, re.M)))


def test_header_symbols_are_exported():
    names = _declared_functions()
    assert set(names) == set(b.EXPORTED)
    L = q.lib()
    for n in names:
        assert hasattr(L, n), n
    assert L.ql_abi_version() == 113


def test_nf4_sizes_and_bits_per_param(orc):
    sz = q.nf4_sizes(4096, 4096, True)
    assert sz == [8388608, 0, 262144, 4096, 4]
    n = 4096 * 4096
    assert 8 * sum(sz) / n == 4 + 8 / 64 + 32 / (64 * 256) + 32 / n
    assert sum(q.nf4_sizes(4096, 4096, False)) * 8 / n == 4.5
    # the oracle's storage arithmetic on a small tensor agrees
    w = np.random.default_rng(0).standard_normal(64 * 300).astype(np.float32) * 0.02
    st = orc.quantize_nf4(w, double_quant=True)
    assert sum(q.nf4_sizes(300, 64, True)) * 8 / w.size == orc.bits_per_param(st)
    # ragged and odd sizes
    assert q.nf4_sizes(3, 7, False) == [11, 4, 0, 0, 0]
    assert q.nf4_sizes(1, 64 * 257, True) == [32 * 257, 0, 257, 8, 4]


def test_nf4_sizes_block_128():
    """Blocks of 128 weights (one constant per 128): 4.25 bits/param without
    double quantisation, 4 + 8/128 + 32/(128*256) (+ 32/n) with it."""
    n = 4096 * 4096
    sz = q.nf4_sizes(4096, 4096, True, block=128)
    assert sz == [n // 2, 0, n // 128, 4 * (n // 128 // 256), 4]
    assert 8 * sum(sz) / n == 4 + 8 / 128 + 32 / (128 * 256) + 32 / n
    assert 8 * sum(q.nf4_sizes(4096, 4096, False, block=128)) / n == 4.25
    assert q.nf4_sizes(3, 7, False, block=128) == [11, 4, 0, 0, 0]
    with pytest.raises(ValueError):
        q.nf4_sizes(4, 4, False, block=96)


def test_workspace_sizes():
    for op in (q.QL_OP_FWD, q.QL_OP_BWD):
        a = q.workspace_bytes(op, 2048, 4096, 4096, 16)
        bb = q.workspace_bytes(op, 2048, 8192, 8192, 16)
        assert a % 256 == 0 and bb % 256 == 0 and a > 0
        assert bb <= 2.5 * a  # never proportional to N * K (no N x K gradient buffer)
        assert q.workspace_bytes(op, 0, 4096, 4096, 16) == 0
        assert q.workspace_bytes(op, 16, 4096, 4096, 129) == 0
    nb = 4096 * 4096 // 64
    # the fp32 block constants, then 512 exact partial sums of 12 64-bit counters
    assert q.workspace_bytes(q.QL_OP_QUANTIZE, 0, 4096, 4096, 0) == 4 * nb + 512 * 12 * 8
    assert q.workspace_bytes(q.QL_OP_QUANTIZE, 0, 3, 5, 0) == 256 + 512 * 12 * 8
    assert q.workspace_bytes(7, 1, 1, 1, 1) == 0


def _decode_partial_floats(M, N, K, r):
    """The decode forward's fp32 partials: S contraction slices of y [M, N]
    and U slices of u [M, r], for the larger of its launch plans (runs of
    cpw = 2^k <= 8 chunks for double-quantised weights with K % 128 == 0, the
    longest that leaves at least 384 workgroups, else one chunk per wave
    while 3 x 256 workgroups of 4 waves hold them;
    4 cpw chunks per workgroup; u slices of 4 chunks, at most 16)."""
    cdiv = lambda a, b: -(-a // b)
    G, NC, KB = cdiv(N, 64), cdiv(K, 128), K // 64
    S = []
    if K % 128 == 0 and (N * KB) % 16 == 0:
        c = 8
        while c > 1 and (KB % (2 * c) != 0 or G * cdiv(NC, 4 * c) < 384):
            c //= 2
        if KB % (2 * c) == 0:
            S.append(cdiv(NC, 4 * c))
    cpw = 1 if G * NC <= 3 * 256 * 4 else cdiv(G * NC, 3 * 256 * 4)
    S2 = cdiv(NC, 4 * cpw)
    S.append(cdiv(NC, cdiv(NC, S2)))
    U = min(16, cdiv(NC, 4))
    U = cdiv(NC, cdiv(NC, U))
    return max(S) * M * N + U * M * r


@pytest.mark.parametrize("M,N,K,r", [(1, 4096, 4096, 16), (16, 4096, 4096, 16),
                                     (1, 8192, 28672, 64), (16, 14336, 4096, 16),
                                     (5, 200, 4416, 16), (16, 96, 8192, 128),
                                     (2, 2048, 28672, 16), (1, 1, 64, 1)])
def test_workspace_covers_decode_partials(M, N, K, r):
    """qlora_linear_fwd at M <= 16 writes y and u slice sums into its
    workspace after the M x r u region; the reported size must hold them."""
    ws = q.workspace_bytes(q.QL_OP_FWD, M, N, K, r)
    u_region = -(-(M * r * 4) // 256) * 256
    assert ws >= u_region + 4 * _decode_partial_floats(M, N, K, r)
    assert ws % 256 == 0


# Argument checks run before any launch.  The pointers below are fake but
# aligned; every case fails validation, so nothing touches a device.  The
# test is skipped where a GPU is present so a checking bug could never turn
# a fake pointer into a launch.
no_gpu = pytest.mark.skipif(torch.cuda.is_available(), reason="fake-pointer checks run on CPU hosts only")
FAKE = 0x10000


def _desc(rows=64, cols=64, dq=0, **kw):
    d = b.QlNf4(FAKE, FAKE, FAKE, FAKE, FAKE, rows, cols, 64, 256, dq, 0)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@no_gpu
@pytest.mark.parametrize("desc,expect", [
    (dict(rows=0), b.QL_EINVAL), (dict(cols=-1), b.QL_EINVAL), (dict(dq=2), b.QL_EINVAL),
    (dict(block=96), b.QL_EUNSUPPORTED), (dict(block=32), b.QL_EUNSUPPORTED),
    (dict(block2=512), b.QL_EUNSUPPORTED),
    (dict(packed=None), b.QL_EINVAL), (dict(absmax=None), b.QL_EINVAL),
    (dict(dq=1, absmax_mean=None), b.QL_EINVAL), (dict(packed=FAKE + 8), b.QL_EALIGN),
    (dict(reserved=1), b.QL_EINVAL),
])
def test_quantize_rejects_bad_descriptor(desc, expect):
    dq = desc.pop("dq", 0)
    d = _desc(dq=dq, **desc)
    st = q.lib().nf4_quantize(ctypes.c_void_p(FAKE), b.QL_BF16, ctypes.byref(d), None, 0, None)
    assert st == expect
    st = q.lib().nf4_dequantize(ctypes.byref(d), ctypes.c_void_p(FAKE), b.QL_BF16, None)
    assert st == expect


@no_gpu
def test_quantize_rejects_bad_buffers():
    L = q.lib()
    d = _desc()
    assert L.nf4_quantize(None, b.QL_BF16, ctypes.byref(d), None, 0, None) == b.QL_EINVAL
    assert L.nf4_quantize(ctypes.c_void_p(FAKE), 5, ctypes.byref(d), None, 0, None) == b.QL_EINVAL
    assert L.nf4_quantize(ctypes.c_void_p(FAKE + 2), b.QL_F16, ctypes.byref(d), None, 0,
                          None) == b.QL_EALIGN  # fp16 weights are accepted up to alignment
    assert L.nf4_dequantize(ctypes.byref(d), ctypes.c_void_p(FAKE), 3, None) == b.QL_EINVAL
    assert L.nf4_quantize(ctypes.c_void_p(FAKE + 2), b.QL_BF16, ctypes.byref(d), None, 0,
                          None) == b.QL_EALIGN
    d1 = _desc(dq=1)
    assert L.nf4_quantize(ctypes.c_void_p(FAKE), b.QL_BF16, ctypes.byref(d1), ctypes.c_void_p(FAKE),
                          16, None) == b.QL_EWORKSPACE
    assert L.nf4_dequantize(ctypes.byref(d), ctypes.c_void_p(FAKE + 4), b.QL_F32,
                            None) == b.QL_EALIGN


def _many(L, descs, ptrs=None, dtype=b.QL_BF16, ws=None, ws_bytes=0, count=None):
    n = len(descs)
    arr = (b.QlNf4 * max(n, 1))(*descs)
    pv = (ctypes.c_void_p * max(n, 1))(*(ptrs if ptrs is not None else [FAKE] * n))
    return L.nf4_quantize_many(n if count is None else count, pv, dtype, arr,
                               ctypes.c_void_p(ws) if ws else None, ws_bytes, None)


@no_gpu
def test_quantize_many_rejects_bad_arguments():
    """nf4_quantize_many checks every weight before enqueueing anything."""
    L = q.lib()
    ok = _desc()
    assert _many(L, [ok], count=-1) == b.QL_EINVAL
    assert L.nf4_quantize_many(1, None, b.QL_BF16, ctypes.byref(ok), None, 0, None) == b.QL_EINVAL
    assert _many(L, [ok, ok], dtype=5) == b.QL_EINVAL
    # an invalid descriptor anywhere in the list, with its own error code
    assert _many(L, [ok, _desc(rows=0)]) == b.QL_EINVAL
    assert _many(L, [ok, ok, _desc(block=96)]) == b.QL_EUNSUPPORTED
    assert _many(L, [ok, _desc(packed=FAKE + 8)]) == b.QL_EALIGN
    # mixed block size or form
    assert _many(L, [ok, _desc(block=128)]) == b.QL_EINVAL
    assert _many(L, [ok, _desc(dq=1)]) == b.QL_EINVAL
    # a NULL or misaligned weight pointer
    assert _many(L, [ok, ok], ptrs=[FAKE, 0]) == b.QL_EINVAL
    assert _many(L, [ok, ok], ptrs=[FAKE, FAKE + 2]) == b.QL_EALIGN
    # the double-quantised form needs the sum of the per-weight workspaces
    d1, d2 = _desc(dq=1, rows=128), _desc(dq=1, rows=4096, cols=4096)
    need = (q.workspace_bytes(q.QL_OP_QUANTIZE, 0, 128, 64, 0)
            + q.workspace_bytes(q.QL_OP_QUANTIZE, 0, 4096, 4096, 0))
    assert q.quantize_many_workspace_bytes([(128, 64), (4096, 4096)]) == need
    assert _many(L, [d1, d2]) == b.QL_EWORKSPACE
    assert _many(L, [d1, d2], ws=FAKE, ws_bytes=need - 256) == b.QL_EWORKSPACE
    assert _many(L, [d1, d2], ws=FAKE + 16, ws_bytes=need) == b.QL_EALIGN
    # nothing to do
    assert _many(L, [], count=0) == b.QL_OK


def _fwd(L, M=16, r=8, act=b.QL_BF16, lora=b.QL_BF16, alpha=16.0, x=FAKE, y=FAKE, A=FAKE,
         ws=FAKE, ws_bytes=1 << 30, desc=None):
    d = desc or _desc(rows=128, cols=256)
    return L.qlora_linear_fwd(ctypes.c_void_p(x), act, M, ctypes.byref(d), ctypes.c_void_p(A),
                              ctypes.c_void_p(FAKE), lora, r, alpha, ctypes.c_void_p(y), None,
                              ctypes.c_void_p(ws) if ws else None, ws_bytes, None)


@no_gpu
def test_linear_fwd_rejects_bad_arguments():
    L = q.lib()
    assert _fwd(L, M=0) == b.QL_EINVAL
    assert _fwd(L, r=0) == b.QL_EINVAL
    assert _fwd(L, r=129) == b.QL_EUNSUPPORTED
    assert _fwd(L, act=3) == b.QL_EINVAL
    assert _fwd(L, lora=9) == b.QL_EINVAL
    # a 16-bit LoRA dtype must match 16-bit activations (fp16 compute with
    # bf16 factors, or the reverse, is not a combination the layer runs)
    assert _fwd(L, act=b.QL_F16, lora=b.QL_BF16) == b.QL_EUNSUPPORTED
    assert _fwd(L, act=b.QL_BF16, lora=b.QL_F16) == b.QL_EUNSUPPORTED
    assert _fwd(L, act=b.QL_F16, lora=b.QL_F16, M=0) == b.QL_EINVAL  # fp16 itself is accepted
    assert _fwd(L, act=b.QL_F16, lora=b.QL_F32, ws=0) == b.QL_EWORKSPACE
    assert _fwd(L, alpha=float("inf")) == b.QL_EINVAL
    assert _fwd(L, alpha=float("nan")) == b.QL_EINVAL
    assert _fwd(L, x=0) == b.QL_EINVAL
    assert _fwd(L, y=FAKE + 2) == b.QL_EALIGN
    assert _fwd(L, A=FAKE + 8) == b.QL_EALIGN
    assert _fwd(L, desc=_desc(rows=128, cols=100)) == b.QL_ESHAPE
    assert _fwd(L, desc=_desc(rows=128, cols=192, block=128)) == b.QL_ESHAPE  # K % 128
    assert _fwd(L, ws=0) == b.QL_EWORKSPACE
    assert _fwd(L, ws_bytes=255) == b.QL_EWORKSPACE
    assert _fwd(L, ws=FAKE + 16) == b.QL_EALIGN


@no_gpu
def test_linear_fwd_u_rejects_bad_arguments():
    L = q.lib()
    d = _desc(rows=128, cols=256)

    def fwd_u(M=16, r=8, u=FAKE, x=FAKE, y=FAKE, alpha=16.0, desc=d):
        return L.qlora_linear_fwd_u(ctypes.c_void_p(x) if x else None, b.QL_BF16, M,
                                    ctypes.byref(desc), ctypes.c_void_p(u) if u else None,
                                    ctypes.c_void_p(FAKE), b.QL_BF16, r, alpha,
                                    ctypes.c_void_p(y) if y else None, None)
    assert fwd_u(u=0) == b.QL_EINVAL
    assert fwd_u(x=0) == b.QL_EINVAL
    assert fwd_u(M=0) == b.QL_EINVAL
    assert fwd_u(r=129) == b.QL_EUNSUPPORTED
    assert fwd_u(alpha=float("inf")) == b.QL_EINVAL
    assert fwd_u(u=FAKE + 4) == b.QL_EALIGN
    assert fwd_u(desc=_desc(rows=128, cols=100)) == b.QL_ESHAPE


@no_gpu
def test_linear_bwd_rejects_bad_arguments():
    L = q.lib()
    d = _desc(rows=128, cols=256)

    def bwd(dA=FAKE, dB=FAKE, dx=FAKE, M=32, ws_bytes=1 << 30):
        return L.qlora_linear_bwd(ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), b.QL_BF16, M,
                                  ctypes.byref(d), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
                                  b.QL_BF16, 8, 16.0, None,
                                  ctypes.c_void_p(dx) if dx else None,
                                  ctypes.c_void_p(dA) if dA else None,
                                  ctypes.c_void_p(dB) if dB else None, ctypes.c_void_p(FAKE),
                                  ws_bytes, None)
    assert bwd(dA=0) == b.QL_EINVAL
    assert bwd(dB=0) == b.QL_EINVAL
    assert bwd(dx=FAKE + 4) == b.QL_EALIGN
    assert bwd(M=-1) == b.QL_EINVAL
    assert bwd(ws_bytes=1024) == b.QL_EWORKSPACE


@no_gpu
def test_adamw_rejects_bad_arguments():
    L = q.lib()

    def adam(n=8, step=1, p=FAKE, bf=None, b1=0.9, b2=0.999, eps=1e-8, lr=2e-4):
        return L.ql_adamw_step(ctypes.c_void_p(p) if p else None, ctypes.c_void_p(FAKE),
                               ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
                               ctypes.c_void_p(bf) if bf else None, n, lr, b1, b2, eps, 0.01,
                               step, None)
    assert adam(n=-1) == b.QL_EINVAL
    assert adam(step=0) == b.QL_EINVAL
    assert adam(p=0) == b.QL_EINVAL
    assert adam(p=FAKE + 4) == b.QL_EALIGN
    assert adam(bf=FAKE + 2) == b.QL_EALIGN
    assert adam(b1=1.0) == b.QL_EINVAL
    assert adam(b2=-0.1) == b.QL_EINVAL
    assert adam(eps=0.0) == b.QL_EINVAL
    assert adam(lr=float("nan")) == b.QL_EINVAL
    assert adam(n=0) == b.QL_OK  # nothing to enqueue


def test_strerror_and_python_errors():
    L = q.lib()
    for s in range(7):
        assert L.ql_strerror(s)
    assert L.ql_strerror(99) == b"unknown status"
    with pytest.raises(ValueError):
        b._check(b.QL_ESHAPE, "x")
    with pytest.raises(b.QLoRAError):
        b._check(b.QL_EHIP, "x")


@no_gpu
def test_dropout_entry_points_reject_bad_arguments():
    L = q.lib()
    d = _desc(rows=128, cols=256)

    def fwd(p=0.05, act=b.QL_BF16, M=32, ws_bytes=1 << 30):
        return L.qlora_linear_fwd_dropout(ctypes.c_void_p(FAKE), act, M, ctypes.byref(d),
                                          ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), b.QL_BF16,
                                          8, 16.0, p, 7, ctypes.c_void_p(FAKE), None,
                                          ctypes.c_void_p(FAKE), ws_bytes, None)

    def bwd(p=0.05, act=b.QL_BF16, acc=0, desc=d, dx=FAKE, ws_bytes=1 << 30):
        return L.qlora_linear_bwd_dropout(ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), act, 32,
                                          ctypes.byref(desc), ctypes.c_void_p(FAKE),
                                          ctypes.c_void_p(FAKE), b.QL_BF16, 8, 16.0, p, 7, None,
                                          ctypes.c_void_p(dx) if dx else None,
                                          ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), acc,
                                          ctypes.c_void_p(FAKE), ws_bytes, None)
    for p in (1.0, -0.1, float("nan"), 2.0):
        assert fwd(p=p) == b.QL_EINVAL
        assert bwd(p=p) == b.QL_EINVAL
        assert L.ql_dropout_mask(4, 4, p, 7, ctypes.c_void_p(FAKE), None) == b.QL_EINVAL
    assert fwd(M=0) == b.QL_EINVAL
    assert fwd(ws_bytes=255) == b.QL_EWORKSPACE
    assert bwd(acc=2) == b.QL_EINVAL
    assert bwd(ws_bytes=1024) == b.QL_EWORKSPACE
    # fp32 activations and any N are accepted: the checks after the dtype's run
    assert fwd(act=b.QL_F32, ws_bytes=255) == b.QL_EWORKSPACE
    assert bwd(act=b.QL_F32, ws_bytes=1024) == b.QL_EWORKSPACE
    assert bwd(desc=_desc(rows=100, cols=256), ws_bytes=1024) == b.QL_EWORKSPACE
    assert L.ql_dropout_mask(0, 4, 0.1, 7, ctypes.c_void_p(FAKE), None) == b.QL_EINVAL
    assert L.ql_dropout_mask(4, -1, 0.1, 7, ctypes.c_void_p(FAKE), None) == b.QL_EINVAL
    assert L.ql_dropout_mask(4, 4, 0.1, 7, None, None) == b.QL_EINVAL
    assert L.ql_dropout_mask(4, 4, 0.1, 7, ctypes.c_void_p(FAKE + 1), None) == b.QL_EALIGN
