"""qlora_linear_fwd_noalloc: the forward with the library's own fixed per-GPU
workspace, checked bit for bit against qlora_linear_fwd with a caller
workspace (same kernels, same launch plan), on two calls in a row, the
second with a smaller input; and the host-side rejection of a call whose
workspace exceeds the fixed size (nothing enqueued)."""
import ctypes

import pytest
import torch

import qlora_fine_tuning_quantize_amd as q
import qlora_fine_tuning_quantize_amd.binding as b
import synth_inputs as si

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _case(M, N, K, r, dq, act, lora, seed):
    t = si.linear_inputs(seed, M, N, K, r, act_dtype=act, w_dtype=act, lora_dtype=lora,
                         with_dy=False, device=DEV)
    W = q.nf4_quantize(t["W"], double_quant=dq)
    return t, W


def _both(t, W, alpha):
    M, r = t["x"].shape[0], t["A"].shape[0]
    u_ref = torch.full((M, r), float("nan"), dtype=torch.float32, device=DEV)
    y_ref = q.qlora_linear_fwd(t["x"], W, t["A"], t["B"], alpha, u_save=u_ref)
    u = torch.full((M, r), float("nan"), dtype=torch.float32, device=DEV)
    y = torch.full_like(y_ref, float("nan"))
    b.qlora_linear_fwd_noalloc(t["x"], W, t["A"], t["B"], alpha, y=y, u_save=u)
    torch.cuda.synchronize()
    return y, u, y_ref, u_ref


@pytest.mark.parametrize("first,second", [
    # decode sizes: streamed weight with u slices, then a smaller call
    ((16, 4096, 4096, 16, True, torch.bfloat16, torch.bfloat16),
     (1, 1024, 2048, 8, True, torch.bfloat16, torch.bfloat16)),
    # the matrix-core path (u, GEMM, split-K sum), then a decode-sized call
    ((300, 1024, 2048, 16, True, torch.bfloat16, torch.bfloat16),
     (5, 200, 640, 5, False, torch.float16, torch.float32)),
    # few tokens: 64-token tiles and u slices in one launch, then the slice
    # sum with the bypass; then fewer tokens, ragged, in fp16
    ((48, 2048, 4096, 16, True, torch.bfloat16, torch.bfloat16),
     (20, 200, 1024, 8, False, torch.float16, torch.float32)),
    # 128-token tiles with u slices in the same launch (65..128 tokens), then
    # a decode-sized call
    ((96, 1024, 4096, 16, True, torch.bfloat16, torch.bfloat16),
     (3, 256, 512, 8, True, torch.bfloat16, torch.bfloat16)),
])
def test_noalloc_matches_fwd_twice(first, second):
    for i, (M, N, K, r, dq, act, lora) in enumerate((first, second)):
        print(f"noalloc call {i}: M={M} N={N} K={K} r={r} dq={dq} act={act}", flush=True)
        t, W = _case(M, N, K, r, dq, act, lora, 300 + i)
        y, u, y_ref, u_ref = _both(t, W, 2.0 * r)
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), "y"
        assert torch.equal(u, u_ref), "u_save"


def test_noalloc_rejects_oversize():
    # 512 x 4096 x 14336 at r = 16 needs just over 32 MiB of forward workspace
    M, N, K, r = 512, 4096, 14336, 16
    assert q.workspace_bytes(q.QL_OP_FWD, M, N, K, r) > b.NOALLOC_WORKSPACE_BYTES
    t, W = _case(M, N, K, r, True, torch.bfloat16, torch.bfloat16, 310)
    y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(q.QLoRAArgumentError) as e:
        b.qlora_linear_fwd_noalloc(t["x"], W, t["A"], t["B"], 32.0, y=y)
    assert e.value.status == b.QL_EWORKSPACE
    torch.cuda.synchronize()
    assert torch.all(y == 7.0), "a rejected call must enqueue nothing"
