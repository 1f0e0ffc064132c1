"""GPU parity of the optimizer-side entry points, through the C ABI:
ql_adamw_step against the oracle's AdamW (bit for bit: both sides take the
same fp32 roundings in the same order), and gradient accumulation
(qlora_linear_bwd_acc) against the oracle's summed gradients."""
import numpy as np
import pytest
import torch

import qlora_fine_tuning_quantize_amd as q
import synth_inputs as si
from tests.helpers import BF16_TOL, host, rel_err

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.mark.parametrize("n", [1, 3, 4, 5, 1000, 65537, (1 << 20) + 3])
@pytest.mark.parametrize("with_bf16", [False, True])
def test_adamw_bit_exact(orc, n, with_bf16):
    print(f"adamw n={n} bf16={with_bf16}", flush=True)
    gen = torch.Generator().manual_seed(n)
    p = torch.randn(n, generator=gen)
    m = torch.randn(n, generator=gen) * 0.1
    v = torch.rand(n, generator=gen) * 0.01
    pd, md, vd = p.to(DEV), m.to(DEV), v.to(DEV)
    pb = torch.empty(n, dtype=torch.bfloat16, device=DEV) if with_bf16 else None
    pr, mr, vr = p.numpy(), m.numpy(), v.numpy()
    for step in (1, 2, 3):
        g = torch.randn(n, generator=gen) * (0.5 ** step)
        q.adamw_step(pd, g.to(DEV), md, vd, lr=2e-4, step=step, param_bf16=pb)
        pr, mr, vr, pbr = orc.adamw_step(pr, g.numpy(), mr, vr, 2e-4, step=step,
                                         want_bf16=with_bf16)
        torch.cuda.synchronize()
        assert np.array_equal(pd.cpu().numpy().view(np.uint32), pr.view(np.uint32)), step
        assert np.array_equal(md.cpu().numpy().view(np.uint32), mr.view(np.uint32)), step
        assert np.array_equal(vd.cpu().numpy().view(np.uint32), vr.view(np.uint32)), step
        if with_bf16:
            assert np.array_equal(pb.cpu().view(torch.int16).numpy().view(np.uint16), pbr), step


def test_gradient_accumulation(orc):
    """Three micro-batches through qlora_linear_bwd_acc add up to the oracle's
    summed dA and dB; dx is each micro-batch's own."""
    M, N, K, r = 96, 384, 512, 16
    t = si.linear_inputs(93, M, N, K, r, sub=1)
    W = q.nf4_quantize(t["W"].to(DEV), double_quant=True)
    st = orc.quantize_nf4(host(t["W"]), double_quant=True)
    w_hat = orc.dequantize(st).reshape(N, K)
    A, B = t["A"].to(DEV), t["B"].to(DEV)
    dA = torch.zeros((r, K), dtype=torch.float32, device=DEV)
    dB = torch.zeros((N, r), dtype=torch.float32, device=DEV)
    dA_sum, dB_sum = np.zeros((r, K)), np.zeros((N, r))
    for mb in range(3):
        tm = si.linear_inputs(94, M, N, K, r, sub=mb)
        x, dy = tm["x"].to(DEV), tm["dy"].to(DEV)
        dx, _, _ = q.qlora_linear_bwd(dy, x, W, A, B, 32.0, dA=dA, dB=dB, accumulate=True)
        dx1, _, _ = q.qlora_linear_bwd(dy, x, W, A, B, 32.0)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(dx.float().cpu().numpy(), dx1.float().cpu().numpy())
        _, a_ref, b_ref = orc.linear_bwd(host(tm["x"]), w_hat, host(t["A"]), host(t["B"]),
                                         host(tm["dy"]), 32.0, r, want_dx=False)
        dA_sum += a_ref
        dB_sum += b_ref
        assert rel_err(dA.cpu().numpy(), dA_sum) <= BF16_TOL, mb
        assert rel_err(dB.cpu().numpy(), dB_sum) <= BF16_TOL, mb
