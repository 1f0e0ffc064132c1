"""The layer's launches under HIP graph capture: a captured forward +
backward, replayed several times with eager work and synchronisations in
between, reproduces the eager results bit for bit on every replay (the
library enqueues only kernels on the caller's stream: no allocation, no
memset, no synchronisation)."""
import pytest
import torch

import qlora_fine_tuning_quantize_amd as q
import synth_inputs as si

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.mark.parametrize("M,N,K,r,dropout,block,act", [
    (300, 384, 640, 16, 0.0, 64, torch.bfloat16),   # 256-token GEMMs
    (8, 256, 512, 8, 0.0, 64, torch.bfloat16),      # decode GEMV forward
    (64, 256, 1024, 16, 0.0, 64, torch.bfloat16),   # 64-token forward tiles with split-K
    (300, 384, 640, 16, 0.1, 64, torch.bfloat16),   # LoRA dropout, forward and backward
    (64, 256, 1024, 16, 0.0, 128, torch.bfloat16),  # blocks of 128
    (300, 384, 640, 16, 0.1, 64, torch.float16),    # fp16 compute with dropout
    (8, 256, 512, 8, 0.0, 64, torch.float16),       # fp16 decode GEMV
    (4, 256, 8192, 16, 0.0, 64, torch.bfloat16),    # decode GEMV, contraction split in 2
    (8, 256, 512, 8, 0.1, 64, torch.bfloat16),      # decode forward with LoRA dropout
    (40, 256, 1024, 16, 0.1, 64, torch.bfloat16),   # few-token forward with LoRA dropout
])
def test_graph_replay_matches_eager(M, N, K, r, dropout, block, act):
    print(f"graph replay M={M} N={N} K={K} r={r} dropout={dropout} block={block} act={act}",
          flush=True)
    t = {k: v.to(DEV) for k, v in si.linear_inputs(92, M, N, K, r, act_dtype=act, w_dtype=act,
                                                   lora_dtype=act, sub=M).items()}
    W = q.nf4_quantize(t["W"], double_quant=True, block=block)
    bufs = dict(y=torch.empty((M, N), dtype=act, device=DEV),
                u=torch.empty((M, r), dtype=torch.float32, device=DEV),
                dx=torch.empty((M, K), dtype=act, device=DEV),
                dA=torch.empty((r, K), dtype=torch.float32, device=DEV),
                dB=torch.empty((N, r), dtype=torch.float32, device=DEV))
    wsf = q.workspace(q.QL_OP_FWD, M, N, K, r, DEV)
    wsb = q.workspace(q.QL_OP_BWD, M, N, K, r, DEV)

    def step():
        if dropout > 0:
            q.qlora_linear_fwd_dropout(t["x"], W, t["A"], t["B"], 32.0, dropout, 77, y=bufs["y"],
                                       u_save=bufs["u"], ws=wsf)
            q.qlora_linear_bwd_dropout(t["dy"], t["x"], W, t["A"], t["B"], 32.0, dropout, 77,
                                       u_saved=bufs["u"], dx=bufs["dx"], dA=bufs["dA"],
                                       dB=bufs["dB"], ws=wsb)
            return
        q.qlora_linear_fwd(t["x"], W, t["A"], t["B"], 32.0, y=bufs["y"], u_save=bufs["u"], ws=wsf)
        q.qlora_linear_bwd(t["dy"], t["x"], W, t["A"], t["B"], 32.0, u_saved=bufs["u"],
                           dx=bufs["dx"], dA=bufs["dA"], dB=bufs["dB"], ws=wsb)

    step()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in bufs.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    other = torch.randn((M, K), device=DEV).to(act)
    for rep in range(3):
        for v in bufs.values():
            v.fill_(float("nan"))
        # eager work of the library between replays
        q.qlora_linear_fwd(other, W, t["A"], t["B"], 32.0, ws=wsf)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in bufs:
            assert torch.equal(bufs[k], ref[k]), (rep, k)
