"""GPU parity of nf4_quantize_many (several weights per launch) against the
oracle: every weight's packed codes, block constants, double-quantisation
codes, scales and mean bit-exact, as for nf4_quantize (Gemma lesson 09,
sec. 9.2.1 and 9.2.2).  Lists longer than one launch's eight weights, mixed
sizes (one element to several workgroups' grid-stride steps), every input
dtype, both block sizes and both forms."""
import numpy as np
import pytest
import torch

import qlora_fine_tuning_quantize_amd as q
import synth_inputs as si
from tests.helpers import host

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

SHAPES = [(1, 1), (3, 5), (1, 65), (7, 129), (64, 64), (300, 1000), (33, 64 * 257), (1, 7),
          (1024, 4096), (2, 128), (129, 384)]


def _say(*a):
    print(*a, flush=True)


def _expect_oracle(orc, w_cpu, Wq, dq, block):
    st = orc.quantize_nf4(host(w_cpu).reshape(-1), double_quant=dq, block=block)
    np.testing.assert_array_equal(host(Wq.packed)[:st["packed"].size], st["packed"])
    if dq:
        np.testing.assert_array_equal(host(Wq.absmax_q)[:st["absmax_q"].size], st["absmax_q"])
        np.testing.assert_array_equal(
            host(Wq.absmax_scale)[:st["absmax_scale"].size].view(np.uint32),
            st["absmax_scale"].view(np.uint32))
        assert (host(Wq.absmax_mean)[:1].view(np.uint32)[0]
                == np.float32(st["absmax_mean"]).view(np.uint32))
    else:
        np.testing.assert_array_equal(host(Wq.absmax)[:st["absmax"].size].view(np.uint32),
                                      st["absmax"].view(np.uint32))


def _weights(dtype, seed0):
    ws = []
    for i, (rows, cols) in enumerate(SHAPES):
        w = si.normal((rows, cols), 0.02 * (1 + i), seed=seed0 + 7 * i, dtype=dtype)
        flat = w.view(-1)
        if flat.numel() >= 512:
            flat[128:256] = 0                  # all-zero blocks
            flat[5] = 0.4 * (1 + i)            # outliers
            flat[300] = -0.4 * (1 + i)
        ws.append(w)
    return ws


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("block", [64, 128])
@pytest.mark.parametrize("dq", [False, True])
def test_quantize_many_bit_exact(orc, dtype, block, dq):
    _say(f"quantize_many dtype={dtype} block={block} dq={dq} weights={len(SHAPES)}")
    ws = _weights(dtype, 1000 + block + 3 * dq)
    outs = q.nf4_quantize_many([w.to(DEV) for w in ws], double_quant=dq, block=block)
    torch.cuda.synchronize()
    for w, Wq in zip(ws, outs):
        _expect_oracle(orc, w, Wq, dq, block)


def test_quantize_many_means_stay_per_weight(orc):
    """Weights whose constants lie 2^60 .. 2^-100 apart next to ordinary ones:
    each weight's mean comes from its own constants only (the tie case needs
    the exact sum: 2^58 + 2^35)."""
    rng = np.random.default_rng(5)
    blocks = []
    for a in (2.0 ** 60, 2.0 ** 36, 2.0 ** 7, 2.0 ** -100):
        b = (rng.uniform(-1, 1, 64) * a).astype(np.float32)
        b[3] = np.float32(a)
        blocks.append(b)
    tie = torch.from_numpy(np.concatenate(blocks).reshape(4, 64))
    scales = np.exp2(np.repeat(rng.integers(-140, 120, 5000), 64).astype(np.float64))
    wide = torch.from_numpy((rng.standard_normal(64 * 5000) * scales).astype(np.float32)
                            .reshape(5000, 64))
    plain = si.normal((256, 512), 0.02, seed=9, dtype=torch.float32)
    ws = [plain, tie, wide, plain.clone()]
    outs = q.nf4_quantize_many([w.to(DEV) for w in ws], double_quant=True)
    torch.cuda.synchronize()
    for w, Wq in zip(ws, outs):
        _expect_oracle(orc, w, Wq, True, 64)
    assert host(outs[1].absmax_mean)[0] == np.float32(2.0 ** 58 + 2.0 ** 35)


def test_quantize_many_weightset_layer(orc):
    """One layer of the 8B-shaped weight set (q, k, v, o, gate, up, down) in one
    call: bit-exact against the oracle and equal to one call per weight."""
    names = si.WEIGHTSET_8B["shapes"]
    ws = [si.weightset_tensor(0, name, device=DEV) for name in names]
    _say(f"quantize_many weight set layer 0: {[tuple(w.shape) for w in ws]}")
    outs = q.nf4_quantize_many(ws, double_quant=True)
    singles = [q.nf4_quantize(w, double_quant=True) for w in ws]
    torch.cuda.synchronize()
    for w, Wq, W1 in zip(ws, outs, singles):
        _expect_oracle(orc, w.cpu(), Wq, True, 64)
        sizes = q.nf4_sizes(Wq.rows, Wq.cols, True)  # bytes; the buffers are padded past them
        for f, nbytes in (("packed", sizes[0]), ("absmax_q", sizes[2]),
                          ("absmax_scale", sizes[3]), ("absmax_mean", sizes[4])):
            a, b = getattr(Wq, f), getattr(W1, f)
            n = nbytes // a.element_size()
            assert torch.equal(a[:n], b[:n]), f


def test_quantize_many_graph_replays(orc):
    """The call captured in a HIP graph and replayed three times, with eager
    calls on other inputs in between: every replay gives the oracle's codes."""
    ws = [si.normal(s, 0.02, seed=40 + i, dtype=torch.bfloat16).to(DEV)
          for i, s in enumerate([(64, 64), (300, 1000), (1024, 4096)])]
    other = [si.normal(w.shape, 0.05, seed=90 + i, dtype=torch.bfloat16).to(DEV)
             for i, w in enumerate(ws)]
    outs = [q.NF4Weight.empty(w.shape[0], w.shape[1], True, DEV) for w in ws]
    wsp = torch.empty(q.quantize_many_workspace_bytes([w.shape for w in ws]), dtype=torch.uint8,
                      device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        q.nf4_quantize_many(ws, double_quant=True, out=outs, ws=wsp)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q.nf4_quantize_many(ws, double_quant=True, out=outs, ws=wsp)
    for rep in range(3):
        q.nf4_quantize_many(other, double_quant=True, out=outs, ws=wsp)  # overwrite eagerly
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _say(f"graph replay {rep}")
        for w, Wq in zip(ws, outs):
            _expect_oracle(orc, w.cpu(), Wq, True, 64)
