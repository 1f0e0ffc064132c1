"""Seeded synthetic inputs for the QLoRA linear layer.

This module only draws random tensors of the stated shapes and distributions;
it holds none of the layer's arithmetic.  Both the GPU tests/benchmark and
the CPU oracle consume the same bytes produced here.

Recipe: normal draws in fp32 (torch generator seeded with 1000*config +
tensor id), multiplied by the stated standard deviation, then stored in the
stated dtype (bf16 by round-to-nearest-even through torch's cast).  Outlier
planting picks positions uniformly without replacement and sets them to
+/- value with a random sign.  CPU and GPU generators produce different
streams, so a caller draws on one device and copies to the other.
"""
from __future__ import annotations

import torch

# tensor ids inside a configuration
T_W, T_X, T_A, T_B, T_DY, T_OUTLIER = 1, 2, 3, 4, 5, 6


def seed_of(config: int, tensor: int, sub: int = 0) -> int:
    return 1000 * config + tensor + 100_000 * sub


def normal(shape, std: float, seed: int, dtype=torch.bfloat16, device="cpu") -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
    t.mul_(std)
    return t.to(dtype)


def plant_outliers(w: torch.Tensor, frac: float, value: float, seed: int) -> torch.Tensor:
    """Set round(frac * numel) uniformly chosen positions (no replacement) of
    w to +/- value, in place; returns w."""
    n = w.numel()
    k = int(round(frac * n))
    if k == 0:
        return w
    g = torch.Generator(device=w.device)
    g.manual_seed(seed)
    pos = torch.randperm(n, generator=g, device=w.device)[:k]
    sign = torch.randint(0, 2, (k,), generator=g, device=w.device).to(torch.float32) * 2 - 1
    flat = w.view(-1)
    flat[pos] = (sign * value).to(w.dtype)
    return w


def linear_inputs(config: int, M: int, N: int, K: int, r: int, *, w_std=0.02, lora_std=0.01,
                  act_dtype=torch.bfloat16, w_dtype=torch.bfloat16, lora_dtype=torch.bfloat16,
                  with_dy=True, sub: int = 0, device="cpu") -> dict:
    """W [N,K] ~ N(0, w_std), x [M,K] ~ N(0,1), A [r,K] and B [N,r] ~ N(0, lora_std),
    dy [M,N] ~ N(0,1)."""
    out = {
        "W": normal((N, K), w_std, seed_of(config, T_W, sub), w_dtype, device),
        "x": normal((M, K), 1.0, seed_of(config, T_X, sub), act_dtype, device),
        "A": normal((r, K), lora_std, seed_of(config, T_A, sub), lora_dtype, device),
        "B": normal((N, r), lora_std, seed_of(config, T_B, sub), lora_dtype, device),
    }
    if with_dy:
        out["dy"] = normal((M, N), 1.0, seed_of(config, T_DY, sub), act_dtype, device)
    return out


# The five workloads (shapes from the layer's benchmark configurations).
SMALL_FP32 = dict(config=1, M=4, N=256, K=256, r=8, alpha=16.0)
DECODE = dict(config=2, N=4096, K=4096, r=16, alpha=32.0, Ms=(1, 4, 16))
MLP_8B = dict(config=3, M=2048, r=16, alpha=32.0,
              projs={"gate": (14336, 4096), "up": (14336, 4096), "down": (4096, 14336)})
MLP_70B = dict(config=4, M=4096, r=64, alpha=16.0,
               projs={"gate": (28672, 8192), "up": (28672, 8192), "down": (8192, 28672)})
WEIGHTSET_8B = dict(config=5, layers=32,
                    shapes={"q": (4096, 4096), "k": (1024, 4096), "v": (1024, 4096),
                            "o": (4096, 4096), "gate": (14336, 4096), "up": (14336, 4096),
                            "down": (4096, 14336)},
                    std=0.02, outlier_frac=1e-3, outlier_sigma=20.0)


def weightset_tensor(layer: int, name: str, device="cpu") -> torch.Tensor:
    """One bf16 weight of the 8B-shaped weight set, N(0, 0.02) with 0.1% of
    positions set to +/- 20 sigma."""
    cfg = WEIGHTSET_8B
    names = list(cfg["shapes"])
    tid = 10 + names.index(name)
    shape = cfg["shapes"][name]
    w = normal(shape, cfg["std"], seed_of(5, tid, layer), torch.bfloat16, device)
    return plant_outliers(w, cfg["outlier_frac"], cfg["outlier_sigma"] * cfg["std"],
                          seed_of(5, tid + 50, layer))
