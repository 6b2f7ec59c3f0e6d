"""Seeded synthetic inputs for the QLoRA layer workloads (shared by tests and
the benchmark).  This module holds no arithmetic of the method: it only draws
random tensors with the shapes and distributions of the workloads.

Distributions use the standard deviation as the second parameter of N(.,.).
Every tensor has its own seed, so the CPU oracle and the GPU path see
identical bits.  Tensors are generated on the CPU with torch.Generator, except
where a `device` is passed (used for inputs too large to draw on the host).
"""
from __future__ import annotations

import torch

LLAMA7B_UP = (11008, 4096)        # (N, K): 4096 -> 11008
LLAMA7B_DOWN = (4096, 11008)      # 11008 -> 4096
LLAMA65B_BLOCK = {                # name: (N, K)
    "q": (8192, 8192), "k": (8192, 8192), "v": (8192, 8192), "o": (8192, 8192),
    "gate": (22016, 8192), "up": (22016, 8192), "down": (8192, 22016),
}


def _gen(seed, device="cpu"):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, std, seed, dtype=torch.bfloat16, device="cpu"):
    x = torch.randn(shape, generator=_gen(seed, device), device=device, dtype=torch.float32)
    return (x * std).to(dtype)


def weight_gaussian(N, K, std, seed, dtype=torch.bfloat16, device="cpu"):
    return normal((N, K), std, seed, dtype, device)


def weight_with_outliers(N, K, std, frac, factor, seed, dtype=torch.bfloat16, device="cpu"):
    """N(0, std) with a Bernoulli(frac) mask of entries multiplied by `factor`."""
    g = _gen(seed, device)
    w = torch.randn((N, K), generator=g, device=device, dtype=torch.float32) * std
    mask = torch.rand((N, K), generator=g, device=device) < frac
    w = torch.where(mask, w * factor, w)
    return w.to(dtype)


def weight_row_std(N, K, lo, hi, seed, dtype=torch.bfloat16, device="cpu"):
    """Per-output-row std ~ U(lo, hi), entries N(0, std_row)."""
    g = _gen(seed, device)
    stds = lo + (hi - lo) * torch.rand((N, 1), generator=g, device=device)
    w = torch.randn((N, K), generator=g, device=device, dtype=torch.float32) * stds
    return w.to(dtype)


def weight_student_t(N, K, scale, df, seed, dtype=torch.bfloat16, device="cpu"):
    """scale * t_df, drawn as Z / sqrt(V / df) with V ~ chi2(df) = sum of df squared normals."""
    g = _gen(seed, device)
    z = torch.randn((N, K), generator=g, device=device, dtype=torch.float32)
    v = torch.zeros((N, K), device=device, dtype=torch.float32)
    for _ in range(df):
        e = torch.randn((N, K), generator=g, device=device, dtype=torch.float32)
        v += e * e
    return (scale * z / torch.sqrt(v / df)).to(dtype)


def lora_pair(K, N, r, seed_l1, seed_l2, l2_std=0.01):
    """L1 [K, r] ~ N(0, 1/K) and L2 [r, N] ~ N(0, l2_std), bf16."""
    return normal((K, r), 1.0 / K, seed_l1), normal((r, N), l2_std, seed_l2)


def layer_inputs(N, K, M, r, seed_base, w_kind="gaussian", w_std=0.02, dy_std=1.0, l2_std=0.01,
                 w_dtype=torch.bfloat16):
    """One linear's inputs: W, L1, L2, X, dY with seeds seed_base + (0..4)."""
    if w_kind == "gaussian":
        W = weight_gaussian(N, K, w_std, seed_base + 0, w_dtype)
    elif w_kind == "outliers":
        W = weight_with_outliers(N, K, w_std, 0.001, 10.0, seed_base + 0, w_dtype)
    elif w_kind == "row_std":
        W = weight_row_std(N, K, 0.01, 0.05, seed_base + 0, w_dtype)
    else:
        raise ValueError(w_kind)
    L1, L2 = lora_pair(K, N, r, seed_base + 1, seed_base + 2, l2_std)
    X = normal((M, K), 1.0, seed_base + 3)
    dY = normal((M, N), dy_std, seed_base + 4)
    return {"W": W, "L1": L1, "L2": L2, "X": X, "dY": dY}


def config1():
    """Single linear 512 -> 512, fp32 weights N(0, 0.02) seed 0, r = 8, M = 32."""
    return layer_inputs(512, 512, 32, 8, 0, w_dtype=torch.float32)


def config2(M):
    """LLaMA-7B up-projection 4096 -> 11008 with 0.1% outliers x10, r = 64, decode-sized M."""
    return layer_inputs(11008, 4096, M, 64, 10, w_kind="outliers")


def config3():
    """LLaMA-7B up- and down-projections at M = 4096 tokens, r = 64, dY ~ N(0, 1e-2)."""
    up = layer_inputs(*LLAMA7B_UP, 4096, 64, 20, dy_std=1e-2)
    down = layer_inputs(*LLAMA7B_DOWN, 4096, 64, 30, dy_std=1e-2)
    return {"up": up, "down": down}


def config4_linear(name, M=2048, device="cpu"):
    """One of the 7 linears of a LLaMA-65B block, per-row weight std U(0.01, 0.05), r = 64."""
    i = list(LLAMA65B_BLOCK).index(name)
    N, K = LLAMA65B_BLOCK[name]
    base = 100 * (i + 1)
    W = weight_row_std(N, K, 0.01, 0.05, base, torch.bfloat16, device)
    L1 = normal((K, 64), 1.0 / K, base + 1, device=device)
    L2 = normal((64, N), 0.01, base + 2, device=device)
    X = normal((M, K), 1.0, base + 3, device=device)
    dY = normal((M, N), 1e-2, base + 4, device=device)
    return {"W": W, "L1": L1, "L2": L2, "X": X, "dY": dY}


def config5_weight(layer, name, variant, device="cpu"):
    """Encoder workload: one matrix of layer `layer` of a 65B model, N(0, 0.02)
    (variant "gauss") or 0.02 * t_5 (variant "t5"), bf16."""
    N, K = LLAMA65B_BLOCK[name]
    i = list(LLAMA65B_BLOCK).index(name)
    if variant == "gauss":
        return weight_gaussian(N, K, 0.02, 1000 + 10 * layer + i, torch.bfloat16, device)
    return weight_student_t(N, K, 0.02, 5, 2000 + 10 * layer + i, torch.bfloat16, device)
