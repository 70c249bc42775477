"""Seeded synthetic inputs with the shapes and value distributions of the
workloads (no quantization arithmetic here).

Each generator draws with a torch.Generator seeded as stated, on the device
asked for (the CPU and GPU generators give different streams; a test uses one
device and copies to the other).  Float32 draws are rounded to bf16 where the
workload is bf16.

Recipes:
  mlp_weight_fp32   [3072, 1024] f32 = 0.02 * N(0,1); round(0.1% * n) entries
                    at randperm(n) positions scaled by 50 (outliers).  Seed 0.
  fp8_weight        [7168, 2048] bf16 N(0, 0.02^2).  Seed 1.
  fp8_activation    [8192, 7168] bf16 N(0,1); channels randperm(cols)[:8]
                    scaled by 40 (channel outliers).  Seed 2.
  llama_weight      decoder layer l, projection p (q, k, v, o, gate, up, down):
                    bf16 N(0, 0.02^2) of the Llama-3.1-8B shape.
                    Seed 3000 + 7 l + p.
  kv_layer          K = bias (N(0, 4) per (head, dim), constant over tokens,
                    seed 4000 + l) + 0.1 * N(0,1) per element; V = N(0,1)
                    (seed 5000 + l).  bf16 [tokens, heads, head_dim].
  heavy_tail_weight [28672, 8192] bf16 = 0.02 * Student-t(nu=4), nu=4 drawn as
                    Z / sqrt(mean of 4 squared normals).  Seed 5.
  gaussian          any shape, bf16 N(0,1).  Seed 6 for the 1 GiB sweep.
"""
from __future__ import annotations

import torch

LLAMA_PROJ = (("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
              ("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336))
LLAMA_LAYERS = 32


def _gen(seed: int, device) -> torch.Generator:
    return torch.Generator(device=device).manual_seed(seed)


def mlp_weight_fp32(rows=3072, cols=1024, seed=0, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    x = torch.randn((rows, cols), generator=g, device=device) * 0.02
    n = rows * cols
    k = round(0.001 * n)
    idx = torch.randperm(n, generator=g, device=device)[:k]
    x.view(-1)[idx] *= 50.0
    return x


def fp8_weight(rows=7168, cols=2048, seed=1, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    return (torch.randn((rows, cols), generator=g, device=device) * 0.02).to(torch.bfloat16)


def fp8_activation(rows=8192, cols=7168, seed=2, device="cpu", n_outlier=8) -> torch.Tensor:
    g = _gen(seed, device)
    x = torch.randn((rows, cols), generator=g, device=device)
    ch = torch.randperm(cols, generator=g, device=device)[:n_outlier]
    x[:, ch] *= 40.0
    return x.to(torch.bfloat16)


def llama_weight(layer: int, proj: int, device="cpu", scale_rows=1, scale_cols=1) -> torch.Tensor:
    _, r, c = LLAMA_PROJ[proj]
    g = _gen(3000 + 7 * layer + proj, device)
    w = torch.randn((r // scale_rows, c // scale_cols), generator=g, device=device) * 0.02
    return w.to(torch.bfloat16)


def kv_layer(layer: int, tokens=32768, heads=8, head_dim=128, device="cpu"):
    gk = _gen(4000 + layer, device)
    bias = torch.randn((1, heads, head_dim), generator=gk, device=device) * 2.0
    k = bias + 0.1 * torch.randn((tokens, heads, head_dim), generator=gk, device=device)
    gv = _gen(5000 + layer, device)
    v = torch.randn((tokens, heads, head_dim), generator=gv, device=device)
    return k.to(torch.bfloat16), v.to(torch.bfloat16)


def kv_cache(layers=28, tokens=32768, heads=8, head_dim=128, device="cpu"):
    """K and V as [layers, tokens, heads, head_dim] bf16."""
    k = torch.empty((layers, tokens, heads, head_dim), dtype=torch.bfloat16, device=device)
    v = torch.empty_like(k)
    for l in range(layers):
        k[l], v[l] = kv_layer(l, tokens, heads, head_dim, device)
    return k, v


def heavy_tail_weight(rows=28672, cols=8192, seed=5, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    z = torch.randn((rows, cols), generator=g, device=device)
    chi = torch.zeros((rows, cols), device=device)
    for _ in range(4):
        chi += torch.randn((rows, cols), generator=g, device=device).square_()
    return (0.02 * z / torch.sqrt(chi / 4.0)).to(torch.bfloat16)


def gaussian(rows=65536, cols=8192, seed=6, device="cpu", dtype=torch.bfloat16) -> torch.Tensor:
    g = _gen(seed, device)
    return torch.randn((rows, cols), generator=g, device=device).to(dtype)
