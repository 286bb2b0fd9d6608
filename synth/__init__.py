"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the method: only random tensors with the
shapes and value distributions of the workloads (Wan2.1-T2V-1.3B attention:
12 heads of size 128; latent grids 16x28x56 and 21x30x52; 4x4x8 VSA cubes).
Everything is drawn on the CPU with ``torch.Generator`` so both the HIP path
and the oracle see identical bits.  Tensors are bf16 in the pages' public
[B, L, H, D] layout unless a function says otherwise.
"""
from __future__ import annotations

import torch

HEAD_DIM = 128
WAN_HEADS = 12


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def normal_bf16(shape, seed: int) -> torch.Tensor:
    """N(0, 1) values rounded to bf16."""
    return torch.randn(*shape, generator=_gen(seed), dtype=torch.float32).to(torch.bfloat16)


def qkv_headscaled(B: int, L: int, H: int, D: int, seed: int, scaled: bool = True):
    """Q, K, V in [B, L, H, D] bf16: N(0,1) times an independent per-(tensor, head)
    factor drawn from U(0.5, 2) when ``scaled``."""
    g = _gen(seed)
    out = []
    for _ in range(3):
        x = torch.randn(B, L, H, D, generator=g, dtype=torch.float32)
        if scaled:
            c = 0.5 + 1.5 * torch.rand(H, generator=g, dtype=torch.float32)
            x = x * c.view(1, 1, H, 1)
        out.append(x.to(torch.bfloat16))
    return tuple(out)


def fq_tensor(rows: int = 301056, cols: int = HEAD_DIM, seed: int = 1002,
              outlier_frac: float = 0.001, zero_frac: float = 0.01, outlier_mult: float = 50.0):
    """The standalone fake-quant workload: bf16 [rows, cols] ~ N(0,1), with a
    disjoint random set of ``outlier_frac`` positions multiplied by
    ``outlier_mult`` and ``zero_frac`` positions set to exactly 0."""
    g = _gen(seed)
    n = rows * cols
    x = torch.randn(n, generator=g, dtype=torch.float32)
    perm = torch.randperm(n, generator=g)
    n_out = int(n * outlier_frac)
    n_zero = int(n * zero_frac)
    x[perm[:n_out]] *= outlier_mult
    x[perm[n_out:n_out + n_zero]] = 0.0
    return x.view(rows, cols).to(torch.bfloat16)


def tiny_forward(seed: int = 1001):
    """B=1, H=2, L=256, D=128 non-causal, Q/K/V ~ N(0,1)."""
    return qkv_headscaled(1, 256, 2, HEAD_DIM, seed, scaled=False)


def wan_448x896x61(seed: int = 1003):
    """Wan2.1 1.3B latents at 448x896, 61 frames: L = 16*28*56 = 25088."""
    return qkv_headscaled(1, 16 * 28 * 56, WAN_HEADS, HEAD_DIM, seed, scaled=True)


def wan_480x832x81(seed: int = 1004):
    """Wan2.1 1.3B latents at 480x832, 81 frames: L = 21*30*52 = 32760, plus dO."""
    L = 21 * 30 * 52
    q, k, v = qkv_headscaled(1, L, WAN_HEADS, HEAD_DIM, seed, scaled=True)
    do = normal_bf16((1, L, WAN_HEADS, HEAD_DIM), seed + 100000)
    return q, k, v, do


def vsa_inputs(seed: int = 1005, grid=(16, 28, 56), heads: int = WAN_HEADS):
    """Cube-major Q, K, V ~ N(0,1) for the cube-sparse workload."""
    L = grid[0] * grid[1] * grid[2]
    return qkv_headscaled(1, L, heads, HEAD_DIM, seed, scaled=False)


def wan_ffn(k_in: int = 1536, k_out: int = 8960, tokens: int = 16 * 28 * 56, seed: int = 1006):
    """One feed-forward projection of the Wan2.1 1.3B block at 448x896, 61 frames (25088 tokens,
    model width 1536, FFN width 8960): activations x [tokens, k_in] ~ N(0, 1), weight
    [k_out, k_in] ~ N(0, 0.02^2) (the usual initialiser scale), bias [k_out] ~ N(0, 1) and the
    output gradient [tokens, k_out] ~ N(0, 1), all bf16."""
    x = normal_bf16((tokens, k_in), seed)
    w = (torch.randn(k_out, k_in, generator=_gen(seed + 1)) * 0.02).to(torch.bfloat16)
    b = normal_bf16((k_out,), seed + 2)
    g = normal_bf16((tokens, k_out), seed + 3)
    return x, w, b, g


def sample_rows(L: int, n: int = 64, seed: int = 7, head: int = 8, tail: int = 8):
    """Sorted query/key rows: the first ``head``, the last ``tail`` and the
    rest drawn at random without repetition."""
    g = _gen(seed)
    fixed = list(range(min(head, L))) + list(range(max(0, L - tail), L))
    rest = [r for r in torch.randperm(L, generator=g).tolist() if r not in set(fixed)]
    rows = sorted(set(fixed + rest[:max(0, n - len(set(fixed)))]))
    return torch.tensor(rows, dtype=torch.int64)


def to_bhld_bits(x_blhd: torch.Tensor):
    """bf16 [B, L, H, D] -> numpy uint16 [B, H, L, D] (bit patterns)."""
    return x_blhd.permute(0, 2, 1, 3).contiguous().view(torch.int16).numpy().view("uint16")

