"""Comparison helpers shared by the GPU parity tests.

Attention tolerance (reading of the stated bar): compare the GPU's bf16 output
with the oracle's fp64 result rounded to bf16, and require
  max|gpu - ref| <= 1e-2 * max|ref|   and   sum|gpu - ref| / sum|ref| <= 2e-3.
"""
import numpy as np
import torch

MAX_REL = 1e-2
MEAN_REL = 2e-3


def to_bf16_f64(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 (RNE) and return them as fp64."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)).to(torch.bfloat16).double().numpy()


def metrics(gpu: np.ndarray, ref: np.ndarray):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.abs(gpu - ref)
    return d.max() / max(np.abs(ref).max(), 1e-300), d.sum() / max(np.abs(ref).sum(), 1e-300)


def assert_close(gpu, ref, what="", max_rel=MAX_REL, mean_rel=MEAN_REL, round_ref=True):
    ref = to_bf16_f64(ref) if round_ref else np.asarray(ref, dtype=np.float64)
    mx, mean = metrics(gpu, ref)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite values"
    assert mx <= max_rel and mean <= mean_rel, f"{what}: max rel {mx:.3e} (<= {max_rel}), mean rel {mean:.3e} (<= {mean_rel})"
    return mx, mean


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 numpy bit patterns (CPU copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bhld_bits(t_blhd: torch.Tensor) -> np.ndarray:
    return bits(t_blhd.permute(0, 2, 1, 3))


def bf16_values(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)
