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


# ---- cube-sparse selections -------------------------------------------------------------------
# A selection is an integer decision the kernel takes on fp32 coarse logits and the oracle on fp64,
# from cube means that may differ by one bf16 ulp.  Both must list topk distinct cubes in ascending
# order; where the two lists differ, every differing cube must be a near tie at the top-k boundary.

def assert_valid_selection(sel: np.ndarray, n: int, what: str = "sel") -> None:
    """Every row strictly ascending (so distinct) with entries in [0, n)."""
    sel = np.asarray(sel)
    assert sel.min() >= 0 and sel.max() < n, f"{what}: entries outside [0, {n})"
    if sel.shape[-1] > 1:
        assert np.all(np.diff(sel, axis=-1) > 0), f"{what}: a row is not strictly ascending"


def check_selection(sel_gpu, sel_ref, score, rel_tol=2e-3, min_agree=0.9):
    """Compare two selections [B, H, n, k] (the oracle's coarse scores `score` [B, H, n, n]).
    Returns per-(b, h) masks of the query cubes whose lists agree and of the key cubes on which
    every query cube's choice agrees."""
    sel_gpu, sel_ref = np.asarray(sel_gpu), np.asarray(sel_ref)
    B, H, n, k = sel_ref.shape
    assert sel_gpu.shape == sel_ref.shape, (sel_gpu.shape, sel_ref.shape)
    assert_valid_selection(sel_gpu, n, "gpu sel")
    assert_valid_selection(sel_ref, n, "oracle sel")
    qa = np.all(sel_gpu == sel_ref, axis=-1)
    ka = np.ones((B, H, n), bool)
    spread = np.abs(score).max()
    for b, h, a in zip(*np.nonzero(~qa)):
        s = score[b, h, a]
        kth = np.sort(s)[::-1][k - 1]
        for c in set(sel_gpu[b, h, a].tolist()) ^ set(sel_ref[b, h, a].tolist()):
            assert abs(s[c] - kth) <= rel_tol * spread, (b, h, a, c, s[c], kth)
            ka[b, h, c] = False
    assert qa.mean() >= min_agree, qa.mean()
    return qa, ka
