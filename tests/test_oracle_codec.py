"""Pins for the oracle's NVFP4 codec (CPU only).

The oracle is checked against things other than itself:
  * hand-derived closed forms (tests/golden/codec_closed_forms.txt);
  * PyTorch's own FP8 E4M3FN cast, a library routine, over every input the
    block-scale rounding can see from a bf16 amax;
  * an exact threshold formulation of E2M1 rounding (compare |x| with t*S in
    float64, where t*S is exact) over every E4M3 scale and every bf16 x;
  * invariants of the format (power-of-two equivariance, error bound,
    static-scale bound).
Format sources: "vsqa-preview-1.3b metadata.json" dense precision record
(group_size 16, NVFP4 E2M1 values, FP8 E4M3FN scales); "nvfp4_qad.py"
module docstring and FP4_RANGE / weight_global_sf.
"""
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "codec_closed_forms.txt")


def bits(x):
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def vals(u16):
    return oracle.bf16_bits_to_f32(u16)


def load_golden():
    rows = []
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if line:
            rows.append([float(t) for t in line.split()])
    return rows


@pytest.mark.parametrize("row", load_golden())
def test_closed_forms(row):
    amax, x, scale, y = row
    blk = np.zeros(16, np.float32)
    blk[0] = amax
    blk[1] = x
    out = vals(oracle.fq_bf16(bits(blk)))
    assert oracle.block_scale(amax) == scale
    assert out[1] == y and np.signbit(out[1]) == np.signbit(np.float32(y))


def test_all_ones_block():
    out = vals(oracle.fq_bf16(bits(np.ones(16, np.float32))))
    assert np.all(out == 1.03125)


def test_e4m3_matches_torch_cast_for_every_bf16_amax():
    # Every non-negative finite bf16 amax; the scale input is fp32(amax / 6).
    a = vals(np.arange(0, 0x7F80, dtype=np.uint16))
    v = (a / np.float32(6.0)).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).float().numpy()
    got = np.array([oracle.e4m3(float(t)) for t in v], np.float32)
    inrange = v < 464.0  # torch's cast turns values >= 464 into NaN; the oracle saturates
    assert np.array_equal(got[inrange], ref[inrange])
    assert np.all(got[~inrange] == 448.0)


def test_e4m3_on_fp32_midpoints_and_neighbours():
    # Every E4M3 midpoint, and the fp32 neighbours on both sides of it.
    codes = np.arange(127)
    e, m = codes >> 3, codes & 7
    tab = np.where(e == 0, np.ldexp(m.astype(np.float64), -9), np.ldexp(1 + m / 8.0, e - 7)).astype(np.float32)
    mids = ((tab[:-1].astype(np.float64) + tab[1:]) / 2).astype(np.float32)
    cand = np.concatenate([mids, np.nextafter(mids, 0, dtype=np.float32),
                           np.nextafter(mids, 1e9, dtype=np.float32)])
    ref = torch.from_numpy(cand).to(torch.float8_e4m3fn).float().numpy()
    got = np.array([oracle.e4m3(float(t)) for t in cand], np.float32)
    assert np.array_equal(got, ref)


def _e2m1_exact(x64, S64):
    """E2M1 magnitude of |x|/S decided by exact comparisons |x| vs t*S."""
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    mids = (grid[:-1] + grid[1:]) / 2  # 0.25 0.75 1.25 1.75 2.5 3.5 5
    code = np.zeros(x64.shape, np.int64)
    for k, t in enumerate(mids):
        thr = t * S64
        above = x64 > thr
        tie = x64 == thr
        # past the midpoint -> upper code; on the midpoint -> the even one of (k, k+1)
        up_on_tie = ((k + 1) % 2) == 0
        code = np.where(above | (tie & up_on_tie), k + 1, code)
    return grid[code]


def test_e2m1_exhaustive_over_scales_and_bf16():
    # For every positive E4M3 scale S, every bf16 x in [0, 6S] goes into a block
    # whose amax is 6S (so the block scale is exactly S).
    codes = np.arange(1, 127)
    e, m = codes >> 3, codes & 7
    scales = np.where(e == 0, np.ldexp(m.astype(np.float64), -9), np.ldexp(1 + m / 8.0, e - 7))
    allx = vals(np.arange(0, 0x7F80, dtype=np.uint16)).astype(np.float64)
    blocks, expect = [], []
    for S in scales:
        xs = allx[allx <= 6 * S]
        pad = (-len(xs)) % 15
        xs_p = np.concatenate([xs, np.zeros(pad)])
        b = np.zeros((len(xs_p) // 15, 16))
        b[:, 0] = 6 * S
        b[:, 1:] = xs_p.reshape(-1, 15)
        blocks.append(b)
        ex = np.zeros_like(b)
        ex[:, 0] = 6 * S
        ex[:, 1:] = (_e2m1_exact(xs_p, S) * S).reshape(-1, 15)
        expect.append(ex)
    blocks = np.concatenate(blocks).astype(np.float32)
    expect = np.concatenate(expect).astype(np.float32)
    out = vals(oracle.fq_bf16(bits(blocks)))
    assert np.array_equal(out, expect)


def test_fp32_inputs_match_exact_thresholds():
    # fp32 values (as softmax probabilities are) on and around every decision
    # threshold of every scale.
    codes = np.arange(1, 127)
    e, m = codes >> 3, codes & 7
    scales = np.where(e == 0, np.ldexp(m.astype(np.float64), -9), np.ldexp(1 + m / 8.0, e - 7)).astype(np.float32)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    rows, expect = [], []
    for S in scales:
        thr = (mids * S).astype(np.float32)
        xs = np.concatenate([thr, np.nextafter(thr, 0, dtype=np.float32), np.nextafter(thr, 1e30, dtype=np.float32)])
        xs = xs[xs <= 6 * S]
        pad = (-len(xs)) % 15
        xs = np.concatenate([xs, np.zeros(pad, np.float32)])
        blk = np.zeros((len(xs) // 15, 16), np.float32)
        blk[:, 0] = 6 * S
        blk[:, 1:] = xs.reshape(-1, 15)
        rows.append(blk)
        ex = blk.astype(np.float64).copy()
        ex[:, 1:] = (_e2m1_exact(xs.astype(np.float64), float(S)) * float(S)).reshape(-1, 15)
        expect.append(ex)
    got = oracle.fq_f32_rows(np.concatenate(rows))
    assert np.array_equal(got.astype(np.float64), np.concatenate(expect))


def test_tail_block_equals_zero_padding():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 37)).astype(np.float32)
    y = vals(oracle.fq_bf16(bits(x)))
    xp = np.zeros((5, 48), np.float32)
    xp[:, :37] = x
    yp = vals(oracle.fq_bf16(bits(xp)))
    assert np.array_equal(y, yp[:, :37])


def test_axis_argument_blocks_along_that_axis():
    rng = np.random.default_rng(4)
    x = bits(rng.standard_normal((3, 40, 7)).astype(np.float32))
    y_axis1 = oracle.fq_bf16(x, axis=1)
    y_last = oracle.fq_bf16(np.ascontiguousarray(x.transpose(0, 2, 1)), axis=-1).transpose(0, 2, 1)
    assert np.array_equal(y_axis1, y_last)


def test_power_of_two_equivariance():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2000, 16)).astype(np.float32)
    y = vals(oracle.fq_bf16(bits(x)))
    for k in (-3, -1, 1, 4):
        y2 = vals(oracle.fq_bf16(bits(x * np.float32(2.0 ** k))))
        assert np.array_equal(y2, y * np.float32(2.0 ** k))


def test_error_bound_and_idempotence():
    rng = np.random.default_rng(6)
    x = vals(bits(rng.standard_normal((4000, 16)).astype(np.float32) * 3))
    y = vals(oracle.fq_bf16(bits(x)))
    amax = np.abs(x).max(axis=1)
    S = np.array([oracle.block_scale(float(a)) for a in amax], np.float32)
    # Inside the E2M1 range the error is at most one grid step (2S), and exactly
    # half a step at most where the grid step is S/2 (|x| < 2S).
    assert np.all(np.abs(y - x) <= 1.0 * S[:, None] + 1e-30)
    small = np.abs(x) < 2 * S[:, None]
    assert np.all(np.abs(y - x)[small] <= 0.25 * np.broadcast_to(S[:, None], x.shape)[small])
    # Idempotence is not guaranteed by the format (the block max may move to a
    # different scale); measure it and require it on the vast majority.
    yy = vals(oracle.fq_bf16(bits(y)))
    assert np.mean(yy == y) > 0.99


def test_static_global_scale():
    rng = np.random.default_rng(7)
    x = bits(rng.standard_normal((64, 128)).astype(np.float32) * 7)
    g = oracle.static_scale_bf16(x)
    amax = float(np.abs(vals(x)).max())
    assert g == np.float32(np.float32(2688.0) / np.float32(amax))
    y = vals(oracle.fq_bf16(x, g=g))
    assert np.all(np.abs(y) <= amax * (1 + 2.0 ** -8))
    # the largest element of the tensor lands on the top of the scaled grid
    assert np.isclose(np.abs(y).max(), amax, rtol=2 ** -3)
    # zero tensor: amax clamps at 1e-12
    z = np.zeros((4, 16), np.uint16)
    assert oracle.static_scale_bf16(z) == np.float32(np.float32(2688.0) / np.float32(1e-12))
    assert np.all(vals(oracle.fq_bf16(z, g=oracle.static_scale_bf16(z))) == 0)


def test_unit_scale_outputs_are_exact_bf16():
    # q*S has at most 6 significant bits under a unit scale, so the fp32 result
    # is already a bf16 value: re-rounding changes nothing.
    rng = np.random.default_rng(8)
    x = rng.standard_normal((1000, 16)).astype(np.float32)
    y = oracle.fq_f32_rows(x)
    assert np.array_equal(oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits(y)), y)
