"""GPU parity of the standalone NVFP4 fake quantization (fq_nvfp4) against the
oracle: bit-exact, unit and static global scale, at the full 301056 x 128
workload (25088 tokens x 12 heads x D=128, N(0,1) with 0.1% x50 outliers and
1% exact zeros) and on ragged / strided layouts."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import quantization_aware_attention_nvfp4_amd as m
    return m


def gpu_fq(m, x_cpu, axis=-1, g=None):
    x = x_cpu.cuda()
    y = m.fq_nvfp4(x, axis=axis, global_scale=g)
    torch.cuda.synchronize()
    return bits(y)


def test_full_workload_unit_scale_bit_exact(lib):
    x = synth.fq_tensor()
    got = gpu_fq(lib, x)
    want = oracle.fq_bf16(bits(x))
    mism = np.count_nonzero(got != want)
    assert mism == 0, f"{mism} of {got.size} elements differ"


def test_full_workload_static_scale_bit_exact(lib):
    x = synth.fq_tensor()
    xg = x.cuda()
    g = lib.static_global_scale(xg)
    torch.cuda.synchronize()
    g_ref = oracle.static_scale_bf16(bits(x))
    assert g.item() == np.float32(g_ref)
    y = lib.fq_nvfp4(xg, global_scale=g)
    torch.cuda.synchronize()
    want = oracle.fq_bf16(bits(x), g=g_ref)
    got = bits(y)
    assert np.count_nonzero(got != want) == 0
    # and through the "static" shortcut
    y2 = lib.fq_nvfp4(xg, global_scale="static")
    torch.cuda.synchronize()
    assert np.array_equal(bits(y2), want)


@pytest.mark.parametrize("shape,axis", [((7, 37), -1), ((3, 40, 7), 1), ((1, 16), -1), ((5, 3), -1),
                                        ((2, 33, 12, 128), 1), ((4, 128), 0)])
@pytest.mark.parametrize("static", [False, True])
def test_ragged_and_strided_layouts(lib, shape, axis, static):
    g = torch.Generator().manual_seed(11)
    x = (torch.randn(*shape, generator=g) * 3).to(torch.bfloat16)
    gval = oracle.static_scale_bf16(bits(x)) if static else 1.0
    gt = torch.tensor([gval], dtype=torch.float32, device="cuda") if static else None
    got = gpu_fq(lib, x, axis=axis, g=gt)
    want = oracle.fq_bf16(bits(x), axis=axis, g=gval)
    assert np.array_equal(got, want)


def test_all_bf16_block_maxima(lib):
    # Blocks [amax, x1..x15] for every non-negative finite bf16 amax and 60 x values per amax
    # spread over [-amax, amax] (including +-amax, 0 and the smallest magnitudes).
    amax_bits = np.arange(0, 0x7F80, dtype=np.uint16)
    rng = np.random.default_rng(12)
    rows = []
    for rep in range(4):
        frac = rng.integers(0, 1 << 16, size=(amax_bits.size, 15)).astype(np.uint32)
        xb = ((frac * amax_bits[:, None].astype(np.uint32)) >> 16).astype(np.uint16)  # |x| bits <= amax bits
        sign = (rng.integers(0, 2, size=xb.shape).astype(np.uint16) << 15)
        blk = np.concatenate([amax_bits[:, None], xb | sign], axis=1)
        if rep == 0:
            blk[:, 1] = amax_bits | 0x8000
            blk[:, 2] = 0
        rows.append(blk)
    blocks = np.concatenate(rows).astype(np.uint16)
    x = torch.from_numpy(blocks.view(np.int16)).view(torch.bfloat16)
    got = gpu_fq(lib, x)
    want = oracle.fq_bf16(blocks)
    assert np.array_equal(got, want)


def test_in_place_and_deterministic(lib):
    x = synth.fq_tensor(rows=4096)
    xg = x.cuda()
    y1 = bits(lib.fq_nvfp4(xg))
    y2 = bits(lib.fq_nvfp4(xg))
    lib.fq_nvfp4(xg, out=xg)
    torch.cuda.synchronize()
    assert np.array_equal(y1, y2)
    assert np.array_equal(bits(xg), y1)


def test_every_e2m1_decision_boundary(lib):
    # For every positive E4M3 scale S: blocks whose amax is 6S (so the block scale is S) holding
    # each midpoint t*S of the E2M1 grid, its bf16 neighbours, and their negations.
    codes = np.arange(1, 127)
    e, mnt = codes >> 3, codes & 7
    scales = np.where(e == 0, np.ldexp(mnt.astype(np.float64), -9), np.ldexp(1 + mnt / 8.0, e - 7))
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    rows = []
    for S in scales:
        t = torch.tensor(mids * S, dtype=torch.float32).to(torch.bfloat16)
        tb = t.view(torch.int16).numpy().view(np.uint16)
        vals = np.concatenate([tb, tb - 1, tb + 1])
        vals = np.concatenate([vals, vals | 0x8000]).astype(np.uint16)  # 42 values
        amax = torch.tensor([6 * S], dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        for i in range(0, 42, 14):
            blk = np.zeros(16, np.uint16)
            blk[0] = amax[0]
            blk[1:15] = vals[i:i + 14]
            rows.append(blk)
    blocks = np.stack(rows)
    x = torch.from_numpy(blocks.view(np.int16)).view(torch.bfloat16)
    assert np.array_equal(gpu_fq(lib, x), oracle.fq_bf16(blocks))
