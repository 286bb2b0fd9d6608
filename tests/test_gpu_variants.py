"""GPU parity of the attention variants (AQ_FINAL_MAX, AQ_GSF_QKV, AQ_GSF_P, AQ_SMOOTH_K,
AQ_TWO_LEVEL_P, AQ_SMOOTH_Q, AQ_PV_FP8) against the oracle, within the stated attention tolerance (tests/parity.py).

Dense forward (inference and training outputs) and straight-through backward on ragged, cross
and causal shapes; the cube-sparse forward and backward on a small grid (compared where the two
selections agree, as in the other cube-sparse tests); sampled rows of the 448x896x61 workload
under the final-max statistics, two-level P and smooth-Q.  Properties that hold for any input: under AQ_FINAL_MAX every
chunk-maximum row equals the row's final maximum, and lse is unchanged up to rounding; under
AQ_TWO_LEVEL_P the first-level scales the forward stores match the oracle's to fp32 rounding."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import parity
from tests.parity import assert_close, bf16_values, bhld_bits

pytestmark = pytest.mark.gpu
LOG2E = 1.0 / math.log(2.0)
SCALE = 1.0 / math.sqrt(128)
ALL = 15
FM, GQKV, GP, SK, TWO, SQ, PV8 = 16, 32, 64, 128, 256, 512, 1024
VARIANTS = [ALL | FM, ALL | GQKV, ALL | GP, ALL | SK, SK, ALL | FM | GQKV | GP | SK, ALL | TWO, ALL | TWO | GQKV | SK,
            ALL | SQ, SQ, ALL | SQ | SK | GQKV | FM | GP, ALL | SQ | TWO, ALL | PV8, 8 | PV8, ALL | PV8 | GP | FM,
            ALL | PV8 | TWO | GQKV]


@pytest.fixture(scope="module")
def m():
    import quantization_aware_attention_nvfp4_amd as m
    return m


def rand(B, L, H, seed, mult=1.0, shift=0.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(B, L, H, 128, generator=g) * mult + shift).to(torch.bfloat16)


def bhrd(x_blhd, rows=None):
    x = x_blhd.permute(0, 2, 1, 3)
    if rows is not None:
        x = x[:, :, torch.as_tensor(rows)]
    return bf16_values(x)


@pytest.mark.parametrize("flags", VARIANTS)
@pytest.mark.parametrize("Lq,Lk,causal", [(300, 333, False), (260, 260, True)])
def test_dense_forward_and_backward(m, flags, Lq, Lk, causal):
    q, k, v, do = rand(1, Lq, 2, 201), rand(1, Lk, 2, 202, 1.5, 0.8), rand(1, Lk, 2, 203), rand(1, Lq, 2, 204)
    qg, kg, vg, dog = (t.cuda() for t in (q, k, v, do))
    o_inf = m.attn_qat_fwd(qg, kg, vg, causal=causal, quant_flags=flags)
    o, aux = m.attn_qat_fwd(qg, kg, vg, causal=causal, quant_flags=flags, training=True)
    dq, dk, dv = m.attn_qat_bwd(qg, kg, vg, aux, dog, causal=causal, quant_flags=flags)
    torch.cuda.synchronize()
    args = (bhld_bits(q), bhld_bits(k), bhld_bits(v))
    r = oracle.attn_fwd(*args, SCALE, causal=causal, flags=flags)
    assert_close(bhrd(o_inf), r["o"], f"o inference flags={flags}")
    assert torch.equal(o_inf.view(torch.int16), o.view(torch.int16))  # training adds outputs only
    assert_close(aux["o_hp"].cpu().numpy(), r["o_hp"], f"o_hp flags={flags}")
    lse = aux["lse_log2"].cpu().numpy() / LOG2E
    assert np.abs(lse - r["lse"]).max() < 1e-4
    if flags & TWO:
        # the first-level scales of the live (row, chunk) pairs
        ps = aux["p_scale"].cpu().numpy()
        for c in range(ps.shape[2]):
            reach = np.ones(Lq, bool) if not causal else (np.arange(Lq) >= 128 * c)
            assert np.allclose(ps[:, :, c][..., reach], r["pscale"][..., c][..., reach], rtol=1e-5, atol=0)
    if flags & FM:
        # every chunk-maximum row holds the final row maximum
        cm = aux["chunk_max_log2"].cpu().numpy()
        fin = r["cmax"][..., 0] * LOG2E
        for c in range(cm.shape[2]):
            reach = np.ones(Lq, bool) if not causal else (np.arange(Lq) >= 128 * c)
            assert np.abs(cm[:, :, c][..., reach] - fin[..., reach]).max() < 1e-4 * max(1.0, np.abs(fin).max())
    b = oracle.attn_bwd(*args, bhld_bits(do), SCALE, causal=causal, flags=flags)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert_close(bhrd(t), b[name], f"{name} flags={flags}")


def test_static_scales_differ_from_unit(m):
    # the variants change the result (the flags reach the kernels)
    q, k, v = rand(1, 256, 2, 205), rand(1, 256, 2, 206), rand(1, 256, 2, 207)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    base = m.attn_qat_fwd(qg, kg, vg)
    for fl in (ALL | FM, ALL | GQKV, ALL | GP, ALL | SK, ALL | TWO, ALL | SQ, ALL | PV8):
        assert not torch.equal(m.attn_qat_fwd(qg, kg, vg, quant_flags=fl), base), fl




@pytest.mark.parametrize("flags", [ALL | FM, ALL | FM | GQKV | GP | SK, ALL | TWO | GQKV, ALL | SQ | SK, ALL | PV8 | SK])
def test_cube_sparse_forward_and_backward(m, flags):
    grid, L = (4, 8, 32), 1024
    q, k, v = synth.qkv_headscaled(1, L, 2, 128, seed=208, scaled=False)
    do = synth.normal_bf16(q.shape, 209)
    qg, kg, vg, dog = (t.cuda() for t in (q, k, v, do))
    o, aux = m.vsa_qat_fwd(qg, kg, vg, grid=grid, sparsity=0.6, quant_flags=flags, training=True)
    dq, dk, dv = m.vsa_qat_bwd(qg, kg, vg, aux, dog, grid=grid, sparsity=0.6, quant_flags=flags)
    torch.cuda.synchronize()
    args = (bhld_bits(q), bhld_bits(k), bhld_bits(v))
    rf = oracle.vsa_fwd(*args, SCALE, sparsity=0.6, flags=flags)
    rb = oracle.vsa_bwd(*args, bhld_bits(do), SCALE, sparsity=0.6, flags=flags)
    # selection is not affected by the variants (coarse stage unquantized): near ties only
    qa, ka = parity.check_selection(aux["sel"].cpu().numpy(), rf["sel"], rf["score"], min_agree=0.75)
    qmask, kmask = np.repeat(qa, 128, -1), np.repeat(ka, 128, -1)
    assert_close(bhrd(o)[qmask], rf["o_fine"][qmask], f"o_fine flags={flags}")
    for name, t, mask in (("dq", dq, qmask), ("dk", dk, kmask), ("dv", dv, kmask)):
        assert_close(bhrd(t)[mask], rb[name][mask], f"vsa {name} flags={flags}")


@pytest.mark.parametrize("flags", [ALL | FM, ALL | TWO, ALL | SQ, ALL | PV8])
def test_wan_448x896x61_sampled_rows(m, flags):
    q, k, v = synth.wan_448x896x61()
    L = q.shape[1]
    o = m.attn_qat_fwd(q.cuda(), k.cuda(), v.cuda(), quant_flags=flags)
    torch.cuda.synchronize()
    rows = synth.sample_rows(L, 32, seed=12).numpy()
    h = [0, 7]
    r = oracle.attn_fwd(bhld_bits(q[:, :, h]), bhld_bits(k[:, :, h]), bhld_bits(v[:, :, h]), SCALE,
                        flags=flags, rows=rows)
    assert_close(bhrd(o[:, :, h], rows), r["o"], f"o at 448x896x61 flags={flags}")


def test_two_level_rejections(m):
    q = rand(1, 128, 1, 221).cuda()
    for extra in (FM, GP):
        with pytest.raises(NotImplementedError):
            m.attn_qat_fwd(q, q, q, quant_flags=ALL | TWO | extra)


def test_pv_fp8_needs_quantized_p(m):
    q = rand(1, 128, 1, 222).cuda()
    for fl in (PV8, 7 | PV8):
        with pytest.raises(NotImplementedError):
            m.attn_qat_fwd(q, q, q, quant_flags=fl)


@pytest.mark.parametrize("causal", [False, True])
def test_smooth_q_offset_query(m, causal):
    # a query with a large common offset (the case the smoothing is for): forward, training outputs
    # and backward against the oracle
    L = 300 if not causal else 260
    q, k, v, do = rand(1, L, 2, 231, 1.0, 3.0), rand(1, L, 2, 232), rand(1, L, 2, 233), rand(1, L, 2, 234)
    flags = ALL | SQ
    qg, kg, vg, dog = (t.cuda() for t in (q, k, v, do))
    o, aux = m.attn_qat_fwd(qg, kg, vg, causal=causal, quant_flags=flags, training=True)
    dq, dk, dv = m.attn_qat_bwd(qg, kg, vg, aux, dog, causal=causal, quant_flags=flags)
    torch.cuda.synchronize()
    args = (bhld_bits(q), bhld_bits(k), bhld_bits(v))
    r = oracle.attn_fwd(*args, SCALE, causal=causal, flags=flags)
    assert_close(bhrd(o), r["o"], "smooth-Q o")
    b = oracle.attn_bwd(*args, bhld_bits(do), SCALE, causal=causal, flags=flags)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert_close(bhrd(t), b[name], f"smooth-Q {name}")
