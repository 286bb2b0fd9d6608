"""GPU parity of the cube-sparse straight-through backward (vsa_qat_bwd) against the
oracle (oracle.vsa_bwd), within the stated attention tolerance (tests/parity.py).

The selection is an integer decision that the kernel takes on fp32 coarse logits and
the oracle on fp64, from cube means that may differ by one bf16 ulp.  Gradients are
compared where the two selections agree: dQ on query cubes whose lists agree, dK/dV on
key cubes that every query cube selected (or not) on both sides.  On the full
448x896x61 workload (196 cubes, top-20) the test samples rows of one head against the
oracle and checks two identities on every head that hold for any selection:
sum_j <dV_j, V-hat_j> = sum_i <dO_i, O_i> (O built from P-hat) and sum_j <dK_j, K-hat_j> = sum_i <dQ_i, Q-hat_i>."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import parity
from tests.parity import assert_close, bf16_values, bhld_bits

pytestmark = pytest.mark.gpu
SCALE = 1.0 / math.sqrt(128)
CUBE = (4, 4, 8)


@pytest.fixture(scope="module")
def m():
    import quantization_aware_attention_nvfp4_amd as m
    return m


def gpu_fwd_bwd(m, q, k, v, do, grid, sparsity, flags=15):
    qg, kg, vg, dog = (t.cuda() for t in (q, k, v, do))
    o, aux = m.vsa_qat_fwd(qg, kg, vg, grid=grid, cube=CUBE, sparsity=sparsity, quant_flags=flags, training=True)
    dq, dk, dv = m.vsa_qat_bwd(qg, kg, vg, aux, dog, grid=grid, cube=CUBE, sparsity=sparsity, quant_flags=flags)
    torch.cuda.synchronize()
    return o, aux["sel"].cpu().numpy(), dq, dk, dv


def agreement(sel_gpu, q, k, sparsity, min_agree=0.9):
    """Per (b, h): query cubes whose lists agree with the oracle's, and key cubes whose selectors
    agree; every differing cube must be a near tie (tests/parity.py)."""
    r = oracle.vsa_fwd(bhld_bits(q), bhld_bits(k), bhld_bits(k), SCALE, sparsity=sparsity,
                       rows=np.zeros(0, np.int64))
    return parity.check_selection(sel_gpu, r["sel"], r["score"], min_agree=min_agree)


def rows_of(mask_bhn, cube=128):
    return np.repeat(mask_bhn, cube, axis=-1)


@pytest.mark.parametrize("grid,sparsity,flags", [((4, 8, 16), 0.5, 15), ((4, 8, 32), 0.6, 15),
                                                 ((4, 8, 32), 0.6, 0)])
def test_full_gradients(m, grid, sparsity, flags):
    L = grid[0] * grid[1] * grid[2]
    q, k, v = synth.qkv_headscaled(1, L, 2, 128, seed=93 + L, scaled=False)
    do = synth.normal_bf16(q.shape, 95 + L)
    o, sel, dq, dk, dv = gpu_fwd_bwd(m, q, k, v, do, grid, sparsity, flags)
    r = oracle.vsa_bwd(bhld_bits(q), bhld_bits(k), bhld_bits(v), bhld_bits(do), SCALE, sparsity=sparsity,
                       flags=flags)
    assert sel.shape == r["sel"].shape
    qa, ka = agreement(sel, q, k, sparsity, min_agree=0.75)
    assert np.array_equal(qa, np.all(r["sel"] == sel, axis=-1))  # vsa_bwd selects as vsa_fwd does
    qmask, kmask = rows_of(qa), rows_of(ka)
    for name, t, mask in (("dq", dq, qmask), ("dk", dk, kmask), ("dv", dv, kmask)):
        got = bf16_values(t.permute(0, 2, 1, 3))
        assert_close(got[mask], r[name][mask], f"{name} L={L} flags={flags}")


def test_autograd_function_matches_explicit_calls(m):
    grid = (4, 8, 32)
    L = 1024
    q, k, v = synth.qkv_headscaled(1, L, 2, 128, seed=97, scaled=False)
    do = synth.normal_bf16(q.shape, 98)
    _, _, dq, dk, dv = gpu_fwd_bwd(m, q, k, v, do, grid, 0.6)
    qg, kg, vg = (t.cuda().requires_grad_() for t in (q, k, v))
    out = m.vsa_qat_train(qg, kg, vg, grid=grid, cube=CUBE, sparsity=0.6)
    out.backward(do.cuda())
    torch.cuda.synchronize()
    for a, b in ((qg.grad, dq), (kg.grad, dk), (vg.grad, dv)):
        assert torch.equal(a, b)


def test_deterministic(m):
    grid = (4, 8, 32)
    q, k, v = synth.qkv_headscaled(1, 1024, 2, 128, seed=99, scaled=False)
    do = synth.normal_bf16(q.shape, 100)
    a = gpu_fwd_bwd(m, q, k, v, do, grid, 0.6)
    b = gpu_fwd_bwd(m, q, k, v, do, grid, 0.6)
    for x, y in zip(a[2:], b[2:]):
        assert torch.equal(x, y)


def test_wan_448x896x61_sampled_rows_and_identities(m):
    grid = (16, 28, 56)
    q, k, v = synth.vsa_inputs()
    do = synth.normal_bf16(q.shape, 1105)
    o, sel, dq, dk, dv = gpu_fwd_bwd(m, q, k, v, do, grid, 0.9)
    B, L, H, D = q.shape
    assert sel.shape == (1, H, 196, 20)
    # Identities on every head, from the kernel's own outputs.  Both sides are sums of
    # products whose terms carry independent bf16 roundings (dV, dK, dQ are bf16), so the
    # difference is measured against the root-sum-square of the terms: that noise is about
    # 2^-9 of it, a wrong gradient row moves the sums by about its own size.
    bhld = lambda t: t.double().cpu().permute(0, 2, 1, 3)
    hat = lambda t, axis: torch.from_numpy(oracle.bf16_bits_to_f32(oracle.fq_bf16(bhld_bits(t), axis=axis))
                                           .astype(np.float64))
    qh, kh, vh = hat(q, -1), hat(k, -1), hat(v, 2)
    # O here is the output built from P-hat (O^hp, from the unquantized P, is what D uses).
    pairs = (("dV", bhld(do) * bhld(o), bhld(dv) * vh), ("dK", bhld(dq) * qh, bhld(dk) * kh))
    for what, ta, tb in pairs:
        a, b = ta.sum(dim=(2, 3)), tb.sum(dim=(2, 3))
        norm = tb.pow(2).sum(dim=(2, 3)).sqrt()
        worst = ((a - b).abs() / norm).max().item()
        assert worst <= 2e-2, f"{what} identity: |a-b| / rss {worst:.3e}"
    # sampled rows of head 0 against the oracle
    h = 0
    rows = synth.sample_rows(L, 48, seed=11).numpy()
    r = oracle.vsa_bwd(bhld_bits(q[:, :, h:h + 1]), bhld_bits(k[:, :, h:h + 1]), bhld_bits(v[:, :, h:h + 1]),
                       bhld_bits(do[:, :, h:h + 1]), SCALE, sparsity=0.9, qrows=rows, krows=rows)
    qa, ka = agreement(sel[:, h:h + 1], q[:, :, h:h + 1], k[:, :, h:h + 1], 0.9, min_agree=0.95)
    parity.assert_valid_selection(sel, 196)
    qok, kok = qa[0, 0][rows // 128], ka[0, 0][rows // 128]
    for name, t, ok in (("dq", dq, qok), ("dk", dk, kok), ("dv", dv, kok)):
        got = bf16_values(t[:, torch.as_tensor(rows), h].unsqueeze(1))  # [1, 1, R, D]
        assert_close(got[0, 0][ok], r[name][0, 0][ok], f"{name} sampled rows")
