"""GPU parity of the cube-sparse forward (vsa_qat_fwd) against the oracle.

Selection is an integer decision taken on fp32 coarse logits by the kernel and on
fp64 by the oracle, from cube means that may differ by one bf16 ulp; where the two
selections differ, the differing cubes must be a near tie at the top-k boundary,
and the fine output is compared on the query cubes whose selections agree.  The
fine and coarse outputs use the stated attention tolerance (tests/parity.py)."""
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


@pytest.fixture(scope="module")
def m():
    import quantization_aware_attention_nvfp4_amd as m
    return m


def run(m, q, k, v, grid, sparsity):
    o, oc, sel = m.vsa_qat_fwd(q.cuda(), k.cuda(), v.cuda(), grid=grid, cube=(4, 4, 8), sparsity=sparsity,
                               coarse=True, return_sel=True)
    torch.cuda.synchronize()
    return o, oc, sel.cpu().numpy()


def check_selection(sel_gpu, r):
    """Selections must be ascending, distinct and agree except at near ties; returns a mask of
    agreeing query cubes."""
    qa, _ = parity.check_selection(sel_gpu, r["sel"], r["score"], min_agree=0.97)
    return qa


def test_small_grid(m):
    grid = (4, 8, 32)  # 8 cubes of 128 tokens
    q, k, v = synth.qkv_headscaled(1, 1024, 2, 128, seed=91, scaled=False)
    o, oc, sel = run(m, q, k, v, grid, 0.6)
    rows = np.arange(0, 1024, 3)
    r = oracle.vsa_fwd(bhld_bits(q), bhld_bits(k), bhld_bits(v), SCALE, sparsity=0.6, rows=rows)
    assert r["topk"] == 4 and sel.shape[-1] == 4
    agree = check_selection(sel, r)
    ok = agree[:, :, rows // 128]  # [B, H, R]
    got = bf16_values(o.permute(0, 2, 1, 3)[:, :, torch.as_tensor(rows)])
    assert_close(got[ok], r["o_fine"][ok], "vsa fine")
    gotc = bf16_values(oc.permute(0, 2, 1, 3)[:, :, torch.as_tensor(rows)])
    assert_close(gotc, r["o_coarse"], "vsa coarse")


def test_sparsity_zero_equals_dense(m):
    # Every cube selected: each query walks the dense chunk order with the dense kernels'
    # arithmetic (inference and training), so the outputs are the dense ones bit for bit.
    grid = (4, 8, 16)  # 4 cubes
    q, k, v = synth.qkv_headscaled(1, 512, 3, 128, seed=92, scaled=False)
    o, oc, sel = run(m, q, k, v, grid, 0.0)
    assert np.array_equal(sel, np.broadcast_to(np.arange(4), sel.shape))
    dense = m.attn_qat_fwd(q.cuda(), k.cuda(), v.cuda())
    o_tr, _ = m.vsa_qat_fwd(q.cuda(), k.cuda(), v.cuda(), grid=grid, cube=(4, 4, 8), sparsity=0.0, training=True)
    dense_tr, _ = m.attn_qat_fwd(q.cuda(), k.cuda(), v.cuda(), training=True)
    torch.cuda.synchronize()
    assert torch.equal(o_tr.cpu().view(torch.int16), dense_tr.cpu().view(torch.int16))
    assert torch.equal(o.cpu().view(torch.int16), dense.cpu().view(torch.int16))
    r = oracle.attn_fwd(bhld_bits(q), bhld_bits(k), bhld_bits(v), SCALE)
    assert_close(bf16_values(o.permute(0, 2, 1, 3)), r["o"], "vsa at sparsity 0")


@pytest.mark.parametrize("grid", [(4, 8, 16), (4, 12, 8)])
def test_outputs_at_sparsity_zero_equal_dense(m, grid):
    # Every cube selected, every list in ascending order: each query walks the dense chunk order
    # with the dense kernels' arithmetic, so O (inference and training), lse, the chunk maxima and
    # O^hp are the dense ones bit for bit.  (4, 12, 8) has 3 cubes: the last workgroup's second
    # cube is missing.
    L = grid[0] * grid[1] * grid[2]
    q, k, v = synth.qkv_headscaled(1, L, 3, 128, seed=97 + L, scaled=False)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    o_tr, aux = m.vsa_qat_fwd(qg, kg, vg, grid=grid, cube=(4, 4, 8), sparsity=0.0, training=True)
    d_tr, daux = m.attn_qat_fwd(qg, kg, vg, training=True)
    torch.cuda.synchronize()
    assert torch.equal(o_tr.cpu().view(torch.int16), d_tr.cpu().view(torch.int16))
    o_inf = m.vsa_qat_fwd(qg, kg, vg, grid=grid, cube=(4, 4, 8), sparsity=0.0)
    d_inf = m.attn_qat_fwd(qg, kg, vg)
    assert torch.equal(o_inf.cpu().view(torch.int16), d_inf.cpu().view(torch.int16))
    for name in ("lse_log2", "chunk_max_log2", "o_hp"):
        assert torch.equal(aux[name].cpu().view(torch.int32), daux[name].cpu().view(torch.int32)), name


def test_odd_cube_count(m):
    # 3 cubes, top-2: the last workgroup's second wave group has no cube; inference and training
    # outputs against the oracle on every row of the agreeing query cubes.
    grid = (4, 12, 8)
    L = 384
    q, k, v = synth.qkv_headscaled(1, L, 2, 128, seed=98, scaled=False)
    o, oc, sel = run(m, q, k, v, grid, 0.4)
    o_tr, aux = m.vsa_qat_fwd(q.cuda(), k.cuda(), v.cuda(), grid=grid, cube=(4, 4, 8), sparsity=0.4, training=True)
    torch.cuda.synchronize()
    r = oracle.vsa_fwd(bhld_bits(q), bhld_bits(k), bhld_bits(v), SCALE, sparsity=0.4, rows=np.arange(L))
    assert r["topk"] == 2 and sel.shape == (1, 2, 3, 2)
    assert np.array_equal(aux["sel"].cpu().numpy(), sel)
    agree = check_selection(sel, r)
    ok = np.repeat(agree, 128, axis=-1)
    assert_close(bf16_values(o.permute(0, 2, 1, 3))[ok], r["o_fine"][ok], "vsa fine, 3 cubes")
    assert_close(bf16_values(o_tr.permute(0, 2, 1, 3))[ok], r["o_fine"][ok], "vsa fine training, 3 cubes")


def test_batch_of_two(m):
    grid = (4, 8, 16)  # 4 cubes, top-3
    q, k, v = synth.qkv_headscaled(2, 512, 3, 128, seed=96, scaled=False)
    o, oc, sel = run(m, q, k, v, grid, 0.4)
    r = oracle.vsa_fwd(bhld_bits(q), bhld_bits(k), bhld_bits(v), SCALE, sparsity=0.4, rows=np.arange(512))
    assert r["topk"] == 3 and sel.shape == (2, 3, 4, 3)
    agree = check_selection(sel, r)
    ok = np.repeat(agree, 128, axis=-1)
    assert_close(bf16_values(o.permute(0, 2, 1, 3))[ok], r["o_fine"][ok], "vsa fine B=2")


@pytest.mark.parametrize("sparsity,topk", [(0.7, 3), (0.9, 1), (0.5, 4)])
def test_list_lengths(m, sparsity, topk):
    # odd lists (the second wave group's last position is empty), a single cube, an even list
    grid = (4, 8, 32)  # 8 cubes
    q, k, v = synth.qkv_headscaled(1, 1024, 2, 128, seed=95 + topk, scaled=False)
    o, oc, sel = run(m, q, k, v, grid, sparsity)
    rows = np.arange(1, 1024, 5)
    r = oracle.vsa_fwd(bhld_bits(q), bhld_bits(k), bhld_bits(v), SCALE, sparsity=sparsity, rows=rows)
    assert r["topk"] == topk and sel.shape[-1] == topk
    agree = check_selection(sel, r)
    ok = agree[:, :, rows // 128]
    got = bf16_values(o.permute(0, 2, 1, 3)[:, :, torch.as_tensor(rows)])
    assert_close(got[ok], r["o_fine"][ok], f"vsa fine topk={topk}")


def test_wan_vsa_workload(m):
    q, k, v = synth.vsa_inputs()
    o, oc, sel = run(m, q, k, v, (16, 28, 56), 0.9)
    L = q.shape[1]
    rows = synth.sample_rows(L, 64, seed=9).numpy()
    r = oracle.vsa_fwd(bhld_bits(q), bhld_bits(k), bhld_bits(v), SCALE, sparsity=0.9, rows=rows)
    assert r["topk"] == 20 and sel.shape == (1, 12, 196, 20)
    agree = check_selection(sel, r)
    ok = agree[:, :, rows // 128]
    got = bf16_values(o.permute(0, 2, 1, 3)[:, :, torch.as_tensor(rows)])
    assert_close(got[ok], r["o_fine"][ok], "Wan VSA fine")
    gotc = bf16_values(oc.permute(0, 2, 1, 3)[:, :, torch.as_tensor(rows)])
    assert_close(gotc, r["o_coarse"], "Wan VSA coarse")


@pytest.mark.parametrize("where", ["q", "k"])
def test_nan_token_keeps_selection_valid(m, where):
    # A NaN in one token makes its cube's pooled mean, hence its coarse logits, NaN; those rank
    # below every number, so every list still holds topk distinct ascending cubes and no other
    # query's output is touched.
    grid, L, H = (4, 8, 32), 1024, 2
    q, k, v = synth.qkv_headscaled(1, L, H, 128, seed=94, scaled=False)
    tok = 3 * 128 + 17  # a token of cube 3
    (q if where == "q" else k)[0, tok, 1, 5] = float("nan")
    o, oc, sel = run(m, q, k, v, grid, 0.6)
    n, topk = 8, 4
    assert sel.shape == (1, H, n, topk)
    parity.assert_valid_selection(sel, n)
    on = o.float().cpu().numpy()
    if where == "q":
        # the NaN query cube's logits are all -inf after the mapping: ties to the lowest cubes
        assert np.array_equal(sel[0, 1, 3], np.arange(topk))
        # every other row is finite (the NaN token's own row is whatever the fake quantizer makes
        # of a NaN element: E2M1 has no NaN code)
        bad = np.zeros((L, H), bool)
        bad[tok, 1] = True
        assert np.all(np.isfinite(on[0][~bad]))
    else:
        # the NaN key cube ranks last for every query cube of that head and is never selected
        assert not np.any(sel[0, 1] == 3)
        assert np.all(np.isfinite(on))
