"""GPU parity of the fake-quant attention forward (attn_qat_fwd) against the
oracle, within the stated tolerance (tests/parity.py), on the tiny workload in
full, on ragged / cross / causal shapes that span several 128-key chunks and a
partial last chunk, and on sampled rows of the Wan2.1 448x896x61 workload
(B=1, H=12, L=25088, D=128) in the launch configuration the benchmark times."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import assert_close, bf16_values, bhld_bits

pytestmark = pytest.mark.gpu
LOG2E = 1.0 / math.log(2.0)


@pytest.fixture(scope="module")
def m():
    import quantization_aware_attention_nvfp4_amd as m
    return m


def run(m, q, k, v, causal=False, flags=15, training=False, scale=None):
    out = m.attn_qat_fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, sm_scale=scale, quant_flags=flags,
                         training=training)
    torch.cuda.synchronize()
    return out


def rand_qkv(B, Lq, Lk, H, seed, mult=1.0):
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn(B, Lq, H, 128, generator=g) * mult).to(torch.bfloat16)
    k = (torch.randn(B, Lk, H, 128, generator=g) * mult).to(torch.bfloat16)
    v = torch.randn(B, Lk, H, 128, generator=g).to(torch.bfloat16)
    return q, k, v


def ref_fwd(q, k, v, causal=False, flags=15, rows=None, scale=None):
    scale = 1.0 / math.sqrt(128) if scale is None else scale
    return oracle.attn_fwd(bhld_bits(q), bhld_bits(k), bhld_bits(v), scale, causal=causal, flags=flags,
                           rows=rows)


def gpu_rows(o_blhd, rows):
    # [B, L, H, D] -> [B, H, R, D]
    return bf16_values(o_blhd.permute(0, 2, 1, 3)[:, :, torch.as_tensor(rows)])


def test_tiny_workload_full(m):
    q, k, v = synth.tiny_forward()
    o = run(m, q, k, v)
    r = ref_fwd(q, k, v)
    assert_close(gpu_rows(o, r["rows"]), r["o"], "tiny fwd")


@pytest.mark.parametrize("flags", [0, 1 | 2, 4, 8, 15])
def test_quantizer_subsets(m, flags):
    q, k, v = rand_qkv(1, 200, 300, 2, seed=5, mult=1.5)
    o = run(m, q, k, v, flags=flags)
    r = ref_fwd(q, k, v, flags=flags)
    assert_close(gpu_rows(o, r["rows"]), r["o"], f"flags {flags}")


@pytest.mark.parametrize("Lq,Lk,causal", [(300, 300, False), (200, 333, False), (77, 1000, False),
                                          (300, 300, True), (129, 129, True), (1, 17, False),
                                          (520, 128, False), (513, 513, True)])
def test_ragged_cross_and_causal(m, Lq, Lk, causal):
    q, k, v = rand_qkv(2, Lq, Lk, 3, seed=Lq * 7 + Lk, mult=2.0)
    o = run(m, q, k, v, causal=causal)
    r = ref_fwd(q, k, v, causal=causal)
    assert_close(gpu_rows(o, r["rows"]), r["o"], f"Lq={Lq} Lk={Lk} causal={causal}")


def test_training_outputs(m):
    q, k, v = rand_qkv(1, 260, 390, 2, seed=21, mult=2.0)
    o, aux = run(m, q, k, v, training=True)
    r = ref_fwd(q, k, v)
    assert_close(gpu_rows(o, r["rows"]), r["o"], "o")
    ohp = aux["o_hp"].cpu().numpy().astype(np.float64)
    assert_close(ohp, r["o_hp"], "o_hp", round_ref=False)
    lse = aux["lse_log2"].cpu().numpy().astype(np.float64)
    assert np.allclose(lse, r["lse"] * LOG2E, rtol=1e-5, atol=1e-5)
    cmax = aux["chunk_max_log2"].cpu().numpy().astype(np.float64)  # [B, H, C, Lq]
    assert np.allclose(cmax, np.moveaxis(r["cmax"], -1, 2) * LOG2E, rtol=1e-5, atol=1e-5)
    # the inference path gives the same o bit for bit
    o2 = run(m, q, k, v)
    assert torch.equal(o.view(torch.int16).cpu(), o2.view(torch.int16).cpu())


def test_causal_training_statistics(m):
    q, k, v = rand_qkv(1, 300, 300, 1, seed=23)
    o, aux = run(m, q, k, v, causal=True, training=True)
    r = ref_fwd(q, k, v, causal=True)
    cmax = aux["chunk_max_log2"].cpu().numpy()[0, 0]  # [C, L]
    for i in (0, 5, 127, 128, 200, 299):
        for c in range(i // 128 + 1):
            assert abs(cmax[c, i] - r["cmax"][0, 0, i, c] * LOG2E) <= 1e-5 * max(1.0, abs(cmax[c, i]))


def test_layouts_and_determinism(m):
    q, k, v = rand_qkv(1, 256, 256, 4, seed=31)
    o1 = run(m, q, k, v)
    # the same data in [B, H, L, D] memory, passed as strided [B, L, H, D] views
    qh, kh, vh = (t.permute(0, 2, 1, 3).contiguous().cuda().permute(0, 2, 1, 3) for t in (q, k, v))
    o2 = m.attn_qat_fwd(qh, kh, vh)
    o3 = run(m, q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o1.cpu().view(torch.int16), o2.cpu().view(torch.int16))
    assert torch.equal(o1.cpu().view(torch.int16), o3.cpu().view(torch.int16))


def test_wan_448x896x61_sampled_rows(m):
    q, k, v = synth.wan_448x896x61()
    o = run(m, q, k, v)
    rows = synth.sample_rows(q.shape[1], 64, seed=3).numpy()
    r = ref_fwd(q, k, v, rows=rows)
    assert_close(gpu_rows(o, rows), r["o"], "Wan 448x896x61 forward")
