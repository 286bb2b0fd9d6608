"""GPU parity of the straight-through backward (attn_qat_bwd) against the oracle,
within the stated tolerance (tests/parity.py): full gradients on shapes that span
several 128-key chunks with ragged tails, cross attention and causal masking; on
the Wan2.1 480x832x81 workload (B=1, H=12, L=32760, D=128, L = 8 mod 16, so the
last V/P block is partial) sampled dQ rows of every head and sampled dK/dV key rows
of one head (chunk edges and the whole last partial block included), plus
properties that hold at any size for dK and dV there; on the 448x896x61 workload
(L=25088) the training forward's outputs (o, lse, chunk maxima, o_hp) at sampled
rows and sampled dQ/dK/dV rows, all in the benchmark's launch configuration, on a head
whose work units run whole and on one whose units are split into pieces (the last
round of workgroups).  The small non-causal shapes run every unit as pieces (fewer
units than CUs), the 480x832x81 workload none (its unit counts fill whole rounds)."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import assert_close, bf16_values, bhld_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import quantization_aware_attention_nvfp4_amd as m
    return m


def rand(B, L, H, seed, mult=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(B, L, H, 128, generator=g) * mult).to(torch.bfloat16)


def gpu_grads(m, q, k, v, do, causal=False, flags=15):
    qg, kg, vg, dog = (t.cuda() for t in (q, k, v, do))
    o, aux = m.attn_qat_fwd(qg, kg, vg, causal=causal, quant_flags=flags, training=True)
    dq, dk, dv = m.attn_qat_bwd(qg, kg, vg, aux, dog, causal=causal, quant_flags=flags)
    torch.cuda.synchronize()
    return o, dq, dk, dv


def bhrd(x_blhd, rows=None):
    x = x_blhd.permute(0, 2, 1, 3)
    if rows is not None:
        x = x[:, :, torch.as_tensor(rows)]
    return bf16_values(x)


def ref_bwd(q, k, v, do, causal=False, flags=15, qrows=None, krows=None):
    return oracle.attn_bwd(bhld_bits(q), bhld_bits(k), bhld_bits(v), bhld_bits(do), 1.0 / math.sqrt(128),
                           causal=causal, flags=flags, qrows=qrows, krows=krows)


@pytest.mark.parametrize("Lq,Lk,causal,flags", [(256, 256, False, 15), (300, 300, False, 15), (200, 333, False, 15),
                                                (300, 300, True, 15), (190, 260, False, 0), (130, 130, True, 0),
                                                # one 64-query tile per key chunk; a last tile of one row
                                                (40, 300, False, 15), (65, 200, False, 15), (65, 65, True, 15)])
def test_full_gradients(m, Lq, Lk, causal, flags):
    B, H = 1, 2
    q, do = rand(B, Lq, H, 100 + Lq, 1.5), rand(B, Lq, H, 300 + Lq)
    k, v = rand(B, Lk, H, 200 + Lk, 1.5), rand(B, Lk, H, 400 + Lk)
    o, dq, dk, dv = gpu_grads(m, q, k, v, do, causal=causal, flags=flags)
    r = ref_bwd(q, k, v, do, causal=causal, flags=flags)
    assert_close(bhrd(dq), r["dq"], "dq")
    assert_close(bhrd(dk), r["dk"], "dk")
    assert_close(bhrd(dv), r["dv"], "dv")


def test_tiny_workload(m):
    q, k, v = synth.tiny_forward()
    do = rand(1, 256, 2, 77)
    o, dq, dk, dv = gpu_grads(m, q, k, v, do)
    r = ref_bwd(q, k, v, do)
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert_close(bhrd(g), r[name], name)


def test_medium_length_sampled_keys(m):
    # L = 2056 (= 8 mod 16): full oracle statistics per head, sampled key rows incl. chunk edges
    # and the partial last block.
    L, H = 2056, 2
    q, k, v, do = (rand(1, L, H, s, 1.5 if s < 3 else 1.0) for s in range(4))
    o, dq, dk, dv = gpu_grads(m, q, k, v, do)
    krows = np.array([0, 1, 127, 128, 129, 1023, 1024, 2047, 2048, 2050, 2055])
    qrows = np.array([0, 5, 127, 128, 1000, 2048, 2055])
    r = ref_bwd(q, k, v, do, qrows=qrows, krows=krows)
    assert_close(bhrd(dq, qrows), r["dq"], "dq")
    assert_close(bhrd(dk, krows), r["dk"], "dk")
    assert_close(bhrd(dv, krows), r["dv"], "dv")


def test_deterministic(m):
    q, k, v, do = (rand(1, 300, 2, 50 + s) for s in range(4))
    a = gpu_grads(m, q, k, v, do)
    b = gpu_grads(m, q, k, v, do)
    for x, y in zip(a, b):
        assert torch.equal(x.cpu().view(torch.int16), y.cpu().view(torch.int16))


def test_autograd_function(m):
    q, k, v, do = (rand(1, 200, 2, 60 + s) for s in range(4))
    qg, kg, vg = (t.cuda().requires_grad_() for t in (q, k, v))
    o = m.attn_qat_train(qg, kg, vg)
    o.backward(do.cuda())
    _, dq, dk, dv = gpu_grads(m, q, k, v, do)
    assert torch.equal(qg.grad.view(torch.int16).cpu(), dq.view(torch.int16).cpu())
    assert torch.equal(vg.grad.view(torch.int16).cpu(), dv.view(torch.int16).cpu())


def key_rows(L, n=64, seed=13):
    """Sampled key rows: the first keys, both sides of the first chunk edge, the last full chunk's
    edge, every key of the last 16-key block (partial when L is not a multiple of 16), then
    seeded random keys up to n."""
    last_chunk = (L - 1) // 128 * 128
    fixed = {0, 1, 127, 128, last_chunk - 1, last_chunk, *range((L - 1) // 16 * 16, L)}
    rng = np.random.default_rng(seed)
    rest = [int(x) for x in rng.permutation(L) if int(x) not in fixed][: n - len(fixed)]
    return np.array(sorted(fixed | set(rest)), np.int64)


def one_head_bwd(q, k, v, do, h, qrows, krows):
    sl = slice(h, h + 1)
    return ref_bwd(q[:, :, sl], k[:, :, sl], v[:, :, sl], do[:, :, sl], qrows=qrows, krows=krows)


def test_wan_480x832x81_fwd_bwd(m):
    q, k, v, do = synth.wan_480x832x81()
    L = q.shape[1]
    o, dq, dk, dv = gpu_grads(m, q, k, v, do)
    qrows = synth.sample_rows(L, 32, seed=5).numpy()
    r = ref_bwd(q, k, v, do, qrows=qrows, krows=np.zeros(0, np.int64))
    assert_close(bhrd(dq, qrows), r["dq"], "Wan 480x832x81 dq")
    # dK and dV element by element at 64 key rows of one head (the oracle needs every row's
    # statistics for a key gradient, so one head): keys 0, 1, 127, 128, 32639, 32640 and the
    # partial last block 32752..32759 among them.
    h = 4
    krows = key_rows(L)
    assert {0, 1, 127, 128, 32639, 32640, *range(32752, 32760)} <= set(krows.tolist()) and krows.size == 64
    rk = one_head_bwd(q, k, v, do, h, np.zeros(0, np.int64), krows)
    assert_close(bhrd(dk[:, :, h:h + 1], krows), rk["dk"], "Wan 480x832x81 dk rows")
    assert_close(bhrd(dv[:, :, h:h + 1], krows), rk["dv"], "Wan 480x832x81 dv rows")
    # dK and dV at full size, through identities that hold at any size (non-causal):
    #   sum_j dK_j = scale * sum_i (sum_j dS_ij) Q-hat_i = 0, since every row of dS sums to 0;
    #   sum_j <dV_j, V-hat_j> = sum_i <dO_i, O_i>, since O = A-hat V-hat and dV = A-hat^T dO.
    vh = oracle.bf16_bits_to_f32(oracle.fq_bf16(bhld_bits(v), axis=2)).astype(np.float64)
    dkv, dvv = bhrd(dk), bhrd(dv)
    lhs = np.einsum("bhjd,bhjd->bh", dvv, vh)
    terms = np.einsum("bhid,bhid->bhi", bhrd(do), bhrd(o))
    rhs = terms.sum(-1)
    # the sums cancel heavily, so compare against the size of their terms
    assert np.all(np.abs(lhs - rhs) <= 2e-3 * np.abs(terms).sum(-1)), (lhs, rhs)
    colsum = np.abs(dkv.sum(axis=2)).max()
    assert colsum <= 2e-3 * np.abs(dkv).sum(axis=2).max(), colsum


LOG2E = 1.0 / math.log(2.0)


def test_wan_448x896x61_training(m):
    # The benchmark's timed path at its own size: training forward (o, lse, chunk maxima, o_hp)
    # and the backward, compared with the oracle at sampled rows.
    q, k, v = synth.wan_448x896x61()
    L = q.shape[1]
    do = synth.normal_bf16(q.shape, 2003)
    qg, kg, vg, dog = (t.cuda() for t in (q, k, v, do))
    o, aux = m.attn_qat_fwd(qg, kg, vg, training=True)
    dq, dk, dv = m.attn_qat_bwd(qg, kg, vg, aux, dog)
    torch.cuda.synchronize()
    rows = synth.sample_rows(L, 64, seed=21).numpy()
    # On 256 CUs the last, partly filled round of backward work units is split into pieces: heads 1
    # and 2 have their dQ and dK/dV units run whole; head 11's dQ units and its dK/dV units of key
    # chunks 148-195 are pieces.
    heads = [1, 2, 11]
    hs = torch.as_tensor(heads)
    rf = oracle.attn_fwd(bhld_bits(q[:, :, hs]), bhld_bits(k[:, :, hs]), bhld_bits(v[:, :, hs]),
                         1.0 / math.sqrt(128), rows=rows)
    ri = torch.as_tensor(rows)
    assert_close(bhrd(o[:, :, hs], rows), rf["o"], "448x896x61 training o")
    assert_close(aux["o_hp"][:, hs][:, :, ri].cpu().numpy(), rf["o_hp"], "448x896x61 o_hp")
    lse = aux["lse_log2"][:, hs][:, :, ri].cpu().numpy().astype(np.float64) / LOG2E
    assert np.abs(lse - rf["lse"]).max() <= 1e-5 * max(1.0, np.abs(rf["lse"]).max())
    cm = aux["chunk_max_log2"][:, hs][:, :, :, ri].cpu().numpy().astype(np.float64) / LOG2E  # [1, heads, C, R]
    ref_cm = np.moveaxis(rf["cmax"], -1, 2)
    assert cm.shape == ref_cm.shape == (1, len(heads), 196, rows.size)
    assert np.abs(cm - ref_cm).max() <= 1e-5 * max(1.0, np.abs(ref_cm).max())
    # gradients: dQ rows of these heads, dK/dV key rows of one
    rb = oracle.attn_bwd(bhld_bits(q[:, :, hs]), bhld_bits(k[:, :, hs]), bhld_bits(v[:, :, hs]),
                         bhld_bits(do[:, :, hs]), 1.0 / math.sqrt(128), qrows=rows, krows=np.zeros(0, np.int64))
    assert_close(bhrd(dq[:, :, hs], rows), rb["dq"], "448x896x61 dq rows")
    h = 11
    krows = np.union1d(key_rows(L, seed=22), [148 * 128 - 1, 148 * 128])  # the last whole / first split unit
    rk = one_head_bwd(q, k, v, do, h, np.zeros(0, np.int64), krows)
    assert_close(bhrd(dk[:, :, h:h + 1], krows), rk["dk"], "448x896x61 dk rows")
    assert_close(bhrd(dv[:, :, h:h + 1], krows), rk["dv"], "448x896x61 dv rows")
