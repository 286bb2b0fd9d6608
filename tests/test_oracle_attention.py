"""Pins for the oracle's attention forward, straight-through backward and
cube-sparse forward (CPU only).

Each check ties the oracle to something other than itself:
  * with fake quantization off, the forward and backward equal textbook
    softmax attention computed by PyTorch in float64 (SDPA and autograd);
  * the straight-through dQ/dK with every quantizer on equal PyTorch float64
    autograd of plain attention on the fake-quantized operands (the
    "consistent STE with auxiliary output" of the dense precision record in
    "vsqa-preview-1.3b metadata.json");
  * the online recurrence equals the closed form it unrolls to (each chunk's
    quantized probabilities weighted by exp(m_c - m_final));
  * constant logits give P = 1 and P-hat = fq(1) = 1.03125 exactly;
  * O is linear in V, and <dO, O> = sum_j <dV_j, V-hat_j> ties dV to the forward;
  * cube-sparse attention at sparsity 0 equals dense attention with 128-key
    chunks; the top-k count follows its printed formula; the selection equals
    torch.topk on the coarse scores; the coarse output equals torch softmax;
  * the cube-sparse backward equals the dense backward at sparsity 0, PyTorch
    float64 autograd of block-masked attention without quantization (and for
    dQ/dK on the fake-quantized operands), and pairs dV with the fine output.
"""
import math

import numpy as np
import pytest
import torch

import oracle

D = 128
SCALE = 1.0 / math.sqrt(D)


def rand_bits(shape, seed, mult=1.0):
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn(*shape, generator=g) * mult).to(torch.bfloat16)
    return x.view(torch.int16).numpy().view(np.uint16)


def f64(u16):
    return torch.from_numpy(oracle.bf16_bits_to_f32(u16).astype(np.float64))


def fq_bits(u16, axis):
    return oracle.fq_bf16(u16, axis=axis)


def sdpa64(q, k, v, scale, causal=False):
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale, is_causal=causal)


@pytest.mark.parametrize("Lq,Lk,causal", [(100, 100, False), (70, 300, False), (200, 200, True)])
def test_forward_without_quantization_is_softmax_attention(Lq, Lk, causal):
    q, k, v = rand_bits((1, 2, Lq, D), 1), rand_bits((1, 2, Lk, D), 2), rand_bits((1, 2, Lk, D), 3)
    r = oracle.attn_fwd(q, k, v, SCALE, causal=causal, flags=0)
    ref = sdpa64(f64(q), f64(k), f64(v), SCALE, causal)
    # the oracle rounds logits and probabilities to fp32 before use
    assert np.allclose(r["o"], ref.numpy(), rtol=0, atol=2e-6)
    assert np.allclose(r["o_hp"], r["o"], rtol=0, atol=1e-12)
    s = torch.einsum("bhid,bhjd->bhij", f64(q), f64(k)) * SCALE
    if causal:
        s = s.masked_fill(torch.ones(Lq, Lk, dtype=torch.bool).triu(1), -math.inf)
    assert np.allclose(r["lse"], torch.logsumexp(s, -1).numpy(), atol=1e-5)


def test_chunk_max_is_running_prefix_max():
    q, k, v = rand_bits((1, 1, 40, D), 4), rand_bits((1, 1, 300, D), 5), rand_bits((1, 1, 300, D), 6)
    r = oracle.attn_fwd(q, k, v, SCALE, flags=oracle.QUANT_ALL)
    s = (torch.einsum("id,jd->ij", f64(fq_bits(q, -1))[0, 0], f64(fq_bits(k, -1))[0, 0]) * SCALE).float().double()
    for c in range(3):
        pref = s[:, : min(300, 128 * (c + 1))].max(-1).values
        assert np.array_equal(r["cmax"][0, 0, :, c], pref.numpy())


def test_online_recurrence_equals_unrolled_closed_form():
    Lq, Lk = 24, 300
    q, k, v = rand_bits((1, 1, Lq, D), 7), rand_bits((1, 1, Lk, D), 8, 2.0), rand_bits((1, 1, Lk, D), 9)
    r = oracle.attn_fwd(q, k, v, SCALE, flags=oracle.QUANT_ALL)
    qh = oracle.bf16_bits_to_f32(fq_bits(q, -1))[0, 0].astype(np.float64)
    kh = oracle.bf16_bits_to_f32(fq_bits(k, -1))[0, 0].astype(np.float64)
    vh = oracle.bf16_bits_to_f32(fq_bits(v, 2))[0, 0].astype(np.float64)
    S = (SCALE * (qh @ kh.T)).astype(np.float32)
    out = np.zeros((Lq, D))
    for i in range(Lq):
        C = 3
        mc = [S[i, : min(Lk, 128 * (c + 1))].max() for c in range(C)]
        mfin = mc[-1]
        lsum = 0.0
        acc = np.zeros(D)
        for c in range(C):
            seg = S[i, 128 * c: min(Lk, 128 * (c + 1))]
            # fp32 probabilities relative to the chunk's running max (libm exp,
            # as the oracle uses; numpy's vectorised exp differs in the last bit)
            P = np.array([math.exp(float(t) - float(mc[c])) for t in seg]).astype(np.float32)
            Pp = np.zeros(128, np.float32)
            Pp[: len(P)] = P
            Pq = oracle.fq_f32_rows(Pp[None])[0][: len(P)]
            w = math.exp(float(mc[c]) - float(mfin))
            lsum += w * P.astype(np.float64).sum()
            acc += w * (Pq.astype(np.float64) @ vh[128 * c: 128 * c + len(P)])
        out[i] = acc / lsum
    assert np.allclose(r["o"][0, 0], out, rtol=1e-9, atol=1e-12)


def test_constant_logits_closed_form():
    # K rows all equal -> every logit of a row is the same -> P = 1 -> P-hat =
    # 1.03125 (see the codec closed forms) and O = 1.03125 * mean(V-hat).
    Lk = 200
    q = rand_bits((1, 1, 8, D), 10)
    k = np.tile(rand_bits((1, 1, 1, D), 11), (1, 1, Lk, 1))
    v = rand_bits((1, 1, Lk, D), 12)
    r = oracle.attn_fwd(q, k, v, SCALE, flags=oracle.QUANT_ALL)
    vh = oracle.bf16_bits_to_f32(fq_bits(v, 2))[0, 0].astype(np.float64)
    assert np.allclose(r["o"][0, 0], 1.03125 * vh.mean(0)[None, :], rtol=1e-12, atol=1e-14)
    assert np.allclose(r["o_hp"][0, 0], vh.mean(0)[None, :], rtol=1e-12, atol=1e-14)


def test_single_chunk_equals_final_max_reading():
    q, k, v = rand_bits((1, 1, 16, D), 13), rand_bits((1, 1, 128, D), 14), rand_bits((1, 1, 128, D), 15)
    a = oracle.attn_fwd(q, k, v, SCALE, chunk=128)
    b = oracle.attn_fwd(q, k, v, SCALE, chunk=4096)
    assert np.array_equal(a["o"], b["o"])


def test_output_is_linear_in_v_when_v_is_not_quantized():
    q, k = rand_bits((1, 1, 20, D), 16), rand_bits((1, 1, 260, D), 17)
    g = torch.Generator().manual_seed(18)
    v1 = torch.randint(-8, 8, (1, 1, 260, D), generator=g).to(torch.bfloat16)
    v2 = torch.randint(-8, 8, (1, 1, 260, D), generator=g).to(torch.bfloat16)
    tb = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    fl = oracle.QUANT_Q | oracle.QUANT_K | oracle.QUANT_P
    o1 = oracle.attn_fwd(q, k, tb(v1), SCALE, flags=fl)["o"]
    o2 = oracle.attn_fwd(q, k, tb(v2), SCALE, flags=fl)["o"]
    o12 = oracle.attn_fwd(q, k, tb(v1 + v2), SCALE, flags=fl)["o"]
    assert np.allclose(o12, o1 + o2, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_without_quantization_is_autograd(causal):
    L = 150
    q, k, v, do = (rand_bits((1, 2, L, D), s) for s in (20, 21, 22, 23))
    r = oracle.attn_bwd(q, k, v, do, SCALE, causal=causal, flags=0)
    Q, K, V = (f64(t).requires_grad_() for t in (q, k, v))
    out = sdpa64(Q, K, V, SCALE, causal)
    out.backward(f64(do))
    for name, t in (("dq", Q), ("dk", K), ("dv", V)):
        assert np.allclose(r[name], t.grad.numpy(), rtol=0, atol=5e-6), name


def test_ste_dq_dk_equal_autograd_on_quantized_operands():
    # With every quantizer on, dS uses the unquantized probabilities and
    # D = <dO, O_hp>, so dQ and dK are exactly the gradients of plain attention
    # on (Q-hat, K-hat, V-hat).
    Lq, Lk = 90, 270
    q, do = rand_bits((1, 2, Lq, D), 24), rand_bits((1, 2, Lq, D), 27)
    k, v = rand_bits((1, 2, Lk, D), 25), rand_bits((1, 2, Lk, D), 26)
    r = oracle.attn_bwd(q, k, v, do, SCALE, flags=oracle.QUANT_ALL)
    Q = f64(fq_bits(q, -1)).requires_grad_()
    K = f64(fq_bits(k, -1)).requires_grad_()
    V = f64(fq_bits(v, 2))
    sdpa64(Q, K, V, SCALE).backward(f64(do))
    assert np.allclose(r["dq"], Q.grad.numpy(), rtol=0, atol=5e-6)
    assert np.allclose(r["dk"], K.grad.numpy(), rtol=0, atol=5e-6)


def test_dv_pairs_with_the_forward_output():
    # O = A-hat V-hat (linear in V-hat), dV = A-hat^T dO, so
    # sum_i <dO_i, O_i> = sum_j <dV_j, V-hat_j> per head.
    Lq, Lk = 64, 300
    q, do = rand_bits((1, 2, Lq, D), 28), rand_bits((1, 2, Lq, D), 31)
    k, v = rand_bits((1, 2, Lk, D), 29, 2.0), rand_bits((1, 2, Lk, D), 30)
    f = oracle.attn_fwd(q, k, v, SCALE, flags=oracle.QUANT_ALL)
    b = oracle.attn_bwd(q, k, v, do, SCALE, flags=oracle.QUANT_ALL)
    vh = oracle.bf16_bits_to_f32(fq_bits(v, 2)).astype(np.float64)
    lhs = np.einsum("bhid,bhid->bh", oracle.bf16_bits_to_f32(do).astype(np.float64), f["o"])
    rhs = np.einsum("bhjd,bhjd->bh", b["dv"], vh)
    assert np.allclose(lhs, rhs, rtol=1e-10)


def test_ds_rows_sum_to_zero():
    # Identical K rows: sum_j dS_ij = 0 makes dQ vanish.
    L = 140
    q, v, do = rand_bits((1, 1, L, D), 32), rand_bits((1, 1, L, D), 33), rand_bits((1, 1, L, D), 34)
    k = np.tile(rand_bits((1, 1, 1, D), 35), (1, 1, L, 1))
    r = oracle.attn_bwd(q, k, v, do, SCALE, flags=oracle.QUANT_ALL)
    assert np.abs(r["dq"]).max() < 1e-12


def test_sampled_rows_match_full_rows():
    Lq, Lk = 80, 200
    q, do = rand_bits((1, 1, Lq, D), 36), rand_bits((1, 1, Lq, D), 39)
    k, v = rand_bits((1, 1, Lk, D), 37), rand_bits((1, 1, Lk, D), 38)
    full = oracle.attn_bwd(q, k, v, do, SCALE)
    qr, kr = np.array([0, 17, 79]), np.array([3, 127, 128, 199])
    part = oracle.attn_bwd(q, k, v, do, SCALE, qrows=qr, krows=kr)
    only_q = oracle.attn_bwd(q, k, v, do, SCALE, qrows=qr, krows=np.zeros(0, np.int64))
    assert np.array_equal(part["dq"], full["dq"][:, :, qr])
    assert np.array_equal(only_q["dq"], full["dq"][:, :, qr])
    assert np.array_equal(part["dk"], full["dk"][:, :, kr])
    assert np.array_equal(part["dv"], full["dv"][:, :, kr])
    fr = oracle.attn_fwd(q, k, v, SCALE, rows=qr)
    ff = oracle.attn_fwd(q, k, v, SCALE)
    assert np.array_equal(fr["o"], ff["o"][:, :, qr])


def test_vsa_topk_formula():
    # "vsqa-preview-1.3b metadata.json", attention.selection.effective_topk
    assert oracle.vsa_topk(0.9, 196) == 20
    assert oracle.vsa_topk(0.0, 196) == 196
    assert oracle.vsa_topk(1.0, 196) == 1
    assert oracle.vsa_topk(0.5, 7) == 4


def test_vsa_sparsity_zero_is_dense():
    L, cube = 512, 128
    q, k, v = (rand_bits((1, 2, L, D), s) for s in (40, 41, 42))
    rows = np.array([0, 1, 130, 257, 511])
    sp = oracle.vsa_fwd(q, k, v, SCALE, cube_tokens=cube, sparsity=0.0, rows=rows)
    de = oracle.attn_fwd(q, k, v, SCALE, rows=rows)
    assert sp["topk"] == 4
    assert np.array_equal(sp["o_fine"], de["o"])


def test_vsa_selection_pool_and_coarse_against_torch():
    L, cube = 1024, 128
    q, k, v = (rand_bits((1, 2, L, D), s) for s in (43, 44, 45))
    rows = np.arange(0, L, 37)
    r = oracle.vsa_fwd(q, k, v, SCALE, cube_tokens=cube, sparsity=0.6, rows=rows)
    n, topk = L // cube, r["topk"]
    assert topk == math.ceil(0.4 * n)
    Q, K, V = (f64(t).view(1, 2, n, cube, D) for t in (q, k, v))
    pooled = [t.mean(3).to(torch.bfloat16) for t in (Q, K, V)]
    for name, p in zip(("qpool", "kpool", "vpool"), pooled):
        assert np.array_equal(r[name], p.view(torch.int16).numpy().view(np.uint16)), name
    qc, kc, vc = (p.double() for p in pooled)
    score = torch.einsum("bhad,bhcd->bhac", qc, kc) * SCALE
    assert np.allclose(r["score"], score.numpy(), rtol=1e-13, atol=1e-15)
    sel_ref = torch.topk(score, topk, dim=-1).indices.sort(-1).values
    assert np.array_equal(r["sel"], sel_ref.numpy())
    oc = torch.softmax(score, -1) @ vc  # [1, 2, n, D]
    assert np.allclose(r["o_coarse"], oc[:, :, rows // cube].numpy(), rtol=1e-12, atol=1e-14)
    # the fine output of each row equals dense attention over the selected
    # cubes' keys in ascending order with one chunk per cube
    for bh in range(2):
        for t, i in enumerate(rows[:6]):
            a = i // cube
            keys = np.concatenate([np.arange(c * cube, (c + 1) * cube) for c in r["sel"][0, bh, a]])
            sub = oracle.attn_fwd(q[:, bh:bh + 1], k[:, bh:bh + 1][:, :, keys], v[:, bh:bh + 1][:, :, keys],
                                  SCALE, rows=np.array([i]))
            # V-hat blocks of 16 keys stay inside a cube, so gathering cubes
            # before quantizing V changes nothing
            assert np.array_equal(r["o_fine"][0, bh, t], sub["o"][0, 0, 0])


# ---- cube-sparse backward ----------------------------------------------------

def block_mask(sel, L, cube):
    """Boolean [B, H, L, L] mask: query i may see key j when j's cube is among
    the cubes selected for i's cube."""
    B, H, n, _ = sel.shape
    m = torch.zeros(B, H, n, n, dtype=torch.bool)
    for b in range(B):
        for h in range(H):
            for a in range(n):
                m[b, h, a, torch.as_tensor(sel[b, h, a], dtype=torch.long)] = True
    return m.repeat_interleave(cube, 2).repeat_interleave(cube, 3)


def test_vsa_bwd_sparsity_zero_is_dense_bwd():
    L, cube = 512, 128
    q, k, v, do = (rand_bits((1, 2, L, D), s) for s in (50, 51, 52, 53))
    sp = oracle.vsa_bwd(q, k, v, do, SCALE, cube_tokens=cube, sparsity=0.0)
    de = oracle.attn_bwd(q, k, v, do, SCALE)
    assert sp["topk"] == 4
    for name in ("dq", "dk", "dv"):
        assert np.array_equal(sp[name], de[name]), name


def test_vsa_bwd_without_quantization_is_masked_autograd():
    L, cube = 1024, 128
    q, k, v, do = (rand_bits((1, 2, L, D), s) for s in (54, 55, 56, 57))
    r = oracle.vsa_bwd(q, k, v, do, SCALE, cube_tokens=cube, sparsity=0.6, flags=0)
    assert r["topk"] == 4
    # the selection is the forward's
    assert np.array_equal(r["sel"], oracle.vsa_fwd(q, k, v, SCALE, cube_tokens=cube, sparsity=0.6,
                                                   rows=np.array([0]))["sel"])
    mask = block_mask(r["sel"], L, cube)
    Q, K, V = (f64(t).requires_grad_() for t in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=SCALE)
    out.backward(f64(do))
    for name, t in (("dq", Q), ("dk", K), ("dv", V)):
        assert np.allclose(r[name], t.grad.numpy(), rtol=0, atol=5e-6), name


def test_vsa_bwd_ste_dq_dk_equal_masked_autograd_on_quantized_operands():
    L, cube = 1024, 128
    q, k, v, do = (rand_bits((1, 1, L, D), s) for s in (58, 59, 60, 61))
    r = oracle.vsa_bwd(q, k, v, do, SCALE, cube_tokens=cube, sparsity=0.6)
    mask = block_mask(r["sel"], L, cube)
    Q = f64(fq_bits(q, -1)).requires_grad_()
    K = f64(fq_bits(k, -1)).requires_grad_()
    V = f64(fq_bits(v, 2))
    torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=SCALE).backward(f64(do))
    assert np.allclose(r["dq"], Q.grad.numpy(), rtol=0, atol=5e-6)
    assert np.allclose(r["dk"], K.grad.numpy(), rtol=0, atol=5e-6)


def test_vsa_bwd_dv_pairs_with_the_fine_output_and_rows_sample():
    L, cube = 1024, 128
    q, k, v, do = (rand_bits((1, 2, L, D), s) for s in (62, 63, 64, 65))
    f = oracle.vsa_fwd(q, k, v, SCALE, cube_tokens=cube, sparsity=0.6)
    b = oracle.vsa_bwd(q, k, v, do, SCALE, cube_tokens=cube, sparsity=0.6)
    vh = oracle.bf16_bits_to_f32(fq_bits(v, 2)).astype(np.float64)
    lhs = np.einsum("bhid,bhid->bh", oracle.bf16_bits_to_f32(do).astype(np.float64), f["o_fine"])
    rhs = np.einsum("bhjd,bhjd->bh", b["dv"], vh)
    assert np.allclose(lhs, rhs, rtol=1e-10)
    qr, kr = np.array([0, 300, 1023]), np.array([5, 127, 128, 640])
    part = oracle.vsa_bwd(q, k, v, do, SCALE, cube_tokens=cube, sparsity=0.6, qrows=qr, krows=kr)
    for name, rows in (("dq", qr), ("dk", kr), ("dv", kr)):
        assert np.array_equal(part[name], b[name][:, :, rows]), name
