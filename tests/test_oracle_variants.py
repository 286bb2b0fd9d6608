"""Pins for the oracle's attention variants (CPU only).

The variants are the flags the "attn_qat_train" API page lists and the
"vsqa-preview-1.3b metadata.json" precision records carry (use_global_sf_qkv,
use_global_sf_p, smooth_k), plus the reference-order softmax statistics the
"Attn-QAT Training" guide's environment table names.  Each check ties the
variant to something other than the oracle's own variant code:
  * final max: the output equals the closed form over the whole row (one
    maximum, 16-key blocks from key 0, the pinned fp32 codec); lse equals the
    default reading's; the recorded maximum is the row maximum; dQ/dK equal
    float64 autograd on the quantized operands; dV pairs with the output; at
    sparsity 0 the cube-sparse variant equals the dense one;
  * static Q/K/V scales: attention equals the default attention on operands
    quantized beforehand by the pinned standalone fake quantization with the
    pinned static scale of each tensor;
  * static P scale: the output equals the unrolled closed form with P's blocks
    quantized by the pinned codec under g = 448*6;
  * smooth-K: without quantization the output is softmax attention on the
    smoothed keys, which matches attention on the original keys up to the
    keys' bf16 rounding (the softmax ignores a per-row shift); with
    quantization it equals attention on keys smoothed and quantized by the
    pinned fp32 codec;
  * FP8 P.V product: with every logit of a row equal, P-hat = 1.03125 rounds
    to 1.0 and the output is the key mean of the E4M3-rounded V-hat (torch's
    float8_e4m3fn cast); operands already exact in E4M3 leave the BF16
    path's output unchanged bit for bit; random inputs match the unrolled
    closed form with both operands rounded by that cast; dQ/dK equal float64
    autograd on (Q-hat, K-hat, E4M3(V-hat)) and dV pairs with the output.
"""
import math

import numpy as np
import pytest
import torch

import oracle

D = 128
SCALE = 1.0 / math.sqrt(D)
ALL = oracle.QUANT_ALL


def rand_bits(shape, seed, mult=1.0, shift=0.0):
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn(*shape, generator=g) * mult + shift).to(torch.bfloat16)
    return x.view(torch.int16).numpy().view(np.uint16)


def f32(u16):
    return oracle.bf16_bits_to_f32(u16)


def f64(u16):
    return torch.from_numpy(f32(u16).astype(np.float64))


def bits_of(x32):
    return oracle.f32_to_bf16_bits(np.asarray(x32, np.float32))


def sdpa64(q, k, v, scale, causal=False):
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale, is_causal=causal)


def closed_form(S, vh, gp=1.0, chunk=None, pq_map=None):
    """Per row: the unrolled online recurrence over `chunk`-key chunks (one
    chunk = the whole row when None), fp32 probabilities relative to each
    chunk's running max (libm exp), P-hat from the pinned codec under global
    scale gp rounded to bf16 (then passed through pq_map when given), the
    denominator summing unquantized P."""
    Lq, Lk = S.shape
    chunk = chunk or (Lk + 15) // 16 * 16
    C = (Lk + chunk - 1) // chunk
    out = np.zeros((Lq, vh.shape[1]))
    for i in range(Lq):
        mc = [S[i, : min(Lk, chunk * (c + 1))].max() for c in range(C)]
        lsum, acc = 0.0, np.zeros(vh.shape[1])
        for c in range(C):
            seg = S[i, chunk * c: min(Lk, chunk * (c + 1))]
            P = np.array([math.exp(float(t) - float(mc[c])) for t in seg]).astype(np.float32)
            Pp = np.zeros((len(P) + 15) // 16 * 16, np.float32)
            Pp[: len(P)] = P
            Pq = f32(bits_of(oracle.fq_f32_rows(Pp[None], g=gp)[0][: len(P)]))
            if pq_map is not None:
                Pq = pq_map(Pq)
            w = math.exp(float(mc[c]) - float(mc[-1]))
            lsum += w * P.astype(np.float64).sum()
            acc += w * (Pq.astype(np.float64) @ vh[chunk * c: chunk * c + len(P)])
        out[i] = acc / lsum
    return out


def quantized_ops(q, k, v):
    qh = f32(oracle.fq_bf16(q, -1))[0, 0].astype(np.float64)
    kh = f32(oracle.fq_bf16(k, -1))[0, 0].astype(np.float64)
    vh = f32(oracle.fq_bf16(v, 2))[0, 0].astype(np.float64)
    return qh, kh, vh


# ---------------------------------------------------------------- final max

def test_final_max_equals_whole_row_closed_form():
    Lq, Lk = 20, 300
    q, k, v = rand_bits((1, 1, Lq, D), 101), rand_bits((1, 1, Lk, D), 102, 2.0), rand_bits((1, 1, Lk, D), 103)
    r = oracle.attn_fwd(q, k, v, SCALE, flags=ALL | oracle.FINAL_MAX)
    qh, kh, vh = quantized_ops(q, k, v)
    S = (SCALE * (qh @ kh.T)).astype(np.float32)
    assert np.allclose(r["o"][0, 0], closed_form(S, vh), rtol=1e-9, atol=1e-12)
    # one recorded maximum: the row maximum; lse does not depend on the reading
    # beyond the fp32 rounding of P relative to a different maximum
    assert r["cmax"].shape[-1] == 1
    assert np.array_equal(r["cmax"][0, 0, :, 0], S.max(-1).astype(np.float64))
    d = oracle.attn_fwd(q, k, v, SCALE, flags=ALL)
    assert np.allclose(r["lse"], d["lse"], rtol=0, atol=1e-6)
    # the readings differ (P is not scale-equivariant)
    assert not np.array_equal(r["o"], d["o"])


def test_final_max_backward_identities():
    Lq, Lk = 60, 270
    q, do = rand_bits((1, 2, Lq, D), 104), rand_bits((1, 2, Lq, D), 107)
    k, v = rand_bits((1, 2, Lk, D), 105, 2.0), rand_bits((1, 2, Lk, D), 106)
    fl = ALL | oracle.FINAL_MAX
    b = oracle.attn_bwd(q, k, v, do, SCALE, flags=fl)
    Q = f64(oracle.fq_bf16(q, -1)).requires_grad_()
    K = f64(oracle.fq_bf16(k, -1)).requires_grad_()
    sdpa64(Q, K, f64(oracle.fq_bf16(v, 2)), SCALE).backward(f64(do))
    assert np.allclose(b["dq"], Q.grad.numpy(), rtol=0, atol=5e-6)
    assert np.allclose(b["dk"], K.grad.numpy(), rtol=0, atol=5e-6)
    f = oracle.attn_fwd(q, k, v, SCALE, flags=fl)
    vh = f32(oracle.fq_bf16(v, 2)).astype(np.float64)
    lhs = np.einsum("bhid,bhid->bh", f32(do).astype(np.float64), f["o"])
    rhs = np.einsum("bhjd,bhjd->bh", b["dv"], vh)
    assert np.allclose(lhs, rhs, rtol=1e-10)


def test_final_max_causal_matches_closed_form():
    L = 150
    q, k, v = (rand_bits((1, 1, L, D), s) for s in (108, 109, 110))
    r = oracle.attn_fwd(q, k, v, SCALE, causal=True, flags=ALL | oracle.FINAL_MAX, rows=np.arange(0, L, 7))
    qh, kh, vh = quantized_ops(q, k, v)
    S = (SCALE * (qh @ kh.T)).astype(np.float32)
    for n, i in enumerate(range(0, L, 7)):
        want = closed_form(S[i: i + 1, : i + 1], vh[: i + 1])
        assert np.allclose(r["o"][0, 0, n], want[0], rtol=1e-9, atol=1e-12)


def test_vsa_final_max_sparsity_zero_is_dense_final_max():
    L = 512
    q, k, v = (rand_bits((1, 2, L, D), s) for s in (111, 112, 113))
    fl = ALL | oracle.FINAL_MAX
    s = oracle.vsa_fwd(q, k, v, SCALE, sparsity=0.0, flags=fl)
    d = oracle.attn_fwd(q, k, v, SCALE, flags=fl)
    assert np.array_equal(s["o_fine"], d["o"])
    do = rand_bits((1, 2, L, D), 114)
    sb = oracle.vsa_bwd(q, k, v, do, SCALE, sparsity=0.0, flags=fl)
    db = oracle.attn_bwd(q, k, v, do, SCALE, flags=fl)
    for name in ("dq", "dk", "dv"):
        assert np.allclose(sb[name], db[name], rtol=0, atol=1e-12), name


# ---------------------------------------------------------- static scales

@pytest.mark.parametrize("smooth", [False, True])
def test_static_qkv_scales_compose_the_standalone_fake_quant(smooth):
    Lq, Lk = 40, 200
    q = rand_bits((1, 2, Lq, D), 115, 3.0)
    k = rand_bits((1, 2, Lk, D), 116, 0.5, 0.7)
    v = rand_bits((1, 2, Lk, D), 117, 2.0)
    fl = ALL | oracle.GSF_QKV | (oracle.SMOOTH_K if smooth else 0)
    r = oracle.attn_fwd(q, k, v, SCALE, flags=fl)
    if smooth:
        ks = smoothed_f32(k)
        amax = np.abs(ks).max()
        gk = np.float32(np.float32(2688.0) / np.float32(max(amax, 1e-12)))
        kq = bits_of(oracle.fq_f32_rows(ks, g=float(gk)))
    else:
        kq = oracle.fq_bf16(k, -1, g=oracle.static_scale_bf16(k))
    qq = oracle.fq_bf16(q, -1, g=oracle.static_scale_bf16(q))
    vq = oracle.fq_bf16(v, 2, g=oracle.static_scale_bf16(v))
    ref = oracle.attn_fwd(qq, kq, vq, SCALE, flags=oracle.QUANT_P)
    assert np.array_equal(r["o"], ref["o"])
    assert np.array_equal(r["lse"], ref["lse"])
    b = oracle.attn_bwd(q, k, v, rand_bits((1, 2, Lq, D), 118), SCALE, flags=fl)
    bref = oracle.attn_bwd(qq, kq, vq, rand_bits((1, 2, Lq, D), 118), SCALE, flags=oracle.QUANT_P)
    for name in ("dq", "dk", "dv"):
        assert np.array_equal(b[name], bref[name]), name


def test_static_p_scale_equals_closed_form():
    Lq, Lk = 16, 300
    q, k, v = rand_bits((1, 1, Lq, D), 119), rand_bits((1, 1, Lk, D), 120, 2.0), rand_bits((1, 1, Lk, D), 121)
    r = oracle.attn_fwd(q, k, v, SCALE, flags=ALL | oracle.GSF_P)
    qh, kh, vh = quantized_ops(q, k, v)
    S = (SCALE * (qh @ kh.T)).astype(np.float32)
    assert np.allclose(r["o"][0, 0], closed_form(S, vh, gp=2688.0, chunk=128), rtol=1e-9, atol=1e-12)
    # the P scale changes the result (P-hat is not bf16-exact under it)
    assert not np.array_equal(r["o"], oracle.attn_fwd(q, k, v, SCALE, flags=ALL)["o"])


# ----------------------------------------------------------------- smooth K

def smoothed_f32(k_bits):
    """fp32(k - mean) with the mean per (b, h, channel): fp64 sum / L, rounded to fp32."""
    kf = f32(k_bits)
    mean = (kf.astype(np.float64).sum(axis=2, keepdims=True) / kf.shape[2]).astype(np.float32)
    return (kf - mean).astype(np.float32)


def test_smooth_k_without_quantization_is_softmax_on_smoothed_keys():
    Lq, Lk = 50, 230
    q = rand_bits((1, 2, Lq, D), 122)
    k = rand_bits((1, 2, Lk, D), 123, 1.0, 1.5)  # keys with a large common offset
    v = rand_bits((1, 2, Lk, D), 124)
    r = oracle.attn_fwd(q, k, v, SCALE, flags=oracle.SMOOTH_K)
    ks = torch.from_numpy(f32(bits_of(smoothed_f32(k))).astype(np.float64))
    want = sdpa64(f64(q), ks, f64(v), SCALE).numpy()
    assert np.allclose(r["o"], want, rtol=0, atol=1e-6)  # the oracle's S and P are fp32
    # the softmax ignores the per-row shift: close to attention on the original keys
    orig = sdpa64(f64(q), f64(k), f64(v), SCALE).numpy()
    assert np.abs(r["o"] - orig).max() < 2e-2 * np.abs(orig).max()


def test_smooth_k_with_quantization_composes_the_fp32_codec():
    Lq, Lk = 30, 200
    q = rand_bits((1, 1, Lq, D), 125)
    k = rand_bits((1, 1, Lk, D), 126, 1.0, -2.0)
    v = rand_bits((1, 1, Lk, D), 127)
    r = oracle.attn_fwd(q, k, v, SCALE, flags=ALL | oracle.SMOOTH_K)
    kq = bits_of(oracle.fq_f32_rows(smoothed_f32(k)))
    ref = oracle.attn_fwd(q, kq, v, SCALE, flags=ALL & ~oracle.QUANT_K)
    assert np.array_equal(r["o"], ref["o"])
    do = rand_bits((1, 1, Lq, D), 128)
    b = oracle.attn_bwd(q, k, v, do, SCALE, flags=ALL | oracle.SMOOTH_K)
    bref = oracle.attn_bwd(q, kq, v, do, SCALE, flags=ALL & ~oracle.QUANT_K)
    for name in ("dq", "dk", "dv"):
        assert np.array_equal(b[name], bref[name]), name


# -------------------------------------------------------------- two-level P

TWO = oracle.TWO_LEVEL_P


@pytest.mark.parametrize("Lk", [128, 100])
def test_two_level_p_single_chunk_is_the_static_p_scale(Lk):
    # One chunk: the row's largest P in it is exp(0) = 1, so the first level is 448*6 / 1, the
    # static P scale, and every output (forward and backward) is the static-scale one.
    Lq = 24
    q, k, v = rand_bits((1, 2, Lq, D), 131), rand_bits((1, 2, Lk, D), 132, 2.0), rand_bits((1, 2, Lk, D), 133)
    a = oracle.attn_fwd(q, k, v, SCALE, flags=ALL | TWO)
    b = oracle.attn_fwd(q, k, v, SCALE, flags=ALL | oracle.GSF_P)
    for name in ("o", "o_hp", "lse", "cmax"):
        assert np.array_equal(a[name], b[name]), name
    assert np.all(a["pscale"] == 2688.0)
    do = rand_bits((1, 2, Lq, D), 134)
    ab = oracle.attn_bwd(q, k, v, do, SCALE, flags=ALL | TWO)
    bb = oracle.attn_bwd(q, k, v, do, SCALE, flags=ALL | oracle.GSF_P)
    for name in ("dq", "dk", "dv"):
        assert np.array_equal(ab[name], bb[name]), name


def chunk_constant(seed, Lq=16, C=4):
    """Q ~ N(0,1); keys constant within each 128-key chunk (chunk bases N(0, 2^2)); V ~ N(0,1)."""
    q = rand_bits((1, 1, Lq, D), seed)
    base = rand_bits((C, D), seed + 1, 2.0)
    k = np.repeat(base, 128, axis=0).reshape(1, 1, C * 128, D)
    v = rand_bits((1, 1, C * 128, D), seed + 2)
    return q, k, v


def test_two_level_p_recovers_constant_chunks():
    # Keys constant within each chunk make every P of a (row, chunk) equal to that chunk's largest
    # P, so the first level maps it to 448*6: the block scale is E4M3(448) = 448, the value codes to
    # 6, and P-hat is P up to fp32 and bf16 rounding.  With Q, K, V unquantized the output is then
    # softmax attention to within the bf16 rounding of the chunk weights; the static P scale rounds
    # E4M3(448 P) instead and lands further away.
    q, k, v = chunk_constant(135)
    exact = sdpa64(f64(q), f64(k), f64(v), SCALE).numpy()
    two = oracle.attn_fwd(q, k, v, SCALE, flags=oracle.QUANT_P | TWO)
    stat = oracle.attn_fwd(q, k, v, SCALE, flags=oracle.QUANT_P | oracle.GSF_P)
    scale = np.abs(exact).max()
    e_two = np.abs(two["o"] - exact).max() / scale
    e_stat = np.abs(stat["o"] - exact).max() / scale
    assert e_two < 2.0 ** -8
    assert e_stat > 4 * e_two
    # the first level is 448*6 exactly where the chunk holds the running maximum, larger elsewhere
    cm = two["cmax"][0, 0]
    first = np.concatenate([np.ones((cm.shape[0], 1), bool), cm[:, 1:] > cm[:, :-1]], axis=1)
    ps = two["pscale"][0, 0]
    assert np.all(ps[first] == 2688.0)
    assert np.all(ps[~first] > 2688.0)
    assert (~first).any()


def test_two_level_p_backward_identities():
    # dQ and dK take the unquantized probabilities, so with Q, K, V unquantized they equal float64
    # autograd whatever P's quantizer; dV pairs with the output (<dO, O> = sum_j <dV_j, V_j>),
    # which ties the backward's P-hat to the forward's; on chunk-constant keys dV is autograd's
    # to the bf16 rounding of the chunk weights.
    q, k, v = chunk_constant(137)
    do = rand_bits((1, 1, 16, D), 140)
    fl = oracle.QUANT_P | TWO
    b = oracle.attn_bwd(q, k, v, do, SCALE, flags=fl)
    Q, K, V = (f64(t).requires_grad_() for t in (q, k, v))
    sdpa64(Q, K, V, SCALE).backward(f64(do))
    # (to the fp32 rounding of the logits the oracle forms)
    assert np.abs(b["dq"] - Q.grad.numpy()).max() < 1e-6 * np.abs(Q.grad.numpy()).max()
    assert np.abs(b["dk"] - K.grad.numpy()).max() < 1e-6 * np.abs(K.grad.numpy()).max()
    assert np.abs(b["dv"] - V.grad.numpy()).max() < 2.0 ** -8 * np.abs(V.grad.numpy()).max()
    f = oracle.attn_fwd(q, k, v, SCALE, flags=fl)
    lhs = np.einsum("bhid,bhid->bh", f32(do).astype(np.float64), f["o"])
    rhs = np.einsum("bhjd,bhjd->bh", b["dv"], f32(v).astype(np.float64))
    assert np.allclose(lhs, rhs, rtol=1e-10)
    # random keys: the same pairing, and the cube-sparse backward agrees with the dense one at
    # sparsity 0
    q, k, v = rand_bits((1, 1, 40, D), 141), rand_bits((1, 1, 384, D), 142, 2.0), rand_bits((1, 1, 384, D), 143)
    do = rand_bits((1, 1, 40, D), 144)
    b = oracle.attn_bwd(q, k, v, do, SCALE, flags=ALL | TWO)
    f = oracle.attn_fwd(q, k, v, SCALE, flags=ALL | TWO)
    vh = f32(oracle.fq_bf16(v, 2)).astype(np.float64)
    lhs = np.einsum("bhid,bhid->bh", f32(do).astype(np.float64), f["o"])
    rhs = np.einsum("bhjd,bhjd->bh", b["dv"], vh)
    assert np.allclose(lhs, rhs, rtol=1e-10)


def test_two_level_p_vsa_sparsity_zero_is_dense():
    L = 512
    q, k, v = (rand_bits((1, 1, L, D), s) for s in (145, 146, 147))
    fl = ALL | TWO
    s = oracle.vsa_fwd(q, k, v, SCALE, sparsity=0.0, flags=fl)
    d = oracle.attn_fwd(q, k, v, SCALE, flags=fl)
    assert np.array_equal(s["o_fine"], d["o"])
    do = rand_bits((1, 1, L, D), 148)
    sb = oracle.vsa_bwd(q, k, v, do, SCALE, sparsity=0.0, flags=fl, krows=np.arange(0, L, 37))
    db = oracle.attn_bwd(q, k, v, do, SCALE, flags=fl, krows=np.arange(0, L, 37))
    for name in ("dq", "dk", "dv"):
        assert np.allclose(sb[name], db[name], rtol=0, atol=1e-12), name


def test_two_level_p_rejects_final_max_and_static_p():
    q, k, v = (rand_bits((1, 1, 64, D), s) for s in (149, 150, 151))
    for extra in (oracle.FINAL_MAX, oracle.GSF_P):
        with pytest.raises(ValueError):
            oracle.attn_fwd(q, k, v, SCALE, flags=ALL | TWO | extra)
        with pytest.raises(ValueError):
            oracle.vsa_fwd(q, k, v, SCALE, cube_tokens=64, sparsity=0.0, flags=ALL | TWO | extra)


# ----------------------------------------------------------------- smooth Q

SQ = oracle.SMOOTH_Q


def q_smoothed_eff(q_bits, g=1.0, quant=True):
    """The query the method multiplies with under smooth-Q: fq(fp32(q - mean)) (without `quant`,
    fp32(q - mean)) rounded to bf16 as the matmul operand, plus the mean (per (b, h, channel): fp64
    sum / L rounded to fp32), in fp64; built from the pinned fp32 codec."""
    qf = f32(q_bits)
    mean = (qf.astype(np.float64).sum(axis=2, keepdims=True) / qf.shape[2]).astype(np.float32)
    qs = (qf - mean).astype(np.float32)
    if quant:
        qs = oracle.fq_f32_rows(qs.reshape(-1, D), g=g).reshape(qs.shape)
    qq = f32(bits_of(qs))
    return torch.from_numpy(qq.astype(np.float64) + mean.astype(np.float64))


def test_smooth_q_without_quantization_is_softmax_attention():
    # the subtracted mean's share of every logit is added back: attention on the restored query
    # (the smoothed query rounded to bf16 as the matmul operand, plus the mean), which is plain
    # attention on the original Q up to that bf16 rounding
    Lq, Lk = 40, 200
    q, k, v = rand_bits((1, 2, Lq, D), 161, 1.0, 2.0), rand_bits((1, 2, Lk, D), 162), rand_bits((1, 2, Lk, D), 163)
    r = oracle.attn_fwd(q, k, v, SCALE, flags=SQ)
    ref = sdpa64(q_smoothed_eff(q, quant=False), f64(k), f64(v), SCALE).numpy()
    assert np.abs(r["o"] - ref).max() < 1e-6 * np.abs(ref).max()
    plain = sdpa64(f64(q), f64(k), f64(v), SCALE).numpy()
    assert np.abs(r["o"] - plain).max() < 2.0 ** -7 * np.abs(plain).max()


@pytest.mark.parametrize("causal", [False, True])
def test_smooth_q_is_attention_on_the_restored_query(causal):
    # With Q and K quantized (P unquantized) the output is softmax attention with the query
    # fq(q - mean) + mean and the quantized keys; the backward is float64 autograd of it (dQ passes
    # straight through to q, dK sees the restored query).
    L = 150
    q, k, v = rand_bits((1, 2, L, D), 164, 1.0, 1.5), rand_bits((1, 2, L, D), 165), rand_bits((1, 2, L, D), 166)
    do = rand_bits((1, 2, L, D), 167)
    fl = oracle.QUANT_Q | oracle.QUANT_K | oracle.QUANT_V | SQ
    r = oracle.attn_fwd(q, k, v, SCALE, causal=causal, flags=fl)
    Qe = q_smoothed_eff(q).requires_grad_()
    K = f64(oracle.fq_bf16(k, -1)).requires_grad_()
    V = f64(oracle.fq_bf16(v, 2)).requires_grad_()
    ref = sdpa64(Qe, K, V, SCALE, causal)
    assert np.abs(r["o"] - ref.detach().numpy()).max() < 1e-6 * np.abs(ref.detach().numpy()).max()
    ref.backward(f64(do))
    b = oracle.attn_bwd(q, k, v, do, SCALE, causal=causal, flags=fl)
    for name, want in (("dq", Qe.grad), ("dk", K.grad), ("dv", V.grad)):
        w = want.numpy()
        assert np.abs(b[name] - w).max() < 1e-6 * np.abs(w).max(), name


def test_smooth_q_reduces_the_quantization_error_of_an_offset_query():
    # the point of the smoothing: a query with a large common offset loses less to its quantization
    Lq, Lk = 32, 256
    q, k, v = rand_bits((1, 1, Lq, D), 168, 1.0, 4.0), rand_bits((1, 1, Lk, D), 169), rand_bits((1, 1, Lk, D), 170)
    exact = sdpa64(f64(q), f64(k), f64(v), SCALE).numpy()
    plain = oracle.attn_fwd(q, k, v, SCALE, flags=oracle.QUANT_Q)["o"]
    smooth = oracle.attn_fwd(q, k, v, SCALE, flags=oracle.QUANT_Q | SQ)["o"]
    assert np.abs(smooth - exact).mean() < 0.5 * np.abs(plain - exact).mean()


def test_smooth_q_with_static_scale_and_smooth_k_and_sparse():
    # the static Q scale is taken on the smoothed queries; with smooth-K as well the keys are
    # smoothed first (the logits' per-row shift cancels in the softmax); at sparsity 0 the
    # cube-sparse variant equals the dense one, forward and backward
    L = 256
    q, k, v = rand_bits((1, 1, L, D), 171, 1.0, 2.0), rand_bits((1, 1, L, D), 172, 1.0, 1.0), rand_bits((1, 1, L, D), 173)
    fl = oracle.QUANT_Q | oracle.QUANT_K | oracle.QUANT_V | SQ | oracle.GSF_QKV
    r = oracle.attn_fwd(q, k, v, SCALE, flags=fl)
    qf = f32(q)
    mean = (qf.astype(np.float64).sum(axis=2, keepdims=True) / L).astype(np.float32)
    gq = np.float32(np.float32(2688.0) / np.float32(np.abs((qf - mean).astype(np.float32)).max()))
    Qe = q_smoothed_eff(q, g=float(gq))
    K = f64(oracle.fq_bf16(k, -1, g=oracle.static_scale_bf16(k)))
    V = f64(oracle.fq_bf16(v, 2, g=oracle.static_scale_bf16(v)))
    ref = sdpa64(Qe, K, V, SCALE).numpy()
    assert np.abs(r["o"] - ref).max() < 1e-6 * np.abs(ref).max()
    fl2 = ALL | SQ | oracle.SMOOTH_K
    s = oracle.vsa_fwd(q, k, v, SCALE, sparsity=0.0, flags=fl2)
    d = oracle.attn_fwd(q, k, v, SCALE, flags=fl2)
    assert np.array_equal(s["o_fine"], d["o"])
    do = rand_bits((1, 1, L, D), 174)
    sb = oracle.vsa_bwd(q, k, v, do, SCALE, sparsity=0.0, flags=fl2, krows=np.arange(0, L, 29))
    db = oracle.attn_bwd(q, k, v, do, SCALE, flags=fl2, krows=np.arange(0, L, 29))
    for name in ("dq", "dk", "dv"):
        assert np.allclose(sb[name], db[name], rtol=0, atol=1e-12), name


# ---------------------------------------------------------------- FP8 P.V product

PVF8 = oracle.PV_FP8


def fp8(x):
    """Nearest FP8 E4M3FN value (torch's float8_e4m3fn cast: ties to even, subnormals kept; the
    values here stay far below its 448 limit), as float64."""
    return torch.as_tensor(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_pv_fp8_constant_logits_closed_form():
    # every key equal: every logit of a row is equal, so P = 1 everywhere, P-hat = 6 * E4M3(1/6) =
    # 1.03125 (l = Lk), and E4M3 rounds it to 1.0: O_i = mean_j E4M3(V-hat_j).  The last chunk is
    # partial (200 keys) and its last block has 8 keys.
    Lq, Lk = 8, 200
    q = rand_bits((1, 1, Lq, D), 401)
    k = np.repeat(rand_bits((1, 1, 1, D), 402), Lk, axis=2)
    v = rand_bits((1, 1, Lk, D), 403, 3.0)
    assert fp8(1.03125) == 1.0
    vh = f32(oracle.fq_bf16(v, 2))[0, 0]
    r = oracle.attn_fwd(q, k, v, SCALE, flags=ALL | PVF8)
    assert np.allclose(r["o"][0, 0], np.broadcast_to(fp8(vh).mean(0), (Lq, D)), rtol=1e-12, atol=1e-14)
    d = oracle.attn_fwd(q, k, v, SCALE, flags=ALL)
    assert np.allclose(d["o"][0, 0], np.broadcast_to(1.03125 * vh.astype(np.float64).mean(0), (Lq, D)),
                       rtol=1e-12, atol=1e-14)


def test_pv_fp8_exact_operands_leave_the_bf16_path_unchanged():
    # P unquantized and every logit equal: P = 1 (exact in E4M3); V in 16-key blocks whose abs-max is 6
    # has the unit E4M3 block scale, so V-hat is an E2M1 value (exact in E4M3).  Both readings then
    # multiply the same operands: identical outputs, bit for bit.
    Lq, Lk = 6, 160
    q = rand_bits((1, 1, Lq, D), 404)
    k = np.repeat(rand_bits((1, 1, 1, D), 405), Lk, axis=2)
    g = torch.Generator().manual_seed(406)
    vv = torch.rand(1, 1, Lk, D, generator=g) * 12 - 6
    vv[:, :, ::16, :] = 6.0  # one entry of 6 in every block along the keys
    v = vv.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    vh = f32(oracle.fq_bf16(v, 2))[0, 0]
    assert np.array_equal(fp8(vh), vh.astype(np.float64))
    fl = oracle.QUANT_Q | oracle.QUANT_K | oracle.QUANT_V
    a = oracle.attn_fwd(q, k, v, SCALE, flags=fl | PVF8)
    b = oracle.attn_fwd(q, k, v, SCALE, flags=fl)
    assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["o_hp"], b["o_hp"])


def test_pv_fp8_random_inputs_match_the_unrolled_closed_form():
    Lq, Lk = 12, 300
    q, k, v = rand_bits((1, 1, Lq, D), 407), rand_bits((1, 1, Lk, D), 408, 2.0), rand_bits((1, 1, Lk, D), 409)
    r = oracle.attn_fwd(q, k, v, SCALE, flags=ALL | PVF8)
    qh, kh, vh = quantized_ops(q, k, v)
    S = (SCALE * (qh @ kh.T)).astype(np.float32)
    want = closed_form(S, fp8(vh), chunk=128, pq_map=fp8)
    assert np.allclose(r["o"][0, 0], want, rtol=1e-9, atol=1e-12)
    # and the rounding changes the result (the flag reaches the arithmetic)
    assert not np.allclose(r["o"], oracle.attn_fwd(q, k, v, SCALE, flags=ALL)["o"], rtol=0, atol=1e-6)


def test_pv_fp8_backward():
    Lq, Lk = 50, 200
    q, do = rand_bits((1, 2, Lq, D), 410), rand_bits((1, 2, Lq, D), 413)
    k, v = rand_bits((1, 2, Lk, D), 411, 1.5), rand_bits((1, 2, Lk, D), 412)
    fl = ALL | PVF8
    b = oracle.attn_bwd(q, k, v, do, SCALE, flags=fl)
    # dS uses the unquantized probabilities and dP the rounded V-hat: dQ, dK are plain attention's
    # gradients on (Q-hat, K-hat, E4M3(V-hat))
    Q = f64(oracle.fq_bf16(q, -1)).requires_grad_()
    K = f64(oracle.fq_bf16(k, -1)).requires_grad_()
    V8 = torch.from_numpy(fp8(f32(oracle.fq_bf16(v, 2))))
    sdpa64(Q, K, V8, SCALE).backward(f64(do))
    assert np.allclose(b["dq"], Q.grad.numpy(), rtol=0, atol=5e-6)
    assert np.allclose(b["dk"], K.grad.numpy(), rtol=0, atol=5e-6)
    # dV = A-hat^T dO with the forward's rounded P-hat: <dO, O> = sum_j <dV_j, E4M3(V-hat)_j>
    o = oracle.attn_fwd(q, k, v, SCALE, flags=fl)["o"]
    lhs = np.einsum("bhid,bhid->bh", f64(do).numpy(), o)
    rhs = np.einsum("bhjd,bhjd->bh", b["dv"], V8.numpy())
    assert np.allclose(lhs, rhs, rtol=1e-10, atol=1e-10)
