"""attn_qat_fwd_noalloc, the forward for callers that cannot allocate: called through the C ABI,
its outputs must equal attn_qat_fwd's (the same kernels over the library's fixed device scratch
instead of a caller workspace) bit for bit, on two calls in a row (the second smaller, so it runs
over the scratch the first one left behind), under variants whose per-call statistics live in the
scratch, and at the 448x896x61 workload's size.  Calls beyond the scratch are refused on the host,
before any HIP call."""
import ctypes

import numpy as np
import pytest
import torch

import synth


def rand(B, L, H, seed, mult=1.0, shift=0.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(B, L, H, 128, generator=g) * mult + shift).to(torch.bfloat16)


def same(a, b):
    return torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                       b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16))


@pytest.fixture(scope="module")
def m():
    import quantization_aware_attention_nvfp4_amd as m
    return m


def direct_call(m, q, k, v, o, flags, aux=None, causal=False):
    """The C entry point itself (ctypes), with caller-owned outputs."""
    from quantization_aware_attention_nvfp4_amd import _lib, ops
    B, Lq, H, D = q.shape
    Lk = k.shape[1]
    p = lambda t: None if t is None else t.data_ptr()
    a = aux or {}
    rc = _lib.load().attn_qat_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B, H, H, D, Lq, Lk,
                                          ops._strides_blhd(q), ops._strides_blhd(k), ops._strides_blhd(v),
                                          ops._strides_blhd(o), float(1.0 / np.sqrt(128)), int(causal), int(flags),
                                          p(a.get("lse_log2")), p(a.get("chunk_max_log2")), p(a.get("o_hp")),
                                          torch.cuda.current_stream().cuda_stream)
    assert rc == 0, _lib.load().aq_last_error()


@pytest.mark.gpu
@pytest.mark.parametrize("flags", [15, 15 | 32 | 128])
def test_two_calls_match_the_workspace_entry_point(m, flags):
    # first call: 3 heads, 1000 tokens (ragged last chunk), training outputs
    q, k, v = rand(1, 1000, 3, 301, 1.5, 0.3), rand(1, 1000, 3, 302, 1.2, -0.5), rand(1, 1000, 3, 303)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    o_ref, aux_ref = m.attn_qat_fwd(qg, kg, vg, quant_flags=flags, training=True)
    o = torch.empty_like(o_ref)
    aux = {n: torch.empty_like(t) for n, t in aux_ref.items() if n != "p_scale"}
    direct_call(m, qg, kg, vg, o, flags, aux)
    torch.cuda.synchronize()
    assert same(o, o_ref)
    for n in ("lse_log2", "chunk_max_log2", "o_hp"):
        assert same(aux[n], aux_ref[n]), n
    # second call: smaller (2 heads, 300 tokens, causal, inference) over the scratch the first left
    q2, k2, v2 = rand(1, 300, 2, 304, 0.8), rand(1, 300, 2, 305, 2.0), rand(1, 300, 2, 306)
    q2g, k2g, v2g = q2.cuda(), k2.cuda(), v2.cuda()
    o2_ref = m.attn_qat_fwd(q2g, k2g, v2g, causal=True, quant_flags=flags)
    o2 = torch.empty_like(o2_ref)
    direct_call(m, q2g, k2g, v2g, o2, flags, causal=True)
    torch.cuda.synchronize()
    assert same(o2, o2_ref)


@pytest.mark.gpu
def test_binding_and_wan_448x896x61(m):
    # the binding with preallocated outputs, at the 448x896x61 workload (about 159 MB of scratch),
    # then a tiny call after it
    q, k, v = (t.cuda() for t in synth.wan_448x896x61())
    o_ref = m.attn_qat_fwd(q, k, v)
    out = torch.empty_like(o_ref)
    o = m.attn_qat_fwd_noalloc(q, k, v, out=out)
    torch.cuda.synchronize()
    assert o.data_ptr() == out.data_ptr() and same(o, o_ref)
    qt, kt, vt = (t.cuda() for t in synth.tiny_forward())
    o_tiny, aux = m.attn_qat_fwd_noalloc(qt, kt, vt, training=True)
    o_tiny_ref, aux_ref = m.attn_qat_fwd(qt, kt, vt, training=True)
    torch.cuda.synchronize()
    assert same(o_tiny, o_tiny_ref) and all(same(aux[n], aux_ref[n]) for n in ("lse_log2", "chunk_max_log2", "o_hp"))


def test_refuses_calls_beyond_the_scratch():
    # 12 heads of 65536 tokens need about 0.4 GB of scratch: refused before any HIP call (no GPU
    # needed; the tensor pointers are never dereferenced)
    from quantization_aware_attention_nvfp4_amd import _lib
    lib = _lib.load()
    S = _lib.aq_strides
    L, H = 65536, 12
    need = lib.attn_qat_workspace_size(0, 1, H, L, L)
    assert need > (256 << 20)
    s = S(L * H * 128, 128, H * 128)
    fake = 1 << 20
    rc = lib.attn_qat_fwd_noalloc(fake, fake, fake, fake, 1, H, H, 128, L, L, s, s, s, s, 0.088, 0, 15, None, None,
                                  None, None)
    assert rc == _lib.AQ_ENOTSUP and b"scratch" in lib.aq_last_error()
    # and a call that fits passes the size check (refused here only for a bad argument)
    rc = lib.attn_qat_fwd_noalloc(fake, fake, fake, fake, 1, 12, 12, 128, 1024, 1024, s, s, s, s, -1.0, 0, 15, None,
                                  None, None, None)
    assert rc == _lib.AQ_EINVAL and b"softmax_scale" in lib.aq_last_error()
