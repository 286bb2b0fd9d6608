"""CPU-side checks of the C ABI: the library loads, exports every symbol that
include/attnqat.h declares, and rejects malformed arguments on the host before
any HIP call (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attnqat.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(os.path.join(ROOT, "quantization_aware_attention_nvfp4_amd", "libattnqat.so")):
        import __graft_entry__
        __graft_entry__._libbuild().build()
    from quantization_aware_attention_nvfp4_amd import _lib
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char\s*\*|const char\s*\*)\s*\**\s*(\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("fq_nvfp4", "fq_nvfp4_static_scale", "attn_qat_fwd", "attn_qat_bwd", "vsa_qat_fwd",
              "vsa_topk", "attn_qat_workspace_size", "aq_last_error"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    from quantization_aware_attention_nvfp4_amd import _lib
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(_lib.EXPORTED) == set(declared_functions())


def S(b=1, h=1, l=1):
    from quantization_aware_attention_nvfp4_amd._lib import aq_strides
    return aq_strides(b, h, l)


def fwd(lib, **kw):
    a = dict(q=16, k=16, v=16, o=16, B=1, H=2, Hkv=2, D=128, lq=64, lk=64, scale=0.088, causal=0, flags=15,
             ws=256, ws_bytes=1 << 40)
    a.update(kw)
    s = a.get("s", S(64 * 256, 128, 256))
    return lib.attn_qat_fwd(a["q"], a["k"], a["v"], a["o"], a["B"], a["H"], a["Hkv"], a["D"], a["lq"], a["lk"],
                            s, s, s, s, a["scale"], a["causal"], a["flags"], None, None, None, a["ws"],
                            a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(D=64), -1, "head_size"),
    (dict(q=None), -1, "null"),
    (dict(lq=0), -1, "positive"),
    (dict(scale=float("nan")), -1, "softmax_scale"),
    (dict(scale=-1.0), -1, "softmax_scale"),
    (dict(flags=2048), -1, "quant_flags"),
    (dict(flags=15 | 256 | 16), -2, "AQ_TWO_LEVEL_P"),
    (dict(flags=15 | 256 | 64), -2, "AQ_TWO_LEVEL_P"),
    (dict(flags=7 | 1024), -2, "AQ_PV_FP8"),
    (dict(Hkv=1), -2, "num_kv_heads"),
    (dict(causal=1, lk=32), -2, "causal"),
    (dict(ws_bytes=100), -1, "workspace"),
    (dict(ws=257), -1, "workspace"),
    (dict(q=8), -1, "16-byte aligned"),
    (dict(s=None), -1, "16-byte aligned"),
])
def test_forward_rejects_bad_arguments(lib, kw, code, msg):
    if "s" in kw:
        kw = dict(kw, s=S(64 * 256, 128, 132))  # row stride not a multiple of 8 elements
    assert fwd(lib, **kw) == code
    assert msg in lib.aq_last_error().decode()


def test_forward_training_outputs_come_together(lib):
    s = S(64 * 256, 128, 256)
    rc = lib.attn_qat_fwd(16, 16, 16, 16, 1, 2, 2, 128, 64, 64, s, s, s, s, 0.088, 0, 15, 256, None, None, 256,
                          1 << 40, None)
    assert rc == -1 and "together" in lib.aq_last_error().decode()


def test_backward_requires_statistics(lib):
    s = S(64 * 256, 128, 256)
    rc = lib.attn_qat_bwd(16, 16, 16, None, 16, None, None, 16, 16, 16, 1, 2, 2, 128, 64, 64, s, s, s, s, s, s, s,
                          0.088, 0, 15, 256, 1 << 40, None)
    assert rc == -1 and "required" in lib.aq_last_error().decode()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(grid=(16, 28, 56), cube=(4, 4, 8), L=25087), -1, "seq_len"),
    (dict(grid=(16, 28, 55), cube=(4, 4, 8), L=16 * 28 * 55), -1, "divisible"),
    (dict(grid=(16, 28, 56), cube=(4, 4, 4), L=25088), -2, "128"),
    (dict(grid=(16, 28, 56), cube=(4, 4, 8), L=25088, sparsity=1.5), -1, "sparsity"),
])
def test_vsa_rejects_bad_arguments(lib, kw, code, msg):
    s = S(25088 * 1536, 128, 1536)
    g, c = kw["grid"], kw["cube"]
    rc = lib.vsa_qat_fwd(16, 16, 16, 16, None, None, 1, 12, 128, kw["L"], g[0], g[1], g[2], c[0], c[1], c[2],
                         kw.get("sparsity", 0.9), s, s, s, s, 0.088, 15, None, None, None, 256, 1 << 40, None)
    assert rc == code
    assert msg in lib.aq_last_error().decode()
    # the backward makes the same shape checks
    rc = lib.vsa_qat_bwd(16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 1, 12, 128, kw["L"], g[0], g[1], g[2], c[0],
                         c[1], c[2], kw.get("sparsity", 0.9), s, s, s, s, s, s, s, 0.088, 15, 256, 1 << 40, None)
    assert rc == code
    assert msg in lib.aq_last_error().decode()


def test_vsa_training_outputs_and_backward_inputs(lib):
    s = S(25088 * 1536, 128, 1536)
    rc = lib.vsa_qat_fwd(16, 16, 16, 16, None, None, 1, 12, 128, 25088, 16, 28, 56, 4, 4, 8, 0.9, s, s, s, s,
                         0.088, 15, 16, None, None, 256, 1 << 40, None)
    assert rc == -1 and "together" in lib.aq_last_error().decode()
    rc = lib.vsa_qat_bwd(16, 16, 16, 16, 16, 16, 16, None, 16, 16, 16, 1, 12, 128, 25088, 16, 28, 56, 4, 4, 8, 0.9,
                         s, s, s, s, s, s, s, 0.088, 15, 256, 1 << 40, None)
    assert rc == -1 and "required" in lib.aq_last_error().decode()


def test_fq_rejects_bad_arguments(lib):
    assert lib.fq_nvfp4(None, 8, 1, 16, 1, None, None) == -1
    assert lib.fq_nvfp4(8, 8, 1, 0, 1, None, None) == -1
    assert lib.fq_nvfp4_static_scale(8, 0, 8, None) == -1


def test_topk_and_workspace(lib):
    assert lib.vsa_topk(0.9, 196) == 20
    assert lib.vsa_topk(0.0, 196) == 196
    assert lib.vsa_topk(1.0, 196) == 1
    assert lib.vsa_topk(2.0, 196) == 0
    # K-hat and V-hat for 12 heads x 25088 keys (2 x 77.07 MB), then the variants' regions: the
    # scales (256 B), key means [12, 128] fp32, their fp64 partial sums [12, 98 slabs, 128], the
    # final row maxima [12, 25088] fp32, then smooth-Q's query means, their partial sums and the
    # per-key delta [12, 25088] fp32, each 256-byte aligned.
    al = lambda n: (n + 255) // 256 * 256
    means = al(12 * 128 * 4) + al(12 * 98 * 128 * 8)
    want = 2 * 12 * 25088 * 128 * 2 + 256 + means + al(12 * 25088 * 4) + means + al(12 * 25088 * 4)
    assert lib.attn_qat_workspace_size(0, 1, 12, 25088, 25088) == want
    assert lib.attn_qat_workspace_size(0, 0, 12, 25088, 25088) == 0


def test_python_binding_validates_before_the_library(lib):
    import torch
    from quantization_aware_attention_nvfp4_amd import ops
    x = torch.zeros(4, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ops.fq_nvfp4(x)  # a CPU tensor is refused
    with pytest.raises(NotImplementedError):
        ops.AttnQatTrainImpl(12, 128, False, 0.088, dropout_p=0.1)
    with pytest.raises(ValueError):
        ops.AttnQatTrainImpl(12, 64, False, 0.088)


def test_missing_library_raises_import_error(tmp_path, monkeypatch):
    from quantization_aware_attention_nvfp4_amd import _lib
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libattnqat.so"))
    with pytest.raises(ImportError):
        _lib.load()


def test_linear_rejects_bad_arguments(lib):
    ws = 1 << 20
    fwd = lambda m, n, k, x=16, ws_bytes=1 << 40: lib.qad_linear_fwd(x, 16, None, 16, m, n, k, None, ws, ws_bytes, None)
    assert fwd(0, 64, 64) == -1 and "positive" in lib.aq_last_error().decode()
    assert fwd(10, 64, 48) == -2 and "multiples of 64" in lib.aq_last_error().decode()
    assert fwd(10, 96, 64) == -2
    assert fwd(10, 64, 64, x=8) == -1 and "aligned" in lib.aq_last_error().decode()
    assert fwd(10, 64, 64, ws_bytes=100) == -1 and "workspace" in lib.aq_last_error().decode()
    assert lib.qad_linear_bwd(16, 16, 16, 16, 16, None, 10, 64, 40, ws, 1 << 40, None) == -2
    assert lib.qad_observe_amax(None, 10, 16, None) == -1
    assert lib.qad_linear_workspace_size(0, 10, 64, 64) > 10 * 64 * 2 + 64 * 64 * 2
    assert lib.qad_linear_workspace_size(2, 10, 64, 64) == 0
