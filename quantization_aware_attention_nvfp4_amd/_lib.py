"""ctypes loader for libattnqat.so (the C ABI declared in include/attnqat.h).

The library is required: there is no fallback.  Like the pages' ATTN_QAT_TRAIN
backend ("Attn-QAT Training" guide, "Prerequisites": it fails instead of falling
back to dense attention when its kernel cannot be loaded), a missing or broken
library raises ImportError carrying the original error.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattnqat.so")

AQ_OK, AQ_EINVAL, AQ_ENOTSUP, AQ_EHIP = 0, -1, -2, -3
AQ_QUANT_Q, AQ_QUANT_K, AQ_QUANT_V, AQ_QUANT_P = 1, 2, 4, 8
AQ_QUANT_ALL = 15
# Variants (include/attnqat.h): final-max statistics, static Q/K/V and P global scales, smooth-K,
# two-level P, smooth-Q, the FP8 P.V product.
AQ_FINAL_MAX, AQ_GSF_QKV, AQ_GSF_P, AQ_SMOOTH_K, AQ_TWO_LEVEL_P, AQ_SMOOTH_Q, AQ_PV_FP8 = 16, 32, 64, 128, 256, 512, 1024
AQ_FLAGS_ALL = 2047

EXPORTED = ("aq_last_error", "fq_nvfp4", "fq_nvfp4_static_scale", "attn_qat_fwd", "attn_qat_bwd",
            "vsa_qat_fwd", "vsa_qat_bwd", "vsa_topk", "attn_qat_workspace_size", "aq_kernel_timing",
            "aq_kernel_times", "qad_linear_workspace_size", "qad_linear_fwd", "qad_linear_bwd", "qad_observe_amax",
            "qad_input_global_sf", "attn_qat_fwd_noalloc")


class aq_strides(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int64), ("h", ctypes.c_int64), ("l", ctypes.c_int64)]


_lib = None
_load_error = None


def _declare(lib):
    P, i32, i64, f32, f64, u32, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                                      ctypes.c_double, ctypes.c_uint, ctypes.c_size_t)
    S = aq_strides
    lib.aq_last_error.argtypes = []
    lib.aq_last_error.restype = ctypes.c_char_p
    lib.fq_nvfp4.argtypes = [P, P, i64, i64, i64, P, P]
    lib.fq_nvfp4.restype = i32
    lib.fq_nvfp4_static_scale.argtypes = [P, i64, P, P]
    lib.fq_nvfp4_static_scale.restype = i32
    lib.attn_qat_fwd.argtypes = [P, P, P, P, i32, i32, i32, i32, i64, i64, S, S, S, S, f32, i32, u32,
                                 P, P, P, P, sz, P]
    lib.attn_qat_fwd.restype = i32
    lib.attn_qat_fwd_noalloc.argtypes = [P, P, P, P, i32, i32, i32, i32, i64, i64, S, S, S, S, f32, i32, u32,
                                         P, P, P, P]
    lib.attn_qat_fwd_noalloc.restype = i32
    lib.attn_qat_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, i32, i32, i32, i32, i64, i64, S, S, S,
                                 S, S, S, S, f32, i32, u32, P, sz, P]
    lib.attn_qat_bwd.restype = i32
    lib.vsa_qat_fwd.argtypes = [P, P, P, P, P, P, i32, i32, i32, i64, i32, i32, i32, i32, i32, i32,
                                f64, S, S, S, S, f32, u32, P, P, P, P, sz, P]
    lib.vsa_qat_fwd.restype = i32
    lib.vsa_qat_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, P, i32, i32, i32, i64, i32, i32, i32, i32, i32,
                                i32, f64, S, S, S, S, S, S, S, f32, u32, P, sz, P]
    lib.vsa_qat_bwd.restype = i32
    lib.vsa_topk.argtypes = [f64, i32]
    lib.vsa_topk.restype = i32
    lib.attn_qat_workspace_size.argtypes = [i32, i32, i32, i64, i64]
    lib.attn_qat_workspace_size.restype = sz
    lib.aq_kernel_timing.argtypes = [i32]
    lib.aq_kernel_timing.restype = i32
    lib.aq_kernel_times.argtypes = [ctypes.c_char_p, sz, i32]
    lib.aq_kernel_times.restype = i32
    lib.qad_linear_workspace_size.argtypes = [i32, i64, i64, i64]
    lib.qad_linear_workspace_size.restype = sz
    lib.qad_linear_fwd.argtypes = [P, P, P, P, i64, i64, i64, P, P, sz, P]
    lib.qad_linear_fwd.restype = i32
    lib.qad_linear_bwd.argtypes = [P, P, P, P, P, P, i64, i64, i64, P, sz, P]
    lib.qad_linear_bwd.restype = i32
    lib.qad_observe_amax.argtypes = [P, i64, P, P]
    lib.qad_observe_amax.restype = i32
    lib.qad_input_global_sf.argtypes = [P, P, P]
    lib.qad_input_global_sf.restype = i32


def load():
    """Load the shared library once; raise ImportError if it is missing or broken."""
    global _lib, _load_error
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libattnqat.so not found at {LIB_PATH}; build it with "
                          "quantization_aware_attention_nvfp4_amd.build.build() "
                          "(there is no fallback implementation)")
    try:
        lib = ctypes.CDLL(LIB_PATH)
        _declare(lib)
    except OSError as e:  # pragma: no cover - depends on the machine
        _load_error = e
        raise ImportError(f"libattnqat.so could not be loaded: {e}") from e
    except AttributeError as e:  # a library built from older sources lacks a symbol
        _load_error = e
        raise ImportError(f"libattnqat.so is out of date ({e}); rebuild it with "
                          "quantization_aware_attention_nvfp4_amd/build.py") from e
    _lib = lib
    return lib


class AttnQatError(RuntimeError):
    pass


def check(rc: int, what: str) -> None:
    """Map a C return code onto a Python exception."""
    if rc == AQ_OK:
        return
    msg = load().aq_last_error().decode(errors="replace")
    if rc == AQ_EINVAL:
        raise ValueError(f"{what}: {msg}")
    if rc == AQ_ENOTSUP:
        raise NotImplementedError(f"{what}: {msg}")
    raise AttnQatError(f"{what}: {msg} (code {rc})")


def kernel_timing(enable: bool) -> None:
    """Bracket every library kernel launch with HIP events (see aq_kernel_timing)."""
    load().aq_kernel_timing(1 if enable else 0)


def kernel_times(reset: bool = True) -> dict:
    """{kernel name: (launches, total ms)} accumulated while timing was enabled."""
    buf = ctypes.create_string_buffer(1 << 16)
    rc = load().aq_kernel_times(buf, len(buf), 1 if reset else 0)
    if rc < 0:
        raise AttnQatError("aq_kernel_times failed")
    out = {}
    for line in buf.value.decode().splitlines():
        name, count, ms = line.split()
        out[name] = (int(count), float(ms))
    return out
