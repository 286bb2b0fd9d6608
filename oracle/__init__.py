"""CPU oracle for NVFP4 fake-quantized attention (Attn-QAT).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library in ``quantization_aware_attention_nvfp4_amd`` and
neither imports the other.

The arithmetic lives in ``nvfp4_oracle.c`` (plain C loops, fp32 codec, fp64
attention).  This module compiles it with gcc on first use (building the
checker is not using it) and wraps it with numpy-facing functions.  All
tensors are numpy arrays; bf16 data travels as ``uint16`` bit patterns.

Sources, cited by page title and section:
  * "nvfp4_qad.py" (FastVideo source page): module docstring, FP4_RANGE,
    weight_global_sf, input_global_sf.
  * "vsqa-preview-1.3b metadata.json": attention.precision, attention.selection,
    attention.cube_shape and the dense parent's precision record.
  * "attn_qat_train" API reference page: attn_qat_train and its fixed flags.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_BUILD = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD, "liboracle.so")
_lock = threading.Lock()
_lib = None

QUANT_Q, QUANT_K, QUANT_V, QUANT_P = 1, 2, 4, 8
QUANT_ALL = 15
# Variants (readings in nvfp4_oracle.c): statistics relative to the final row
# maximum, static per-tensor global scales for Q/K/V, the static global scale
# of P, smooth-K, the two-level (per-row, per-chunk) scale of P, smooth-Q.
FINAL_MAX, GSF_QKV, GSF_P, SMOOTH_K, TWO_LEVEL_P, SMOOTH_Q = 16, 32, 64, 128, 256, 512
# FP8 P.V product: both operands of P.V rounded to FP8 E4M3FN (reading in nvfp4_oracle.c).
PV_FP8 = 1024


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (OpenMP, no FMA contraction)."""
    os.makedirs(_BUILD, exist_ok=True)
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            P = ctypes.c_void_p
            i64, i32, f32, f64, u32 = (ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_double,
                                       ctypes.c_uint)
            lib.oracle_e4m3.argtypes = [f32]
            lib.oracle_e4m3.restype = f32
            lib.oracle_e2m1.argtypes = [f32]
            lib.oracle_e2m1.restype = f32
            lib.oracle_e2m1_code.argtypes = [f32]
            lib.oracle_e2m1_code.restype = i32
            lib.oracle_block_scale.argtypes = [f32, f32]
            lib.oracle_block_scale.restype = f32
            lib.oracle_fq_bf16.argtypes = [P, P, i64, i64, i64, f32]
            lib.oracle_fq_bf16.restype = None
            lib.oracle_static_scale_bf16.argtypes = [P, i64]
            lib.oracle_static_scale_bf16.restype = f32
            lib.oracle_fq_f32_rows.argtypes = [P, P, i64, i64, f32]
            lib.oracle_fq_f32_rows.restype = None
            lib.oracle_attn_fwd.argtypes = [P, P, P, i32, i32, i64, i64, i32, f64, i32, u32, i32, P, i64,
                                            P, P, P, P, P]
            lib.oracle_attn_fwd.restype = i32
            lib.oracle_attn_bwd.argtypes = [P, P, P, P, i32, i32, i64, i64, i32, f64, i32, u32, i32, P, i64,
                                            P, i64, P, P, P]
            lib.oracle_attn_bwd.restype = i32
            lib.oracle_vsa_topk.argtypes = [f64, i32]
            lib.oracle_vsa_topk.restype = i32
            lib.oracle_vsa_fwd.argtypes = [P, P, P, i32, i32, i64, i32, i32, f64, f64, u32, P, i64, P, P, P,
                                           P, P, P, P]
            lib.oracle_vsa_fwd.restype = i32
            lib.oracle_vsa_bwd.argtypes = [P, P, P, P, i32, i32, i64, i32, i32, f64, f64, u32, P, i64, P, i64,
                                           P, P, P, P]
            lib.oracle_vsa_bwd.restype = i32
            lib.oracle_linear_fwd.argtypes = [P, P, P, i64, i64, i64, f32, P]
            lib.oracle_linear_fwd.restype = None
            lib.oracle_linear_bwd.argtypes = [P, P, P, i64, i64, i64, P, P, P]
            lib.oracle_linear_bwd.restype = None
            lib.oracle_observe_amax.argtypes = [P, i64, f32]
            lib.oracle_observe_amax.restype = f32
            _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bf16 data must be passed as uint16 bit patterns")
    return a


def set_threads(n: int) -> None:
    """Set the OpenMP thread count used by the oracle."""
    os.environ["OMP_NUM_THREADS"] = str(int(n))
    try:
        ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))
    except OSError:
        pass


# ----------------------------------------------------------------------------
# Codec
# ----------------------------------------------------------------------------

def e4m3(v: float) -> float:
    """Nearest FP8 E4M3FN value to v >= 0 (ties to even, saturating at 448)."""
    return _load().oracle_e4m3(float(v))


def e2m1(v: float) -> float:
    """Nearest E2M1 magnitude to v >= 0 (ties to even, saturating at 6)."""
    return _load().oracle_e2m1(float(v))


def e2m1_code(v: float) -> int:
    return _load().oracle_e2m1_code(float(v))


def block_scale(amax: float, g: float = 1.0) -> float:
    """Dequantization scale S = E4M3(fp32(amax/6) * g) / g of one block."""
    return _load().oracle_block_scale(float(amax), float(g))


def fq_bf16(x_u16: np.ndarray, axis: int = -1, g: float = 1.0) -> np.ndarray:
    """NVFP4 fake quantization of a bf16 tensor (uint16 bits) in blocks of 16
    along ``axis``; returns bf16 bits of the same shape."""
    x = _u16(x_u16)
    axis = axis % x.ndim
    outer = int(np.prod(x.shape[:axis], dtype=np.int64))
    inner = int(np.prod(x.shape[axis + 1:], dtype=np.int64))
    y = np.empty_like(x)
    _load().oracle_fq_bf16(_ptr(x), _ptr(y), outer, x.shape[axis], inner, float(g))
    return y


def static_scale_bf16(x_u16: np.ndarray) -> float:
    """g = 448*6 / max(amax|x|, 1e-12) in fp32."""
    x = _u16(x_u16)
    return _load().oracle_static_scale_bf16(_ptr(x), x.size)


def fq_f32_rows(x: np.ndarray, g: float = 1.0) -> np.ndarray:
    """Fake quantization of fp32 values in blocks of 16 along the last axis."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty_like(x)
    rows = x.size // x.shape[-1]
    _load().oracle_fq_f32_rows(_ptr(x), _ptr(y), rows, x.shape[-1], float(g))
    return y


# ----------------------------------------------------------------------------
# Attention
# ----------------------------------------------------------------------------

def attn_fwd(q, k, v, scale, causal=False, flags=QUANT_ALL, chunk=128, rows=None):
    """Fake-quant attention forward for query rows ``rows`` of every head.

    q: [B, H, Lq, D], k/v: [B, H, Lk, D] as bf16 bits (uint16).
    Returns dict of fp64 arrays: o, o_hp [B, H, R, D]; lse [B, H, R];
    cmax [B, H, R, ceil(Lk/chunk)] (natural-log units); pscale [B, H, R, ceil(Lk/chunk)], the
    global scale of P's blocks in each chunk."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, H, Lq, D = q.shape
    Lk = k.shape[2]
    rows = np.arange(Lq, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    R = rows.size
    if flags & FINAL_MAX:
        chunk = (Lk + 15) // 16 * 16
    C = (Lk + chunk - 1) // chunk
    o = np.empty((B, H, R, D))
    ohp = np.empty((B, H, R, D))
    lse = np.empty((B, H, R))
    cmax = np.empty((B, H, R, C))
    pscale = np.empty((B, H, R, C))
    rc = _load().oracle_attn_fwd(_ptr(q), _ptr(k), _ptr(v), B, H, Lq, Lk, D, float(scale), int(causal),
                                 int(flags), int(chunk), _ptr(rows), R, _ptr(o), _ptr(ohp), _ptr(lse),
                                 _ptr(cmax), _ptr(pscale))
    if rc != 0:
        raise ValueError("oracle_attn_fwd rejected the arguments")
    return {"o": o, "o_hp": ohp, "lse": lse, "cmax": cmax, "pscale": pscale, "rows": rows}


def attn_bwd(q, k, v, do, scale, causal=False, flags=QUANT_ALL, chunk=128, qrows=None, krows=None):
    """Straight-through backward: dQ at query rows ``qrows``, dK/dV at key
    rows ``krows`` (fp64 arrays [B, H, R, D])."""
    q, k, v, do = _u16(q), _u16(k), _u16(v), _u16(do)
    B, H, Lq, D = q.shape
    Lk = k.shape[2]
    qrows = (np.arange(Lq, dtype=np.int64) if qrows is None
             else np.ascontiguousarray(qrows, dtype=np.int64))
    krows = (np.arange(Lk, dtype=np.int64) if krows is None
             else np.ascontiguousarray(krows, dtype=np.int64))
    dq = np.empty((B, H, qrows.size, D))
    dk = np.empty((B, H, krows.size, D))
    dv = np.empty((B, H, krows.size, D))
    rc = _load().oracle_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(do), B, H, Lq, Lk, D, float(scale),
                                 int(causal), int(flags), int(chunk), _ptr(qrows), qrows.size, _ptr(krows),
                                 krows.size, _ptr(dq), _ptr(dk), _ptr(dv))
    if rc != 0:
        raise ValueError("oracle_attn_bwd rejected the arguments")
    return {"dq": dq, "dk": dk, "dv": dv, "qrows": qrows, "krows": krows}


def vsa_topk(sparsity: float, n: int) -> int:
    """max(1, min(ceil((1 - sparsity) * n), n))."""
    return _load().oracle_vsa_topk(float(sparsity), int(n))


def vsa_fwd(q, k, v, scale, cube_tokens=128, sparsity=0.9, flags=QUANT_ALL, rows=None):
    """Cube-sparse forward on cube-major tokens.  Returns pooled Q/K/V (bf16
    bits), coarse scores (fp64), the selection (int32, ascending) and the
    fine / coarse outputs (fp64) for query rows ``rows``."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, H, L, D = q.shape
    n = L // cube_tokens
    topk = vsa_topk(sparsity, n)
    rows = np.arange(L, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    R = rows.size
    qp = np.empty((B, H, n, D), np.uint16)
    kp = np.empty((B, H, n, D), np.uint16)
    vp = np.empty((B, H, n, D), np.uint16)
    score = np.empty((B, H, n, n))
    sel = np.empty((B, H, n, topk), np.int32)
    of = np.empty((B, H, R, D))
    oc = np.empty((B, H, R, D))
    rc = _load().oracle_vsa_fwd(_ptr(q), _ptr(k), _ptr(v), B, H, L, D, cube_tokens, float(sparsity),
                                float(scale), int(flags), _ptr(rows), R, _ptr(qp), _ptr(kp), _ptr(vp),
                                _ptr(score), _ptr(sel), _ptr(of), _ptr(oc))
    if rc < 0:
        raise ValueError("oracle_vsa_fwd rejected the arguments")
    return {"qpool": qp, "kpool": kp, "vpool": vp, "score": score, "sel": sel, "o_fine": of,
            "o_coarse": oc, "topk": topk, "rows": rows}


def vsa_bwd(q, k, v, do, scale, cube_tokens=128, sparsity=0.9, flags=QUANT_ALL, qrows=None, krows=None):
    """Straight-through backward of the cube-sparse fine stage: dQ at query
    rows ``qrows``, dK/dV at key rows ``krows`` (fp64 [B, H, R, D]), and the
    selection it used (int32 [B, H, n, topk], ascending)."""
    q, k, v, do = _u16(q), _u16(k), _u16(v), _u16(do)
    B, H, L, D = q.shape
    n = L // cube_tokens
    topk = vsa_topk(sparsity, n)
    qrows = (np.arange(L, dtype=np.int64) if qrows is None
             else np.ascontiguousarray(qrows, dtype=np.int64))
    krows = (np.arange(L, dtype=np.int64) if krows is None
             else np.ascontiguousarray(krows, dtype=np.int64))
    dq = np.empty((B, H, qrows.size, D))
    dk = np.empty((B, H, krows.size, D))
    dv = np.empty((B, H, krows.size, D))
    sel = np.empty((B, H, n, topk), np.int32)
    rc = _load().oracle_vsa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(do), B, H, L, D, cube_tokens, float(sparsity),
                                float(scale), int(flags), _ptr(qrows), qrows.size, _ptr(krows), krows.size,
                                _ptr(dq), _ptr(dk), _ptr(dv), _ptr(sel))
    if rc < 0:
        raise ValueError("oracle_vsa_bwd rejected the arguments")
    return {"dq": dq, "dk": dk, "dv": dv, "sel": sel, "topk": topk, "qrows": qrows, "krows": krows}


# ----------------------------------------------------------------------------
# bf16 helpers (bit-pattern conversions, no method arithmetic)
# ----------------------------------------------------------------------------

def bf16_bits_to_f32(x_u16: np.ndarray) -> np.ndarray:
    return (np.asarray(x_u16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16 bits (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


# ----------------------------------------------------------------------------
# NVFP4 QAD linear ("nvfp4_qad.py": nvfp4_gemm, _NVFP4STE, calibration)
# ----------------------------------------------------------------------------

def linear_fwd(x, w, bias=None, gx: float = 1.0) -> np.ndarray:
    """y = fq(x, gx) @ fq(w, 448*6/amax|w|)^T + bias, fp64 [M, N].  x: [M, K], w: [N, K],
    bias: [N] (bf16 bits); gx = 1.0 is the unit activation scale."""
    x, w = _u16(x), _u16(w)
    M, K = x.shape
    N = w.shape[0]
    b = None if bias is None else _u16(bias)
    y = np.empty((M, N))
    _load().oracle_linear_fwd(_ptr(x), _ptr(w), _ptr(b), M, N, K, float(gx), _ptr(y))
    return y


def linear_bwd(g, x, w):
    """Full-precision straight-through gradients: gx = g @ w, gw = g^T @ x, gb = sum_m g (fp64)."""
    g, x, w = _u16(g), _u16(x), _u16(w)
    M, N = g.shape
    K = x.shape[1]
    gx, gw, gb = np.empty((M, K)), np.empty((N, K)), np.empty(N)
    _load().oracle_linear_bwd(_ptr(g), _ptr(x), _ptr(w), M, N, K, _ptr(gx), _ptr(gw), _ptr(gb))
    return {"gx": gx, "gw": gw, "gb": gb}


def observe_amax(x, prev: float = 0.0) -> float:
    """max(prev, amax|x|): one calibrating forward's update of the observed maximum."""
    x = _u16(x)
    return _load().oracle_observe_amax(_ptr(x), x.size, float(prev))
