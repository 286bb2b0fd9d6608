"""Thin torch binding over libattnqat.so.

PyTorch is used only to own device memory and to name the current HIP stream;
every step of the computation runs in the library's gfx950 kernels.  These
functions only validate tensor properties, compute strides and allocate the
outputs and the workspace.

Names follow the pages:
  * ``attn_qat_train(q_BLHD, k_BLHD, v_BLHD, is_causal=False, sm_scale=None)``
    and ``AttnQatTrainImpl`` mirror the "attn_qat_train" API reference page
    (attn_qat_train, AttnQatTrainImpl, AttnQatTrainBackend);
  * ``fq_nvfp4`` / ``static_global_scale`` follow "nvfp4_qad.py" (module
    docstring, weight_global_sf, input_global_sf);
  * ``vsa_qat_fwd`` follows the attention record of "vsqa-preview-1.3b
    metadata.json" (cube_shape, selection.effective_topk).
"""
from __future__ import annotations

import math
from typing import Optional

import torch

from . import _lib
from ._lib import (AQ_FINAL_MAX, AQ_FLAGS_ALL, AQ_GSF_P, AQ_GSF_QKV, AQ_QUANT_ALL, AQ_QUANT_K, AQ_QUANT_P,
                   AQ_QUANT_Q, AQ_QUANT_V, AQ_PV_FP8, AQ_SMOOTH_K, AQ_SMOOTH_Q, AQ_TWO_LEVEL_P, aq_strides, check,
                   load)

HEAD_SIZE = 128
CHUNK = 128


def _stream_ptr(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def _require_bf16_cuda(name: str, t: torch.Tensor):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be bfloat16, got {t.dtype}")


def _strides_blhd(t: torch.Tensor) -> aq_strides:
    """Strides of a [B, L, H, D] tensor as (b, h, l) with D contiguous."""
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("attention tensors must be 4-D [B, L, H, D] with a contiguous last dim")
    return aq_strides(t.stride(0), t.stride(2), t.stride(1))


def _workspace(op: int, B: int, H: int, lq: int, lk: int, device) -> torch.Tensor:
    nbytes = load().attn_qat_workspace_size(op, B, H, lq, lk)
    return torch.empty(nbytes + 256, dtype=torch.uint8, device=device)


def _aligned_ptr(ws: torch.Tensor) -> int:
    p = ws.data_ptr()
    return (p + 255) & ~255


# ----------------------------------------------------------------------------------------------
# Standalone fake quantization
# ----------------------------------------------------------------------------------------------

def static_global_scale(x: torch.Tensor) -> torch.Tensor:
    """g = 448*6 / max(amax|x|, 1e-12) as a 1-element fp32 device tensor."""
    _require_bf16_cuda("x", x)
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    g = torch.empty(1, dtype=torch.float32, device=x.device)
    check(load().fq_nvfp4_static_scale(x.data_ptr(), x.numel(), g.data_ptr(), _stream_ptr(x)),
          "fq_nvfp4_static_scale")
    return g


def fq_nvfp4(x: torch.Tensor, axis: int = -1, global_scale=None,
             out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """NVFP4 fake quantization of a contiguous bf16 tensor in 16-element blocks
    along ``axis``.  ``global_scale``: None (unit), "static" (computed from x),
    or a 1-element fp32 device tensor."""
    _require_bf16_cuda("x", x)
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    axis = axis % x.dim()
    outer = math.prod(x.shape[:axis])
    inner = math.prod(x.shape[axis + 1:])
    if out is None:
        out = torch.empty_like(x)
    elif out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous():
        raise ValueError("out must match x")
    g = None
    if isinstance(global_scale, str):
        if global_scale != "static":
            raise ValueError("global_scale must be None, 'static' or a tensor")
        global_scale = static_global_scale(x)
    if global_scale is not None:
        if global_scale.dtype != torch.float32 or global_scale.numel() != 1 or not global_scale.is_cuda:
            raise ValueError("global_scale must be a 1-element fp32 device tensor")
        g = global_scale.data_ptr()
    check(load().fq_nvfp4(x.data_ptr(), out.data_ptr(), outer, x.shape[axis], inner, g, _stream_ptr(x)),
          "fq_nvfp4")
    return out


# ----------------------------------------------------------------------------------------------
# Dense attention
# ----------------------------------------------------------------------------------------------

def _check_qkv(q, k, v):
    for n, t in (("q", q), ("k", k), ("v", v)):
        _require_bf16_cuda(n, t)
        if t.dim() != 4:
            raise ValueError(f"{n} must be [B, L, H, D]")
    B, Lq, H, D = q.shape
    if k.shape[0] != B or v.shape[0] != B:
        raise ValueError("batch sizes differ")
    if k.shape[1] != v.shape[1]:
        raise ValueError("key and value must have the same sequence length")
    if k.shape[2] != v.shape[2] or k.shape[3] != D or v.shape[3] != D:
        raise ValueError("k and v must be [B, Lk, Hkv, D] with q's D")
    return B, Lq, k.shape[1], H, k.shape[2], D


def _chunk_stats(quant_flags: int, shape, device) -> torch.Tensor:
    """The chunk-maximum array; under AQ_TWO_LEVEL_P with room after it for P's first-level
    scales (include/attnqat.h), returned as the view of its first half."""
    if quant_flags & AQ_TWO_LEVEL_P:
        return torch.empty(2, *shape, dtype=torch.float32, device=device)[0]
    return torch.empty(*shape, dtype=torch.float32, device=device)


def _aux_dict(quant_flags: int, lse, cmax, ohp) -> dict:
    aux = {"lse_log2": lse, "chunk_max_log2": cmax, "o_hp": ohp}
    if quant_flags & AQ_TWO_LEVEL_P:
        n = cmax.numel()
        aux["p_scale"] = torch.as_strided(cmax, cmax.shape, cmax.stride(), cmax.storage_offset() + n)
    return aux


def _check_aux(aux: dict, B: int, H: int, Lq: int, C: int, D: int, quant_flags: int) -> None:
    """The forward's auxiliary outputs, as the backward reads them: contiguous fp32 device tensors
    lse_log2 [B, H, Lq], chunk_max_log2 [B, H, C, Lq] (C = key chunks, or selected cubes) and
    o_hp [B, H, Lq, D].  Any other shape would make the kernels read past the buffers."""
    want = {"lse_log2": (B, H, Lq), "chunk_max_log2": (B, H, C, Lq), "o_hp": (B, H, Lq, D)}
    for name, shape in want.items():
        t = aux.get(name)
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"aux[{name!r}] must be a contiguous fp32 device tensor")
        if tuple(t.shape) != shape:
            raise ValueError(f"aux[{name!r}] has shape {tuple(t.shape)}, expected {shape} "
                             "(pass the aux of the forward call with the same arguments)")
    _check_chunk_stats(quant_flags, aux["chunk_max_log2"])


def _check_chunk_stats(quant_flags: int, cmax: torch.Tensor) -> None:
    if quant_flags & AQ_TWO_LEVEL_P:
        need = (cmax.storage_offset() + 2 * cmax.numel()) * 4
        if cmax.untyped_storage().nbytes() < need:
            raise ValueError("under AQ_TWO_LEVEL_P aux['chunk_max_log2'] must be followed in its storage "
                             "by the first-level P scales the forward wrote (pass the forward's aux)")


def attn_qat_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                 sm_scale: Optional[float] = None, quant_flags: int = AQ_QUANT_ALL,
                 training: bool = False):
    """Fake-quant attention forward on [B, L, H, D] bf16 tensors.

    Returns o [B, Lq, H, D] bf16; with ``training`` also a dict holding the
    auxiliary outputs the backward needs: lse_log2 [B, H, Lq], chunk_max_log2
    [B, H, ceil(Lk/128), Lq] and o_hp [B, H, Lq, D] (fp32); under AQ_TWO_LEVEL_P also p_scale,
    P's first-level scale per (row, chunk), which lives right after chunk_max_log2 in one buffer."""
    B, Lq, Lk, H, Hkv, D = _check_qkv(q, k, v)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)  # the pages' default (attn_qat_train)
    o = torch.empty(B, Lq, H, D, dtype=torch.bfloat16, device=q.device)
    lse = cmax = ohp = None
    if training:
        C = (Lk + CHUNK - 1) // CHUNK
        lse = torch.empty(B, H, Lq, dtype=torch.float32, device=q.device)
        cmax = _chunk_stats(quant_flags, (B, H, C, Lq), q.device)
        ohp = torch.empty(B, H, Lq, D, dtype=torch.float32, device=q.device)
    ws = _workspace(0, B, H, Lq, Lk, q.device) if D == HEAD_SIZE and Hkv == H else torch.empty(
        256, dtype=torch.uint8, device=q.device)
    p = lambda t: None if t is None else t.data_ptr()
    check(load().attn_qat_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B, H, Hkv, D, Lq,
                              Lk, _strides_blhd(q), _strides_blhd(k), _strides_blhd(v), _strides_blhd(o),
                              float(sm_scale), int(bool(causal)), int(quant_flags), p(lse), p(cmax),
                              p(ohp), _aligned_ptr(ws), ws.numel() - 256, _stream_ptr(q)),
          "attn_qat_fwd")
    if training:
        return o, _aux_dict(quant_flags, lse, cmax, ohp)
    return o


def attn_qat_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                         sm_scale: Optional[float] = None, quant_flags: int = AQ_QUANT_ALL,
                         training: bool = False, out: Optional[torch.Tensor] = None, aux: Optional[dict] = None):
    """attn_qat_fwd through attn_qat_fwd_noalloc: the library uses its fixed device scratch instead
    of a workspace, so a call with ``out`` (and, with ``training``, ``aux``) given allocates
    nothing.  Returns what attn_qat_fwd returns."""
    B, Lq, Lk, H, Hkv, D = _check_qkv(q, k, v)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    o = out if out is not None else torch.empty(B, Lq, H, D, dtype=torch.bfloat16, device=q.device)
    _require_bf16_cuda("out", o)
    if tuple(o.shape) != (B, Lq, H, D):
        raise ValueError(f"out must be [B, Lq, H, D] = {(B, Lq, H, D)}")
    lse = cmax = ohp = None
    if training:
        C = (Lk + CHUNK - 1) // CHUNK
        if aux is None:
            lse = torch.empty(B, H, Lq, dtype=torch.float32, device=q.device)
            cmax = _chunk_stats(quant_flags, (B, H, C, Lq), q.device)
            ohp = torch.empty(B, H, Lq, D, dtype=torch.float32, device=q.device)
            aux = _aux_dict(quant_flags, lse, cmax, ohp)
        _check_aux(aux, B, H, Lq, C, D, quant_flags)
        lse, cmax, ohp = aux["lse_log2"], aux["chunk_max_log2"], aux["o_hp"]
    p = lambda t: None if t is None else t.data_ptr()
    check(load().attn_qat_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B, H, Hkv, D, Lq,
                                      Lk, _strides_blhd(q), _strides_blhd(k), _strides_blhd(v), _strides_blhd(o),
                                      float(sm_scale), int(bool(causal)), int(quant_flags), p(lse), p(cmax),
                                      p(ohp), _stream_ptr(q)),
          "attn_qat_fwd_noalloc")
    if training:
        return o, aux
    return o


def attn_qat_bwd(q, k, v, aux, d_o, causal: bool = False, sm_scale: Optional[float] = None,
                 quant_flags: int = AQ_QUANT_ALL):
    """Straight-through backward.  ``aux`` is the dict returned by
    ``attn_qat_fwd(..., training=True)``.  Returns dq, dk, dv [B, L, H, D] bf16."""
    B, Lq, Lk, H, Hkv, D = _check_qkv(q, k, v)
    _require_bf16_cuda("d_o", d_o)
    if d_o.shape != q.shape:
        raise ValueError("d_o must have q's shape")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    dq = torch.empty_like(q, memory_format=torch.contiguous_format)
    dk = torch.empty_like(k, memory_format=torch.contiguous_format)
    dv = torch.empty_like(v, memory_format=torch.contiguous_format)
    ws = _workspace(1, B, H, Lq, Lk, q.device) if D == HEAD_SIZE and Hkv == H else torch.empty(
        256, dtype=torch.uint8, device=q.device)
    _check_aux(aux, B, H, Lq, (Lk + CHUNK - 1) // CHUNK, D, quant_flags)
    check(load().attn_qat_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), aux["o_hp"].data_ptr(),
                              d_o.data_ptr(), aux["lse_log2"].data_ptr(), aux["chunk_max_log2"].data_ptr(),
                              dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Hkv, D, Lq, Lk,
                              _strides_blhd(q), _strides_blhd(k), _strides_blhd(v), _strides_blhd(d_o),
                              _strides_blhd(dq), _strides_blhd(dk), _strides_blhd(dv), float(sm_scale),
                              int(bool(causal)), int(quant_flags), _aligned_ptr(ws), ws.numel() - 256,
                              _stream_ptr(q)),
          "attn_qat_bwd")
    return dq, dk, dv


class _AttnQatTrain(torch.autograd.Function):
    """Forward = fake-quant attention; backward = the consistent straight-through
    estimator of the library (fake-quant Jacobians are the identity)."""

    @staticmethod
    def forward(ctx, q, k, v, is_causal, sm_scale, quant_flags):
        o, aux = attn_qat_fwd(q, k, v, causal=is_causal, sm_scale=sm_scale, quant_flags=quant_flags, training=True)
        ctx.save_for_backward(q, k, v, aux["lse_log2"], aux["chunk_max_log2"], aux["o_hp"])
        ctx.is_causal, ctx.sm_scale, ctx.quant_flags = is_causal, sm_scale, quant_flags
        return o

    @staticmethod
    def backward(ctx, d_o):
        q, k, v, lse, cmax, ohp = ctx.saved_tensors
        aux = {"lse_log2": lse, "chunk_max_log2": cmax, "o_hp": ohp}
        dq, dk, dv = attn_qat_bwd(q, k, v, aux, d_o.contiguous(), causal=ctx.is_causal,
                                  sm_scale=ctx.sm_scale, quant_flags=ctx.quant_flags)
        return dq, dk, dv, None, None, None


def attn_qat_train(q_BLHD: torch.Tensor, k_BLHD: torch.Tensor, v_BLHD: torch.Tensor,
                   is_causal: bool = False, sm_scale: Optional[float] = None,
                   quant_flags: int = AQ_QUANT_ALL) -> torch.Tensor:
    """Fake-quant attention with the straight-through backward, [B, L, H, D] in and out
    ("attn_qat_train" page: attn_qat_train; the kernel reads the strided BLHD tensors
    directly, so no permuted copies are made).  quant_flags: quantizers and variants
    (AQ_* constants); the page's call is AQ_QUANT_ALL."""
    return _AttnQatTrain.apply(q_BLHD, k_BLHD, v_BLHD, bool(is_causal), sm_scale, int(quant_flags))


class AttnQatTrainImpl:
    """Mirror of the pages' AttnQatTrainImpl: refuses dropout, forwards to attn_qat_train."""

    def __init__(self, num_heads: int, head_size: int, causal: bool, softmax_scale: float,
                 num_kv_heads: Optional[int] = None, prefix: str = "", **extra_impl_args) -> None:
        if head_size != HEAD_SIZE:
            raise ValueError(f"head_size {head_size} is not supported (supported: [128])")
        self.num_heads = num_heads
        self.num_kv_heads = num_heads if num_kv_heads is None else num_kv_heads
        self.causal = causal
        self.softmax_scale = softmax_scale
        dropout_p = extra_impl_args.get("dropout_p", 0.0)
        if dropout_p > 0:
            raise NotImplementedError(f"attn_qat_train does not support dropout (got dropout_p={dropout_p})")

    def forward(self, query, key, value, attn_metadata=None):
        return attn_qat_train(query, key, value, is_causal=self.causal, sm_scale=self.softmax_scale)


# ----------------------------------------------------------------------------------------------
# Cube-sparse attention
# ----------------------------------------------------------------------------------------------

def vsa_topk(sparsity: float, n_cubes: int) -> int:
    return load().vsa_topk(float(sparsity), int(n_cubes))


def vsa_qat_fwd(q, k, v, grid=(16, 28, 56), cube=(4, 4, 8), sparsity: float = 0.9,
                sm_scale: Optional[float] = None, quant_flags: int = AQ_QUANT_ALL,
                coarse: bool = False, return_sel: bool = False, training: bool = False):
    """Cube-sparse fake-quant forward on cube-major [B, L, H, D] bf16 tensors.
    Returns o_fine (and o_coarse, sel when requested).  With ``training`` the
    return value is (o_fine, aux), aux holding the selection and the fine
    stage's statistics for ``vsa_qat_bwd`` (sel, lse_log2, chunk_max_log2,
    o_hp), and o_coarse when requested."""
    B, L, Lk, H, Hkv, D = _check_qkv(q, k, v)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    n = L // max(1, cube[0] * cube[1] * cube[2])
    topk = vsa_topk(sparsity, n) if n > 0 else 0
    o = torch.empty(B, L, H, D, dtype=torch.bfloat16, device=q.device)
    oc = torch.empty_like(o) if coarse else None
    want_sel = return_sel or training
    sel = torch.empty(B, H, n, max(topk, 1), dtype=torch.int32, device=q.device) if want_sel else None
    lse = cmax = ohp = None
    if training:
        lse = torch.empty(B, H, L, dtype=torch.float32, device=q.device)
        cmax = _chunk_stats(quant_flags, (B, H, max(topk, 1), L), q.device)
        ohp = torch.empty(B, H, L, D, dtype=torch.float32, device=q.device)
    ws = _workspace(2, B, H, L, L, q.device) if D == HEAD_SIZE and L > 0 else torch.empty(
        256, dtype=torch.uint8, device=q.device)
    p = lambda t: None if t is None else t.data_ptr()
    check(load().vsa_qat_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), p(oc), p(sel), B, H, D,
                             L, grid[0], grid[1], grid[2], cube[0], cube[1], cube[2], float(sparsity),
                             _strides_blhd(q), _strides_blhd(k), _strides_blhd(v), _strides_blhd(o),
                             float(sm_scale), int(quant_flags), p(lse), p(cmax), p(ohp), _aligned_ptr(ws),
                             ws.numel() - 256, _stream_ptr(q)),
          "vsa_qat_fwd")
    if training:
        aux = {"sel": sel, **_aux_dict(quant_flags, lse, cmax, ohp)}
        if coarse:
            aux["o_coarse"] = oc
        return o, aux
    out = [o]
    if coarse:
        out.append(oc)
    if return_sel:
        out.append(sel)
    return out[0] if len(out) == 1 else tuple(out)


def vsa_qat_bwd(q, k, v, aux, d_o, grid=(16, 28, 56), cube=(4, 4, 8), sparsity: float = 0.9,
                sm_scale: Optional[float] = None, quant_flags: int = AQ_QUANT_ALL):
    """Straight-through backward of the cube-sparse fine stage.  ``aux`` is the
    dict returned by ``vsa_qat_fwd(..., training=True)`` with the same
    arguments.  Returns dq, dk, dv [B, L, H, D] bf16."""
    B, L, Lk, H, Hkv, D = _check_qkv(q, k, v)
    _require_bf16_cuda("d_o", d_o)
    if d_o.shape != q.shape:
        raise ValueError("d_o must have q's shape")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    n = L // max(1, cube[0] * cube[1] * cube[2])
    topk = vsa_topk(sparsity, n) if n > 0 else 0
    sel = aux.get("sel")
    if not isinstance(sel, torch.Tensor) or sel.dtype != torch.int32 or not sel.is_contiguous() or not sel.is_cuda:
        raise ValueError("aux['sel'] must be a contiguous int32 device tensor")
    if tuple(sel.shape) != (B, H, n, topk):
        raise ValueError(f"aux['sel'] has shape {tuple(sel.shape)}, expected {(B, H, n, topk)} for "
                         f"{n} cubes at sparsity {sparsity} (pass the forward's aux and sparsity)")
    _check_aux(aux, B, H, L, topk, D, quant_flags)
    dq = torch.empty_like(q, memory_format=torch.contiguous_format)
    dk = torch.empty_like(k, memory_format=torch.contiguous_format)
    dv = torch.empty_like(v, memory_format=torch.contiguous_format)
    ws = _workspace(3, B, H, L, L, q.device) if D == HEAD_SIZE and L > 0 else torch.empty(
        256, dtype=torch.uint8, device=q.device)
    check(load().vsa_qat_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), aux["o_hp"].data_ptr(), d_o.data_ptr(),
                             aux["lse_log2"].data_ptr(), aux["chunk_max_log2"].data_ptr(), sel.data_ptr(),
                             dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, D, L, grid[0], grid[1], grid[2],
                             cube[0], cube[1], cube[2], float(sparsity), _strides_blhd(q), _strides_blhd(k),
                             _strides_blhd(v), _strides_blhd(d_o), _strides_blhd(dq), _strides_blhd(dk),
                             _strides_blhd(dv), float(sm_scale), int(quant_flags), _aligned_ptr(ws),
                             ws.numel() - 256, _stream_ptr(q)),
          "vsa_qat_bwd")
    return dq, dk, dv


class _VsaQatTrain(torch.autograd.Function):
    """Forward = the cube-sparse fine stage; backward = its straight-through
    estimator (vsa_qat_bwd)."""

    @staticmethod
    def forward(ctx, q, k, v, grid, cube, sparsity, sm_scale, quant_flags):
        o, aux = vsa_qat_fwd(q, k, v, grid=grid, cube=cube, sparsity=sparsity, sm_scale=sm_scale,
                             quant_flags=quant_flags, training=True)
        ctx.save_for_backward(q, k, v, aux["sel"], aux["lse_log2"], aux["chunk_max_log2"], aux["o_hp"])
        ctx.args = (grid, cube, sparsity, sm_scale, quant_flags)
        return o

    @staticmethod
    def backward(ctx, d_o):
        q, k, v, sel, lse, cmax, ohp = ctx.saved_tensors
        grid, cube, sparsity, sm_scale, quant_flags = ctx.args
        aux = {"sel": sel, "lse_log2": lse, "chunk_max_log2": cmax, "o_hp": ohp}
        dq, dk, dv = vsa_qat_bwd(q, k, v, aux, d_o.contiguous(), grid=grid, cube=cube, sparsity=sparsity,
                                 sm_scale=sm_scale, quant_flags=quant_flags)
        return dq, dk, dv, None, None, None, None, None


def vsa_qat_train(q_BLHD: torch.Tensor, k_BLHD: torch.Tensor, v_BLHD: torch.Tensor, grid=(16, 28, 56),
                  cube=(4, 4, 8), sparsity: float = 0.9, sm_scale: Optional[float] = None,
                  quant_flags: int = AQ_QUANT_ALL) -> torch.Tensor:
    """Cube-sparse fine stage with the straight-through backward, cube-major [B, L, H, D] in and out."""
    return _VsaQatTrain.apply(q_BLHD, k_BLHD, v_BLHD, tuple(grid), tuple(cube), float(sparsity), sm_scale,
                              int(quant_flags))


# ----------------------------------------------------------------------------------------------
# NVFP4 QAD linear ("nvfp4_qad.py": nvfp4_gemm, _NVFP4STE, NVFP4QADLinearMethod)
# ----------------------------------------------------------------------------------------------

FP4_RANGE = 448.0 * 6.0


def _linear_ws(op: int, m: int, n: int, k: int, device) -> torch.Tensor:
    return torch.empty(load().qad_linear_workspace_size(op, m, n, k), dtype=torch.uint8, device=device)


def _rows(x: torch.Tensor, k: int) -> torch.Tensor:
    if x.shape[-1] != k:
        raise ValueError(f"last dimension {x.shape[-1]} != in_features {k}")
    return x.reshape(-1, k).contiguous()


def input_global_sf(amax: torch.Tensor) -> torch.Tensor:
    """The static activation scale (input_global_sf) of a calibrated maximum, formed by the library
    (qad_input_global_sf): ``amax`` and the result are one-element fp32 device tensors."""
    if not isinstance(amax, torch.Tensor) or amax.dtype != torch.float32 or not amax.is_cuda or amax.numel() != 1:
        raise ValueError("amax must be a one-element fp32 device tensor")
    g = torch.empty(1, dtype=torch.float32, device=amax.device)
    check(load().qad_input_global_sf(amax.data_ptr(), g.data_ptr(), _stream_ptr(amax)), "qad_input_global_sf")
    return g


def qad_linear_fwd(x: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor] = None,
                   input_sf: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = fq(x, input_sf) fq(weight, 448*6/amax|weight|)^T + bias (nvfp4_gemm on the fake-quant +
    BF16 MFMA path).  x [..., k], weight [n, k], bias [n]: bf16 on the device; input_sf: device fp32
    scalar (static scale) or None (unit scale)."""
    for name, t in (("x", x), ("weight", weight)):
        _require_bf16_cuda(name, t)
    n, k = weight.shape
    x2 = _rows(x, k)
    w = weight.contiguous()
    b = None
    if bias is not None:
        _require_bf16_cuda("bias", bias)
        b = bias.contiguous()
    if input_sf is not None and (input_sf.dtype != torch.float32 or not input_sf.is_cuda or input_sf.numel() != 1):
        raise ValueError("input_sf must be a one-element fp32 device tensor")
    m = x2.shape[0]
    y = torch.empty(m, n, dtype=torch.bfloat16, device=x.device)
    ws = _linear_ws(0, m, n, k, x.device)
    check(load().qad_linear_fwd(x2.data_ptr(), w.data_ptr(), None if b is None else b.data_ptr(), y.data_ptr(), m,
                                n, k, None if input_sf is None else input_sf.data_ptr(), ws.data_ptr(), ws.numel(),
                                _stream_ptr(x)), "qad_linear_fwd")
    return y.view(*x.shape[:-1], n)


def qad_linear_bwd(grad_y: torch.Tensor, x: torch.Tensor, weight: torch.Tensor, need_bias: bool = True):
    """Full-precision straight-through gradients (_NVFP4STE.backward): grad_x = grad_y W,
    grad_w = grad_y^T x, grad_b = column sums of grad_y."""
    n, k = weight.shape
    g2 = grad_y.reshape(-1, n).contiguous()
    x2 = _rows(x, k)
    m = x2.shape[0]
    gx = torch.empty(m, k, dtype=torch.bfloat16, device=x.device)
    gw = torch.empty(n, k, dtype=torch.bfloat16, device=x.device)
    gb = torch.empty(n, dtype=torch.bfloat16, device=x.device) if need_bias else None
    ws = _linear_ws(1, m, n, k, x.device)
    check(load().qad_linear_bwd(g2.data_ptr(), x2.data_ptr(), weight.contiguous().data_ptr(), gx.data_ptr(),
                                gw.data_ptr(), None if gb is None else gb.data_ptr(), m, n, k, ws.data_ptr(),
                                ws.numel(), _stream_ptr(x)), "qad_linear_bwd")
    return gx.view(x.shape), gw, gb


class _QadLinearSTE(torch.autograd.Function):
    """Forward = the NVFP4 linear; backward = full-precision linear gradients (straight-through)."""

    @staticmethod
    def forward(ctx, x, weight, bias, input_sf):
        ctx.save_for_backward(x, weight)
        ctx.has_bias = bias is not None
        return qad_linear_fwd(x, weight, bias, input_sf)

    @staticmethod
    def backward(ctx, grad_y):
        x, weight = ctx.saved_tensors
        gx, gw, gb = qad_linear_bwd(grad_y, x, weight, need_bias=ctx.has_bias)
        return gx, gw, gb, None


def qad_linear(x: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor] = None,
               input_sf: Optional[torch.Tensor] = None) -> torch.Tensor:
    """NVFP4 QAD linear with the straight-through backward when gradients are needed."""
    if torch.is_grad_enabled() and (x.requires_grad or weight.requires_grad):
        return _QadLinearSTE.apply(x, weight, bias, input_sf)
    return qad_linear_fwd(x, weight, bias, input_sf)


def qad_observe_amax(x: torch.Tensor, amax: torch.Tensor) -> torch.Tensor:
    """Max calibration: amax (one-element fp32 device tensor) = max(amax, max|x|), in place."""
    _require_bf16_cuda("x", x)
    if amax.dtype != torch.float32 or not amax.is_cuda or amax.numel() != 1:
        raise ValueError("amax must be a one-element fp32 device tensor")
    xc = x.contiguous()
    check(load().qad_observe_amax(xc.data_ptr(), xc.numel(), amax.data_ptr(), _stream_ptr(x)), "qad_observe_amax")
    return amax


class QADLinear:
    """An NVFP4 QAD linear layer (NVFP4QADLinearMethod): act_scale "unit" (attention projections,
    gates) or "static" (FFN linears, 448*6 / calibrated amax).  Inside calibrating() the dense
    linear runs and every input's abs-max is folded into the observed maximum; enabled = False
    runs the dense linear."""

    def __init__(self, weight: torch.Tensor, bias: Optional[torch.Tensor] = None, act_scale: str = "unit"):
        if act_scale not in ("unit", "static"):
            raise ValueError(f"act_scale must be 'unit' or 'static', got {act_scale!r}")
        self.weight, self.bias, self.act_scale = weight, bias, act_scale
        self.enabled, self.calibrating = True, False
        self.observed_amax = torch.zeros(1, dtype=torch.float32, device=weight.device)
        self.input_amax: Optional[float] = None
        self.input_sf: Optional[torch.Tensor] = None

    def set_input_amax(self, amax: float) -> None:
        """Fix the activation's calibrated maximum; the static scale is formed on the device."""
        if not amax > 0:
            raise ValueError(f"calibrated amax must be positive, got {amax}")
        self.input_amax = float(amax)
        dev_amax = torch.tensor([self.input_amax], dtype=torch.float32).to(self.weight.device)
        self.input_sf = input_global_sf(dev_amax)

    def finish_calibration(self) -> None:
        self.calibrating = False
        amax = float(self.observed_amax.item())
        if not amax > 0:
            raise ValueError(f"calibrated amax must be positive, got {amax}")
        self.input_amax = amax
        self.input_sf = input_global_sf(self.observed_amax)

    def __call__(self, x: torch.Tensor) -> torch.Tensor:
        if self.calibrating:
            qad_observe_amax(x, self.observed_amax)
            return torch.nn.functional.linear(x, self.weight, self.bias)
        if not self.enabled:
            return torch.nn.functional.linear(x, self.weight, self.bias)
        sf = None
        if self.act_scale == "static":
            if self.input_sf is None:
                raise RuntimeError("static activation scale used before calibration")
            sf = self.input_sf
        return qad_linear(x, self.weight, self.bias, sf)


__all__ = ["AQ_QUANT_ALL", "AQ_QUANT_Q", "AQ_QUANT_K", "AQ_QUANT_V", "AQ_QUANT_P", "AQ_FINAL_MAX", "AQ_GSF_QKV",
           "AQ_GSF_P", "AQ_SMOOTH_K", "AQ_SMOOTH_Q", "AQ_TWO_LEVEL_P", "AQ_PV_FP8", "AQ_FLAGS_ALL", "fq_nvfp4",
           "static_global_scale", "attn_qat_fwd", "attn_qat_fwd_noalloc", "attn_qat_bwd", "attn_qat_train", "AttnQatTrainImpl",
           "vsa_qat_fwd", "vsa_qat_bwd", "vsa_qat_train", "vsa_topk", "qad_linear_fwd", "qad_linear_bwd",
           "qad_linear", "qad_observe_amax", "input_global_sf", "QADLinear"]
