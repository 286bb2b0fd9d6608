"""MI355X (gfx950) NVFP4 fake-quantized attention (Attn-QAT).

The computation lives in ``libattnqat.so`` (hand-written HIP kernels behind the
C ABI of ``include/attnqat.h``); this package is a thin torch binding over it.
Importing the package loads the library and fails with ImportError when it is
missing: there is no fallback path.
"""
from ._lib import load as _load

_load()

from .ops import (AQ_FINAL_MAX, AQ_FLAGS_ALL, AQ_GSF_P, AQ_GSF_QKV, AQ_QUANT_ALL, AQ_QUANT_K,  # noqa: E402
                  AQ_QUANT_P, AQ_QUANT_Q, AQ_QUANT_V, AQ_PV_FP8, AQ_SMOOTH_K, AQ_SMOOTH_Q, AQ_TWO_LEVEL_P,
                  AttnQatTrainImpl, attn_qat_bwd, attn_qat_fwd, attn_qat_fwd_noalloc, attn_qat_train, fq_nvfp4,
                  static_global_scale, vsa_qat_bwd, vsa_qat_fwd, vsa_qat_train, vsa_topk, QADLinear,
                  input_global_sf, qad_linear, qad_linear_bwd, qad_linear_fwd, qad_observe_amax)

__all__ = ["AQ_QUANT_ALL", "AQ_QUANT_Q", "AQ_QUANT_K", "AQ_QUANT_V", "AQ_QUANT_P", "AQ_FINAL_MAX", "AQ_GSF_QKV",
           "AQ_GSF_P", "AQ_SMOOTH_K", "AQ_SMOOTH_Q", "AQ_TWO_LEVEL_P", "AQ_PV_FP8", "AQ_FLAGS_ALL", "fq_nvfp4",
           "static_global_scale", "attn_qat_fwd", "attn_qat_fwd_noalloc", "attn_qat_bwd", "attn_qat_train", "AttnQatTrainImpl",
           "vsa_qat_fwd", "vsa_qat_bwd", "vsa_qat_train", "vsa_topk", "qad_linear_fwd", "qad_linear_bwd",
           "qad_linear", "qad_observe_amax", "input_global_sf", "QADLinear"]
