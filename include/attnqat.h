/*
 * attnqat.h - C ABI of the MI355X (gfx950) NVFP4 fake-quantized attention library.
 *
 * The operations follow these web pages (cited by title and section):
 *   [API]  "attn_qat_train" API reference page (fastvideo.attention.backends.attn_qat_train):
 *          attn_qat_train(q_BLHD, k_BLHD, v_BLHD, is_causal, sm_scale), its fixed kernel flags
 *          (use_qat_qkv_backward, fake_quant_p_bwd, use_high_prec_o, unit global scales),
 *          AttnQatTrainBackend.get_supported_head_sizes() == [128], AttnQatTrainImpl (dropout
 *          refused), AttentionImpl(num_heads, head_size, softmax_scale, causal, num_kv_heads).
 *   [DOC]  "Attn-QAT Training" guide: "Prerequisites" (fail instead of falling back to dense
 *          attention), "Architecture-specific Triton routing" (query and key/value lengths may
 *          differ; key and value lengths must match).
 *   [QAD]  "nvfp4_qad.py" source page: module docstring (per-16 E4M3 block scales under a unit or
 *          static global scale), FP4_RANGE = 448*6, weight_global_sf / input_global_sf.
 *   [META] "vsqa-preview-1.3b metadata.json": attention.precision (NVFP4 fake-quant with BF16
 *          matmul; quant_p, quant_v; coarse BF16, quantize_coarse false), attention.selection
 *          (effective_topk formula), attention.cube_shape [4,4,8]; the dense parent's precision
 *          record (group_size 16, E2M1 values, FP8 E4M3FN scales, backward "consistent STE with
 *          auxiliary output").
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE memory owned by the caller.  The library never allocates or
 *     frees memory and keeps no pointer after the call returns.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream).  No call
 *     synchronises the host; results are ready when the stream reaches them.
 *   - bf16 tensors are IEEE bfloat16 bit patterns; fp32 tensors are IEEE binary32.
 *   - Attention tensors are 4-D with a contiguous head dimension D = 128.  Their layout is given
 *     by element strides {b, h, l} (batch, head, token), so both the pages' public [B, L, H, D]
 *     layout and the kernel-side [B, H, L, D] layout are accepted without copies.
 *   - Return value: AQ_OK (0) on success, a negative code on failure.  On failure nothing has
 *     been enqueued and aq_last_error() returns a message (thread-local, valid until the next
 *     call on the same thread).  Argument checks run on the host before any launch.
 *   - Calls that overlap on one stream are ordered by the stream; the library holds no state
 *     between calls, so calls on different streams are independent when their buffers are.
 */
#ifndef ATTNQAT_H
#define ATTNQAT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    AQ_OK = 0,
    AQ_EINVAL = -1,  /* malformed argument: null pointer, size, stride, scale, flag, workspace */
    AQ_ENOTSUP = -2, /* well-formed but outside what the kernels implement */
    AQ_EHIP = -3     /* a HIP launch failed */
};

/* Which operands are fake-quantized ([API] is_qat with unit global scales; [META] quant_p,
   quant_v).  AQ_QUANT_ALL is the pages' configuration. */
enum {
    AQ_QUANT_Q = 1, /* Q in 16-element blocks along D */
    AQ_QUANT_K = 2, /* K in 16-element blocks along D */
    AQ_QUANT_V = 4, /* V in 16-element blocks along the key axis */
    AQ_QUANT_P = 8, /* softmax probabilities in 16-key blocks along the key axis */
    AQ_QUANT_ALL = 15
};

/* Variants, OR-ed into the same flags word.  [API] lists the kernel flags use_global_sf_qkv,
   use_global_sf_p, smooth_k, smooth_q and two_level_quant_p_sage3 (all off in attn_qat_train) and
   [META]'s precision records carry the first three; [DOC]'s environment table names reference-order softmax statistics
   (FASTVIDEO_ATTN_QAT_FWD_EXACT_M).  None is defined on the pages; the readings implemented:
     AQ_FINAL_MAX  every P relative to its row's final maximum over all keys (the selected keys for
                   vsa_qat_fwd) instead of the running maximum of 128-key chunks; the forward
                   first runs a row-maximum pass (+50% QK^T work).  The training outputs then hold
                   that maximum in every chunk-maximum row, which the backward uses unchanged.
     AQ_GSF_QKV    static global scale per tensor for Q, K, V: g = 448*6 / max(amax, 1e-12) over
                   the whole tensor (["nvfp4_qad.py"] input_global_sf), computed on the device
                   for every call; the dequantized values are rounded to bf16.
     AQ_GSF_P      static global scale of P's blocks, g = 448*6 (P's largest value is 1).
     AQ_SMOOTH_K   the keys' per-channel mean over the sequence (fp64 sum / L, rounded to fp32)
                   subtracted before quantization; the softmax of a row ignores the shift and the
                   gradient passes to K unchanged.
     AQ_TWO_LEVEL_P  two-level P, SageAttention3's recipe: per row and 128-key chunk (selected cube
                   for vsa_qat_fwd) a first level g = 448*6 / (the row's largest P in the chunk;
                   448*6 when it is 0) serves as the global scale of P's 16-key blocks, quantized as
                   under a static scale.  Training calls then pass a chunk_max_log2 array of TWICE
                   the size: its second half, laid out like the first, receives g of every
                   (row, chunk), which the backward reads.  Not combinable with AQ_FINAL_MAX or
                   AQ_GSF_P (AQ_ENOTSUP).
     AQ_SMOOTH_Q   SageAttention2's smoothing of Q: the queries' per-channel mean over the sequence
                   (the AQ_SMOOTH_K reading) is subtracted before quantization and its share of the
                   logits, delta_j = <mean, k-hat_j> (fp32), is added back to every logit of key j.
                   The backward's key gradients see the restored query q-hat + mean; dQ is
                   unchanged.  Under AQ_GSF_QKV the static Q scale is taken on the smoothed Q.
     AQ_PV_FP8     the FP8 P.V product ([META]'s precision records carry pv_fp8, undefined there):
                   both operands of the P-hat V-hat product, as the bf16 path forms them, rounded
                   to the nearest FP8 E4M3FN value (ties to even, subnormals kept, saturating at
                   448, sign kept), then multiplied with fp32 accumulation; P's blocks are
                   quantized under a global scale of 1 (448*6 with AQ_GSF_P, the two-level scale
                   with AQ_TWO_LEVEL_P), which is the plain block scale.  The backward uses the
                   same operands: dP against the rounded V-hat, dV from the rounded P-hat, O^hp
                   from the rounded V-hat.  Requires AQ_QUANT_P (else AQ_ENOTSUP).  The forward
                   multiplies these operands on the fp16 MFMA (every E4M3FN value is exact in fp16,
                   so the products are the FP8 ones), which also carries O^hp's unquantized P.
   Otherwise, under AQ_GSF_QKV, AQ_GSF_P or AQ_TWO_LEVEL_P the P-hat V-hat product runs in bf16 (the
   values are no longer exact in fp16). */
enum {
    AQ_FINAL_MAX = 16,
    AQ_GSF_QKV = 32,
    AQ_GSF_P = 64,
    AQ_SMOOTH_K = 128,
    AQ_TWO_LEVEL_P = 256,
    AQ_SMOOTH_Q = 512,
    AQ_PV_FP8 = 1024,
    AQ_FLAGS_ALL = 2047
};

/* Element strides of a 4-D attention tensor, indexed (batch, head, token, d) with d contiguous. */
typedef struct {
    int64_t b, h, l;
} aq_strides;

/* Message describing the most recent failure on this thread ("" if none). */
const char *aq_last_error(void);

/* ---------------------------------------------------------------------------------------------
 * fq_nvfp4 - standalone NVFP4 fake quantization ([QAD] module docstring; [META] group_size 16,
 * E2M1 values, FP8 E4M3FN block scales).
 *
 * x, y   : bf16 tensors viewed as [outer, axis_len, inner], row-major and contiguous; y may equal
 *          x (in place).  Blocks are 16 consecutive positions along `axis`; the last block of an
 *          axis whose length is not a multiple of 16 is shorter.
 * global_scale : NULL for the unit global scale g = 1 (the attention setting), or a DEVICE
 *          pointer to one fp32 g (for instance from fq_nvfp4_static_scale).
 * Per block with abs-max a: s = E4M3(fp32(fp32(a/6)*g)) (round to nearest, ties to even,
 * saturating at 448, subnormals kept), S = fp32(s/g); each element becomes
 * bf16(sign(x) * E2M1(fp32(|x|/S)) * S), E2M1 rounding to nearest with ties to the even code and
 * saturating at 6; a block whose S is 0 becomes signed zeros.
 * Errors: AQ_EINVAL for null x/y or non-positive sizes.
 * ------------------------------------------------------------------------------------------- */
int fq_nvfp4(const void *x, void *y, int64_t outer, int64_t axis_len, int64_t inner,
             const float *global_scale, void *stream);

/* Static global scale ([QAD] weight_global_sf and input_global_sf):
 * *g_out = fp32(448*6 / max(a, 1e-12)) with a = max |x| over the n bf16 elements of x (NaN read
 * as 0).  g_out is a DEVICE pointer to one fp32.  Errors: AQ_EINVAL for null pointers or n <= 0. */
int fq_nvfp4_static_scale(const void *x, int64_t n, float *g_out, void *stream);

/* ---------------------------------------------------------------------------------------------
 * attn_qat_fwd - fake-quantized attention forward ([API] attn_qat_train; [META] "NVFP4
 * fake-quant with BF16 matmul").
 *
 * q [B, H, lq, 128], k and v [B, H, lk, 128], o [B, H, lq, 128]: bf16, layout by strides.
 * Every bf16 tensor of the attention entry points starts 16-byte aligned and has strides that
 * are multiples of 8 elements and below 2^24 (rows move in 16-byte pieces); lq, lk <= 2^30.
 * Q-hat, K-hat along D and V-hat along keys are fake-quantized per quant_flags (quantizers and
 * the AQ_FINAL_MAX / AQ_GSF_QKV / AQ_GSF_P / AQ_SMOOTH_K / AQ_TWO_LEVEL_P / AQ_SMOOTH_Q / AQ_PV_FP8 variants above).  The keys are
 * visited in chunks of 128 ([0,128), [128,256), ...); in chunk c the running row maximum m_c of
 * the logits softmax_scale * <q-hat, k-hat> is refreshed first, then P = exp(logit - m_c) is
 * formed, fake-quantized in 16-key blocks (AQ_QUANT_P) and multiplied with V-hat on BF16 MFMA;
 * the denominator sums the unquantized P.  o = acc / l rounded to bf16.
 * softmax_scale : finite and > 0 ([API] default 1/sqrt(D) is applied by the caller).
 * causal        : top-left causal mask; requires lq == lk.
 * Optional training outputs (all three or none; attn_qat_bwd needs all three):
 *   lse_log2       [B, H, lq] fp32 contiguous: log2 of the softmax denominator in base-2 logit
 *                  units, i.e. log2(e) * (m + ln l) with m the final row maximum.
 *   chunk_max_log2 [B, H, ceil(lk/128), lq] fp32 contiguous: log2(e) * m_c after each chunk
 *                  (under AQ_TWO_LEVEL_P twice that: then [2, B, H, ceil(lk/128), lq], the second
 *                  half P's first-level scale of each chunk)
 *                  (entries of chunks a causal row never reaches are left unwritten).
 *   o_hp           [B, H, lq, 128] fp32 contiguous: the auxiliary high-precision output with
 *                  unquantized P ([API] use_high_prec_o).
 * workspace : DEVICE scratch of at least attn_qat_workspace_size(0, ...) bytes, 256-byte aligned.
 * Errors: AQ_EINVAL (null q/k/v/o/workspace, head_size != 128 [API]
 * get_supported_head_sizes, sizes <= 0, non-finite or non-positive softmax_scale, flags outside
 * AQ_FLAGS_ALL, strides that are not positive, misaligned tensors or strides, workspace too
 * small, only some of the training outputs); AQ_ENOTSUP (num_kv_heads != num_heads, causal with
 * lq != lk, lengths above 2^30).
 * ------------------------------------------------------------------------------------------- */
int attn_qat_fwd(const void *q, const void *k, const void *v, void *o, int batch, int num_heads,
                 int num_kv_heads, int head_size, int64_t lq, int64_t lk, aq_strides sq,
                 aq_strides sk, aq_strides sv, aq_strides so, float softmax_scale, int causal,
                 unsigned quant_flags, float *lse_log2, float *chunk_max_log2, float *o_hp,
                 void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * attn_qat_fwd_noalloc - attn_qat_fwd for callers that cannot allocate device memory: code under
 * HIP stream capture, serving loops and harnesses that forbid hipMalloc.
 *
 * Same arguments, checks, kernels and results as attn_qat_fwd, without the workspace: the library
 * uses a fixed scratch of AQ_NOALLOC_SCRATCH_BYTES in a file-scope device array, one copy per
 * device, present from the library's first use of that device until the process ends.  The
 * scratch of the CURRENT device (hipGetDevice) is used; `stream` must belong to it.  Nothing is
 * allocated or freed (leave aq_kernel_timing off: its events are created per launch).
 * Every call on a device shares that device's scratch and finds it as the last call left it;
 * nothing in it needs to start at zero.  Calls that can overlap on one device (different streams,
 * or different host threads) race on the scratch: the caller orders them.
 * Errors: as attn_qat_fwd (the workspace ones aside), plus AQ_ENOTSUP when the call's workspace,
 * attn_qat_workspace_size(0, batch, num_heads, lq, lk), exceeds AQ_NOALLOC_SCRATCH_BYTES (for
 * example 12 heads of 32768 tokens fit: about 208 MB), and AQ_EHIP when the scratch's device
 * address cannot be obtained.  Size checks come before any HIP call.
 * ------------------------------------------------------------------------------------------- */
#define AQ_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int attn_qat_fwd_noalloc(const void *q, const void *k, const void *v, void *o, int batch, int num_heads,
                         int num_kv_heads, int head_size, int64_t lq, int64_t lk, aq_strides sq,
                         aq_strides sk, aq_strides sv, aq_strides so, float softmax_scale, int causal,
                         unsigned quant_flags, float *lse_log2, float *chunk_max_log2, float *o_hp,
                         void *stream);

/* ---------------------------------------------------------------------------------------------
 * attn_qat_bwd - straight-through backward ([META] backward "consistent STE with auxiliary
 * output"; [API] use_qat_qkv_backward, fake_quant_p_bwd, use_high_prec_o).
 *
 * Fake-quant nodes pass gradients unchanged and the chunk maxima are constants.  With
 * A = exp(logit - lse) and A-hat = fq(exp(logit - m_c)) * exp(m_c - lse) (bit-for-bit the P-hat
 * the forward used): D_i = <dO_i, o_hp_i>, dV = A-hat^T dO, dP = dO V-hat^T,
 * dS = A * (dP - D), dQ = scale dS K-hat, dK = scale dS^T Q-hat.
 * Inputs q, k, v, d_o (bf16, strided as in the forward) and o_hp, lse_log2, chunk_max_log2
 * exactly as written by attn_qat_fwd with the same arguments, quant_flags included (the
 * variants' scales and key means are recomputed from the same tensors): o_hp [B, H, lq, 128],
 * lse_log2 [B, H, lq] and chunk_max_log2 [B, H, ceil(lk/128), lq] (x2 under AQ_TWO_LEVEL_P), fp32
 * contiguous.  The pointers carry no sizes, so the library cannot check these shapes: smaller
 * buffers are read past their end.  Outputs dq, dk, dv bf16 with their own strides.
 * Deterministic: no atomics.  Non-causal calls may compute some (head, 128-row) blocks of the
 * gradients in pieces whose fp32 sums are added in a fixed order, to fill the last round of
 * workgroups; which blocks depends on the device's compute-unit count, so results can differ in
 * the last bits between GPU models, never between runs on one.
 * workspace: at least attn_qat_workspace_size(1, ...) bytes.
 * Errors: as attn_qat_fwd, plus AQ_EINVAL for any null gradient or statistics pointer.
 * ------------------------------------------------------------------------------------------- */
int attn_qat_bwd(const void *q, const void *k, const void *v, const float *o_hp, const void *d_o,
                 const float *lse_log2, const float *chunk_max_log2, void *dq, void *dk, void *dv,
                 int batch, int num_heads, int num_kv_heads, int head_size, int64_t lq,
                 int64_t lk, aq_strides sq, aq_strides sk, aq_strides sv, aq_strides sdo,
                 aq_strides sdq, aq_strides sdk, aq_strides sdv, float softmax_scale, int causal,
                 unsigned quant_flags, void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * vsa_qat_fwd - cube-sparse fake-quant attention forward ([META] attention kind "vsa",
 * cube_shape [4,4,8], coarse "BF16" not quantized, fine "NVFP4 fake-quant with BF16 matmul",
 * selection effective_topk = max(1, min(ceil((1-sparsity)*n), n))).
 *
 * Tokens are cube-major: the grid grid_t x grid_h x grid_w is cut into cubes of
 * cube_t x cube_h x cube_w tokens and each cube's tokens are contiguous along l (cube index
 * raster order over the cube grid).  n = number of cubes.
 *   1. Qc, Kc (and Vc when o_coarse is requested) = per-cube means in fp32, rounded to bf16.
 *   2. coarse logits softmax_scale * <Qc, Kc>; each query cube keeps the topk highest-scoring
 *      key cubes (ties to the lower cube index), listed in ascending cube order.
 *   3. fine stage: the dense forward restricted to the selected cubes' keys, visited in that
 *      ascending order with one 128-key chunk per cube.
 * o_fine [B, H, L, 128] bf16 (strides so); o_coarse (NULL allowed) receives
 * softmax(coarse logits) @ Vc broadcast to every token of the query cube, bf16, strides so;
 * sel (NULL allowed) receives the [B, H, n, topk] int32 selection.
 * Optional training outputs of the fine stage (all three or none; vsa_qat_bwd needs them and
 * sel): lse_log2 [B, H, L], chunk_max_log2 [B, H, topk, L] (x2 under AQ_TWO_LEVEL_P, as for
 * attn_qat_fwd) (the running maximum after each
 * selected cube, in list order) and o_hp [B, H, L, 128], fp32 contiguous, defined as for
 * attn_qat_fwd.
 * workspace: at least attn_qat_workspace_size(2, ...) bytes with lk = L.
 * A query cube whose coarse logits are NaN (a NaN among its tokens) ranks them below every
 * number, so its list still holds topk distinct cubes (the lowest indices among equals).
 * Errors: AQ_EINVAL (as the forward, plus grid sizes not divisible by the cube, L !=
 * grid_t*grid_h*grid_w, sparsity outside [0,1], only some of the training outputs);
 * AQ_ENOTSUP (cube of other than 128 tokens, more than 4096 cubes, more than 1024 selected cubes
 * per query cube).
 * ------------------------------------------------------------------------------------------- */
int vsa_qat_fwd(const void *q, const void *k, const void *v, void *o_fine, void *o_coarse,
                int32_t *sel, int batch, int num_heads, int head_size, int64_t seq_len,
                int grid_t, int grid_h, int grid_w, int cube_t, int cube_h, int cube_w,
                double sparsity, aq_strides sq, aq_strides sk, aq_strides sv, aq_strides so,
                float softmax_scale, unsigned quant_flags, float *lse_log2, float *chunk_max_log2,
                float *o_hp, void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * vsa_qat_bwd - straight-through backward of the cube-sparse fine stage ([META] attention kind
 * "vsa" with quantize_fine, backward "consistent STE with auxiliary output"; needed to train the
 * sparse model).
 *
 * The dense backward's formulas (attn_qat_bwd) with every query cube attending only to its
 * selected cubes: dQ of a query sums over its cube's selected keys; dK and dV of a key sum over
 * the queries of every cube that selected the key's cube, with the chunk maximum of the
 * selection slot that cube used.  The coarse stage (o_coarse) is not differentiated here.
 * Inputs q, k, v, d_o (bf16 [B, L, H, 128] by strides), sel [B, H, n, topk] int32,
 * lse_log2 [B, H, L], chunk_max_log2 [B, H, topk, L] (x2 under AQ_TWO_LEVEL_P) and o_hp
 * [B, H, L, 128] fp32, exactly as written by vsa_qat_fwd with the same arguments, sparsity
 * included (topk follows from it; the shapes cannot be checked here, and smaller buffers are read
 * past their end).  sel must hold distinct cube indices in ascending order; an entry outside
 * [0, n) is clamped into it, so a malformed list gives meaningless gradients but no access
 * outside the operands.  Outputs dq, dk, dv bf16 with their own strides.
 * workspace: at least attn_qat_workspace_size(3, ...) bytes with lq = lk = L.
 * Errors: as vsa_qat_fwd, plus AQ_EINVAL for a null gradient, statistics or sel pointer and
 * AQ_ENOTSUP for more than 4096 cubes.
 * ------------------------------------------------------------------------------------------- */
int vsa_qat_bwd(const void *q, const void *k, const void *v, const float *o_hp, const void *d_o,
                const float *lse_log2, const float *chunk_max_log2, const int32_t *sel, void *dq, void *dk,
                void *dv, int batch, int num_heads, int head_size, int64_t seq_len, int grid_t, int grid_h,
                int grid_w, int cube_t, int cube_h, int cube_w, double sparsity, aq_strides sq, aq_strides sk,
                aq_strides sv, aq_strides sdo, aq_strides sdq, aq_strides sdk, aq_strides sdv,
                float softmax_scale, unsigned quant_flags, void *workspace, size_t workspace_bytes,
                void *stream);

/* Number of cubes kept per query cube: max(1, min(ceil((1 - sparsity) * n), n)). */
int vsa_topk(double sparsity, int n_cubes);

/* Workspace bytes needed by op 0 = attn_qat_fwd, 1 = attn_qat_bwd, 2 = vsa_qat_fwd and
 * 3 = vsa_qat_bwd (lq = lk = L); 0 for invalid arguments. */
size_t attn_qat_workspace_size(int op, int batch, int num_heads, int64_t lq, int64_t lk);

/* ---------------------------------------------------------------------------------------------
 * NVFP4 QAD linear (["nvfp4_qad.py"] nvfp4_gemm, _NVFP4STE, NVFP4QADLinearMethod.apply).
 *
 * qad_linear_fwd: y [m, n] = fq(x, g_x) [m, k] . fq(w, g_w) [n, k]^T + bias [n], bf16 row-major
 *   contiguous.  g_w = 448*6 / max(amax|w|, 1e-12) (weight_global_sf), computed on the device on
 *   every call; g_x = *input_sf (a DEVICE fp32 scalar, the static input_global_sf
 *   448*6 / calibrated amax) or 1 when input_sf is NULL (the unit scale of the attention
 *   projections).  Blocks of 16 along k, E4M3 block scales, E2M1 values, dequantized and rounded
 *   to bf16 (as fq_nvfp4 outputs them); the product runs on BF16 MFMA with fp32 accumulation and
 *   the bias is added before the bf16 rounding.  bias may be NULL.
 * qad_linear_bwd: the straight-through estimator's full-precision gradients: grad_x [m, k] =
 *   grad_y [m, n] . w, grad_w [n, k] = grad_y^T . x, grad_b [n] = column sums of grad_y, bf16
 *   (fp32 accumulation).  Any output may be NULL to skip it.
 * qad_observe_amax: *amax = max(*amax, max|x|) over numel bf16 values (max calibration; *amax is a
 *   DEVICE fp32 scalar the caller zeroes before the first calibrating call).
 * qad_input_global_sf: *g_out = fp32(448*6 / max(*amax, 1e-12)) ([QAD] input_global_sf after
 *   calibration; NaN read as 0), both DEVICE fp32 scalars; *g_out serves as input_sf.
 * Workspace: qad_linear_workspace_size(0 = forward, 1 = backward, m, n, k) bytes of DEVICE memory
 *   (any alignment).
 * Errors: AQ_EINVAL (null pointers, non-positive sizes, tensors not 16-byte aligned, workspace too
 *   small); AQ_ENOTSUP (k or n not a multiple of 64, rows too long for the kernels' 32-bit tile
 *   offsets).
 * ------------------------------------------------------------------------------------------- */
size_t qad_linear_workspace_size(int op, int64_t m, int64_t n, int64_t k);
int qad_linear_fwd(const void *x, const void *w, const void *bias, void *y, int64_t m, int64_t n, int64_t k,
                   const float *input_sf, void *workspace, size_t workspace_bytes, void *stream);
int qad_linear_bwd(const void *grad_y, const void *x, const void *w, void *grad_x, void *grad_w, void *grad_b,
                   int64_t m, int64_t n, int64_t k, void *workspace, size_t workspace_bytes, void *stream);
int qad_observe_amax(const void *x, int64_t numel, float *amax, void *stream);
int qad_input_global_sf(const float *amax, float *g_out, void *stream);

/* ---------------------------------------------------------------------------------------------
 * Kernel timing (profiling aid, not part of the method).
 * aq_kernel_timing(1) makes every later kernel launch of the library, on any stream, record a
 * HIP event before and after the kernel on that stream; aq_kernel_timing(0) stops it.
 * aq_kernel_times() waits for the recorded events and writes one line per kernel name,
 * "<name> <launches> <total milliseconds>\n", accumulated since the last reset, into buf (at
 * most len bytes, NUL-terminated); reset != 0 clears the totals afterwards.  Returns the length
 * of the full report, or AQ_EHIP if an event could not be read.
 * ------------------------------------------------------------------------------------------- */
int aq_kernel_timing(int enable);
int aq_kernel_times(char *buf, size_t len, int reset);

#ifdef __cplusplus
}
#endif

#endif /* ATTNQAT_H */
