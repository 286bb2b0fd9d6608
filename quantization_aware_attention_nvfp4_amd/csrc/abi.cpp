// abi.cpp - the extern "C" surface declared in include/attnqat.h: argument validation, error
// reporting and dispatch to the gfx950 launchers.  Every check runs on the host before anything
// is enqueued, so a rejected call leaves the stream untouched.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include "attnqat.h"
#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return AQ_OK;
}

int hip_status(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(AQ_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

aq::Strides cvt(aq_strides s) { return aq::Strides{s.b, s.h, s.l}; }

bool strides_ok(aq_strides s) { return s.b > 0 && s.h > 0 && s.l > 0; }

// The attention kernels move rows in 16-byte pieces and keep per-lane row offsets in 32 bits:
// bf16 tensors must start 16-byte aligned, with strides that are multiples of 8 elements and
// below 2^24 elements.
bool tensor_ok(const void *p, aq_strides s) {
  const int64_t lim = (int64_t)1 << 24;
  return ((uintptr_t)p & 15) == 0 && s.b % 8 == 0 && s.h % 8 == 0 && s.l % 8 == 0 && s.b < lim * 64 &&
         s.h < lim * 64 && s.l < lim;
}

// Checks shared by the attention entry points ("attn_qat_train" page: head sizes [128],
// AttentionImpl(num_heads, head_size, softmax_scale, causal, num_kv_heads)).
int check_attention(int batch, int num_heads, int num_kv_heads, int head_size, int64_t lq,
                    int64_t lk, float softmax_scale, int causal, unsigned quant_flags) {
  if (head_size != aq::kHeadDimHost)
    return fail(AQ_EINVAL, "head_size %d is not supported (supported: 128)", head_size);
  if (batch <= 0 || num_heads <= 0 || lq <= 0 || lk <= 0)
    return fail(AQ_EINVAL, "sizes must be positive (batch %d, heads %d, lq %lld, lk %lld)", batch,
                num_heads, (long long)lq, (long long)lk);
  if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale))
    return fail(AQ_EINVAL, "softmax_scale must be finite and > 0 (got %g)", (double)softmax_scale);
  if (quant_flags & ~(unsigned)AQ_FLAGS_ALL)
    return fail(AQ_EINVAL, "quant_flags 0x%x has bits outside AQ_FLAGS_ALL", quant_flags);
  if ((quant_flags & AQ_TWO_LEVEL_P) && (quant_flags & (AQ_FINAL_MAX | AQ_GSF_P)))
    return fail(AQ_ENOTSUP, "AQ_TWO_LEVEL_P does not combine with AQ_FINAL_MAX or AQ_GSF_P (flags 0x%x)",
                quant_flags);
  if ((quant_flags & AQ_PV_FP8) && !(quant_flags & AQ_QUANT_P))
    return fail(AQ_ENOTSUP, "AQ_PV_FP8 needs AQ_QUANT_P (flags 0x%x)", quant_flags);
  if (num_kv_heads != num_heads)
    return fail(AQ_ENOTSUP, "num_kv_heads (%d) must equal num_heads (%d)", num_kv_heads, num_heads);
  if (causal && lq != lk)
    return fail(AQ_ENOTSUP, "causal attention needs lq == lk (got %lld, %lld)", (long long)lq,
                (long long)lk);
  if (lq > ((int64_t)1 << 30) || lk > ((int64_t)1 << 30))
    return fail(AQ_ENOTSUP, "sequence lengths above 2^30 are not supported (lq %lld, lk %lld)", (long long)lq,
                (long long)lk);
  return AQ_OK;
}

}  // namespace

extern "C" {

const char *aq_last_error(void) { return g_err; }

int fq_nvfp4(const void *x, void *y, int64_t outer, int64_t axis_len, int64_t inner,
             const float *global_scale, void *stream) {
  if (!x || !y) return fail(AQ_EINVAL, "fq_nvfp4: null tensor pointer");
  if (outer <= 0 || axis_len <= 0 || inner <= 0)
    return fail(AQ_EINVAL, "fq_nvfp4: sizes must be positive (%lld, %lld, %lld)", (long long)outer,
                (long long)axis_len, (long long)inner);
  return hip_status(aq::launch_fq(x, y, outer, axis_len, inner, global_scale, (hipStream_t)stream),
                    "fq_nvfp4 launch");
}

int fq_nvfp4_static_scale(const void *x, int64_t n, float *g_out, void *stream) {
  if (!x || !g_out) return fail(AQ_EINVAL, "fq_nvfp4_static_scale: null pointer");
  if (n <= 0) return fail(AQ_EINVAL, "fq_nvfp4_static_scale: n must be positive");
  return hip_status(aq::launch_static_scale(x, n, g_out, (hipStream_t)stream),
                    "fq_nvfp4_static_scale launch");
}

int vsa_topk(double sparsity, int n_cubes) {
  if (n_cubes <= 0 || !(sparsity >= 0.0 && sparsity <= 1.0)) return 0;
  const double t = ceil((1.0 - sparsity) * (double)n_cubes);
  int k = (int)t;
  if (k > n_cubes) k = n_cubes;
  if (k < 1) k = 1;
  return k;
}

size_t attn_qat_workspace_size(int op, int batch, int num_heads, int64_t lq, int64_t lk) {
  if (batch <= 0 || num_heads <= 0 || lq <= 0 || lk <= 0 || op < 0 || op > 3) return 0;
  return aq::workspace_bytes(op, batch, num_heads, lq, lk);
}

// Argument checks of attn_qat_fwd and attn_qat_fwd_noalloc (everything but the workspace).
static int check_fwd(const char *fn, const void *q, const void *k, const void *v, void *o, int batch,
                     int num_heads, int num_kv_heads, int head_size, int64_t lq, int64_t lk, aq_strides sq,
                     aq_strides sk, aq_strides sv, aq_strides so, float softmax_scale, int causal,
                     unsigned quant_flags, float *lse_log2, float *chunk_max_log2, float *o_hp) {
  if (!q || !k || !v || !o) return fail(AQ_EINVAL, "%s: null tensor pointer", fn);
  int rc = check_attention(batch, num_heads, num_kv_heads, head_size, lq, lk, softmax_scale, causal,
                           quant_flags);
  if (rc) return rc;
  if (!strides_ok(sq) || !strides_ok(sk) || !strides_ok(sv) || !strides_ok(so))
    return fail(AQ_EINVAL, "%s: strides must be positive with d contiguous", fn);
  if (!tensor_ok(q, sq) || !tensor_ok(k, sk) || !tensor_ok(v, sv) || !tensor_ok(o, so))
    return fail(AQ_EINVAL, "%s: tensors must be 16-byte aligned with strides that are multiples of 8 "
                           "elements and below 2^24", fn);
  if ((lse_log2 || chunk_max_log2 || o_hp) && !(lse_log2 && chunk_max_log2 && o_hp))
    return fail(AQ_EINVAL, "%s: the training outputs lse_log2, chunk_max_log2 and o_hp come together "
                           "(all three or none)", fn);
  return AQ_OK;
}

static int run_fwd(const char *fn, const void *q, const void *k, const void *v, void *o, int batch, int num_heads,
                   int64_t lq, int64_t lk, aq_strides sq, aq_strides sk, aq_strides sv, aq_strides so,
                   float softmax_scale, int causal, unsigned quant_flags, float *lse_log2, float *chunk_max_log2,
                   float *o_hp, void *workspace, void *stream) {
  aq::AttnArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o;
  a.batch = batch; a.heads = num_heads; a.lq = lq; a.lk = lk;
  a.sq = cvt(sq); a.sk = cvt(sk); a.sv = cvt(sv); a.so = cvt(so);
  a.scale = softmax_scale; a.causal = causal != 0; a.flags = quant_flags;
  a.lse = lse_log2; a.cmax = chunk_max_log2; a.o_hp = o_hp;
  a.workspace = workspace;
  return hip_status(aq::launch_attn_fwd(a, (hipStream_t)stream), fn);
}

int attn_qat_fwd(const void *q, const void *k, const void *v, void *o, int batch, int num_heads,
                 int num_kv_heads, int head_size, int64_t lq, int64_t lk, aq_strides sq,
                 aq_strides sk, aq_strides sv, aq_strides so, float softmax_scale, int causal,
                 unsigned quant_flags, float *lse_log2, float *chunk_max_log2, float *o_hp,
                 void *workspace, size_t workspace_bytes, void *stream) {
  int rc = check_fwd("attn_qat_fwd", q, k, v, o, batch, num_heads, num_kv_heads, head_size, lq, lk, sq, sk, sv,
                     so, softmax_scale, causal, quant_flags, lse_log2, chunk_max_log2, o_hp);
  if (rc) return rc;
  const size_t need = aq::workspace_bytes(0, batch, num_heads, lq, lk);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255))
    return fail(AQ_EINVAL, "attn_qat_fwd: workspace must be 256-byte aligned and hold %zu bytes",
                need);
  return run_fwd("attn_qat_fwd launch", q, k, v, o, batch, num_heads, lq, lk, sq, sk, sv, so, softmax_scale,
                 causal, quant_flags, lse_log2, chunk_max_log2, o_hp, workspace, stream);
}

int attn_qat_fwd_noalloc(const void *q, const void *k, const void *v, void *o, int batch, int num_heads,
                         int num_kv_heads, int head_size, int64_t lq, int64_t lk, aq_strides sq,
                         aq_strides sk, aq_strides sv, aq_strides so, float softmax_scale, int causal,
                         unsigned quant_flags, float *lse_log2, float *chunk_max_log2, float *o_hp,
                         void *stream) {
  int rc = check_fwd("attn_qat_fwd_noalloc", q, k, v, o, batch, num_heads, num_kv_heads, head_size, lq, lk, sq,
                     sk, sv, so, softmax_scale, causal, quant_flags, lse_log2, chunk_max_log2, o_hp);
  if (rc) return rc;
  const size_t need = aq::workspace_bytes(0, batch, num_heads, lq, lk);
  if (need > (size_t)AQ_NOALLOC_SCRATCH_BYTES)
    return fail(AQ_ENOTSUP,
                "attn_qat_fwd_noalloc: this call needs %zu bytes of scratch, above the library's fixed %zu "
                "(use attn_qat_fwd with a workspace)", need, (size_t)AQ_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  hipError_t e = aq::noalloc_scratch(&ws);
  if (e != hipSuccess) return hip_status(e, "attn_qat_fwd_noalloc scratch address");
  return run_fwd("attn_qat_fwd_noalloc launch", q, k, v, o, batch, num_heads, lq, lk, sq, sk, sv, so,
                 softmax_scale, causal, quant_flags, lse_log2, chunk_max_log2, o_hp, ws, stream);
}

int attn_qat_bwd(const void *q, const void *k, const void *v, const float *o_hp, const void *d_o,
                 const float *lse_log2, const float *chunk_max_log2, void *dq, void *dk, void *dv,
                 int batch, int num_heads, int num_kv_heads, int head_size, int64_t lq,
                 int64_t lk, aq_strides sq, aq_strides sk, aq_strides sv, aq_strides sdo,
                 aq_strides sdq, aq_strides sdk, aq_strides sdv, float softmax_scale, int causal,
                 unsigned quant_flags, void *workspace, size_t workspace_bytes, void *stream) {
  if (!q || !k || !v || !d_o || !dq || !dk || !dv)
    return fail(AQ_EINVAL, "attn_qat_bwd: null tensor pointer");
  if (!o_hp || !lse_log2 || !chunk_max_log2)
    return fail(AQ_EINVAL, "attn_qat_bwd: o_hp, lse_log2 and chunk_max_log2 are required");
  int rc = check_attention(batch, num_heads, num_kv_heads, head_size, lq, lk, softmax_scale, causal,
                           quant_flags);
  if (rc) return rc;
  if (!strides_ok(sq) || !strides_ok(sk) || !strides_ok(sv) || !strides_ok(sdo) ||
      !strides_ok(sdq) || !strides_ok(sdk) || !strides_ok(sdv))
    return fail(AQ_EINVAL, "attn_qat_bwd: strides must be positive with d contiguous");
  if (!tensor_ok(q, sq) || !tensor_ok(k, sk) || !tensor_ok(v, sv) || !tensor_ok(d_o, sdo) || !tensor_ok(dq, sdq) ||
      !tensor_ok(dk, sdk) || !tensor_ok(dv, sdv))
    return fail(AQ_EINVAL, "attn_qat_bwd: tensors must be 16-byte aligned with strides that are multiples of 8 "
                           "elements and below 2^24");
  const size_t need = aq::workspace_bytes(1, batch, num_heads, lq, lk);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255))
    return fail(AQ_EINVAL, "attn_qat_bwd: workspace must be 256-byte aligned and hold %zu bytes",
                need);
  aq::AttnArgs a{};
  a.q = q; a.k = k; a.v = v;
  a.batch = batch; a.heads = num_heads; a.lq = lq; a.lk = lk;
  a.sq = cvt(sq); a.sk = cvt(sk); a.sv = cvt(sv);
  a.scale = softmax_scale; a.causal = causal != 0; a.flags = quant_flags;
  a.lse = const_cast<float *>(lse_log2); a.cmax = const_cast<float *>(chunk_max_log2);
  a.o_hp = const_cast<float *>(o_hp);
  a.workspace = workspace;
  aq::BwdArgs b{};
  b.d_o = d_o; b.dq = dq; b.dk = dk; b.dv = dv;
  b.sdo = cvt(sdo); b.sdq = cvt(sdq); b.sdk = cvt(sdk); b.sdv = cvt(sdv);
  return hip_status(aq::launch_attn_bwd(a, b, (hipStream_t)stream), "attn_qat_bwd launch");
}

// Shape checks shared by the cube-sparse entry points.
static int check_vsa(const char *fn, int batch, int num_heads, int head_size, int64_t seq_len, int grid_t,
              int grid_h, int grid_w, int cube_t, int cube_h, int cube_w, double sparsity, float softmax_scale,
              unsigned quant_flags) {
  int rc = check_attention(batch, num_heads, num_heads, head_size, seq_len, seq_len, softmax_scale,
                           0, quant_flags);
  if (rc) return rc;
  if (grid_t <= 0 || grid_h <= 0 || grid_w <= 0 || cube_t <= 0 || cube_h <= 0 || cube_w <= 0)
    return fail(AQ_EINVAL, "%s: grid and cube sizes must be positive", fn);
  if (grid_t % cube_t || grid_h % cube_h || grid_w % cube_w)
    return fail(AQ_EINVAL, "%s: grid %dx%dx%d is not divisible by cube %dx%dx%d", fn, grid_t, grid_h, grid_w,
                cube_t, cube_h, cube_w);
  if ((int64_t)grid_t * grid_h * grid_w != seq_len)
    return fail(AQ_EINVAL, "%s: seq_len %lld != grid_t*grid_h*grid_w", fn, (long long)seq_len);
  if (!(sparsity >= 0.0 && sparsity <= 1.0))
    return fail(AQ_EINVAL, "%s: sparsity must lie in [0, 1] (got %g)", fn, sparsity);
  if (cube_t * cube_h * cube_w != aq::kChunkHost)
    return fail(AQ_ENOTSUP, "%s: cubes of %d tokens are not supported (only 128)", fn, cube_t * cube_h * cube_w);
  return AQ_OK;
}

int vsa_qat_fwd(const void *q, const void *k, const void *v, void *o_fine, void *o_coarse,
                int32_t *sel, int batch, int num_heads, int head_size, int64_t seq_len,
                int grid_t, int grid_h, int grid_w, int cube_t, int cube_h, int cube_w,
                double sparsity, aq_strides sq, aq_strides sk, aq_strides sv, aq_strides so,
                float softmax_scale, unsigned quant_flags, float *lse_log2, float *chunk_max_log2,
                float *o_hp, void *workspace, size_t workspace_bytes, void *stream) {
  if (!q || !k || !v || !o_fine) return fail(AQ_EINVAL, "vsa_qat_fwd: null tensor pointer");
  int rc = check_vsa("vsa_qat_fwd", batch, num_heads, head_size, seq_len, grid_t, grid_h, grid_w, cube_t, cube_h,
                     cube_w, sparsity, softmax_scale, quant_flags);
  if (rc) return rc;
  if ((lse_log2 || chunk_max_log2 || o_hp) && !(lse_log2 && chunk_max_log2 && o_hp))
    return fail(AQ_EINVAL, "vsa_qat_fwd: the training outputs lse_log2, chunk_max_log2 and o_hp come together "
                           "(all three or none)");
  if (!strides_ok(sq) || !strides_ok(sk) || !strides_ok(sv) || !strides_ok(so))
    return fail(AQ_EINVAL, "vsa_qat_fwd: strides must be positive with d contiguous");
  if (!tensor_ok(q, sq) || !tensor_ok(k, sk) || !tensor_ok(v, sv) || !tensor_ok(o_fine, so) ||
      (o_coarse && !tensor_ok(o_coarse, so)))
    return fail(AQ_EINVAL, "vsa_qat_fwd: tensors must be 16-byte aligned with strides that are multiples of 8 "
                           "elements and below 2^24");
  const size_t need = aq::workspace_bytes(2, batch, num_heads, seq_len, seq_len);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255))
    return fail(AQ_EINVAL, "vsa_qat_fwd: workspace must be 256-byte aligned and hold %zu bytes",
                need);
  aq::AttnArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o_fine;
  a.batch = batch; a.heads = num_heads; a.lq = seq_len; a.lk = seq_len;
  a.sq = cvt(sq); a.sk = cvt(sk); a.sv = cvt(sv); a.so = cvt(so);
  a.scale = softmax_scale; a.causal = false; a.flags = quant_flags;
  a.lse = lse_log2; a.cmax = chunk_max_log2; a.o_hp = o_hp;
  a.workspace = workspace;
  aq::VsaArgs s{};
  s.o_coarse = o_coarse; s.sel = sel;
  s.n_cubes = (int)(seq_len / aq::kChunkHost);
  s.topk = vsa_topk(sparsity, s.n_cubes);
  // The backward walks lists of at most kMaxCubesHost query cubes per key cube, and the top-k
  // kernel keeps every cube's score in LDS (8 bytes per cube): the same cap for both directions.
  if (s.n_cubes > aq::kMaxCubesHost)
    return fail(AQ_ENOTSUP, "vsa_qat_fwd: at most %d cubes (got %d)", aq::kMaxCubesHost, s.n_cubes);
  if (s.topk > 1024)
    return fail(AQ_ENOTSUP, "vsa_qat_fwd: at most 1024 selected cubes per query cube (got %d)", s.topk);
  return hip_status(aq::launch_vsa_fwd(a, s, (hipStream_t)stream), "vsa_qat_fwd launch");
}

int vsa_qat_bwd(const void *q, const void *k, const void *v, const float *o_hp, const void *d_o,
                const float *lse_log2, const float *chunk_max_log2, const int32_t *sel, void *dq, void *dk,
                void *dv, int batch, int num_heads, int head_size, int64_t seq_len, int grid_t, int grid_h,
                int grid_w, int cube_t, int cube_h, int cube_w, double sparsity, aq_strides sq, aq_strides sk,
                aq_strides sv, aq_strides sdo, aq_strides sdq, aq_strides sdk, aq_strides sdv,
                float softmax_scale, unsigned quant_flags, void *workspace, size_t workspace_bytes,
                void *stream) {
  if (!q || !k || !v || !d_o || !dq || !dk || !dv) return fail(AQ_EINVAL, "vsa_qat_bwd: null tensor pointer");
  if (!o_hp || !lse_log2 || !chunk_max_log2 || !sel)
    return fail(AQ_EINVAL, "vsa_qat_bwd: o_hp, lse_log2, chunk_max_log2 and sel are required");
  int rc = check_vsa("vsa_qat_bwd", batch, num_heads, head_size, seq_len, grid_t, grid_h, grid_w, cube_t, cube_h,
                     cube_w, sparsity, softmax_scale, quant_flags);
  if (rc) return rc;
  if (!strides_ok(sq) || !strides_ok(sk) || !strides_ok(sv) || !strides_ok(sdo) || !strides_ok(sdq) ||
      !strides_ok(sdk) || !strides_ok(sdv))
    return fail(AQ_EINVAL, "vsa_qat_bwd: strides must be positive with d contiguous");
  if (!tensor_ok(q, sq) || !tensor_ok(k, sk) || !tensor_ok(v, sv) || !tensor_ok(d_o, sdo) || !tensor_ok(dq, sdq) ||
      !tensor_ok(dk, sdk) || !tensor_ok(dv, sdv))
    return fail(AQ_EINVAL, "vsa_qat_bwd: tensors must be 16-byte aligned with strides that are multiples of 8 "
                           "elements and below 2^24");
  const int n = (int)(seq_len / aq::kChunkHost);
  if (n > aq::kMaxCubesHost)
    return fail(AQ_ENOTSUP, "vsa_qat_bwd: at most %d cubes (got %d)", aq::kMaxCubesHost, n);
  const size_t need = aq::workspace_bytes(3, batch, num_heads, seq_len, seq_len);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255))
    return fail(AQ_EINVAL, "vsa_qat_bwd: workspace must be 256-byte aligned and hold %zu bytes", need);
  aq::AttnArgs a{};
  a.q = q; a.k = k; a.v = v;
  a.batch = batch; a.heads = num_heads; a.lq = seq_len; a.lk = seq_len;
  a.sq = cvt(sq); a.sk = cvt(sk); a.sv = cvt(sv);
  a.scale = softmax_scale; a.causal = false; a.flags = quant_flags;
  a.lse = const_cast<float *>(lse_log2); a.cmax = const_cast<float *>(chunk_max_log2);
  a.o_hp = const_cast<float *>(o_hp);
  a.workspace = workspace;
  aq::BwdArgs b{};
  b.d_o = d_o; b.dq = dq; b.dk = dk; b.dv = dv;
  b.sdo = cvt(sdo); b.sdq = cvt(sdq); b.sdk = cvt(sdk); b.sdv = cvt(sdv);
  return hip_status(aq::launch_vsa_bwd(a, b, sel, n, vsa_topk(sparsity, n), (hipStream_t)stream),
                    "vsa_qat_bwd launch");
}

// ---- NVFP4 QAD linear ---------------------------------------------------------------------------

// Shapes the GEMM kernel takes: contractions over k (forward) and n (grad_x) in steps of 64,
// 16-byte aligned contiguous rows, 32-bit row offsets inside one 256-row tile.
static int check_linear(const char *what, int64_t m, int64_t n, int64_t k) {
  if (m <= 0 || n <= 0 || k <= 0)
    return fail(AQ_EINVAL, "%s: sizes must be positive (m %lld, n %lld, k %lld)", what, (long long)m,
                (long long)n, (long long)k);
  if (k % 64 || n % 64)
    return fail(AQ_ENOTSUP, "%s: in_features (%lld) and out_features (%lld) must be multiples of 64", what,
                (long long)k, (long long)n);
  const int64_t mp = (m + 63) / 64 * 64;
  if (256 * (k > n ? k : n) * 2 >= ((int64_t)1 << 32) || 256 * mp * 2 >= ((int64_t)1 << 32))
    return fail(AQ_ENOTSUP, "%s: rows too long for 32-bit tile offsets", what);
  return AQ_OK;
}

static bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

size_t qad_linear_workspace_size(int op, int64_t m, int64_t n, int64_t k) {
  if (m <= 0 || n <= 0 || k <= 0 || op < 0 || op > 1) return 0;
  return aq::linear_workspace(op, m, n, k).total + 256;
}

int qad_linear_fwd(const void *x, const void *w, const void *bias, void *y, int64_t m, int64_t n, int64_t k,
                   const float *input_sf, void *workspace, size_t workspace_bytes, void *stream) {
  if (!x || !w || !y || !workspace) return fail(AQ_EINVAL, "qad_linear_fwd: null pointer");
  int rc = check_linear("qad_linear_fwd", m, n, k);
  if (rc) return rc;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || (bias && !aligned16(bias)))
    return fail(AQ_EINVAL, "qad_linear_fwd: tensors must be 16-byte aligned");
  const aq::LinearWorkspace lw = aq::linear_workspace(0, m, n, k);
  uint8_t *ws = (uint8_t *)(((uintptr_t)workspace + 255) & ~(uintptr_t)255);
  if ((size_t)(ws - (uint8_t *)workspace) + lw.total > workspace_bytes)
    return fail(AQ_EINVAL, "qad_linear_fwd: workspace of %zu bytes is too small (need %zu)", workspace_bytes,
                qad_linear_workspace_size(0, m, n, k));
  hipStream_t st = (hipStream_t)stream;
  float *gw = (float *)(ws + lw.gw);
  hipError_t e;
  if ((e = aq::launch_static_scale(w, n * k, gw, st))) return hip_status(e, "qad_linear_fwd weight scale");
  if ((e = aq::launch_fq(w, ws + lw.wq, n, k, 1, gw, st))) return hip_status(e, "qad_linear_fwd weight");
  if ((e = aq::launch_fq(x, ws + lw.xq, m, k, 1, input_sf, st))) return hip_status(e, "qad_linear_fwd input");
  return hip_status(aq::launch_gemm_tn(ws + lw.xq, k, ws + lw.wq, k, y, n, bias, m, n, k, st), "qad_linear_fwd gemm");
}

int qad_linear_bwd(const void *grad_y, const void *x, const void *w, void *grad_x, void *grad_w, void *grad_b,
                   int64_t m, int64_t n, int64_t k, void *workspace, size_t workspace_bytes, void *stream) {
  if (!grad_y || !x || !w || !workspace) return fail(AQ_EINVAL, "qad_linear_bwd: null pointer");
  int rc = check_linear("qad_linear_bwd", m, n, k);
  if (rc) return rc;
  if (!aligned16(grad_y) || !aligned16(x) || !aligned16(w) || (grad_x && !aligned16(grad_x)) ||
      (grad_w && !aligned16(grad_w)) || (grad_b && !aligned16(grad_b)))
    return fail(AQ_EINVAL, "qad_linear_bwd: tensors must be 16-byte aligned");
  const aq::LinearWorkspace lw = aq::linear_workspace(1, m, n, k);
  uint8_t *ws = (uint8_t *)(((uintptr_t)workspace + 255) & ~(uintptr_t)255);
  if ((size_t)(ws - (uint8_t *)workspace) + lw.total > workspace_bytes)
    return fail(AQ_EINVAL, "qad_linear_bwd: workspace of %zu bytes is too small (need %zu)", workspace_bytes,
                qad_linear_workspace_size(1, m, n, k));
  hipStream_t st = (hipStream_t)stream;
  const int64_t mp = (m + 63) / 64 * 64;
  hipError_t e;
  if (grad_x) {
    if ((e = aq::launch_transpose(w, k, n, k, ws + lw.wt, n, st))) return hip_status(e, "qad_linear_bwd W^T");
    if ((e = aq::launch_gemm_tn(grad_y, n, ws + lw.wt, n, grad_x, k, nullptr, m, k, n, st)))
      return hip_status(e, "qad_linear_bwd grad_x");
  }
  if (grad_w) {
    // g^T, with grad_b's column sums taken in the same pass
    if (grad_b)
      e = aq::launch_transpose_colsum(grad_y, m, n, ws + lw.gt, mp, grad_b, (float *)(ws + lw.part), st);
    else
      e = aq::launch_transpose(grad_y, n, m, n, ws + lw.gt, mp, st);
    if (e) return hip_status(e, "qad_linear_bwd g^T");
    if ((e = aq::launch_transpose(x, k, m, k, ws + lw.xt, mp, st))) return hip_status(e, "qad_linear_bwd x^T");
    if ((e = aq::launch_gemm_tn(ws + lw.gt, mp, ws + lw.xt, mp, grad_w, k, nullptr, n, k, mp, st)))
      return hip_status(e, "qad_linear_bwd grad_w");
  }
  if (grad_b && !grad_w)
    return hip_status(aq::launch_colsum(grad_y, m, n, grad_b, (float *)(ws + lw.part), st), "qad_linear_bwd grad_b");
  return ok();
}

int qad_input_global_sf(const float *amax, float *g_out, void *stream) {
  if (!amax || !g_out) return fail(AQ_EINVAL, "qad_input_global_sf: null pointer");
  return hip_status(aq::launch_scale_from_amax(amax, g_out, (hipStream_t)stream), "qad_input_global_sf launch");
}

int qad_observe_amax(const void *x, int64_t numel, float *amax, void *stream) {
  if (!x || !amax) return fail(AQ_EINVAL, "qad_observe_amax: null pointer");
  if (numel <= 0) return fail(AQ_EINVAL, "qad_observe_amax: numel must be positive");
  return hip_status(aq::launch_observe_amax(x, numel, amax, (hipStream_t)stream), "qad_observe_amax launch");
}

}  // extern "C"
