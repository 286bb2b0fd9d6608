/*
 * Plain CPU oracle for NVFP4 fake-quantized attention (Attn-QAT).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or constant with the
 * HIP library.
 *
 * Sources (web pages, cited by title and section):
 *  [QAD]  "nvfp4_qad.py" (FastVideo fastvideo/layers/quantization source page):
 *         module docstring (per-16 E4M3 block scales under a unit or static
 *         global scale), FP4_RANGE = 448*6, weight_global_sf (nan_to_num and
 *         the 1e-12 clamp), NVFP4QADLinearMethod.input_global_sf.
 *  [META] "vsqa-preview-1.3b metadata.json": attention.precision ("fine":
 *         NVFP4 fake-quant with BF16 matmul, quant_p, quant_v, quantize_coarse
 *         false), attention.selection (effective_topk formula, sparsity 0.9),
 *         attention.cube_shape [4,4,8]; the dense parent's precision record
 *         (group_size 16, qk/pv_format NVFP4 E2M1, scale dtype FP8 E4M3FN,
 *         backward "consistent STE with auxiliary output").
 *  [API]  "attn_qat_train" API reference page: attn_qat_train (BHLD layout,
 *         default sm_scale 1/sqrt(D), use_high_prec_o, fake_quant_p_bwd,
 *         use_qat_qkv_backward, unit global scales).
 *
 * Readings where the pages are silent are listed in the design notes; the
 * ones that shape arithmetic here are: the running max is refreshed once per
 * 128-key chunk (the chunk length is a parameter), the softmax denominator
 * sums unquantized P, the quotient |x|/S and amax/6 are fp32 IEEE divisions,
 * E4M3 saturates at 448 and keeps subnormals, E2M1 saturates at 6, ties go to
 * the even code, and a zero block scale gives signed zeros.
 *
 * Precision: the codec runs in fp32 (the precision both sides take the
 * rounding decisions in); dot products, softmax sums and gradients run in
 * fp64.  Build with -ffp-contract=off so no FMA contraction changes fp32
 * results.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* bf16 <-> fp32                                                            */
/* ------------------------------------------------------------------------ */

static float bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round-to-nearest-even fp32 -> bf16 (inputs here are always finite). */
static uint16_t f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

static uint16_t f64_to_bf16(double d)
{
    /* Exact RNE of a double to bf16: find the two neighbouring bf16 values
       by truncating toward zero, then compare distances in double. */
    if (d == 0.0) return signbit(d) ? 0x8000 : 0x0000;
    float f = (float)d; /* nearest fp32 */
    uint32_t u;
    memcpy(&u, &f, 4);
    uint16_t lo = (uint16_t)(u >> 16);           /* truncated magnitude */
    uint16_t hi = (uint16_t)(lo + 1);            /* next magnitude away from 0 */
    double vlo = bf16_to_f32(lo), vhi = bf16_to_f32(hi);
    double dlo = fabs(d - vlo), dhi = fabs(d - vhi);
    if (dlo < dhi) return lo;
    if (dhi < dlo) return hi;
    return (lo & 1u) ? hi : lo;
}

/* ------------------------------------------------------------------------ */
/* Codec: value tables and nearest-value search.                            */
/* ------------------------------------------------------------------------ */

/* FP8 E4M3FN ([META] qk_scale_dtype "FP8 E4M3FN"): bias 7, 3 mantissa bits,
   no infinities, code 0x7F is NaN, largest finite value 448 ([QAD] FP4_RANGE
   = 448 * 6).  Codes 0..126 are the non-negative finite values in
   increasing order. */
static float e4m3_table[127];
/* E2M1 magnitudes ([META] qk_format "NVFP4 E2M1"): codes 0..7. */
static const float e2m1_table[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

static void init_tables(void)
{
    static int done = 0;
    if (done) return;
    for (int code = 0; code < 127; ++code) {
        int e = code >> 3, m = code & 7;
        e4m3_table[code] = (e == 0) ? ldexpf((float)m, -9)
                                    : ldexpf(1.0f + (float)m / 8.0f, e - 7);
    }
    done = 1;
}

/* Nearest entry of an increasing table to v >= 0; on an exact tie the even
   code wins; values above the last entry saturate to it. */
static int nearest_code(const float *table, int n, float v)
{
    if (v >= table[n - 1]) return n - 1;
    int best = 0;
    double bestd = fabs((double)v - (double)table[0]);
    for (int c = 1; c < n; ++c) {
        double d = fabs((double)v - (double)table[c]);
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            bestd = d;
        }
    }
    return best;
}

float oracle_e4m3(float v) { init_tables(); return e4m3_table[nearest_code(e4m3_table, 127, v)]; }
float oracle_e2m1(float v) { return e2m1_table[nearest_code(e2m1_table, 8, v)]; }
int oracle_e2m1_code(float v) { return nearest_code(e2m1_table, 8, v); }

/* Block scale actually used to dequantize, for a block with abs-max `amax`
   under global scale g: s = E4M3(fp32(fp32(amax / 6) * g)), S = fp32(s / g). */
float oracle_block_scale(float amax, float g)
{
    init_tables();
    volatile float a6 = amax / 6.0f;
    volatile float sg = a6 * g;
    float s = oracle_e4m3(sg);
    volatile float S = s / g;
    return S;
}

/* One fake-quantized element given its block scale S: E2M1 of fp32(|x|/S),
   times S, sign restored. */
static float fq_elem(float x, float S)
{
    if (S == 0.0f) return copysignf(0.0f, x);
    volatile float r = fabsf(x) / S;
    float q = oracle_e2m1(r);
    volatile float y = q * S;
    return copysignf(y, x);
}

/* Exported for element-level checks: one value with a given block scale. */
float oracle_fq_value(float x, float S)
{
    init_tables();
    return fq_elem(x, S);
}

/* Fake-quantize one block of n (<= 16) fp32 values in place. */
static void fq_block_f32(float *x, int n, float g)
{
    float amax = 0.0f;
    for (int i = 0; i < n; ++i)
        if (fabsf(x[i]) > amax) amax = fabsf(x[i]);
    float S = oracle_block_scale(amax, g);
    for (int i = 0; i < n; ++i) x[i] = fq_elem(x[i], S);
}

/* Standalone fake-quant of a bf16 tensor viewed as [outer, axis, inner],
   blocks of 16 consecutive positions along `axis` (the last block may be
   shorter), global scale g (1.0 = unit).  Output is bf16 RNE of the fp32
   dequantized value.  [QAD] module docstring; [META] group_size 16. */
void oracle_fq_bf16(const uint16_t *x, uint16_t *y, int64_t outer, int64_t axis, int64_t inner,
                    float g)
{
    init_tables();
#pragma omp parallel for schedule(static)
    for (int64_t o = 0; o < outer; ++o)
        for (int64_t a0 = 0; a0 < axis; a0 += 16) {
            int n = (int)((axis - a0) < 16 ? (axis - a0) : 16);
            float buf[16];
            for (int64_t in = 0; in < inner; ++in) {
                for (int i = 0; i < n; ++i)
                    buf[i] = bf16_to_f32(x[(o * axis + a0 + i) * inner + in]);
                fq_block_f32(buf, n, g);
                for (int i = 0; i < n; ++i)
                    y[(o * axis + a0 + i) * inner + in] = f32_to_bf16(buf[i]);
            }
        }
}

/* Static global scale [QAD] weight_global_sf / input_global_sf:
   g = 448*6 / max(nan_to_num(amax|x|), 1e-12), in fp32. */
float oracle_static_scale_bf16(const uint16_t *x, int64_t n)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float v = fabsf(bf16_to_f32(x[i]));
        if (isnan(v)) v = 0.0f;
        if (v > amax) amax = v;
    }
    if (amax < 1e-12f) amax = 1e-12f;
    volatile float g = (448.0f * 6.0f) / amax;
    return g;
}

/* Fake-quant of fp32 values in blocks of 16 along a contiguous vector (used by
   the tests to exercise the codec on fp32 inputs such as softmax
   probabilities). */
void oracle_fq_f32_rows(const float *x, float *y, int64_t rows, int64_t len, float g)
{
    init_tables();
    float buf[16];
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t a0 = 0; a0 < len; a0 += 16) {
            int n = (int)((len - a0) < 16 ? (len - a0) : 16);
            for (int i = 0; i < n; ++i) buf[i] = x[r * len + a0 + i];
            fq_block_f32(buf, n, g);
            for (int i = 0; i < n; ++i) y[r * len + a0 + i] = buf[i];
        }
}

/* ------------------------------------------------------------------------ */
/* Attention.  Tensors are [B, H, L, D] bf16 (row-major); D is the head size. */
/* ------------------------------------------------------------------------ */

enum { QF_Q = 1, QF_K = 2, QF_V = 4, QF_P = 8 };
/* Variants named by the [API] flag list and the [META] precision records
   (use_global_sf_qkv, use_global_sf_p, smooth_k; "sm100_exact_m" and the
   reference-order statistics of the "Attn-QAT Training" guide); their
   arithmetic is the reading given with each use below. */
enum { QF_FINAL_MAX = 16, QF_GSF_QKV = 32, QF_GSF_P = 64, QF_SMOOTH_K = 128, QF_TWO_LEVEL_P = 256,
       QF_SMOOTH_Q = 512, QF_PV_FP8 = 1024 };

/* FP8 P.V product ([META] precision records, flag pv_fp8; named there, not
   defined).  Reading: both operands of the P.V product, as the BF16 path forms
   them (P-hat, or P rounded to bf16 when P is not quantized; V-hat rounded to
   bf16), are rounded to FP8 E4M3FN - nearest value with ties to the even
   code, subnormals kept, saturating at 448, sign kept - and multiplied with
   fp32 accumulation (a product of two E4M3 values is exact).  The
   straight-through backward uses the same operands: dP against the rounded
   V, dV from the rounded P-hat times exp(m_c - lse), and o_hp (unquantized P
   times the rounded V) for D. */
static void round_e4m3_vals(float *x, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) x[i] = copysignf(oracle_e4m3(fabsf(x[i])), x[i]);
}

/* Two-level quantization of P ([API] two_level_quant_p_sage3; the
   SageAttention3 recipe the flag is named after): a first, per-row level maps
   the largest P of the row within the chunk to 448*6, and the NVFP4 blocks are
   quantized under that scale as under a static global scale (E4M3 block
   scales of fp32(amax/6)*g, S = fp32(s/g)).  Per chunk and row:
   g = fp32(448*6 / max_t P[t]) over the chunk's live keys (448*6 when that
   maximum is 0).  Not combined with QF_FINAL_MAX or QF_GSF_P. */
static float two_level_scale(const float *P, const int64_t *kc, int chunk)
{
    float rm = 0.0f;
    for (int t = 0; t < chunk; ++t)
        if (kc[t] >= 0 && P[t] > rm) rm = P[t];
    if (!(rm > 0.0f)) return 448.0f * 6.0f;
    volatile float g = (448.0f * 6.0f) / rm;
    return g;
}

/* Per-head operands after fake quantization: Q and K along D, V along the
   key axis ([META] quant_v, qk_format/pv_format).  They are the operands of a
   BF16 matmul ([META] "NVFP4 fake-quant with BF16 matmul"), so each value is
   rounded to bf16 after dequantization; under the unit global scale this
   changes nothing (an E2M1 value times an E4M3 scale is exact in bf16). */
typedef struct {
    float *qh;     /* [Lq, D] */
    float *kh;     /* [Lk, D] */
    float *vh;     /* [Lk, D] */
    float gp;      /* global scale of P's blocks */
    float *qbar;   /* smooth-Q: [D] the queries' mean, else NULL */
    double *delta; /* smooth-Q: [Lk] <qbar, k-hat_j>, else NULL */
} head_ops;

/* Global scales of one call: unit, or static per tensor (QF_GSF_QKV: the
   [QAD] input_global_sf formula 448*6/amax over the whole tensor, taken on
   the values that are quantized, i.e. after smoothing), and for P
   (QF_GSF_P: 448*6 / 1, P's largest value being exp(0) = 1). */
typedef struct {
    float gq, gk, gv, gp;
} call_scales;

static void load_head(const uint16_t *src, float *dst, int64_t L, int D)
{
    for (int64_t i = 0; i < L * D; ++i) dst[i] = bf16_to_f32(src[i]);
}

static void quant_rows_D(float *x, int64_t L, int D, float g)
{
    for (int64_t i = 0; i < L; ++i)
        for (int d0 = 0; d0 < D; d0 += 16) fq_block_f32(x + i * D + d0, D - d0 < 16 ? D - d0 : 16, g);
}

static void quant_cols_L(float *x, int64_t L, int D, float g)
{
    float buf[16];
    for (int d = 0; d < D; ++d)
        for (int64_t j0 = 0; j0 < L; j0 += 16) {
            int n = (int)((L - j0) < 16 ? (L - j0) : 16);
            for (int i = 0; i < n; ++i) buf[i] = x[(j0 + i) * D + d];
            fq_block_f32(buf, n, g);
            for (int i = 0; i < n; ++i) x[(j0 + i) * D + d] = buf[i];
        }
}

static void round_bf16(float *x, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) x[i] = bf16_to_f32(f32_to_bf16(x[i]));
}

/* Smooth-K (flag smooth_k): the keys' mean over the sequence, per channel,
   is subtracted before quantization.  Reading: the mean is the fp64 sum over
   the L keys divided by L, rounded to fp32; the smoothed key is
   fp32(k - mean).  Every logit of a query row moves by the same amount, so
   the softmax is unchanged. */
static void smooth_rows(float *x, int64_t L, int D)
{
    for (int d = 0; d < D; ++d) {
        double s = 0.0;
        for (int64_t j = 0; j < L; ++j) s += (double)x[j * D + d];
        float mean = (float)(s / (double)L);
        for (int64_t j = 0; j < L; ++j) {
            volatile float t = x[j * D + d] - mean;
            x[j * D + d] = t;
        }
    }
}

/* Smooth-Q (flag smooth_q; SageAttention2's smoothing of Q): the queries'
   mean over the sequence, per channel (the smooth-K reading: fp64 sum / L,
   rounded to fp32), is subtracted before quantization, and its part of every
   logit is added back in full precision: S_ij = scale * (<q-hat'_i, k-hat_j>
   + delta_j) with q-hat' = fq(fp32(q - mean)) and delta_j = <mean, k-hat_j>
   (fp64).  Unlike smooth-K the shift is per key, so it must be restored.
   Under the straight-through estimator the effective query is q-hat' + mean:
   dQ is unchanged (dS k-hat) and dK_j = scale * sum_i dS_ij (q-hat'_i + mean). */
static void smooth_rows_mean(float *x, int64_t L, int D, float *mean)
{
    for (int d = 0; d < D; ++d) {
        double s = 0.0;
        for (int64_t j = 0; j < L; ++j) s += (double)x[j * D + d];
        mean[d] = (float)(s / (double)L);
    }
    smooth_rows(x, L, D);
}

/* 448*6 / max(amax, 1e-12) over all B*H heads of a [B*H, L, D] tensor, on
   the values that are quantized (smoothed first when `smooth`). */
static float tensor_scale(const uint16_t *x, int64_t BH, int64_t L, int D, int smooth)
{
    float amax = 0.0f;
    float *buf = (float *)malloc(sizeof(float) * L * D);
    for (int64_t bh = 0; bh < BH; ++bh) {
        load_head(x + bh * L * D, buf, L, D);
        if (smooth) smooth_rows(buf, L, D);
        for (int64_t i = 0; i < L * D; ++i) {
            float a = fabsf(buf[i]);
            if (isnan(a)) a = 0.0f;
            if (a > amax) amax = a;
        }
    }
    free(buf);
    if (amax < 1e-12f) amax = 1e-12f;
    volatile float g = (448.0f * 6.0f) / amax;
    return g;
}

static call_scales make_scales(const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t BH, int64_t Lq,
                               int64_t Lk, int D, unsigned flags)
{
    call_scales c = {1.0f, 1.0f, 1.0f, 1.0f};
    if (flags & QF_GSF_QKV) {
        c.gq = tensor_scale(q, BH, Lq, D, (flags & QF_SMOOTH_Q) != 0);
        c.gk = tensor_scale(k, BH, Lk, D, (flags & QF_SMOOTH_K) != 0);
        c.gv = tensor_scale(v, BH, Lk, D, 0);
    }
    if (flags & QF_GSF_P) c.gp = 448.0f * 6.0f;
    return c;
}

static void make_head_ops(head_ops *h, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                          int64_t Lq, int64_t Lk, int D, unsigned flags, const call_scales *cs)
{
    h->qh = (float *)malloc(sizeof(float) * Lq * D);
    h->kh = (float *)malloc(sizeof(float) * Lk * D);
    h->vh = (float *)malloc(sizeof(float) * Lk * D);
    h->gp = cs->gp;
    h->qbar = NULL;
    h->delta = NULL;
    load_head(q, h->qh, Lq, D);
    load_head(k, h->kh, Lk, D);
    load_head(v, h->vh, Lk, D);
    if (flags & QF_SMOOTH_K) smooth_rows(h->kh, Lk, D);
    if (flags & QF_SMOOTH_Q) {
        h->qbar = (float *)malloc(sizeof(float) * D);
        smooth_rows_mean(h->qh, Lq, D, h->qbar);
    }
    if (flags & QF_Q) quant_rows_D(h->qh, Lq, D, cs->gq);
    if (flags & QF_K) quant_rows_D(h->kh, Lk, D, cs->gk);
    if (flags & QF_V) quant_cols_L(h->vh, Lk, D, cs->gv);
    round_bf16(h->qh, Lq * D);
    round_bf16(h->kh, Lk * D);
    round_bf16(h->vh, Lk * D);
    if (flags & QF_PV_FP8) round_e4m3_vals(h->vh, Lk * D);
    if (h->qbar) {
        h->delta = (double *)malloc(sizeof(double) * Lk);
        for (int64_t j = 0; j < Lk; ++j) {
            double t = 0.0;
            for (int d = 0; d < D; ++d) t += (double)h->qbar[d] * (double)h->kh[j * D + d];
            h->delta[j] = t;
        }
    }
}

static void free_head_ops(head_ops *h)
{
    free(h->qh);
    free(h->kh);
    free(h->vh);
    free(h->qbar);
    free(h->delta);
}

/* S_ij = fp32(scale * (<q_i, k_j> + delta_j)), in fp64 (delta: smooth-Q). */
static float logit(const head_ops *h, int64_t i, int64_t j, int D, double scale)
{
    const float *a = h->qh + i * D, *b = h->kh + j * D;
    double s = 0.0;
    for (int d = 0; d < D; ++d) s += (double)a[d] * (double)b[d];
    if (h->delta) s += h->delta[j];
    return (float)(scale * s);
}

/* The query the key gradients see: q-hat (+ the smoothed-away mean). */
static double q_eff(const head_ops *h, int64_t i, int d, int D)
{
    return (double)h->qh[i * D + d] + (h->qbar ? (double)h->qbar[d] : 0.0);
}

/* Online-softmax forward for one query row (the fine stage of both the dense
   and the cube-sparse method).  The keys are visited as a list of chunks; in
   each chunk the running max is refreshed first, then P = exp(S - m) is
   formed, fake-quantized over 16-key blocks (keys aligned to the chunk start;
   masked or absent keys count as 0), and folded into the accumulators.
   keys[c*chunk + t] is the key index of position t of chunk c, or -1 when
   the position is masked/absent.
   Outputs: o (quantized-P output), o_hp (auxiliary high-precision output,
   unquantized P; [API] use_high_prec_o), lse = m + ln l, and the running
   max after every chunk (cmax[c], -inf for a chunk that had no live key). */
static void row_forward(const head_ops *h, int64_t i, const int64_t *keys, int64_t nchunks, int chunk,
                        int D, double scale, unsigned flags, double *o, double *o_hp, double *lse,
                        double *cmax, double *pscale)
{
    float *S = (float *)malloc(sizeof(float) * chunk);
    float *P = (float *)malloc(sizeof(float) * chunk);
    float *Pq = (float *)malloc(sizeof(float) * chunk);
    double *acc = (double *)calloc(D, sizeof(double));
    double *acc_hp = (double *)calloc(D, sizeof(double));
    float m = -INFINITY;
    double l = 0.0;
    for (int64_t c = 0; c < nchunks; ++c) {
        const int64_t *kc = keys + c * chunk;
        int live = 0;
        float cm = -INFINITY;
        for (int t = 0; t < chunk; ++t) {
            if (kc[t] < 0) continue;
            S[t] = logit(h, i, kc[t], D, scale);
            if (S[t] > cm) cm = S[t];
            live = 1;
        }
        if (!live) {
            if (cmax) cmax[c] = -INFINITY;
            if (pscale) pscale[c] = h->gp;
            continue;
        }
        float m_new = m > cm ? m : cm;
        for (int t = 0; t < chunk; ++t)
            P[t] = (kc[t] < 0) ? 0.0f : (float)exp((double)S[t] - (double)m_new);
        memcpy(Pq, P, sizeof(float) * chunk);
        const float gp = (flags & QF_TWO_LEVEL_P) ? two_level_scale(P, kc, chunk) : h->gp;
        if (pscale) pscale[c] = gp;
        if (flags & QF_P) {
            for (int t0 = 0; t0 < chunk; t0 += 16) fq_block_f32(Pq + t0, chunk - t0 < 16 ? chunk - t0 : 16, gp);
            round_bf16(Pq, chunk); /* the P-hat V-hat matmul operand */
        }
        if (flags & QF_PV_FP8) {
            round_bf16(Pq, chunk); /* the BF16 path's operand (no change when P is quantized) */
            round_e4m3_vals(Pq, chunk);
        }
        double alpha = (m == -INFINITY) ? 0.0 : exp((double)m - (double)m_new);
        double psum = 0.0;
        for (int t = 0; t < chunk; ++t) psum += (double)P[t];
        l = alpha * l + psum;
        for (int d = 0; d < D; ++d) {
            double a = 0.0, ahp = 0.0;
            for (int t = 0; t < chunk; ++t) {
                if (kc[t] < 0) continue;
                double vv = (double)h->vh[kc[t] * D + d];
                a += (double)Pq[t] * vv;
                ahp += (double)P[t] * vv;
            }
            acc[d] = alpha * acc[d] + a;
            acc_hp[d] = alpha * acc_hp[d] + ahp;
        }
        if (cmax) cmax[c] = m_new;
        m = m_new;
    }
    for (int d = 0; d < D; ++d) {
        if (o) o[d] = acc[d] / l;
        if (o_hp) o_hp[d] = acc_hp[d] / l;
    }
    if (lse) *lse = (double)m + log(l);
    free(S);
    free(P);
    free(Pq);
    free(acc);
    free(acc_hp);
}

/* Dense key schedule: chunk c holds keys [c*chunk, c*chunk+chunk) clipped to
   Lk; with causal masking, keys after the query row are masked (top-left
   alignment, Lq == Lk). */
static int64_t *dense_keys(int64_t Lk, int chunk, int64_t i, int causal, int64_t *nchunks)
{
    int64_t C = (Lk + chunk - 1) / chunk;
    int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * C * chunk);
    for (int64_t p = 0; p < C * chunk; ++p) {
        int64_t j = p;
        keys[p] = (j >= Lk || (causal && j > i)) ? -1 : j;
    }
    *nchunks = C;
    return keys;
}

/* Forward for the requested query rows of every (b, h).
   Outputs (any may be NULL), indexed [bh][r] for row rows[r]:
     o, o_hp : [B*H, nrows, D] fp64
     lse     : [B*H, nrows]
     cmax    : [B*H, nrows, ceil(Lk/chunk)]
     pscale  : [B*H, nrows, ceil(Lk/chunk)], the global scale P's blocks
               had in each chunk (two_level_scale under QF_TWO_LEVEL_P).  */
int oracle_attn_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, int B, int H, int64_t Lq,
                    int64_t Lk, int D, double scale, int causal, unsigned flags, int chunk,
                    const int64_t *rows, int64_t nrows, double *o, double *o_hp, double *lse,
                    double *cmax, double *pscale)
{
    init_tables();
    if (causal && Lq != Lk) return -1;
    if ((flags & QF_TWO_LEVEL_P) && (flags & (QF_FINAL_MAX | QF_GSF_P))) return -2;
    if (flags & QF_FINAL_MAX) chunk = (int)((Lk + 15) / 16 * 16);
    int64_t C = (Lk + chunk - 1) / chunk;
    const call_scales cs = make_scales(q, k, v, (int64_t)B * H, Lq, Lk, D, flags);
    for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
        head_ops hd;
        make_head_ops(&hd, q + bh * Lq * D, k + bh * Lk * D, v + bh * Lk * D, Lq, Lk, D, flags, &cs);
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t nc;
            int64_t *keys = dense_keys(Lk, chunk, rows[r], causal, &nc);
            int64_t idx = bh * nrows + r;
            row_forward(&hd, rows[r], keys, nc, chunk, D, scale, flags, o ? o + idx * D : NULL,
                        o_hp ? o_hp + idx * D : NULL, lse ? lse + idx : NULL,
                        cmax ? cmax + idx * C : NULL, pscale ? pscale + idx * C : NULL);
            free(keys);
        }
        free_head_ops(&hd);
    }
    return 0;
}

/* Straight-through backward ([META] backward "consistent STE with auxiliary
   output"; [API] use_qat_qkv_backward, fake_quant_p_bwd, use_high_prec_o).
   Fake-quant nodes pass gradients unchanged and the running maxima are
   constants, so with A = exp(S - LSE) (unquantized probabilities) and
   Ahat = fq(exp(S - m_c)) * exp(m_c - LSE) (the probabilities the forward
   multiplied V with):
     D_i   = <dO_i, Ohp_i>
     dV_j  = sum_i Ahat_ij dO_i
     dP_ij = <dO_i, Vhat_j>
     dS_ij = A_ij (dP_ij - D_i)
     dQ_i  = scale sum_j dS_ij Khat_j,   dK_j = scale sum_i dS_ij Qhat_i. */

typedef struct {
    const head_ops *hd;
    const uint16_t *dO; /* [Lq, D] bf16 of this head */
    int64_t Lk, C;
    int D, chunk, causal;
    unsigned flags;
    double scale;
} bwd_head;

/* The 16-key block that holds key j (blocks start at multiples of 16 from
   the start of j's chunk): first key and length. */
static void key_block(const bwd_head *x, int64_t j, int64_t *b0, int *nb)
{
    int64_t c0 = (j / x->chunk) * x->chunk;
    int64_t s = c0 + ((j - c0) / 16) * 16;
    int64_t e = s + 16;
    if (e > c0 + x->chunk) e = c0 + x->chunk;
    if (e > x->Lk) e = x->Lk;
    *b0 = s;
    *nb = (int)(e - s);
}

/* For row i with forward statistics (lse, m_c the running max after the
   chunk that holds the block, and g the global scale its P blocks had) and
   key block [b0, b0+nb):
   A[t] = exp(S - lse), Ahat[t] = fq(exp(S - m_c), g)[t] * exp(m_c - lse),
   for the block's keys (masked keys give 0). */
static void block_weights_mc(const bwd_head *x, int64_t i, int64_t b0, int nb, double lse, double mc, float g,
                             double *A, double *Ahat)
{
    float P[16];
    float S[16];
    for (int t = 0; t < nb; ++t) {
        int live = !(x->causal && b0 + t > i);
        S[t] = live ? logit(x->hd, i, b0 + t, x->D, x->scale) : -INFINITY;
        P[t] = live ? (float)exp((double)S[t] - mc) : 0.0f;
    }
    if (x->flags & QF_P) {
        fq_block_f32(P, nb, g);
        round_bf16(P, nb);
    }
    if (x->flags & QF_PV_FP8) {
        round_bf16(P, nb);
        round_e4m3_vals(P, nb);
    }
    for (int t = 0; t < nb; ++t) {
        int live = !(x->causal && b0 + t > i);
        A[t] = live ? exp((double)S[t] - lse) : 0.0;
        Ahat[t] = (double)P[t] * exp(mc - lse);
    }
}

/* Dense schedule: the block's chunk is the one its keys fall in. */
static void block_weights(const bwd_head *x, int64_t i, int64_t b0, int nb, double lse, const double *cmax,
                          const double *pscale, double *A, double *Ahat)
{
    block_weights_mc(x, i, b0, nb, lse, cmax[b0 / x->chunk], (float)pscale[b0 / x->chunk], A, Ahat);
}

static double dot_do_v(const bwd_head *x, int64_t i, int64_t j)
{
    double s = 0.0;
    for (int d = 0; d < x->D; ++d)
        s += (double)bf16_to_f32(x->dO[i * x->D + d]) * (double)x->hd->vh[j * x->D + d];
    return s;
}

/* Forward statistics of row i: lse, running max and P's global scale per
   chunk, and D_i = <dO_i, Ohp_i>. */
static void row_stats(const bwd_head *x, int64_t i, double *lse, double *cmax, double *pscale, double *Di)
{
    int64_t nc;
    int64_t *keys = dense_keys(x->Lk, x->chunk, i, x->causal, &nc);
    double *ohp = (double *)malloc(sizeof(double) * x->D);
    row_forward(x->hd, i, keys, nc, x->chunk, x->D, x->scale, x->flags, NULL, ohp, lse, cmax, pscale);
    double s = 0.0;
    for (int d = 0; d < x->D; ++d) s += (double)bf16_to_f32(x->dO[i * x->D + d]) * ohp[d];
    *Di = s;
    free(ohp);
    free(keys);
}

/* Computes dQ for query rows qrows and dK, dV for key rows krows, per (b,h).
   Outputs fp64: dq [B*H, nq, D], dk/dv [B*H, nk, D]. */
int oracle_attn_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *dout, int B,
                    int H, int64_t Lq, int64_t Lk, int D, double scale, int causal, unsigned flags,
                    int chunk, const int64_t *qrows, int64_t nq, const int64_t *krows, int64_t nk,
                    double *dq, double *dk, double *dv)
{
    init_tables();
    if (causal && Lq != Lk) return -1;
    if ((flags & QF_TWO_LEVEL_P) && (flags & (QF_FINAL_MAX | QF_GSF_P))) return -2;
    if (flags & QF_FINAL_MAX) chunk = (int)((Lk + 15) / 16 * 16);
    int64_t C = (Lk + chunk - 1) / chunk;
    const call_scales cs = make_scales(q, k, v, (int64_t)B * H, Lq, Lk, D, flags);
    for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
        head_ops hd;
        make_head_ops(&hd, q + bh * Lq * D, k + bh * Lk * D, v + bh * Lk * D, Lq, Lk, D, flags, &cs);
        bwd_head x = {&hd, dout + bh * Lq * D, Lk, C, D, chunk, causal, flags, scale};

        if (dq && nq > 0) {
#pragma omp parallel for schedule(dynamic, 1)
            for (int64_t a = 0; a < nq; ++a) {
                int64_t i = qrows[a];
                double lse, Di, A[16], Ah[16];
                double *cmax = (double *)malloc(sizeof(double) * C);
                double *pg = (double *)malloc(sizeof(double) * C);
                row_stats(&x, i, &lse, cmax, pg, &Di);
                double *out = dq + (bh * nq + a) * D;
                for (int d = 0; d < D; ++d) out[d] = 0.0;
                for (int64_t b0 = 0; b0 < Lk;) {
                    int64_t s;
                    int nb;
                    key_block(&x, b0, &s, &nb);
                    block_weights(&x, i, s, nb, lse, cmax, pg, A, Ah);
                    for (int t = 0; t < nb; ++t) {
                        int64_t j = s + t;
                        if (causal && j > i) continue;
                        double dS = A[t] * (dot_do_v(&x, i, j) - Di);
                        for (int d = 0; d < D; ++d) out[d] += scale * dS * (double)hd.kh[j * D + d];
                    }
                    b0 = s + nb;
                }
                free(cmax);
                free(pg);
            }
        }

        if (nk > 0 && (dk || dv)) {
            /* Key gradients need every row's statistics. */
            double *lse = (double *)malloc(sizeof(double) * Lq);
            double *cmax = (double *)malloc(sizeof(double) * Lq * C);
            double *pg = (double *)malloc(sizeof(double) * Lq * C);
            double *Dv = (double *)malloc(sizeof(double) * Lq);
#pragma omp parallel for schedule(dynamic, 16)
            for (int64_t i = 0; i < Lq; ++i) row_stats(&x, i, lse + i, cmax + i * C, pg + i * C, Dv + i);
#pragma omp parallel for schedule(dynamic, 1)
            for (int64_t a = 0; a < nk; ++a) {
                int64_t j = krows[a];
                int64_t s;
                int nb;
                key_block(&x, j, &s, &nb);
                double *ok = dk ? dk + (bh * nk + a) * D : NULL;
                double *ov = dv ? dv + (bh * nk + a) * D : NULL;
                for (int d = 0; d < D; ++d) {
                    if (ok) ok[d] = 0.0;
                    if (ov) ov[d] = 0.0;
                }
                double A[16], Ah[16];
                for (int64_t i = 0; i < Lq; ++i) {
                    if (causal && j > i) continue;
                    block_weights(&x, i, s, nb, lse[i], cmax + i * C, pg + i * C, A, Ah);
                    double dS = A[j - s] * (dot_do_v(&x, i, j) - Dv[i]);
                    for (int d = 0; d < D; ++d) {
                        if (ok) ok[d] += scale * dS * q_eff(&hd, i, d, D);
                        if (ov) ov[d] += Ah[j - s] * (double)bf16_to_f32(x.dO[i * D + d]);
                    }
                }
            }
            free(lse);
            free(cmax);
            free(pg);
            free(Dv);
        }
        free_head_ops(&hd);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Cube-sparse (VSA) forward.  [META] attention: kind "vsa", cube_shape
   [4,4,8], precision.coarse "BF16", quantize_coarse false, quantize_fine
   true, selection.effective_topk = max(1, min(ceil((1-sparsity)*n), n)).  */
/* ------------------------------------------------------------------------ */

int oracle_vsa_topk(double sparsity, int n)
{
    double t = ceil((1.0 - sparsity) * (double)n);
    int k = (int)t;
    if (k > n) k = n;
    if (k < 1) k = 1;
    return k;
}

/* Mean over each cube of `ct` consecutive tokens (tokens are cube-major),
   computed in fp64 and rounded to bf16. out: [ncubes, D] bf16. */
static void pool_cubes(const uint16_t *x, int64_t ncubes, int ct, int D, uint16_t *out)
{
    for (int64_t c = 0; c < ncubes; ++c)
        for (int d = 0; d < D; ++d) {
            double s = 0.0;
            for (int t = 0; t < ct; ++t) s += (double)bf16_to_f32(x[(c * ct + t) * D + d]);
            out[c * D + d] = f64_to_bf16(s / (double)ct);
        }
}

/* The selection of one head: cube means of Q and K (fp64, rounded to bf16),
   coarse logits scale * <Qc, Kc>, and for every query cube the topk highest
   scoring key cubes (ties to the lower cube index) listed in ascending order.
   qp, kp: [n, D] bf16; sc: [n, n]; sl: [n, topk]. */
static void vsa_select_head(const uint16_t *qh, const uint16_t *kh, int64_t n, int ct, int D, double scale,
                            int topk, uint16_t *qp, uint16_t *kp, double *sc, int32_t *sl)
{
    pool_cubes(qh, n, ct, D, qp);
    pool_cubes(kh, n, ct, D, kp);
    for (int64_t a = 0; a < n; ++a)
        for (int64_t b = 0; b < n; ++b) {
            double s = 0.0;
            for (int d = 0; d < D; ++d) s += (double)bf16_to_f32(qp[a * D + d]) * (double)bf16_to_f32(kp[b * D + d]);
            sc[a * n + b] = scale * s;
        }
    for (int64_t a = 0; a < n; ++a) {
        char *taken = (char *)calloc(n, 1);
        for (int t = 0; t < topk; ++t) {
            int64_t best = -1;
            for (int64_t b = 0; b < n; ++b)
                if (!taken[b] && (best < 0 || sc[a * n + b] > sc[a * n + best])) best = b;
            taken[best] = 1;
        }
        int t = 0;
        for (int64_t b = 0; b < n; ++b)
            if (taken[b]) sl[a * topk + t++] = (int32_t)b;
        free(taken);
    }
}

/* Key list of a query cube: its selected cubes' tokens, one chunk per cube. */
static int64_t *vsa_keys(const int32_t *sl_row, int topk, int ct)
{
    int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * topk * ct);
    for (int t = 0; t < topk; ++t)
        for (int u = 0; u < ct; ++u) keys[t * ct + u] = (int64_t)sl_row[t] * ct + u;
    return keys;
}

/* Outputs per (b,h):
     qpool, kpool, vpool : [B*H, n, D] bf16 (may be NULL)
     score   : [B*H, n, n] fp64 coarse logits scale * <Qc, Kc> (may be NULL)
     sel     : [B*H, n, topk] int32, selected cubes in ascending order
     o_fine  : [B*H, nrows, D] fp64 for the query rows `rows`
     o_coarse: [B*H, nrows, D] fp64 softmax(score) @ Vc of the row's cube
   The fine stage reuses the dense forward with the selected cubes' keys in
   ascending cube order, one chunk per cube. */
int oracle_vsa_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, int B, int H, int64_t L, int D,
                   int cube_tokens, double sparsity, double scale, unsigned flags, const int64_t *rows,
                   int64_t nrows, uint16_t *qpool, uint16_t *kpool, uint16_t *vpool, double *score,
                   int32_t *sel, double *o_fine, double *o_coarse)
{
    init_tables();
    if (L % cube_tokens) return -1;
    if ((flags & QF_TWO_LEVEL_P) && (flags & (QF_FINAL_MAX | QF_GSF_P))) return -2;
    int64_t n = L / cube_tokens;
    int topk = oracle_vsa_topk(sparsity, (int)n);
    uint16_t *qp = (uint16_t *)malloc(2 * n * D), *kp = (uint16_t *)malloc(2 * n * D),
             *vp = (uint16_t *)malloc(2 * n * D);
    double *sc = (double *)malloc(sizeof(double) * n * n);
    int32_t *sl = (int32_t *)malloc(sizeof(int32_t) * n * topk);
    /* Reference-order statistics over the selected keys: one chunk. */
    const int64_t nchunk = (flags & QF_FINAL_MAX) ? 1 : topk;
    const int chunk = (flags & QF_FINAL_MAX) ? topk * cube_tokens : cube_tokens;
    const call_scales cs = make_scales(q, k, v, (int64_t)B * H, L, L, D, flags);
    for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
        const uint16_t *qh = q + bh * L * D, *kh = k + bh * L * D, *vh = v + bh * L * D;
        vsa_select_head(qh, kh, n, cube_tokens, D, scale, topk, qp, kp, sc, sl);
        pool_cubes(vh, n, cube_tokens, D, vp);
        if (qpool) memcpy(qpool + bh * n * D, qp, 2 * n * D);
        if (kpool) memcpy(kpool + bh * n * D, kp, 2 * n * D);
        if (vpool) memcpy(vpool + bh * n * D, vp, 2 * n * D);
        if (score) memcpy(score + bh * n * n, sc, sizeof(double) * n * n);
        if (sel) memcpy(sel + bh * n * topk, sl, sizeof(int32_t) * n * topk);

        head_ops hd;
        make_head_ops(&hd, qh, kh, vh, L, L, D, flags, &cs);
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t i = rows[r];
            int64_t a = i / cube_tokens;
            int64_t *keys = vsa_keys(sl + a * topk, topk, cube_tokens);
            if (o_fine)
                row_forward(&hd, i, keys, nchunk, chunk, D, scale, flags, o_fine + (bh * nrows + r) * D,
                            NULL, NULL, NULL, NULL);
            if (o_coarse) {
                double mx = -INFINITY, l = 0.0;
                for (int64_t b = 0; b < n; ++b)
                    if (sc[a * n + b] > mx) mx = sc[a * n + b];
                double *out = o_coarse + (bh * nrows + r) * D;
                for (int d = 0; d < D; ++d) out[d] = 0.0;
                for (int64_t b = 0; b < n; ++b) {
                    double p = exp(sc[a * n + b] - mx);
                    l += p;
                    for (int d = 0; d < D; ++d) out[d] += p * (double)bf16_to_f32(vp[b * D + d]);
                }
                for (int d = 0; d < D; ++d) out[d] /= l;
            }
            free(keys);
        }
        free_head_ops(&hd);
    }
    free(qp);
    free(kp);
    free(vp);
    free(sc);
    free(sl);
    return topk;
}

/* Straight-through backward of the fine stage (the same formulas as
   oracle_attn_bwd) with each query cube attending to its selected cubes only,
   visited in ascending order with one chunk per cube.  The running max of row
   i after its t-th selected cube is the chunk max of every key block of that
   cube.  Computes dQ for query rows qrows and dK, dV for key rows krows, per
   (b,h); outputs fp64 [B*H, nq, D] and [B*H, nk, D]; sel [B*H, n, topk] (may
   be NULL).  Returns topk, or -1 when L is not a whole number of cubes. */
int oracle_vsa_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *dout, int B, int H,
                   int64_t L, int D, int cube_tokens, double sparsity, double scale, unsigned flags,
                   const int64_t *qrows, int64_t nq, const int64_t *krows, int64_t nk, double *dq, double *dk,
                   double *dv, int32_t *sel)
{
    init_tables();
    if (L % cube_tokens) return -1;
    if ((flags & QF_TWO_LEVEL_P) && (flags & (QF_FINAL_MAX | QF_GSF_P))) return -2;
    const int64_t n = L / cube_tokens;
    const int ct = cube_tokens;
    const int topk = oracle_vsa_topk(sparsity, (int)n);
    uint16_t *qp = (uint16_t *)malloc(2 * n * D), *kp = (uint16_t *)malloc(2 * n * D);
    double *sc = (double *)malloc(sizeof(double) * n * n);
    int32_t *sl = (int32_t *)malloc(sizeof(int32_t) * n * topk);
    /* Reference-order statistics over the selected keys: one chunk, whose
       maximum every block of every selected cube uses. */
    const int fm = (flags & QF_FINAL_MAX) != 0;
    const int64_t nchunk = fm ? 1 : topk;
    const call_scales cs = make_scales(q, k, v, (int64_t)B * H, L, L, D, flags);
    for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
        const uint16_t *qh = q + bh * L * D, *kh = k + bh * L * D, *vh = v + bh * L * D;
        vsa_select_head(qh, kh, n, ct, D, scale, topk, qp, kp, sc, sl);
        if (sel) memcpy(sel + bh * n * topk, sl, sizeof(int32_t) * n * topk);
        head_ops hd;
        make_head_ops(&hd, qh, kh, vh, L, L, D, flags, &cs);
        bwd_head x = {&hd, dout + bh * L * D, L, n, D, ct, 0, flags, scale};

        /* Row statistics (lse, running max after each selected cube, D_i). */
        double *lse = (double *)malloc(sizeof(double) * L);
        double *cmax = (double *)malloc(sizeof(double) * L * topk);
        double *pg = (double *)malloc(sizeof(double) * L * topk);
        double *Dv = (double *)malloc(sizeof(double) * L);
        char *need = (char *)calloc(L, 1);
        for (int64_t a = 0; a < nq; ++a) need[qrows[a]] = 1;
        if (nk > 0 && (dk || dv))
            for (int64_t i = 0; i < L; ++i) need[i] = 1;
#pragma omp parallel for schedule(dynamic, 16)
        for (int64_t i = 0; i < L; ++i) {
            if (!need[i]) continue;
            int64_t *keys = vsa_keys(sl + (i / ct) * topk, topk, ct);
            double *ohp = (double *)malloc(sizeof(double) * D);
            row_forward(&hd, i, keys, nchunk, fm ? topk * ct : ct, D, scale, flags, NULL, ohp, lse + i,
                        cmax + i * topk, pg + i * topk);
            double s = 0.0;
            for (int d = 0; d < D; ++d) s += (double)bf16_to_f32(x.dO[i * D + d]) * ohp[d];
            Dv[i] = s;
            free(ohp);
            free(keys);
        }

        if (dq && nq > 0) {
#pragma omp parallel for schedule(dynamic, 1)
            for (int64_t a = 0; a < nq; ++a) {
                int64_t i = qrows[a];
                const int32_t *row_sel = sl + (i / ct) * topk;
                double *out = dq + (bh * nq + a) * D;
                double A[16], Ah[16];
                for (int d = 0; d < D; ++d) out[d] = 0.0;
                for (int t = 0; t < topk; ++t)
                    for (int64_t b0 = (int64_t)row_sel[t] * ct; b0 < (int64_t)(row_sel[t] + 1) * ct; b0 += 16) {
                        int64_t s;
                        int nb;
                        key_block(&x, b0, &s, &nb);
                        block_weights_mc(&x, i, s, nb, lse[i], cmax[i * topk + (fm ? 0 : t)],
                                         (float)pg[i * topk + (fm ? 0 : t)], A, Ah);
                        for (int u = 0; u < nb; ++u) {
                            int64_t j = s + u;
                            double dS = A[u] * (dot_do_v(&x, i, j) - Dv[i]);
                            for (int d = 0; d < D; ++d) out[d] += scale * dS * (double)hd.kh[j * D + d];
                        }
                    }
            }
        }

        if (nk > 0 && (dk || dv)) {
#pragma omp parallel for schedule(dynamic, 1)
            for (int64_t a = 0; a < nk; ++a) {
                int64_t j = krows[a];
                int64_t s;
                int nb;
                key_block(&x, j, &s, &nb);
                double *ok = dk ? dk + (bh * nk + a) * D : NULL;
                double *ov = dv ? dv + (bh * nk + a) * D : NULL;
                for (int d = 0; d < D; ++d) {
                    if (ok) ok[d] = 0.0;
                    if (ov) ov[d] = 0.0;
                }
                double A[16], Ah[16];
                const int64_t b = j / ct;
                for (int64_t qc = 0; qc < n; ++qc) {
                    int t = -1;
                    for (int u = 0; u < topk; ++u)
                        if (sl[qc * topk + u] == b) t = u;
                    if (t < 0) continue;  /* this query cube did not select j's cube */
                    for (int64_t i = qc * ct; i < (qc + 1) * ct; ++i) {
                        block_weights_mc(&x, i, s, nb, lse[i], cmax[i * topk + (fm ? 0 : t)],
                                         (float)pg[i * topk + (fm ? 0 : t)], A, Ah);
                        double dS = A[j - s] * (dot_do_v(&x, i, j) - Dv[i]);
                        for (int d = 0; d < D; ++d) {
                            if (ok) ok[d] += scale * dS * q_eff(&hd, i, d, D);
                            if (ov) ov[d] += Ah[j - s] * (double)bf16_to_f32(x.dO[i * D + d]);
                        }
                    }
                }
            }
        }
        free(lse);
        free(cmax);
        free(pg);
        free(Dv);
        free(need);
        free_head_ops(&hd);
    }
    free(qp);
    free(kp);
    free(sc);
    free(sl);
    return topk;
}

/* ------------------------------------------------------------------------ */
/* NVFP4 QAD linear.  ["nvfp4_qad.py"] module docstring and nvfp4_gemm: the    */
/* weight is RTN NVFP4 under g_w = 448*6 / amax(|W|) (weight_global_sf), the   */
/* activation per-16 E4M3 blocks under a unit or static global scale          */
/* (input_global_sf), blocks along the input features (the contraction axis); */
/* the product of the dequantized operands plus the bias.  _NVFP4STE backward: */
/* full-precision grad_x = grad @ W, grad_w = grad^T @ x, grad_b = sum grad.  */
/* Reading: the operands of the (BF16) matmul are the dequantized values      */
/* rounded to bf16 (as fq_nvfp4 outputs them); sums are fp64.                 */
/* ------------------------------------------------------------------------ */

/* y [M, N] fp64 = fq(x, gx) [M, K] . fq(w, g_w) [N, K]^T + bias, with
   g_w = oracle_static_scale_bf16(w).  bias may be NULL.  gx = 1: unit scale. */
void oracle_linear_fwd(const uint16_t *x, const uint16_t *w, const uint16_t *bias, int64_t M, int64_t N,
                       int64_t K, float gx, double *y)
{
    init_tables();
    uint16_t *xq = (uint16_t *)malloc(2 * M * K), *wq = (uint16_t *)malloc(2 * N * K);
    oracle_fq_bf16(x, xq, M, K, 1, gx);
    oracle_fq_bf16(w, wq, N, K, 1, oracle_static_scale_bf16(w, N * K));
    float *xf = (float *)malloc(sizeof(float) * M * K), *wf = (float *)malloc(sizeof(float) * N * K);
    for (int64_t i = 0; i < M * K; ++i) xf[i] = bf16_to_f32(xq[i]);
    for (int64_t i = 0; i < N * K; ++i) wf[i] = bf16_to_f32(wq[i]);
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double s = bias ? (double)bf16_to_f32(bias[n]) : 0.0;
            for (int64_t k = 0; k < K; ++k) s += (double)xf[m * K + k] * (double)wf[n * K + k];
            y[m * N + n] = s;
        }
    free(xq);
    free(wq);
    free(xf);
    free(wf);
}

/* Straight-through backward of the linear: gx [M, K] = g [M, N] . w [N, K],
   gw [N, K] = g^T . x, gb [N] = column sums of g (any output may be NULL).
   Inputs bf16, outputs fp64. */
void oracle_linear_bwd(const uint16_t *g, const uint16_t *x, const uint16_t *w, int64_t M, int64_t N, int64_t K,
                       double *gx, double *gw, double *gb)
{
    if (gx) {
#pragma omp parallel for schedule(static)
        for (int64_t m = 0; m < M; ++m)
            for (int64_t k = 0; k < K; ++k) {
                double s = 0.0;
                for (int64_t n = 0; n < N; ++n) s += (double)bf16_to_f32(g[m * N + n]) * (double)bf16_to_f32(w[n * K + k]);
                gx[m * K + k] = s;
            }
    }
    if (gw) {
#pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < N; ++n)
            for (int64_t k = 0; k < K; ++k) {
                double s = 0.0;
                for (int64_t m = 0; m < M; ++m) s += (double)bf16_to_f32(g[m * N + n]) * (double)bf16_to_f32(x[m * K + k]);
                gw[n * K + k] = s;
            }
    }
    if (gb) {
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0;
            for (int64_t m = 0; m < M; ++m) s += (double)bf16_to_f32(g[m * N + n]);
            gb[n] = s;
        }
    }
}

/* Max calibration ["nvfp4_qad.py"] NVFP4QADLinearMethod.apply while calibrating:
   the running maximum folds in amax(|x|) of every input.  Returns
   max(prev, amax|x|) (NaN inputs count as 0, as the static-scale formula's nan_to_num). */
float oracle_observe_amax(const uint16_t *x, int64_t n, float prev)
{
    float amax = prev;
    for (int64_t i = 0; i < n; ++i) {
        float v = fabsf(bf16_to_f32(x[i]));
        if (isnan(v)) v = 0.0f;
        if (v > amax) amax = v;
    }
    return amax;
}
