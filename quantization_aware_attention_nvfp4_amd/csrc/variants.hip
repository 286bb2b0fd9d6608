// variants.hip - per-call quantities of the attention variants, computed on the device before the
// operands are quantized.
//
// The "attn_qat_train" API page lists the kernel flags use_global_sf_qkv, use_global_sf_p and
// smooth_k (all off in its call), and the "vsqa-preview-1.3b metadata.json" precision records
// carry the same names; the pages do not define them.  The readings built here:
//   * smooth-K: the keys' per-channel mean over the sequence, the fp64 sum over the L keys divided
//     by L and rounded to fp32, is subtracted from every key before quantization (the softmax of a
//     row ignores the common shift of its logits);
//   * static Q/K/V scales: one global scale per tensor, g = 448*6 / max(amax, 1e-12) over the
//     whole tensor ("nvfp4_qad.py": input_global_sf), on the values that are quantized (the
//     smoothed keys under smooth-K);
//   * static P scale: g = 448*6 / 1, P's largest value being exp(0) = 1 (a constant; no kernel);
//   * smooth-Q (SageAttention2's smoothing): the queries' per-channel mean (the smooth-K reading)
//     is subtracted before quantization and delta_j = <mean, k-hat_j> per key is added back to the
//     logits; the mean comes from the same slab kernels, delta from qk_delta_kernel.
//
// Both reductions are deterministic: the mean's fp64 partial sums are combined in a fixed order,
// and the abs-max is order-independent (one atomic maximum per workgroup on the float's bits,
// which order like the values for non-negative floats).
#include "aq_device.hpp"
#include "launch.hpp"
#include "timing.hpp"

namespace aq {
namespace {

constexpr int kD = kHeadDim;

__global__ __launch_bounds__(64) void fill_u32_kernel(uint32_t *__restrict__ p, int n, uint32_t v) {
  if ((int)threadIdx.x < n) p[threadIdx.x] = v;
}

// Partial sums of one slab of kMeanSlab keys of one head: part[(bh, slab), d] = sum over the
// slab's keys of k[b, l, h, d] in fp64.  Lane t reads 8 channels (one 16-byte load) of every 16th
// key of the slab, starting at key t/16; the 16 lanes that share a channel group are then added
// in key-group order through LDS.
__global__ __launch_bounds__(256) void kmean_partial_kernel(const uint16_t *__restrict__ k, Strides s, int heads,
                                                            int64_t L, int nslab, double *__restrict__ part) {
  __shared__ double acc_lds[16][kD];
  const int64_t bh = blockIdx.x / nslab;
  const int slab = (int)(blockIdx.x % nslab);
  const int64_t b = bh / heads, h = bh % heads;
  const int grp = threadIdx.x & 15, sub = threadIdx.x >> 4;
  const int64_t l0 = (int64_t)slab * kMeanSlab, l1 = l0 + kMeanSlab < L ? l0 + kMeanSlab : L;
  const uint16_t *base = k + b * s.b + h * s.h + 8 * grp;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int64_t l = l0 + sub; l < l1; l += 16) {
    const u32x4 v = *(const u32x4 *)(base + l * s.l);
    acc[0] += (double)bf16lo(v.x); acc[1] += (double)bf16hi(v.x);
    acc[2] += (double)bf16lo(v.y); acc[3] += (double)bf16hi(v.y);
    acc[4] += (double)bf16lo(v.z); acc[5] += (double)bf16hi(v.z);
    acc[6] += (double)bf16lo(v.w); acc[7] += (double)bf16hi(v.w);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) acc_lds[sub][8 * grp + j] = acc[j];
  __syncthreads();
  if (threadIdx.x < kD) {
    double t = 0.0;
    for (int i = 0; i < 16; ++i) t += acc_lds[i][threadIdx.x];
    part[(bh * nslab + slab) * kD + threadIdx.x] = t;
  }
}

// mean[bh, d] = fp32(sum of the slabs' partial sums, in slab order, / L).
__global__ __launch_bounds__(256) void kmean_final_kernel(const double *__restrict__ part, int nslab, int64_t L,
                                                          int64_t total, float *__restrict__ mean) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= total) return;
  const int64_t bh = id / kD, d = id % kD;
  double acc = 0.0;
  for (int i = 0; i < nslab; ++i) acc += part[(bh * nslab + i) * kD + d];
  mean[id] = (float)(acc / (double)L);
}

// Abs-max of a strided [B, L, H, 128] bf16 tensor (of fp32(x - mean) when mean is given) into
// *out as float bits, by an atomic maximum per workgroup.  One workgroup: one head and 64 rows;
// a lane reads 8 consecutive channels (16 bytes).
__global__ __launch_bounds__(256) void amax_kernel(const uint16_t *__restrict__ x, Strides s, int heads, int64_t L,
                                                   int64_t nblk, const float *__restrict__ mean,
                                                   uint32_t *__restrict__ out) {
  __shared__ float red[4];
  const int64_t bh = blockIdx.x / nblk, blk = blockIdx.x % nblk;
  const int64_t b = bh / heads, h = bh % heads;
  const int tid = threadIdx.x, part = tid & 15;
  const float *mrow = mean ? mean + bh * kD + 8 * part : nullptr;
  float am = 0.0f;
  for (int i = 0; i < 4; ++i) {
    const int64_t r = blk * 64 + 16 * i + (tid >> 4);
    if (r >= L) break;
    const u32x4 v = *(const u32x4 *)(x + b * s.b + h * s.h + r * s.l + 8 * part);
    float f[8] = {bf16lo(v.x), bf16hi(v.x), bf16lo(v.y), bf16hi(v.y),
                  bf16lo(v.z), bf16hi(v.z), bf16lo(v.w), bf16hi(v.w)};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float y = mrow ? f[j] - mrow[j] : f[j];
      am = fmaxf(am, __builtin_fabsf(y));
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
  if ((tid & 63) == 0) red[tid >> 6] = am;
  __syncthreads();
  if (tid == 0) {
    const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    atomicMax(out, f2u(m));
  }
}

// g[i] = 2688 / max(amax_i, 1e-12) for Q, K, V (1 without the static Q/K/V scales), g[3] = the P
// scale.  Layout of scal: float g[4], then uint32 amax bits[3].
__global__ void gsf_final_kernel(float *__restrict__ scal, int qkv, int pscale) {
  if (threadIdx.x != 0) return;
  const uint32_t *bits = (const uint32_t *)(scal + 4);
  for (int i = 0; i < 3; ++i) {
    float amax = u2f(bits[i]);
    if (amax < 1e-12f) amax = 1e-12f;
    scal[i] = qkv ? (448.0f * 6.0f) / amax : 1.0f;
  }
  scal[3] = pscale ? 448.0f * 6.0f : 1.0f;
}

// delta[row] = <qmean[bh], kq[row]> for the K-hat rows (256 bytes each, plain layout) of every
// head: 16 lanes per row, lane i taking channels 8i .. 8i+7 in order (fp32 fma), then a fixed
// butterfly over the 16 lanes.
__global__ __launch_bounds__(256) void qk_delta_kernel(const u32x4 *__restrict__ kq, const float *__restrict__ qmean,
                                                       int64_t rows_per_head, int64_t total_rows,
                                                       float *__restrict__ delta) {
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int part = threadIdx.x & 15;
  float acc = 0.0f;
  if (row < total_rows) {
    const u32x4 v = kq[row * 16 + part];
    const float *m = qmean + (row / rows_per_head) * kD + 8 * part;
    const float f[8] = {bf16lo(v.x), bf16hi(v.x), bf16lo(v.y), bf16hi(v.y),
                        bf16lo(v.z), bf16hi(v.z), bf16lo(v.w), bf16hi(v.w)};
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = __builtin_fmaf(f[i], m[i], acc);
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) acc += __shfl_xor(acc, o, 64);
  if (part == 0 && row < total_rows) delta[row] = acc;
}

hipError_t launch_amax(const void *x, Strides s, int batch, int heads, int64_t L, const float *mean, uint32_t *out,
                       hipStream_t stream) {
  const int64_t nblk = (L + 63) / 64;
  const int64_t blocks = (int64_t)batch * heads * nblk;
  AQ_LAUNCH("amax", amax_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const uint16_t *)x, s, heads, L,
            nblk, mean, out);
  return hipGetLastError();
}

}  // namespace

VariantPtrs variant_ptrs(const AttnArgs &a, const Workspace &w) {
  uint8_t *ws = (uint8_t *)a.workspace;
  const float *scal = (const float *)(ws + w.scal);
  const bool qkv = (a.flags & kFlagGsfQkv) != 0;
  const bool sq = (a.flags & kFlagSmoothQ) != 0;
  return VariantPtrs{qkv ? scal : nullptr, qkv ? scal + 1 : nullptr, qkv ? scal + 2 : nullptr,
                     (a.flags & kFlagGsfP) ? scal + 3 : nullptr,
                     (a.flags & kFlagSmoothK) ? (const float *)(ws + w.kmean) : nullptr,
                     sq ? (const float *)(ws + w.qmean) : nullptr, sq ? (const float *)(ws + w.delta) : nullptr};
}

hipError_t launch_variant_prep(const AttnArgs &a, const Workspace &w, hipStream_t stream) {
  const bool smooth = (a.flags & kFlagSmoothK) != 0, qkv = (a.flags & kFlagGsfQkv) != 0,
             pscale = (a.flags & kFlagGsfP) != 0, smooth_q = (a.flags & kFlagSmoothQ) != 0;
  if (!smooth && !qkv && !pscale && !smooth_q) return hipSuccess;
  uint8_t *ws = (uint8_t *)a.workspace;
  float *scal = (float *)(ws + w.scal);
  float *kmean = (float *)(ws + w.kmean);
  hipError_t e;
  const int64_t bh = (int64_t)a.batch * a.heads;
  if (smooth) {
    const int nslab = (int)((a.lk + kMeanSlab - 1) / kMeanSlab);
    double *part = (double *)(ws + w.kpart);
    AQ_LAUNCH("kmean_partial", kmean_partial_kernel, dim3((unsigned)(bh * nslab)), dim3(256), 0, stream,
              (const uint16_t *)a.k, a.sk, a.heads, a.lk, nslab, part);
    if ((e = hipGetLastError())) return e;
    const int64_t total = bh * kD;
    AQ_LAUNCH("kmean_final", kmean_final_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, part,
              nslab, a.lk, total, kmean);
    if ((e = hipGetLastError())) return e;
  }
  float *qmean = (float *)(ws + w.qmean);
  if (smooth_q) {
    const int nslab = (int)((a.lq + kMeanSlab - 1) / kMeanSlab);
    double *part = (double *)(ws + w.qpart);
    AQ_LAUNCH("qmean_partial", kmean_partial_kernel, dim3((unsigned)(bh * nslab)), dim3(256), 0, stream,
              (const uint16_t *)a.q, a.sq, a.heads, a.lq, nslab, part);
    if ((e = hipGetLastError())) return e;
    const int64_t total = bh * kD;
    AQ_LAUNCH("qmean_final", kmean_final_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, part,
              nslab, a.lq, total, qmean);
    if ((e = hipGetLastError())) return e;
  }
  if (qkv) {
    uint32_t *bits = (uint32_t *)(scal + 4);
    AQ_LAUNCH("fill_u32", fill_u32_kernel, dim3(1), dim3(64), 0, stream, bits, 3, 0u);
    if ((e = hipGetLastError())) return e;
    if ((e = launch_amax(a.q, a.sq, a.batch, a.heads, a.lq, smooth_q ? qmean : nullptr, bits, stream))) return e;
    if ((e = launch_amax(a.k, a.sk, a.batch, a.heads, a.lk, smooth ? kmean : nullptr, bits + 1, stream))) return e;
    if ((e = launch_amax(a.v, a.sv, a.batch, a.heads, a.lk, nullptr, bits + 2, stream))) return e;
  }
  AQ_LAUNCH("gsf_final", gsf_final_kernel, dim3(1), dim3(64), 0, stream, scal, (int)qkv, (int)pscale);
  return hipGetLastError();
}

hipError_t launch_qk_delta(const AttnArgs &a, const Workspace &w, hipStream_t stream) {
  if (!(a.flags & kFlagSmoothQ)) return hipSuccess;
  uint8_t *ws = (uint8_t *)a.workspace;
  const int64_t per_head = (a.lk + kChunk - 1) / kChunk * kChunk;
  const int64_t total = (int64_t)a.batch * a.heads * per_head;
  AQ_LAUNCH("qk_delta", qk_delta_kernel, dim3((unsigned)((total + 15) / 16)), dim3(256), 0, stream,
            (const u32x4 *)(ws + w.kq), (const float *)(ws + w.qmean), per_head, total, (float *)(ws + w.delta));
  return hipGetLastError();
}

}  // namespace aq
