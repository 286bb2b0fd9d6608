// vsa.hip - cube-sparse (VSA) NVFP4 fake-quant attention forward on gfx950.
//
// "vsqa-preview-1.3b metadata.json", attention: kind "vsa", cube_shape [4,4,8] (128 tokens),
// precision.coarse "BF16" with quantize_coarse false, fine "NVFP4 fake-quant with BF16 matmul"
// with quantize_fine true, selection.effective_topk = max(1, min(ceil((1-sparsity)*n), n)).
// Tokens arrive cube-major (each cube's 128 tokens contiguous), so a cube is exactly one 128-key
// chunk of the dense kernels and V-hat's 16-key blocks never straddle cubes.
//
//   pool_kernel    cube means of Q, K (and V for the coarse output) in fp32, rounded to bf16.
//   select_kernel  per (head, query cube): coarse logits against every key cube in fp32, top-k
//                  by repeated block-wide argmax (ties to the lower index), the selected cubes
//                  listed in ascending order; optionally the coarse output softmax(logits) @ Vc.
//   fine stage     the dense forward kernel with each query cube's chunk list (attn_fwd.hip).
#include "attn_common.hpp"
#include "launch.hpp"
#include "timing.hpp"

namespace aq {
namespace {

constexpr int kD = kHeadDim;

// One workgroup per (head, cube, tensor): 256 lanes = 128 d x 2 halves of the cube's tokens.
__global__ __launch_bounds__(256) void pool_kernel(const uint16_t *__restrict__ q, Strides sq,
                                                   const uint16_t *__restrict__ k, Strides sk,
                                                   const uint16_t *__restrict__ v, Strides sv,
                                                   uint16_t *__restrict__ pool, int heads, int64_t n,
                                                   int64_t bhn) {
  __shared__ float part[kD];
  const int64_t id = blockIdx.x % bhn;
  const int which = (int)(blockIdx.x / bhn);
  const int64_t bh = id / n, cube = id % n;
  const int64_t b = bh / heads, h = bh % heads;
  const uint16_t *src = which == 0 ? q : (which == 1 ? k : v);
  const Strides s = which == 0 ? sq : (which == 1 ? sk : sv);
  const int d = threadIdx.x & (kD - 1), half = threadIdx.x >> 7;
  const uint16_t *base = src + b * s.b + h * s.h + (cube * kChunk + half * 64) * s.l + d;
  float acc = 0.0f;
  for (int t = 0; t < 64; ++t) acc += bf16lo(base[t * s.l]);
  if (half == 1) part[d] = acc;
  __syncthreads();
  if (half == 0) {
    const float mean = (acc + part[d]) * (1.0f / kChunk);
    pool[((int64_t)which * bhn + id) * kD + d] = (uint16_t)f32_to_bf16_rne(mean);
  }
}

// Block-wide argmax of (score, -index) over 256 lanes.
__device__ __forceinline__ void argmax_step(float &s, int &i, float s2, int i2) {
  if (s2 > s || (s2 == s && i2 < i)) {
    s = s2;
    i = i2;
  }
}

// One workgroup per (head, query cube a).  Handles up to 256 key cubes per lane pass.
__global__ __launch_bounds__(256) void select_kernel(const uint16_t *__restrict__ pool, int64_t bhn, int64_t n,
                                                     int topk, float scale, int32_t *__restrict__ sel,
                                                     uint16_t *__restrict__ o_coarse, Strides so,
                                                     int heads) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float *score = (float *)smem;                  // [n]
  int *taken = (int *)(score + n);               // [n]
  float *qa = (float *)(taken + n);              // [128]
  float *red_s = qa + kD;                        // [4]
  int *red_i = (int *)(red_s + 4);               // [4]
  const int64_t id = blockIdx.x;                 // bh * n + a
  const int64_t bh = id / n, a = id % n;
  const uint16_t *qc = pool + id * kD;
  const uint16_t *kc = pool + (bhn + bh * n) * kD;
  const uint16_t *vc = pool + (2 * bhn + bh * n) * kD;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < kD) qa[tid] = bf16lo(qc[tid]);
  __syncthreads();
  for (int64_t b = tid; b < n; b += 256) {
    const uint16_t *kr = kc + b * kD;
    float acc = 0.0f;
    for (int d = 0; d < kD; ++d) acc = __builtin_fmaf(qa[d], bf16lo(kr[d]), acc);
    // A NaN score (a NaN anywhere in the cube's tokens) ranks below every number, so the top-k
    // always finds topk distinct cubes.
    const float sc = scale * acc;
    score[b] = sc == sc ? sc : -__builtin_inff();
    taken[b] = 0;
  }
  __syncthreads();
  for (int r = 0; r < topk; ++r) {
    float bs = -__builtin_inff();
    int bi = 0x7fffffff;
    for (int64_t b = tid; b < n; b += 256)
      if (!taken[b]) argmax_step(bs, bi, score[b], (int)b);
    for (int off = 32; off > 0; off >>= 1) argmax_step(bs, bi, __shfl_xor(bs, off), __shfl_xor(bi, off));
    if (lane == 0) {
      red_s[wave] = bs;
      red_i[wave] = bi;
    }
    __syncthreads();
    if (tid == 0) {
      float s0 = red_s[0];
      int i0 = red_i[0];
      for (int w = 1; w < 4; ++w) argmax_step(s0, i0, red_s[w], red_i[w]);
      // Every score is a number (at worst -inf, which the tie rule still picks), so i0 is an
      // untaken cube; the lowest untaken one stands in should that ever fail.
      if (i0 < 0 || i0 >= n || taken[i0]) {
        i0 = 0;
        while (i0 < n - 1 && taken[i0]) ++i0;
      }
      taken[i0] = 1;
    }
    __syncthreads();
  }
  // ascending list of the selected cubes
  if (tid == 0) {
    int t = 0;
    int32_t *out = sel + id * topk;
    for (int64_t b = 0; b < n; ++b)
      if (taken[b]) out[t++] = (int32_t)b;
  }
  if (o_coarse) {
    // softmax over all key cubes (not quantized), then the mean values Vc
    __syncthreads();
    float mx = -__builtin_inff();
    for (int64_t b = tid; b < n; b += 256) mx = fmaxf(mx, score[b]);
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if (lane == 0) red_s[wave] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red_s[0], red_s[1]), fmaxf(red_s[2], red_s[3]));
    __syncthreads();
    for (int64_t b = tid; b < n; b += 256) score[b] = __expf(score[b] - mx);
    __syncthreads();
    if (tid < kD) {
      float num = 0.0f, den = 0.0f;
      for (int64_t b = 0; b < n; ++b) {
        num = __builtin_fmaf(score[b], bf16lo(vc[b * kD + tid]), num);
        den += score[b];
      }
      qa[tid] = num / den;
    }
    __syncthreads();
    const int64_t bb = bh / heads, hh = bh % heads;
    const int d = tid & (kD - 1);
    const uint16_t val = (uint16_t)f32_to_bf16_rne(qa[d]);
    for (int t = tid >> 7; t < kChunk; t += 2)
      o_coarse[bb * so.b + hh * so.h + (a * kChunk + t) * so.l + d] = val;
  }
}

}  // namespace

hipError_t launch_vsa_fwd(const AttnArgs &a, const VsaArgs &s, hipStream_t stream) {
  const Workspace w = workspace_layout(2, a.batch, a.heads, a.lq, a.lk);
  uint8_t *ws = (uint8_t *)a.workspace;
  hipError_t e = launch_kv_prepass(a, 2, stream);
  if (e != hipSuccess) return e;
  const int64_t n = s.n_cubes;
  const int64_t bhn = (int64_t)a.batch * a.heads * n;
  uint16_t *pool = (uint16_t *)(ws + w.pool);
  const int ntensors = s.o_coarse ? 3 : 2;
  AQ_LAUNCH("vsa_pool", pool_kernel, dim3((unsigned)(bhn * ntensors)), dim3(256), 0, stream,
                     (const uint16_t *)a.q, a.sq, (const uint16_t *)a.k, a.sk, (const uint16_t *)a.v, a.sv,
                     pool, a.heads, n, bhn);
  if ((e = hipGetLastError())) return e;
  int32_t *sel = s.sel ? s.sel : (int32_t *)(ws + w.selw);
  const size_t smem = (size_t)n * 8 + kD * 4 + 32;
  if ((e = hipFuncSetAttribute((const void *)select_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)(smem < 65536 ? 65536 : smem))))
    return e;
  AQ_LAUNCH("vsa_select", select_kernel, dim3((unsigned)bhn), dim3(256), smem, stream, pool, bhn, n, s.topk,
                     a.scale, sel, (uint16_t *)s.o_coarse, a.so, a.heads);
  if ((e = hipGetLastError())) return e;
  return launch_attn_fwd_sel(a, sel, s.topk, stream);
}

}  // namespace aq
