// vsa.hip - cube-sparse (VSA) NVFP4 fake-quant attention forward on gfx950.
//
// "vsqa-preview-1.3b metadata.json", attention: kind "vsa", cube_shape [4,4,8] (128 tokens),
// precision.coarse "BF16" with quantize_coarse false, fine "NVFP4 fake-quant with BF16 matmul"
// with quantize_fine true, selection.effective_topk = max(1, min(ceil((1-sparsity)*n), n)).
// Tokens arrive cube-major (each cube's 128 tokens contiguous), so a cube is exactly one 128-key
// chunk of the dense kernels and V-hat's 16-key blocks never straddle cubes.
//
//   pool_kernel        cube means of Q, K (and V for the coarse output) in fp32, rounded to bf16.
//   select_lds_kernel  per (head, query cube), one wave, the head's key-cube means staged in LDS
//                      (up to 256 key cubes; select_kernel, the same selection without the
//                      staging, past that): coarse logits against every key cube in fp32, the
//                      top-k (ties to the lower index) listed in ascending order; optionally the
//                      coarse output softmax(logits) @ Vc.
//   fine stage     the dense forward kernel with each query cube's chunk list (attn_fwd.hip).
#include "attn_common.hpp"
#include "launch.hpp"
#include "timing.hpp"

namespace aq {
namespace {

constexpr int kD = kHeadDim;

// One wave per (tensor, head, cube), four per workgroup, heads fastest (a workgroup reads
// neighbouring heads' columns of the same token rows): lane (token quarter g = lane/16, 16-byte
// column c = lane%16) adds the 8 values of column c over the 32 tokens of quarter g in token order,
// sixteen rows in flight at a time; the quarters' sums are added pairwise ((0+1)+(2+3)), scaled by
// 1/128 and rounded to bf16.
__global__ __launch_bounds__(256) void pool_kernel(const uint16_t *__restrict__ q, Strides sq,
                                                   const uint16_t *__restrict__ k, Strides sk,
                                                   const uint16_t *__restrict__ v, Strides sv,
                                                   uint16_t *__restrict__ pool, int heads, int64_t n,
                                                   int64_t bhn, int64_t items) {
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= items) return;  // whole waves
  const int64_t h = item % heads, r = item / heads, cube = r % n, r2 = r / n;
  const int64_t nb = bhn / ((int64_t)heads * n), b = r2 % nb;
  const int which = (int)(r2 / nb);
  const int64_t id = (b * heads + h) * n + cube;
  const uint16_t *src = which == 0 ? q : (which == 1 ? k : v);
  const Strides s = which == 0 ? sq : (which == 1 ? sk : sv);
  const int l = threadIdx.x & 63, c = l & 15, g = l >> 4;
  const uint16_t *base = src + b * s.b + h * s.h + (cube * kChunk + g * 32) * s.l + 8 * c;
  float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  for (int t0 = 0; t0 < 32; t0 += 16) {
    u32x4 x[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) x[t] = *(const u32x4 *)(base + (t0 + t) * s.l);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      acc[0] += bf16lo(x[t].x);
      acc[1] += bf16hi(x[t].x);
      acc[2] += bf16lo(x[t].y);
      acc[3] += bf16hi(x[t].y);
      acc[4] += bf16lo(x[t].z);
      acc[5] += bf16hi(x[t].z);
      acc[6] += bf16lo(x[t].w);
      acc[7] += bf16hi(x[t].w);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    acc[i] += __shfl_xor(acc[i], 16, 64);  // quarters 0+1, 2+3
    acc[i] += __shfl_xor(acc[i], 32, 64);  // (0+1) + (2+3)
  }
  if (g == 0) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = f32_to_bf16_rne(acc[2 * i] * (1.0f / kChunk)) | (f32_to_bf16_rne(acc[2 * i + 1] * (1.0f / kChunk)) << 16);
    *(u32x4 *)(pool + ((int64_t)which * bhn + id) * kD + 8 * c) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// One wave per (head, query cube a), four per workgroup, no workgroup barrier.  LDS per wave: the
// n coarse logits, their exponentials (coarse output) and the query cube's pooled row.  The
// logits: lanes over key cubes, each a dot product in d order in fp32.  Top-k: the largest topk,
// ties to the lower index, listed in ascending order.  Optionally the coarse output
// softmax(logits) @ Vc, broadcast to the cube's 128 tokens.
__global__ __launch_bounds__(256) void select_kernel(const uint16_t *__restrict__ pool, int64_t bhn, int64_t n,
                                                     int topk, float scale, int32_t *__restrict__ sel,
                                                     uint16_t *__restrict__ o_coarse, Strides so,
                                                     int heads) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t id = (int64_t)blockIdx.x * 4 + wave;  // bh * n + a
  if (id >= bhn) return;
  const int64_t n4 = (n + 3) & ~(int64_t)3;    // 16-byte aligned regions
  float *score = smem + wave * (2 * n4 + kD);  // [n]
  float *ex = score + n4;                      // [n]
  float *qa = ex + n4;                         // [128]
  const int64_t bh = id / n, a = id % n;
  const uint16_t *qc = pool + id * kD;
  const uint16_t *kc = pool + (bhn + bh * n) * kD;
  const uint16_t *vc = pool + (2 * bhn + bh * n) * kD;
  {
    const uint32_t x = *(const uint32_t *)(qc + 2 * lane);
    qa[2 * lane] = bf16lo(x);
    qa[2 * lane + 1] = bf16hi(x);
  }
  for (int64_t b = lane; b < n; b += 64) {
    const u32x4 *kr = (const u32x4 *)(kc + b * kD);
    float acc = 0.0f;
    u32x4 xs[kD / 8];
#pragma unroll
    for (int j = 0; j < kD / 8; ++j) xs[j] = kr[j];
#pragma unroll
    for (int j = 0; j < kD / 8; ++j) {
      const u32x4 x = xs[j];
      const f32x4 q0 = *(const f32x4 *)(qa + 8 * j), q1 = *(const f32x4 *)(qa + 8 * j + 4);
      acc = __builtin_fmaf(q0[0], bf16lo(x.x), acc);
      acc = __builtin_fmaf(q0[1], bf16hi(x.x), acc);
      acc = __builtin_fmaf(q0[2], bf16lo(x.y), acc);
      acc = __builtin_fmaf(q0[3], bf16hi(x.y), acc);
      acc = __builtin_fmaf(q1[0], bf16lo(x.z), acc);
      acc = __builtin_fmaf(q1[1], bf16hi(x.z), acc);
      acc = __builtin_fmaf(q1[2], bf16lo(x.w), acc);
      acc = __builtin_fmaf(q1[3], bf16hi(x.w), acc);
    }
    // A NaN score (a NaN anywhere in the cube's tokens) ranks below every number, so the top-k
    // always finds topk distinct cubes.
    const float sc = scale * acc;
    score[b] = sc == sc ? sc : -__builtin_inff();
  }
  if (o_coarse) {
    // softmax over all key cubes (not quantized), then the mean values Vc
    float mx = -__builtin_inff();
    for (int64_t b = lane; b < n; b += 64) mx = fmaxf(mx, score[b]);
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    for (int64_t b = lane; b < n; b += 64) ex[b] = __expf(score[b] - mx);
    float num0 = 0.0f, num1 = 0.0f, den = 0.0f;
    for (int64_t b = 0; b < n; ++b) {
      const float e = ex[b];
      const uint32_t x = *(const uint32_t *)(vc + b * kD + 2 * lane);
      num0 = __builtin_fmaf(e, bf16lo(x), num0);
      num1 = __builtin_fmaf(e, bf16hi(x), num1);
      den += e;
    }
    const uint32_t val = f32_to_bf16_rne(num0 / den) | (f32_to_bf16_rne(num1 / den) << 16);
    const int64_t bb = bh / heads, hh = bh % heads;
    uint16_t *dst = o_coarse + bb * so.b + hh * so.h + a * kChunk * so.l + 2 * lane;
    for (int t = 0; t < kChunk; ++t) *(uint32_t *)(dst + t * so.l) = val;
  }
  // The topk-th largest logit T by bisection over order-preserving keys (no NaN is left: those
  // became -inf), then every logit above T and, of those equal to T, the lowest cubes: the same
  // set as topk rounds of argmax with ties to the lower index, listed in ascending order.
  auto okey = [](float x) -> uint32_t {
    const uint32_t u = __builtin_bit_cast(uint32_t, x + 0.0f);  // -0 as +0: they tie
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  };
  auto count_ge = [&](uint32_t t) -> int {
    int c = 0;
    for (int64_t base = 0; base < n; base += 64) {
      const int64_t b = base + lane;
      c += (int)__builtin_popcountll(__builtin_amdgcn_ballot_w64(b < n && okey(score[b]) >= t));
    }
    return c;
  };
  uint32_t lo = 0u, hi = 0xFFFFFFFFu;  // count_ge(lo) >= topk holds throughout
  while (lo < hi) {
    const uint32_t mid = lo + (uint32_t)(((uint64_t)(hi - lo) + 1u) >> 1);
    if (count_ge(mid) >= topk) lo = mid;
    else hi = mid - 1u;
  }
  int need_eq = topk - (lo == 0xFFFFFFFFu ? 0 : count_ge(lo + 1u));  // cubes equal to T to take
  int32_t *out = sel + id * topk;
  int cnt = 0;
  for (int64_t base = 0; base < n; base += 64) {
    const int64_t b = base + lane;
    const uint32_t kb = b < n ? okey(score[b]) : 0u;
    const uint64_t meq = __builtin_amdgcn_ballot_w64(b < n && kb == lo);
    const int eq_before = (int)__builtin_popcountll(meq & ((1ull << lane) - 1ull));
    const bool take = b < n && (kb > lo || (kb == lo && eq_before < need_eq));
    const uint64_t m = __builtin_amdgcn_ballot_w64(take);
    if (take) out[cnt + (int)__builtin_popcountll(m & ((1ull << lane) - 1ull))] = (int32_t)b;
    cnt += (int)__builtin_popcountll(m);
    const int eq_all = (int)__builtin_popcountll(meq);
    need_eq -= eq_all < need_eq ? eq_all : need_eq;
  }
}

// The same selection for n <= 256 key cubes, with the head's key-cube means staged once per
// workgroup: one workgroup per (head, group of 4 * kSelPerWave query cubes), the n pooled K rows
// in LDS as bf16 (rows padded to 272 bytes, so the 16-byte reads of 16 lanes at one column cover
// all 64 banks), each wave walking its query cubes.  Lane l scores key cubes l, l+64, l+128, l+192
// (the same d-order fp32 chains as select_kernel) and keeps them in registers for the top-k
// bisection.  The coarse output, when asked for, as in select_kernel.
constexpr int kSelPerWave = 2;
constexpr int kSelRow = 272;  // bytes per staged key-cube row
__global__ __launch_bounds__(256) void select_lds_kernel(const uint16_t *__restrict__ pool, int64_t bhn, int64_t n,
                                                         int64_t groups, int topk, float scale,
                                                         int32_t *__restrict__ sel, uint16_t *__restrict__ o_coarse,
                                                         Strides so, int heads) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t bh = blockIdx.x / groups, grp = blockIdx.x % groups;
  uint8_t *kl = (uint8_t *)smem;
  const u32x4 *kc = (const u32x4 *)(pool + (bhn + bh * n) * kD);
  for (int64_t i = threadIdx.x; i < n * (kD / 8); i += 256)
    *(u32x4 *)(kl + (i >> 4) * kSelRow + (i & 15) * 16) = kc[i];
  float *qa = (float *)(kl + n * kSelRow) + wave * (kD + 256);  // [128] query mean, then [n] exponentials
  float *ex = qa + kD;
  __syncthreads();
  const uint16_t *vc = pool + (2 * bhn + bh * n) * kD;
  auto okey = [](float x) -> uint32_t {
    const uint32_t u = __builtin_bit_cast(uint32_t, x + 0.0f);  // -0 as +0: they tie
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  };
  for (int sidx = 0; sidx < kSelPerWave; ++sidx) {
    const int64_t a = (grp * 4 + wave) * kSelPerWave + sidx;
    if (a >= n) break;  // wave-uniform
    const int64_t id = bh * n + a;
    {
      const uint32_t x = *(const uint32_t *)(pool + id * kD + 2 * lane);
      qa[2 * lane] = bf16lo(x);
      qa[2 * lane + 1] = bf16hi(x);
    }
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    int64_t rb[4];
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) rb[sl] = min((int64_t)lane + 64 * sl, n - 1);  // in bounds; dropped below
#pragma unroll 4
    for (int j = 0; j < kD / 8; ++j) {
      const f32x4 q0 = *(const f32x4 *)(qa + 8 * j), q1 = *(const f32x4 *)(qa + 8 * j + 4);
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        const u32x4 x = *(const u32x4 *)(kl + rb[sl] * kSelRow + 16 * j);
        float t = acc[sl];
        t = __builtin_fmaf(q0[0], bf16lo(x.x), t);
        t = __builtin_fmaf(q0[1], bf16hi(x.x), t);
        t = __builtin_fmaf(q0[2], bf16lo(x.y), t);
        t = __builtin_fmaf(q0[3], bf16hi(x.y), t);
        t = __builtin_fmaf(q1[0], bf16lo(x.z), t);
        t = __builtin_fmaf(q1[1], bf16hi(x.z), t);
        t = __builtin_fmaf(q1[2], bf16lo(x.w), t);
        t = __builtin_fmaf(q1[3], bf16hi(x.w), t);
        acc[sl] = t;
      }
    }
    // NaN scores rank below every number; key cubes past n are not counted
    float sc[4];
    uint32_t key[4];
    bool live[4];
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      live[sl] = lane + 64 * sl < n;
      const float x = scale * acc[sl];
      sc[sl] = x == x ? x : -__builtin_inff();
      key[sl] = okey(sc[sl]);
    }
    if (o_coarse) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int sl = 0; sl < 4; ++sl)
        if (live[sl]) mx = fmaxf(mx, sc[sl]);
      for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
#pragma unroll
      for (int sl = 0; sl < 4; ++sl)
        if (live[sl]) ex[lane + 64 * sl] = __expf(sc[sl] - mx);
      float num0 = 0.0f, num1 = 0.0f, den = 0.0f;
      for (int64_t b = 0; b < n; ++b) {
        const float e = ex[b];
        const uint32_t x = *(const uint32_t *)(vc + b * kD + 2 * lane);
        num0 = __builtin_fmaf(e, bf16lo(x), num0);
        num1 = __builtin_fmaf(e, bf16hi(x), num1);
        den += e;
      }
      const uint32_t val = f32_to_bf16_rne(num0 / den) | (f32_to_bf16_rne(num1 / den) << 16);
      const int64_t bb = bh / heads, hh = bh % heads;
      uint16_t *dst = o_coarse + bb * so.b + hh * so.h + a * kChunk * so.l + 2 * lane;
      for (int t = 0; t < kChunk; ++t) *(uint32_t *)(dst + t * so.l) = val;
    }
    auto count_ge = [&](uint32_t t) -> int {
      int c = 0;
#pragma unroll
      for (int sl = 0; sl < 4; ++sl)
        c += (int)__builtin_popcountll(__builtin_amdgcn_ballot_w64(live[sl] && key[sl] >= t));
      return c;
    };
    uint32_t lo = 0u, hi = 0xFFFFFFFFu;  // count_ge(lo) >= topk holds throughout
    while (lo < hi) {
      const uint32_t mid = lo + (uint32_t)(((uint64_t)(hi - lo) + 1u) >> 1);
      if (count_ge(mid) >= topk) lo = mid;
      else hi = mid - 1u;
    }
    int need_eq = topk - (lo == 0xFFFFFFFFu ? 0 : count_ge(lo + 1u));
    int32_t *out = sel + id * topk;
    int cnt = 0;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      const uint64_t meq = __builtin_amdgcn_ballot_w64(live[sl] && key[sl] == lo);
      const int eq_before = (int)__builtin_popcountll(meq & ((1ull << lane) - 1ull));
      const bool take = live[sl] && (key[sl] > lo || (key[sl] == lo && eq_before < need_eq));
      const uint64_t m = __builtin_amdgcn_ballot_w64(take);
      if (take) out[cnt + (int)__builtin_popcountll(m & ((1ull << lane) - 1ull))] = (int32_t)(lane + 64 * sl);
      cnt += (int)__builtin_popcountll(m);
      const int eq_all = (int)__builtin_popcountll(meq);
      need_eq -= eq_all < need_eq ? eq_all : need_eq;
    }
  }
}

}  // namespace

hipError_t launch_vsa_select(const AttnArgs &a, const VsaArgs &s, const Workspace &w, hipStream_t stream);

hipError_t launch_vsa_fwd(const AttnArgs &a, const VsaArgs &s, hipStream_t stream) {
  const Workspace w = workspace_layout(2, a.batch, a.heads, a.lq, a.lk);
  uint8_t *ws = (uint8_t *)a.workspace;
  // The cube means and the selection (workspace regions pool, selw) on the side stream, beside
  // the K/V prepass (regions kq, vt), which moves more bytes and so stays on the call's stream;
  // both read only the caller's Q, K and V.
  SideFork f;
  hipError_t e = side_fork(stream, f);
  if (e != hipSuccess) return e;
  e = launch_vsa_select(a, s, w, f.stream);
  if (e == hipSuccess) e = launch_kv_prepass(a, 2, stream);
  const hipError_t j = side_join(stream, f);
  if (e != hipSuccess) return e;
  if (j != hipSuccess) return j;
  int32_t *sel = s.sel ? s.sel : (int32_t *)(ws + w.selw);
  return launch_attn_fwd_sel(a, sel, s.topk, stream);
}

// The cube means and the coarse selection (and the coarse output when asked for).
hipError_t launch_vsa_select(const AttnArgs &a, const VsaArgs &s, const Workspace &w, hipStream_t stream) {
  uint8_t *ws = (uint8_t *)a.workspace;
  hipError_t e;
  const int64_t n = s.n_cubes;
  const int64_t bhn = (int64_t)a.batch * a.heads * n;
  uint16_t *pool = (uint16_t *)(ws + w.pool);
  const int ntensors = s.o_coarse ? 3 : 2;
  const int64_t items = bhn * ntensors;
  AQ_LAUNCH("vsa_pool", pool_kernel, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, stream,
                     (const uint16_t *)a.q, a.sq, (const uint16_t *)a.k, a.sk, (const uint16_t *)a.v, a.sv,
                     pool, a.heads, n, bhn, items);
  if ((e = hipGetLastError())) return e;
  int32_t *sel = s.sel ? s.sel : (int32_t *)(ws + w.selw);
  if (n <= 256) {
    const int64_t groups = (n + 4 * kSelPerWave - 1) / (4 * kSelPerWave);
    const size_t lds = (size_t)n * kSelRow + (size_t)4 * (kD + 256) * 4;
    if ((e = hipFuncSetAttribute((const void *)select_lds_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)(lds < 65536 ? 65536 : lds))))
      return e;
    AQ_LAUNCH("vsa_select", select_lds_kernel, dim3((unsigned)((bhn / n) * groups)), dim3(256), lds, stream, pool,
              bhn, n, groups, s.topk, a.scale, sel, (uint16_t *)s.o_coarse, a.so, a.heads);
    return hipGetLastError();
  }
  const size_t smem = (size_t)4 * (2 * ((n + 3) & ~(int64_t)3) + kD) * 4;
  if ((e = hipFuncSetAttribute((const void *)select_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)(smem < 65536 ? 65536 : smem))))
    return e;
  AQ_LAUNCH("vsa_select", select_kernel, dim3((unsigned)((bhn + 3) / 4)), dim3(256), smem, stream, pool, bhn, n,
                     s.topk, a.scale, sel, (uint16_t *)s.o_coarse, a.so, a.heads);
  return hipGetLastError();
}

}  // namespace aq
