// fq.hip - standalone NVFP4 fake quantization on gfx950 ("nvfp4_qad.py" module docstring:
// per-16 E4M3 block scales under a unit or static global scale; weight_global_sf and
// input_global_sf for the static scale g = 448*6 / amax).
//
// The op streams HBM: 2 bytes read and 2 written per element.  The contiguous kernel gives each
// lane 8 bf16 (one 16-byte load); two neighbouring lanes hold one 16-element block and exchange
// their partial abs-max through one DPP move, so every load and store instruction of a wave
// covers 1 KiB of consecutive memory.
#include "aq_device.hpp"
#include "launch.hpp"
#include "timing.hpp"

namespace aq {
namespace {

constexpr int kThreads = 256;
// Contiguous kernel: one-wave workgroups stream fastest (measured on MI355X: 64 lanes 6.4 TB/s,
// 256 lanes 5.9 TB/s on the [301056, 128] workload).
constexpr int kContigThreads = 64;

template <bool kUnit>
__device__ __forceinline__ u32x4 fq8(u32x4 v, float g) {
  float f[8] = {bf16lo(v.x), bf16hi(v.x), bf16lo(v.y), bf16hi(v.y),
                bf16lo(v.z), bf16hi(v.z), bf16lo(v.w), bf16hi(v.w)};
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) am = fmaxf(am, __builtin_fabsf(f[i]));
  am = fmaxf(am, xor1(am));
  uint32_t w[4];
  if (kUnit) {
    // The signed quotient goes through the E2M1 conversion (round half to even is symmetric), so
    // only a zero result needs its sign back: OR-ing the input's two bf16 sign bits into the
    // packed pair restores -0 and leaves every nonzero result unchanged.
    const float S = block_scale_unit(am);
    const float inv = S == 0.0f ? 0.0f : recip_e4m3(S);
    const uint32_t vin[4] = {v.x, v.y, v.z, v.w};
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = div_e4m3(f[i], S, inv);
    e2m1_decode8(e2m1_codes8(q), S, q);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = __builtin_amdgcn_perm(f2u(q[2 * i + 1]), f2u(q[2 * i]), 0x07060302u) | (vin[i] & 0x80008000u);
  } else {
    const float s = round_e4m3((am / 6.0f) * g);
    const float S = s / g;
    const bool zero = !(S > 0.0f);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = zero ? 0.0f * f[2 * i] : fq_general(f[2 * i], S);
      const float b = zero ? 0.0f * f[2 * i + 1] : fq_general(f[2 * i + 1], S);
      w[i] = f32_to_bf16_rne(a) | (f32_to_bf16_rne(b) << 16);
    }
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

// Blocks are contiguous: inner == 1 and axis % 16 == 0, so the tensor is n8 chunks of 8 values
// and chunk pairs (2j, 2j+1) are blocks.  One chunk per lane and one pass: many small
// workgroups with a single non-temporal 16-byte load and store per lane stream HBM faster than a
// grid-stride loop with several loads in flight per lane (measured on MI355X: 6.1 against
// 5.4 TB/s for a plain copy).  n8 is even and lane pairs start at even indexes, so a lane's
// partner (lane ^ 1) is in range exactly when the lane is.
template <bool kUnit>
__global__ __launch_bounds__(kContigThreads) void fq_contig_kernel(const u32x4 *__restrict__ x,
                                                                   u32x4 *__restrict__ y, int64_t n8,
                                                                   const float *__restrict__ gptr) {
  const float g = kUnit ? 1.0f : *gptr;
  const int64_t j = (int64_t)blockIdx.x * kContigThreads + threadIdx.x;
  const u32x4 v = j < n8 ? __builtin_nontemporal_load(x + j) : u32x4{0u, 0u, 0u, 0u};
  const u32x4 r = fq8<kUnit>(v, g);
  if (j < n8) __builtin_nontemporal_store(r, y + j);
}

// General layout: one lane per block column (outer o, block b, inner position t).  Consecutive
// lanes take consecutive t, so loads are coalesced whenever inner > 1.
template <bool kUnit>
__global__ __launch_bounds__(kThreads) void fq_general_kernel(const uint16_t *__restrict__ x,
                                                              uint16_t *__restrict__ y,
                                                              int64_t outer, int64_t axis,
                                                              int64_t inner,
                                                              const float *__restrict__ gptr) {
  const float g = kUnit ? 1.0f : *gptr;
  const int64_t nblk = (axis + kBlock - 1) / kBlock;
  const int64_t total = outer * nblk * inner;
  for (int64_t id = (int64_t)blockIdx.x * kThreads + threadIdx.x; id < total;
       id += (int64_t)gridDim.x * kThreads) {
    const int64_t t = id % inner;
    const int64_t b = (id / inner) % nblk;
    const int64_t o = id / (inner * nblk);
    const int64_t a0 = b * kBlock;
    const int n = (int)((axis - a0) < kBlock ? (axis - a0) : kBlock);
    const int64_t base = (o * axis + a0) * inner + t;
    float f[kBlock];
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < kBlock; ++i) {
      f[i] = i < n ? bf16lo(x[base + i * inner]) : 0.0f;
      am = fmaxf(am, __builtin_fabsf(f[i]));
    }
    if (kUnit) {
      const float S = block_scale_unit(am);
      const float inv = S == 0.0f ? 0.0f : recip_e4m3(S);
#pragma unroll
      for (int i = 0; i < kBlock; i += 2) fq_unit_pair(f[i], f[i + 1], S, inv);
#pragma unroll
      for (int i = 0; i < kBlock; ++i)
        if (i < n) y[base + i * inner] = (uint16_t)(f2u(f[i]) >> 16);
    } else {
      const float s = round_e4m3((am / 6.0f) * g);
      const float S = s / g;
      const bool zero = !(S > 0.0f);
#pragma unroll
      for (int i = 0; i < kBlock; ++i)
        if (i < n) y[base + i * inner] = (uint16_t)f32_to_bf16_rne(zero ? 0.0f * f[i] : fq_general(f[i], S));
    }
  }
}

__global__ void static_scale_init(float *g) { *(uint32_t *)g = 0u; }

// max |x| over n bf16 values, folded into *g (as fp32 bits: for non-negative floats the unsigned
// order is the numeric order).  fmaxf drops NaN, which reads NaN as 0.
__global__ __launch_bounds__(kThreads) void static_scale_reduce(const uint16_t *__restrict__ x,
                                                                int64_t n, float *g) {
  float m = 0.0f;
  const int64_t n8 = n / 8;
  const u32x4 *x8 = (const u32x4 *)x;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n8; i += (int64_t)gridDim.x * kThreads) {
    const u32x4 v = x8[i];
    m = fmaxf(m, fmaxf(fmaxf(__builtin_fabsf(bf16lo(v.x)), __builtin_fabsf(bf16hi(v.x))),
                       fmaxf(__builtin_fabsf(bf16lo(v.y)), __builtin_fabsf(bf16hi(v.y)))));
    m = fmaxf(m, fmaxf(fmaxf(__builtin_fabsf(bf16lo(v.z)), __builtin_fabsf(bf16hi(v.z))),
                       fmaxf(__builtin_fabsf(bf16lo(v.w)), __builtin_fabsf(bf16hi(v.w)))));
  }
  for (int64_t i = n8 * 8 + (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads)
    m = fmaxf(m, __builtin_fabsf(bf16lo(x[i])));
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) atomicMax((unsigned int *)g, f2u(m));
}

__global__ void static_scale_final(float *g) {
  const float a = fmaxf(*g, 1e-12f);
  *g = 2688.0f / a;  // FP4_RANGE = 448 * 6
}

// The same scale from an observed maximum (a calibrated activation's amax; fmaxf reads NaN as 0).
__global__ void scale_from_amax_kernel(const float *amax, float *g) {
  const float a = fmaxf(fmaxf(*amax, 0.0f), 1e-12f);
  *g = 2688.0f / a;
}

int grid_for(int64_t work_items, int per_thread) {
  int64_t blocks = (work_items + (int64_t)kThreads * per_thread - 1) / ((int64_t)kThreads * per_thread);
  if (blocks < 1) blocks = 1;
  if (blocks > 8192) blocks = 8192;
  return (int)blocks;
}

}  // namespace

hipError_t launch_fq(const void *x, void *y, int64_t outer, int64_t axis, int64_t inner,
                     const float *g, hipStream_t stream) {
  const bool contiguous = inner == 1 && axis % kBlock == 0 &&
                          ((uintptr_t)x % 16 == 0) && ((uintptr_t)y % 16 == 0);
  if (contiguous) {
    const int64_t n8 = outer * axis / 8;
    const int64_t grid = (n8 + kContigThreads - 1) / kContigThreads;  // one 16-byte chunk per lane
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    if (g == nullptr)
      AQ_LAUNCH("fq_contig_unit", fq_contig_kernel<true>, dim3((unsigned)grid), dim3(kContigThreads), 0, stream,
                         (const u32x4 *)x, (u32x4 *)y, n8, g);
    else
      AQ_LAUNCH("fq_contig_static", fq_contig_kernel<false>, dim3((unsigned)grid), dim3(kContigThreads), 0, stream,
                         (const u32x4 *)x, (u32x4 *)y, n8, g);
  } else {
    const int64_t cols = outer * ((axis + kBlock - 1) / kBlock) * inner;
    const int grid = grid_for(cols, 1);
    if (g == nullptr)
      AQ_LAUNCH("fq_general_unit", fq_general_kernel<true>, dim3(grid), dim3(kThreads), 0, stream,
                         (const uint16_t *)x, (uint16_t *)y, outer, axis, inner, g);
    else
      AQ_LAUNCH("fq_general_static", fq_general_kernel<false>, dim3(grid), dim3(kThreads), 0, stream,
                         (const uint16_t *)x, (uint16_t *)y, outer, axis, inner, g);
  }
  return hipGetLastError();
}

hipError_t launch_scale_from_amax(const float *amax, float *g_out, hipStream_t stream) {
  AQ_LAUNCH("scale_from_amax", scale_from_amax_kernel, dim3(1), dim3(1), 0, stream, amax, g_out);
  return hipGetLastError();
}

hipError_t launch_static_scale(const void *x, int64_t n, float *g_out, hipStream_t stream) {
  AQ_LAUNCH("static_scale_init", static_scale_init, dim3(1), dim3(1), 0, stream, g_out);
  AQ_LAUNCH("static_scale_reduce", static_scale_reduce, dim3(grid_for(n / 8 + 1, 16)), dim3(kThreads), 0, stream,
                     (const uint16_t *)x, n, g_out);
  AQ_LAUNCH("static_scale_final", static_scale_final, dim3(1), dim3(1), 0, stream, g_out);
  return hipGetLastError();
}

}  // namespace aq
