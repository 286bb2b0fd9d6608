// prepass.hip - fake quantization of whole attention operands into the workspace, once per call.
//
// Q-hat and K-hat are fake-quantized along D, V-hat along the key axis, in 16-element blocks with
// E4M3 scales and E2M1 values under the unit global scale ("vsqa-preview-1.3b metadata.json":
// dense precision record, group_size 16, qk/pv_format NVFP4 E2M1, use_global_sf_qkv false).
// Quantizing each operand once here keeps the codec out of the attention kernels' inner loops,
// where it would be repeated by every query tile of a head.
//
// kQuantRowsF16 writes the V-hat values as fp16 instead of bf16 (exact, see below) for the
// forward's fp16 P-hat V-hat product.  `out` (TileOut) then rounds every value, after its
// quantization, to the nearest FP8 E4M3FN value (the FP8 P.V product variant), kept as bf16
// (kOutFp8Bf16) or as fp16 (kOutFp8F16: every E4M3FN value is exact in fp16, for the forward's
// fp16 product), or stores the value as fp16 unchanged (kOutF16: K-hat rows under the unit scale,
// exact NVFP4 values, for the training forward's fp16 logits).
//
// Variants (readings stated in variants.hip): a static global scale g (block scale
// s = E4M3(fp32(fp32(amax / 6) * g)), S = fp32(s / g), value E2M1(fp32(|x| / S)) * S rounded to
// bf16, as "nvfp4_qad.py" quantizes under input_global_sf), and the smooth-K mean subtracted in
// fp32 before quantization (rows past L stay zero).
//
// tile_prepass (every mode): one workgroup per 128-row chunk of one head, staged in LDS as
// [row][d] (rows past L read as zero), quantized in place, then written as
//   rows_out  [B*H, C*128, 128]       row-major (the MFMA operand rows of the attention kernels)
//   tiles_out [B*H, C, 128 d, 128 rows] d-major (operands whose contraction runs over rows).
// rows_prepass streams the common row case (unit scale, no smoothing); kv_prepass writes the
// forward's K-hat rows and V-hat tiles of the common case in one launch.
#include "aq_device.hpp"
#include "launch.hpp"
#include "timing.hpp"

namespace aq {
namespace {

constexpr int kD = kHeadDim;

// Fake quantization of one 16-value block in place under the static global scale g; the values
// come back rounded to bf16 (as fp32).
__device__ __forceinline__ void fq_block_static(float (&f)[16], float g) {
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) am = fmaxf(am, __builtin_fabsf(f[i]));
  const float sc = round_e4m3((am / 6.0f) * g);
  const float S = sc / g;
  const bool zero = !(S > 0.0f);
#pragma unroll
  for (int i = 0; i < 16; ++i) f[i] = bf16lo(f32_to_bf16_rne(zero ? 0.0f * f[i] : fq_general(f[i], S)));
}

__global__ __launch_bounds__(256) void tile_prepass(const uint16_t *__restrict__ src, Strides s,
                                                    int heads, int64_t L, int64_t C, int quant,
                                                    u32x4 *__restrict__ rows_out,
                                                    uint16_t *__restrict__ tiles_out,
                                                    const float *__restrict__ gptr,
                                                    const float *__restrict__ mean, int out) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kChunk][kD];
  const int64_t bh = blockIdx.x / C;
  const int64_t c = blockIdx.x % C;
  const int64_t b = bh / heads, h = bh % heads;
  const uint16_t *base = src + b * s.b + h * s.h;
  const int tid = threadIdx.x;

  for (int i = tid; i < kChunk * kD / 8; i += 256) {
    const int row = i >> 4, part = i & 15;
    const int64_t r = c * kChunk + row;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (r < L) x = *(const u32x4 *)(base + r * s.l + part * 8);
    *(u32x4 *)&tile[row][part * 8] = x;
  }
  __syncthreads();

  const float g = gptr ? *gptr : 1.0f;
  if (quant == kQuantD || (quant == kQuantNone && mean)) {
    // lane: row tid/2, d in [64*(tid&1), +64): four 16-element blocks
    const int row = tid >> 1, d0 = (tid & 1) * 64;
    const bool live = c * kChunk + row < L;
    const float *mrow = (mean && live) ? mean + bh * kD + d0 : nullptr;
    for (int blk = 0; blk < 4; ++blk) {
      u32x4 *p = (u32x4 *)&tile[row][d0 + 16 * blk];
      float f[16];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const u32x4 v = p[i];
        f[8 * i + 0] = bf16lo(v.x); f[8 * i + 1] = bf16hi(v.x);
        f[8 * i + 2] = bf16lo(v.y); f[8 * i + 3] = bf16hi(v.y);
        f[8 * i + 4] = bf16lo(v.z); f[8 * i + 5] = bf16hi(v.z);
        f[8 * i + 6] = bf16lo(v.w); f[8 * i + 7] = bf16hi(v.w);
      }
      if (mrow) {
#pragma unroll
        for (int i = 0; i < 16; ++i) f[i] = f[i] - mrow[16 * blk + i];
      }
      if (quant == kQuantD && !gptr) {
        float am = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) am = fmaxf(am, __builtin_fabsf(f[i]));
        const float S = block_scale_unit(am);
        const float inv = S == 0.0f ? 0.0f : recip_e4m3(S);
#pragma unroll
        for (int i = 0; i < 16; i += 2) fq_unit_pair(f[i], f[i + 1], S, inv);  // exact in bf16
      } else if (quant == kQuantD) {
        fq_block_static(f, g);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) f[i] = bf16lo(f32_to_bf16_rne(f[i]));  // smoothed, unquantized
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
        p[i] = u32x4{pack_exact_bf16(f[8 * i], f[8 * i + 1]), pack_exact_bf16(f[8 * i + 2], f[8 * i + 3]),
                     pack_exact_bf16(f[8 * i + 4], f[8 * i + 5]), pack_exact_bf16(f[8 * i + 6], f[8 * i + 7])};
    }
    __syncthreads();
  } else if ((quant == kQuantRows || quant == kQuantRowsF16) && gptr) {
    // static global scale (bf16 values): lane column d = tid%128, rows [64*(tid/128), +64)
    const int d = tid & (kD - 1), r0 = (tid >> 7) * 64;
    for (int blk = 0; blk < 4; ++blk) {
      float f[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) f[i] = bf16lo(tile[r0 + 16 * blk + i][d]);
      fq_block_static(f, g);
#pragma unroll
      for (int i = 0; i < 16; ++i) tile[r0 + 16 * blk + i][d] = (uint16_t)(f2u(f[i]) >> 16);
    }
    __syncthreads();
  } else if (quant == kQuantRows || quant == kQuantRowsF16) {
    // lane: column d = tid%128, rows [64*(tid/128), +64): four 16-row blocks
    const int d = tid & (kD - 1), r0 = (tid >> 7) * 64;
    for (int blk = 0; blk < 4; ++blk) {
      float f[16];
      float am = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        f[i] = bf16lo(tile[r0 + 16 * blk + i][d]);
        am = fmaxf(am, __builtin_fabsf(f[i]));
      }
      const float S = block_scale_unit(am);
      const float inv = S == 0.0f ? 0.0f : recip_e4m3(S);
#pragma unroll
      for (int i = 0; i < 16; i += 2) fq_unit_pair(f[i], f[i + 1], S, inv);
      // kQuantRowsF16: the value as fp16 bits.  Every unit-scale NVFP4 value (|x| <= 6 * 448,
      // nonzero |x| >= 2^-10, at most 6 significant bits) is exact in fp16.
      if (quant == kQuantRowsF16) {
#pragma unroll
        for (int i = 0; i < 16; ++i) tile[r0 + 16 * blk + i][d] = __builtin_bit_cast(uint16_t, (_Float16)f[i]);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) tile[r0 + 16 * blk + i][d] = (uint16_t)(f2u(f[i]) >> 16);
      }
    }
    __syncthreads();
  }

  if (out != kOutBf16) {
    // FP8 P.V product: every (bf16) value rounded to the nearest E4M3FN value, sign kept (exact in
    // bf16 and in fp16); kOutF16: the value itself; rows past L stay zero
    for (int i = tid; i < kChunk * kD / 2; i += 256) {
      uint32_t *w = (uint32_t *)&tile[0][0] + i;
      const float a = bf16lo(*w), b = bf16hi(*w);
      const bool e4m3 = out == kOutFp8Bf16 || out == kOutFp8F16;
      const float ra = e4m3 ? u2f(f2u(round_e4m3(__builtin_fabsf(a))) | (f2u(a) & 0x80000000u)) : a;
      const float rb = e4m3 ? u2f(f2u(round_e4m3(__builtin_fabsf(b))) | (f2u(b) & 0x80000000u)) : b;
      if (out == kOutFp8Bf16)
        *w = pack_exact_bf16(ra, rb);
      else
        *w = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)ra) |
             ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)rb) << 16);
    }
    __syncthreads();
  }

  if (rows_out) {
    u32x4 *dst = rows_out + (bh * C + c) * (kChunk * kD / 8);
    for (int i = tid; i < kChunk * kD / 8; i += 256) dst[i] = *(const u32x4 *)&tile[i >> 4][(i & 15) * 8];
  }
  if (tiles_out) {
    // lane: d = tid/2, rows [64*(tid&1), +64)
    const int d = tid >> 1, r0 = (tid & 1) * 64;
    uint16_t *dst = tiles_out + ((bh * C + c) * kD + d) * kChunk + r0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = (uint32_t)tile[r0 + 8 * i + 2 * j][d] | ((uint32_t)tile[r0 + 8 * i + 2 * j + 1][d] << 16);
      *(u32x4 *)(dst + 8 * i) = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
}

// The common row case (D-axis blocks under the unit scale, no smoothing, bf16 or fp16 values) as
// a stream: one lane per 16-byte piece (8 values) of an output row, two neighbouring lanes per
// 16-value block exchanging their partial abs-max through one DPP move (the standalone fake
// quantizer's arrangement); rows past L come out zero.  The values are those of tile_prepass: the
// same scale, quotient and E2M1 rounding, the input's sign kept on zeros.  j: the piece's index
// over all rows of all heads; whole waves only, so every lane's partner is live.
__device__ __forceinline__ u32x4 rows_load(const uint16_t *__restrict__ src, Strides s, int heads, int64_t L,
                                           int64_t C, int64_t j) {
  const int64_t row = j >> 4, part = j & 15;
  const int64_t bh = row / (C * kChunk), r = row % (C * kChunk);
  const int64_t b = bh / heads, h = bh % heads;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (r < L) v = __builtin_nontemporal_load((const u32x4 *)(src + b * s.b + h * s.h + r * s.l + part * 8));
  return v;
}
__device__ __forceinline__ void rows_store(u32x4 v, int64_t j, u32x4 *__restrict__ rows_out, int f16) {
  float f[8] = {bf16lo(v.x), bf16hi(v.x), bf16lo(v.y), bf16hi(v.y), bf16lo(v.z), bf16hi(v.z), bf16lo(v.w), bf16hi(v.w)};
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) am = fmaxf(am, __builtin_fabsf(f[i]));
  am = fmaxf(am, xor1(am));
  const float S = block_scale_unit(am);
  const float inv = S == 0.0f ? 0.0f : recip_e4m3(S);
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = div_e4m3(f[i], S, inv);
  e2m1_decode8(e2m1_codes8(q), S, q);
  const uint32_t vin[4] = {v.x, v.y, v.z, v.w};
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (f16)  // exact: at most 6 significant bits in [2^-10, 6 * 448]
      w[i] = ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)q[2 * i]) |
              ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)q[2 * i + 1]) << 16)) |
             (vin[i] & 0x80008000u);
    else
      w[i] = __builtin_amdgcn_perm(f2u(q[2 * i + 1]), f2u(q[2 * i]), 0x07060302u) | (vin[i] & 0x80008000u);
  }
  __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]}, rows_out + j);
}

__global__ __launch_bounds__(64) void rows_prepass(const uint16_t *__restrict__ src, Strides s, int heads, int64_t L,
                                                   int64_t C, int64_t n8, u32x4 *__restrict__ rows_out, int f16) {
  const int64_t j = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (j >= n8) return;  // n8 is a multiple of 64
  rows_store(rows_load(src, s, heads, L, C, j), j, rows_out, f16);
}

// V-hat of one 128-row chunk (blocks of 16 rows per column under the unit scale), d-major: wave w
// loads rows [32w, 32w+32) of columns 2*lane and 2*lane+1 (one 32-bit load per row: 256
// contiguous bytes per row and wave), quantizes its two 16-row blocks of each column in registers
// and writes the column's 32 values into the LDS tile [128 d][128 rows]; after one barrier every
// wave stores four whole 256-byte tile rows per instruction.  The tile's 16-byte pieces are
// swizzled by d (physical piece = piece ^ ((d >> 1) & 15)), so the 16 lanes of one LDS access
// touch 16 different piece positions: all 64 banks, no conflicts.  Rows past L read as zero.  The
// values are tile_prepass's for kQuantRows (bf16) and kQuantRowsF16 (fp16) under the unit scale:
// the same blocks, scale, quotient and rounding.
__device__ __forceinline__ uint32_t vt_piece(int d, int piece) {
  return (uint32_t)(d * 256 + ((piece ^ ((d >> 1) & 15)) << 4));
}
__device__ __forceinline__ void vtile_chunk(const uint16_t *__restrict__ src, Strides s, int heads, int64_t L,
                                            int64_t C, int64_t chunk, uint16_t *__restrict__ tiles_out, int f16,
                                            uint8_t *lds) {
  const int64_t bh = chunk / C, c = chunk % C;
  const int64_t b = bh / heads, h = bh % heads;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t r0 = c * kChunk + 32 * wave;
  const uint16_t *base = src + b * s.b + h * s.h + 2 * lane;
  uint32_t x[32];
#pragma unroll
  for (int i = 0; i < 32; ++i)
    x[i] = r0 + i < L ? __builtin_nontemporal_load((const uint32_t *)(base + (r0 + i) * s.l)) : 0u;
#pragma unroll
  for (int col = 0; col < 2; ++col) {
    uint32_t w[16];  // the column's 32 values, two per word, in row order
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      float f[16];
      float am = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        f[i] = col ? bf16hi(x[16 * blk + i]) : bf16lo(x[16 * blk + i]);
        am = fmaxf(am, __builtin_fabsf(f[i]));
      }
      const float S = block_scale_unit(am);
      const float inv = S == 0.0f ? 0.0f : recip_e4m3(S);
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        fq_unit_pair(f[i], f[i + 1], S, inv);
        w[8 * blk + i / 2] =
            f16 ? ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f[i]) |
                   ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f[i + 1]) << 16))
                : ((f2u(f[i]) >> 16) | (f2u(f[i + 1]) & 0xFFFF0000u));
      }
    }
    const int d = 2 * lane + col;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *(u32x4 *)(lds + vt_piece(d, 4 * wave + q)) = u32x4{w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]};
  }
  __syncthreads();
  // instruction i of wave w: tile rows d = 16i + 4w + lane/16, piece lane%16
  u32x4 *dst = (u32x4 *)(tiles_out + (bh * C + c) * kD * kChunk);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int d = 16 * i + 4 * wave + (lane >> 4), piece = lane & 15;
    __builtin_nontemporal_store(*(const u32x4 *)(lds + vt_piece(d, piece)), dst + d * 16 + piece);
  }
}

// K-hat rows and V-hat tiles of heads [bh0, bh0 + nbh) in one launch: the first kblocks
// workgroups stream K rows (64 rows each: four 16-byte pieces per lane, loaded together), the rest
// one V chunk each.
__global__ __launch_bounds__(256) void kv_prepass(const uint16_t *__restrict__ k, Strides sk,
                                                  const uint16_t *__restrict__ v, Strides sv, int heads, int64_t L,
                                                  int64_t C, int64_t bh0, int64_t kblocks,
                                                  u32x4 *__restrict__ krows, int kf16,
                                                  uint16_t *__restrict__ vtiles, int vf16) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kD * kChunk * 2];
  if ((int64_t)blockIdx.x < kblocks) {
    const int64_t j0 = (bh0 * C * kChunk + (int64_t)blockIdx.x * 64) * 16 + threadIdx.x;
    u32x4 x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = rows_load(k, sk, heads, L, C, j0 + 256 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) rows_store(x[i], j0 + 256 * i, krows, kf16);
    return;
  }
  vtile_chunk(v, sv, heads, L, C, bh0 * C + ((int64_t)blockIdx.x - kblocks), vtiles, vf16, lds);
}

}  // namespace

hipError_t launch_tile_prepass(const void *src, Strides s, int batch, int heads, int64_t L,
                               TileQuant quant, void *rows_out, void *tiles_out, const float *g,
                               const float *mean, hipStream_t stream, TileOut out) {
  const int64_t C = (L + kChunk - 1) / kChunk;
  const int64_t blocks = (int64_t)batch * heads * C;
  if (quant == kQuantD && !g && !mean && rows_out && !tiles_out && (out == kOutBf16 || out == kOutF16)) {
    const int64_t n8 = blocks * kChunk * (kD / 8);
    AQ_LAUNCH("tile_prepass", rows_prepass, dim3((unsigned)(n8 / 64)), dim3(64), 0, stream, (const uint16_t *)src, s,
              heads, L, C, n8, (u32x4 *)rows_out, (int)(out == kOutF16));
    return hipGetLastError();
  }
  AQ_LAUNCH("tile_prepass", tile_prepass, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const uint16_t *)src, s, heads, L, C, (int)quant, (u32x4 *)rows_out,
                     (uint16_t *)tiles_out, g, mean, (int)out);
  return hipGetLastError();
}

hipError_t launch_kv_stream(const void *k, Strides sk, const void *v, Strides sv, int batch, int heads, int64_t L,
                            int64_t bh0, int64_t nbh, void *krows, bool kf16, void *vtiles, bool vf16,
                            hipStream_t stream) {
  const int64_t C = (L + kChunk - 1) / kChunk;
  if (bh0 < 0 || nbh < 0 || bh0 + nbh > (int64_t)batch * heads) return hipErrorInvalidValue;
  if (nbh == 0 || C == 0) return hipSuccess;
  const int64_t kblocks = nbh * C * (kChunk / 64);  // 64 K rows per workgroup
  const int64_t blocks = kblocks + nbh * C;
  AQ_LAUNCH("kv_prepass", kv_prepass, dim3((unsigned)blocks), dim3(256), 0, stream, (const uint16_t *)k, sk,
            (const uint16_t *)v, sv, heads, L, C, bh0, kblocks, (u32x4 *)krows, (int)kf16, (uint16_t *)vtiles,
            (int)vf16);
  return hipGetLastError();
}

}  // namespace aq
