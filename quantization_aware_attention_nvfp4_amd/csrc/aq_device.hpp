// aq_device.hpp - device helpers shared by the gfx950 kernels: bf16 packing, the NVFP4 codec
// and MFMA operand types.
//
// Format ("vsqa-preview-1.3b metadata.json", dense precision record: group_size 16, qk/pv_format
// NVFP4 E2M1, qk/pv_scale_dtype FP8 E4M3FN; "nvfp4_qad.py" module docstring: per-16 E4M3 block
// scales under a unit or static global scale, FP4_RANGE = 448*6).
//
// Every function here is __host__ __device__ so the arithmetic can be checked exhaustively on the
// CPU; the CPU and gfx950 both round fp32 add/mul/fma/div to nearest-even, so results agree bit
// for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace aq {

constexpr int kHeadDim = 128;  // the only supported head size ("attn_qat_train" page,
                               // get_supported_head_sizes)
constexpr int kBlock = 16;     // fake-quant block length
constexpr int kChunk = 128;    // keys per online-softmax chunk

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__host__ __device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
__host__ __device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }

// bf16 bits <-> fp32.  The round-to-nearest-even conversion is only used where the kernels need
// it outside the packed hardware conversion.
__host__ __device__ __forceinline__ float bf16lo(uint32_t w) { return u2f(w << 16); }
__host__ __device__ __forceinline__ float bf16hi(uint32_t w) { return u2f(w & 0xFFFF0000u); }
__host__ __device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = f2u(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
// Two fp32 values whose bf16 rounding is exact (every fake-quantized value is): truncate.
__host__ __device__ __forceinline__ uint32_t pack_exact_bf16(float lo, float hi) {
  return (f2u(lo) >> 16) | (f2u(hi) & 0xFFFF0000u);
}

// Round v >= 0 (finite) to the nearest FP8 E4M3FN value: 3 mantissa bits, smallest normal
// exponent -6 (subnormals are multiples of 2^-9), ties to even, saturating at 448.
// Adding c = 2^(max(e, -6) + 20), e the exponent of v, leaves exactly the bits of v above
// 2^(max(e,-6)-3) after the fp32 round-to-nearest-even; subtracting c restores the value.
__host__ __device__ __forceinline__ float round_e4m3(float v) {
  uint32_t e = f2u(v) & 0x7F800000u;
  e = e > 0x3C800000u ? e : 0x3C800000u;  // 2^-6
  const float c = u2f(e + (20u << 23));
  const float r = (v + c) - c;
  return r < 448.0f ? r : 448.0f;
}

// Round r >= 0 to the nearest E2M1 magnitude {0, .5, 1, 1.5, 2, 3, 4, 6}: one mantissa bit,
// smallest normal exponent 0 (step 0.5 below 2), ties to the even code, saturating at 6.
// Same construction with c = 2^(max(e, 0) + 22): the grid step is 0.5 on [0,2), 1 on [2,4) and 2
// on [4,8); the even multiple of the step is the even code.
__host__ __device__ __forceinline__ float round_e2m1(float r) {
  uint32_t e = f2u(r) & 0x7F800000u;
  e = e > 0x3F800000u ? e : 0x3F800000u;  // 2^0
  const float c = u2f(e + (22u << 23));
  const float y = (r + c) - c;
  return y < 6.0f ? y : 6.0f;
}

// fp32(a / 6) without a division: q0 = a * RN(1/6), one Markstein correction.  Equal to the
// IEEE quotient for every fp32 a >= 2^-120; below that both round to the E4M3 scale 0 (checked
// exhaustively on the host).
__host__ __device__ __forceinline__ float div6(float a) {
  const float inv6 = 0.16666667163372039794921875f;  // RN(1/6)
  const float q0 = a * inv6;
  const float rem = __builtin_fmaf(-q0, 6.0f, a);
  return __builtin_fmaf(rem, inv6, q0);
}

// fp32(x / S) for an E4M3 value S > 0 given inv = fp32(1 / S): one Markstein correction.
// Equal to the IEEE quotient for every such S and every fp32 x with |x/S| in [2^-5, 2^7)
// (checked exhaustively on the host over the 8 significands of S; the sequence is odd in x and
// invariant under power-of-two scaling).  Smaller quotients round to 0 either way.
__host__ __device__ __forceinline__ float div_e4m3(float x, float S, float inv) {
  const float q0 = x * inv;
  const float rem = __builtin_fmaf(-q0, S, x);
  return __builtin_fmaf(rem, inv, q0);
}

// One Newton step that turns any approximation y0 within 2 ulps of 1/S into fp32(1/S) for every
// positive E4M3 value S (checked on the host for all 126 values and all such y0).
__host__ __device__ __forceinline__ float newton_recip(float S, float y0) {
  const float e = __builtin_fmaf(-S, y0, 1.0f);
  return __builtin_fmaf(e, y0, y0);
}

// fp32(1/S) for an E4M3 value S > 0: hardware reciprocal (about 1 ulp) plus the Newton step.
__device__ __forceinline__ float recip_e4m3(float S) { return newton_recip(S, __builtin_amdgcn_rcpf(S)); }

// Unit-global-scale block scale: S = E4M3(fp32(amax / 6)).
__host__ __device__ __forceinline__ float block_scale_unit(float amax) { return round_e4m3(div6(amax)); }

// Fake-quantize one value with block scale S (> 0) and inv = 1/S under the unit global scale:
// sign(x) * E2M1(|x| / S) * S.  The product has at most 6 significant bits, so it is exact.
__host__ __device__ __forceinline__ float fq_unit(float x, float S, float inv) {
  const float ax = __builtin_fabsf(x);
  const float q = round_e2m1(div_e4m3(ax, S, inv));
  return u2f(f2u(q * S) | (f2u(x) & 0x80000000u));
}

// Same under a general global scale: S = s/g is not an E4M3 value, so the quotient is an IEEE
// division.  Returns the fp32 dequantized value (the caller rounds to bf16).
__host__ __device__ __forceinline__ float fq_general(float x, float S) {
  const float ax = __builtin_fabsf(x);
  const float q = round_e2m1(ax / S);
  return u2f(f2u(q * S) | (f2u(x) & 0x80000000u));
}

// Cross-lane exchanges inside a 64-wide wavefront.
// Value of lane (l ^ 1): DPP quad permutation [1, 0, 3, 2].
__device__ __forceinline__ float xor1(float v) {
  return u2f(__builtin_amdgcn_mov_dpp((int)f2u(v), 0xB1, 0xF, 0xF, true));
}
// The larger of two values in one v_max_f32.  fmaxf would first copy each operand through a
// quieting v_max (the compiler cannot know they are not signalling NaNs); the values here are
// logits and running maxima, which come from MFMAs and maxima, never from memory.
__device__ __forceinline__ float max_nq(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// Combine a value with the one in lane (l ^ 32).  v_permlane32_swap exchanges the upper half
// of its first operand with the lower half of its second; with both operands equal to v its two
// results hold (v_l, v_{l^32}) in some order in every lane, so a symmetric combination of the two
// gives both lanes of a pair the same bits.
__device__ __forceinline__ float pair_max(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(f2u(v), f2u(v), false, false);
  return max_nq(u2f(p[0]), u2f(p[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(f2u(v), f2u(v), false, false);
  return u2f(p[0]) + u2f(p[1]);
}

// Two values rounded to the nearest E2M1 value (ties to the even code, saturating at +-6, sign
// kept) by the gfx950 packed FP4 conversion with a unit scale, and converted back.  Equal to
// round_e2m1 with the sign restored (an in-bounds sweep of 11.3M fp32 inputs, every midpoint and
// its neighbours included, and the bit-exact fake-quant tests check this on the GPU).
__device__ __forceinline__ void e2m1_pair(float &a, float &b) {
  const uint32_t code = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0);
  const auto r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, 1.0f, 0);
  a = r[0];
  b = r[1];
}

// ---- Softmax-probability fake quantization in the attention kernels -----------------------
// A P block (16 keys of one query) has P = exp2(y - m) with y = c * logit.  Its scale is
// S = E4M3(amax / 6) with amax = exp2(c * logit_max - m), logit_max the block's largest logit
// (exp2 is monotone).
// The E2M1 argument P / S is taken in one exponential, r = exp2(y - mb) with mb = m + log2(Sd),
// Sd = max(S, 2^-9).  A block whose scale is 0 has amax / 6 <= 2^-10, so its r = 512 P stays at
// most 3 and its dequantized values, code * S, are 0 whatever the codes; Sd = 2^-9 (the smallest
// E4M3 step, an exact power of two) keeps the unquantized P = Sd * r of every block.  Forward and
// backward both use this exact sequence, so they agree on every code.
//
// The E4M3 rounding of amax / 6 runs on the gfx950 FP8 conversions (fp32 -> E4M3FN -> fp32 and
// -> fp16, unit scale): round to nearest even with subnormals kept, equal to round_e4m3 for every
// fp32 in [0, 464] (an in-bounds sweep of every fp32 bit pattern in [0, 0.25] matched bit for bit;
// above 464 the conversion gives NaN instead of saturating, and amax / 6 is at most about 1/6
// here).  amax / 6 is one multiply by RN(1/6), within one ulp of the quotient.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
constexpr float kRcp6 = 0.16666667163372039794921875f;  // RN(1/6)
constexpr float kScaleFloor = 0.001953125f;             // 2^-9

struct ProbBlock {
  float S;      // the block scale (0 for a zero block)
  float Sd;     // max(S, 2^-9)
  float mb;     // m + log2(Sd)
  _Float16 Sh;  // S as fp16 (exact)
};
__device__ __forceinline__ ProbBlock prob_block(float logit_max, float c, float m) {
  const float a6 = __builtin_amdgcn_exp2f(__builtin_fmaf(logit_max, c, -m)) * kRcp6;
  const s16x2 w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s16x2{0, 0}, a6, a6, 1.0f, false);
  const uint32_t wb = __builtin_bit_cast(uint32_t, w);
  const float S = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(wb, 1.0f, false)[0];
  const f16x2 h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wb, 1.0f, false);
  const float Sd = u2f(max(f2u(S), f2u(kScaleFloor)));  // S >= 0: the integer maximum
  return ProbBlock{S, Sd, m + __builtin_amdgcn_logf(Sd), h[0]};
}
// The four blocks of a lane's 64 logits (four 32-key sub-tiles) at once: the conversions take
// two values each.
__device__ __forceinline__ void prob_blocks4(const float *logit_max, float c, float m, ProbBlock *pb) {
  float a6[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) a6[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(logit_max[i], c, -m)) * kRcp6;
  s16x2 w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s16x2{0, 0}, a6[0], a6[1], 1.0f, false);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, a6[2], a6[3], 1.0f, true);
  const uint32_t wb = __builtin_bit_cast(uint32_t, w);
  const auto S01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(wb, 1.0f, false);
  const auto S23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(wb, 1.0f, true);
  const f16x2 h01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wb, 1.0f, false);
  const f16x2 h23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wb, 1.0f, true);
  const float S[4] = {S01[0], S01[1], S23[0], S23[1]};
  const _Float16 h[4] = {h01[0], h01[1], h23[0], h23[1]};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float Sd = u2f(max(f2u(S[i]), f2u(kScaleFloor)));
    pb[i] = ProbBlock{S[i], Sd, m + __builtin_amdgcn_logf(Sd), h[i]};
  }
}
// The same under the static global scale g of P's blocks: s = E4M3(fp32(fp32(amax / 6) * g)),
// S = fp32(s / g).  S is then not an E4M3 value, so the dequantized P-hat is rounded to bf16 as
// the matmul operand.
__device__ __forceinline__ ProbBlock prob_block_static(float logit_max, float c, float m, float g) {
  const float am = __builtin_amdgcn_exp2f(__builtin_fmaf(logit_max, c, -m));
  const float S = round_e4m3((am / 6.0f) * g) / g;
  const float Sd = S == 0.0f ? 1.0f : S;
  return ProbBlock{S, Sd, m + __builtin_amdgcn_logf(Sd), (_Float16)S};
}
// The static scale of P's blocks ("nvfp4_qad.py" FP4_RANGE over P's largest value, 1).
constexpr float kPScaleStatic = 448.0f * 6.0f;
// Two-level P (SageAttention3's recipe, the two_level_quant_p_sage3 flag of the "attn_qat_train"
// API page): the first level of a (row, chunk) maps the chunk's largest P of the row,
// exp2(fma(cm, c, -m)) for the row's largest logit cm in the chunk, to 448*6; 448*6 when that P
// is 0 (no live key).  P's blocks then take it as their global scale.
__device__ __forceinline__ float two_level_scale(float cm, float c, float m) {
  const float rm = __builtin_amdgcn_exp2f(__builtin_fmaf(cm, c, -m));
  return rm > 0.0f ? kPScaleStatic / rm : kPScaleStatic;
}

// Eight values rounded to E2M1 codes in one register (byte i holds pair i; ties to the even
// code, saturating at +-6, sign kept), by the gfx950 packed FP4 conversion with a unit scale.
__device__ __forceinline__ uint32_t e2m1_codes8(const float *r) {
  // Each conversion writes one byte and keeps the rest; all four bytes are written, so the
  // starting value only has to be some defined register (r[0]'s bits: no extra move).
  uint32_t code = __builtin_bit_cast(uint32_t, r[0]);
  code = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(code, r[0], r[1], 1.0f, 0);
  code = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(code, r[2], r[3], 1.0f, 1);
  code = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(code, r[4], r[5], 1.0f, 2);
  code = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(code, r[6], r[7], 1.0f, 3);
  return code;
}
// The eight coded values times f, as fp32.
__device__ __forceinline__ void e2m1_decode8(uint32_t code, float f, float *x) {
  const auto a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, 1.0f, 0);
  const auto b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, 1.0f, 1);
  const auto c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, 1.0f, 2);
  const auto d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, 1.0f, 3);
  x[0] = a[0] * f; x[1] = a[1] * f; x[2] = b[0] * f; x[3] = b[1] * f;
  x[4] = c[0] * f; x[5] = c[1] * f; x[6] = d[0] * f; x[7] = d[1] * f;
}
// The eight coded values times S as fp16 (exact: an E2M1 value times an E4M3 scale has at most 6
// significant bits and lies in [2^-10, 6 * 448]), packed two per register.
__device__ __forceinline__ u32x4 e2m1_decode8_f16(uint32_t code, _Float16 h) {
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(code, 1.0f, 0) * h;
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(code, 1.0f, 1) * h;
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(code, 1.0f, 2) * h;
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(code, 1.0f, 3) * h;
  return u32x4{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
               __builtin_bit_cast(uint32_t, d)};
}

// Fake-quantize two non-negative values of one block (unit global scale, scale S and inv = 1/S,
// inv = 0 for a zero block): E2M1(x / S) * S.
__device__ __forceinline__ void fq_pos_pair(float &a, float &b, float S, float inv) {
  float ra = div_e4m3(a, S, inv), rb = div_e4m3(b, S, inv);
  e2m1_pair(ra, rb);
  a = ra * S;
  b = rb * S;
}

// Same for signed values: the magnitude is quantized and the sign bit of x is put back, so -0
// stays -0.
__device__ __forceinline__ void fq_unit_pair(float &a, float &b, float S, float inv) {
  const uint32_t sa = f2u(a) & 0x80000000u, sb = f2u(b) & 0x80000000u;
  float ra = __builtin_fabsf(a), rb = __builtin_fabsf(b);
  fq_pos_pair(ra, rb, S, inv);
  a = u2f(f2u(ra) | sa);
  b = u2f(f2u(rb) | sb);
}

}  // namespace aq
