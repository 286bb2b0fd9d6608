// attn_fwd.hip - NVFP4 fake-quantized attention forward on gfx950 (MI355X).
//
// Method ("vsqa-preview-1.3b metadata.json", attention.precision: "NVFP4 fake-quant with BF16
// matmul", quant_p, quant_v, unit global scales; "attn_qat_train" API page: attn_qat_train with
// use_high_prec_o): Q-hat and K-hat are fake-quantized along D, V-hat along keys, and the softmax
// probabilities P along keys, all in 16-element blocks with E4M3 scales and E2M1 values; both
// matmuls run on BF16 MFMA with fp32 accumulation inside an online softmax whose running maximum
// is refreshed once per 128-key chunk.
//
// K-hat (rows) and V-hat (d-major chunk tiles) are fake-quantized once per call into the workspace
// by the tile prepass (prepass.hip); the forward kernel runs one workgroup per (head, tile of
// 32*WAVES queries) and each wave owns 32 queries.
//
// Wave data layout (v_mfma_f32_32x32x16_bf16; accumulator element (row i, column j) sits in lane
// j + 32*((i/4)%2), register 4*(i/8) + i%4):
//   S^T = K-hat Q-hat^T: A = 32 K-hat rows, B = Q-hat^T (columns = the wave's 32 queries).  The
//     K rows are fed in the order key(i) = 16*((i/4)%2) + 4*(i/8) + i%4, so lane l holds query
//     l%32 and, in its 16 registers, the 16 consecutive keys 16*(l/32) + r of the 32-key
//     sub-tile: one whole P fake-quant block per lane and sub-tile, no cross-lane traffic.
//   O^T += V-hat^T P-hat^T: A = V-hat^T rows (d), B = P-hat^T taken straight from the registers
//     that held S^T, so P never leaves the lane.  O^T keeps the query in the lane, so the
//     per-row softmax rescale is a per-lane scalar.
//   A row's 128 keys per chunk are split over lanes l and l^32; the chunk max needs one
//   permlane32 swap, the denominator is combined once at the end.
// LDS: one K-hat chunk (32 KiB) and one V-hat^T chunk (32 KiB), 16-byte columns XOR-swizzled by
// row so the A-operand reads of 8 lanes hit 8 different bank groups.
#include <type_traits>

#include "attn_common.hpp"
#include "launch.hpp"
#include "timing.hpp"

namespace aq {
namespace {

constexpr int kD = kHeadDim;
constexpr int kMaxSel = 1024;  // longest cube-sparse chunk list (checked by the launcher)

// ------------------------------------------------------------------------------------------
// Forward kernel
// ------------------------------------------------------------------------------------------

struct FwdParams {
  const uint16_t *q;
  Strides sq;
  uint16_t *o;
  Strides so;
  const u32x4 *kq;   // workspace K-hat
  const u32x4 *vt;   // workspace V-hat^T tiles
  float *lse;        // [BH, lq] or null
  float *cmax;       // [BH, C, lq] or null
  float *o_hp;       // [BH, lq, 128] or null
  const int32_t *sel;  // cube-sparse: [BH, n_cubes, topk] selected chunks, or null (dense)
  int heads;
  int64_t lq, lk;
  int64_t nchunks;   // dense: ceil(lk/128); sparse: topk
  int64_t kchunks;   // chunks of the K/V workspace per head
  int qtiles;        // ceil(lq / (32*WAVES))
  int64_t nblocks;   // heads*batch*qtiles
  int64_t per_xcd;   // ceil(nblocks / 8)
  float c;           // softmax_scale * log2(e)
  bool causal, quant_q;
  const float *gq;      // static global scale of Q (device scalar), or null for the unit scale
  const float *m_init;  // [BH, lq] final row maxima (base 2) seeding the running max, or null
  float *m_out;         // row-max pass: where it writes them
  bool two_level;       // P's global scale per (row, chunk): two_level_scale (GP kernels)
  float *pg;            // training, two-level: [BH, C, lq] those scales, or null
  const float *qmean;   // smooth-Q: [BH, 128] the queries' mean, subtracted before quantization
  const float *delta;   // smooth-Q: [BH, kchunks*128] <mean, k-hat_j>, added to every logit
  float gp_static;      // GP kernels: P's global scale when it is not the two-level one (448*6, or 1)
};

// Copy offsets of this lane's 16-byte pieces of a staged [128][256 B] tile by a workgroup of
// WAVES waves: LDS instruction i of wave w covers rows 4*WAVES*i + 4w .. +3 (physical column
// lane%16); the lane fetches the logical column the swizzle maps there.  Row 4*WAVES*i + 4w +
// lane/16 of the source starts 1024*WAVES*i bytes past the tile base, which the wave-uniform base
// absorbs, so one 32-bit offset serves every i whose swizzle term is the same (sw_kq depends on
// row bit 4, i.e. on i%2 for 4 waves and not on i for 8; sw_row on neither).
struct StageOffsets {
  uint32_t k_even, k_odd, v;
};
template <int WAVES>
__device__ __forceinline__ StageOffsets stage_offsets(int wave, int lane) {
  const int r = 4 * wave + (lane >> 4), pc = lane & 15;
  return StageOffsets{(uint32_t)(r * 256 + ((pc ^ sw_kq(r)) << 4)),
                      (uint32_t)(r * 256 + ((pc ^ sw_kq(r + 4 * WAVES)) << 4)),
                      (uint32_t)(r * 256 + ((pc ^ sw_row(r)) << 4))};
}
template <int WAVES>
__device__ __forceinline__ void stage_k(const uint8_t *gtile, uint8_t *lds, const StageOffsets &so, int wave) {
#pragma unroll
  for (int i = 0; i < 32 / WAVES; ++i)
    load_lds16_s(gtile + 1024 * WAVES * i, (i & 1) ? so.k_odd : so.k_even, lds + 1024 * WAVES * i + 1024 * wave);
}
template <int WAVES>
__device__ __forceinline__ void stage_v(const uint8_t *gtile, uint8_t *lds, const StageOffsets &so, int wave) {
#pragma unroll
  for (int i = 0; i < 32 / WAVES; ++i) load_lds16_s(gtile + 1024 * WAVES * i, so.v, lds + 1024 * WAVES * i + 1024 * wave);
}
// The same copies with the LDS tile given as an LDS byte address.
template <int WAVES>
__device__ __forceinline__ void stage_k_at(const uint8_t *gtile, uint32_t lds, const StageOffsets &so, int wave) {
#pragma unroll
  for (int i = 0; i < 32 / WAVES; ++i)
    load_lds16_sa(gtile + 1024 * WAVES * i, (i & 1) ? so.k_odd : so.k_even, lds + 1024 * WAVES * i + 1024 * wave);
}
template <int WAVES>
__device__ __forceinline__ void stage_v_at(const uint8_t *gtile, uint32_t lds, const StageOffsets &so, int wave) {
#pragma unroll
  for (int i = 0; i < 32 / WAVES; ++i) load_lds16_sa(gtile + 1024 * WAVES * i, so.v, lds + 1024 * WAVES * i + 1024 * wave);
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Q-hat fragment of the lane's query (zero past lq): the S^T B operand, d = 16t + 8hf + (0..7);
// the two lane halves hold the two 8-element halves of each 16-element block along D.
__device__ __forceinline__ void load_q_frags(const FwdParams &p, int64_t bb, int64_t hh, int64_t qrow, bool qvalid,
                                             int hf, bf16x8 (&qf)[8]) {
  const uint16_t *qp = p.q + bb * p.sq.b + hh * p.sq.h + (qvalid ? qrow : 0) * p.sq.l;
  const float g = p.gq ? *p.gq : 1.0f;
  const float *qm = p.qmean ? p.qmean + (bb * p.heads + hh) * kD : nullptr;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (qvalid) v = *(const u32x4 *)(qp + 16 * t + 8 * hf);
    if (qm) {
      // smooth-Q: fp32(q - mean) (rows past lq stay zero), then the quantizer of the K prepass
      // (unit: the exact-quotient pair path; static: the IEEE quotient), rounded to bf16
      float f[8] = {bf16lo(v.x), bf16hi(v.x), bf16lo(v.y), bf16hi(v.y),
                    bf16lo(v.z), bf16hi(v.z), bf16lo(v.w), bf16hi(v.w)};
      if (qvalid) {
        const f32x4 m0 = *(const f32x4 *)(qm + 16 * t + 8 * hf), m1 = *(const f32x4 *)(qm + 16 * t + 8 * hf + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f[i] = f[i] - m0[i];
          f[4 + i] = f[4 + i] - m1[i];
        }
      }
      if (p.quant_q) {
        float am = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) am = fmaxf(am, __builtin_fabsf(f[i]));
        am = pair_max(am);
        if (p.gq) {
          // the prepass's static-scale block arithmetic (fq_block_static), on this lane's half
          const float S = round_e4m3((am / 6.0f) * g) / g;
          const bool zero = !(S > 0.0f);
#pragma unroll
          for (int i = 0; i < 8; ++i) f[i] = zero ? 0.0f * f[i] : fq_general(f[i], S);
        } else {
          const float S = block_scale_unit(am);
          const float inv = S == 0.0f ? 0.0f : recip_e4m3(S);
#pragma unroll
          for (int i = 0; i < 8; i += 2) fq_unit_pair(f[i], f[i + 1], S, inv);
        }
      }
      v = u32x4{f32_to_bf16_rne(f[0]) | (f32_to_bf16_rne(f[1]) << 16), f32_to_bf16_rne(f[2]) | (f32_to_bf16_rne(f[3]) << 16),
                f32_to_bf16_rne(f[4]) | (f32_to_bf16_rne(f[5]) << 16), f32_to_bf16_rne(f[6]) | (f32_to_bf16_rne(f[7]) << 16)};
    } else if (p.quant_q && p.gq) {
      // static global scale: the IEEE quotient and the value rounded to bf16
      float f[8] = {bf16lo(v.x), bf16hi(v.x), bf16lo(v.y), bf16hi(v.y),
                    bf16lo(v.z), bf16hi(v.z), bf16lo(v.w), bf16hi(v.w)};
      float am = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) am = fmaxf(am, __builtin_fabsf(f[i]));
      am = pair_max(am);
      const float S = round_e4m3((am / 6.0f) * g) / g;
      const bool zero = !(S > 0.0f);
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = zero ? 0.0f * f[2 * i] : fq_general(f[2 * i], S);
        const float b = zero ? 0.0f * f[2 * i + 1] : fq_general(f[2 * i + 1], S);
        w[i] = f32_to_bf16_rne(a) | (f32_to_bf16_rne(b) << 16);
      }
      v = u32x4{w[0], w[1], w[2], w[3]};
    } else if (p.quant_q) {
      float f[8] = {bf16lo(v.x), bf16hi(v.x), bf16lo(v.y), bf16hi(v.y),
                    bf16lo(v.z), bf16hi(v.z), bf16lo(v.w), bf16hi(v.w)};
      float am = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) am = fmaxf(am, __builtin_fabsf(f[i]));
      am = pair_max(am);
      const float S = block_scale_unit(am);
      const float inv = S == 0.0f ? 0.0f : recip_e4m3(S);
#pragma unroll
      for (int i = 0; i < 8; i += 2) fq_unit_pair(f[i], f[i + 1], S, inv);
      v = u32x4{pack_exact_bf16(f[0], f[1]), pack_exact_bf16(f[2], f[3]), pack_exact_bf16(f[4], f[5]),
                pack_exact_bf16(f[6], f[7])};
    }
    qf[t] = __builtin_bit_cast(bf16x8, v);
  }
}

// P of one 32-key sub-tile, whose 16 logits in the lane's registers are one P block, as the two
// P-hat V-hat B operands (keys 0-7 and 8-15 of the block); psum gains the block's unquantized sum.
// pb: the block's scale (prob_block, or prob_block_static under P's global scale).  HP: also the
// unquantized P as operands (ph), for O^hp.  GP: P's blocks under a global scale, P-hat rounded to
// bf16.  GP with F16 is the FP8 P.V product: that bf16 P-hat is further rounded to the nearest
// E4M3FN value, which fp16 holds exactly.
template <bool F16, bool HP, bool GP>
__device__ __forceinline__ void form_pq(const f32x16 &s, const ProbBlock &pb, float c, float &psum, u32x4 (&pq)[2],
                                        u32x4 (&ph)[2]) {
  float r[16];
  r[0] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[0], c, -pb.mb));
  float rsum = r[0];  // the same sum as from 0: r >= 0
#pragma unroll
  for (int i = 1; i < 16; ++i) {
    r[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -pb.mb));
    rsum += r[i];
  }
  psum = __builtin_fmaf(pb.Sd, rsum, psum);
  const uint32_t c0 = e2m1_codes8(r), c1 = e2m1_codes8(r + 8);
  if (F16 && !GP) {
    pq[0] = e2m1_decode8_f16(c0, pb.Sh);
    pq[1] = e2m1_decode8_f16(c1, pb.Sh);
  } else {
    float x[8];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      e2m1_decode8(j ? c1 : c0, pb.S, x);
      if (F16) {  // FP8 P.V product (P-hat >= 0)
        f16x8 h;
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = (_Float16)round_e4m3(bf16lo(f32_to_bf16_rne(x[i])));
        pq[j] = __builtin_bit_cast(u32x4, h);
      } else {
        pq[j] = __builtin_bit_cast(u32x4, pack8_cvt(x));
      }
    }
  }
  if (HP) {
#pragma unroll
    for (int i = 0; i < 16; ++i) r[i] *= pb.Sd;  // the unquantized P
    if (F16) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        f16x8 h;
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = (_Float16)r[8 * j + i];
        ph[j] = __builtin_bit_cast(u32x4, h);
      }
    } else {
      ph[0] = __builtin_bit_cast(u32x4, pack8_cvt(r));
      ph[1] = __builtin_bit_cast(u32x4, pack8_cvt(r + 8));
    }
  }
}

// The scale of a P block from its largest logit: unit or global scale g.
template <bool GP>
__device__ __forceinline__ ProbBlock p_block(float bmax, float c, float m_new, float g) {
  return GP ? prob_block_static(bmax, c, m_new, g) : prob_block(bmax, c, m_new);
}

// form_pq with the block's scale computed here; without QP, P itself (bf16) as the operands.
template <bool QP, bool F16, bool HP, bool GP>
__device__ __forceinline__ void form_p(const f32x16 &s, float bmax, float c, float m_new, float g, float &psum,
                                       u32x4 (&pq)[2], u32x4 (&ph)[2]) {
  if (QP) {
    form_pq<F16, HP, GP>(s, p_block<GP>(bmax, c, m_new, g), c, psum, pq, ph);
  } else {
    float P[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      P[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -m_new));
      psum += P[i];
    }
    pq[0] = __builtin_bit_cast(u32x4, pack8_cvt(P));
    pq[1] = __builtin_bit_cast(u32x4, pack8_cvt(P + 8));
  }
}

// TRAIN: also write lse, chunk maxima and O^hp.  QP: P is fake-quantized.  F16: P-hat and V-hat
// (both fake-quantized, hence exact in fp16) multiply on the fp16 MFMA, whose products are the
// same as the bf16 ones for these values.
//
// This kernel serves training, smooth-Q and the cube-sparse calls; other dense inference runs the
// ping-pong kernel below.  Inference: 4 waves (128 queries) per workgroup, two workgroups per CU.  With the
// O^hp product
// the two accumulators leave no room for the Q-hat operand in registers at two waves per SIMD,
// so that variant runs 8 waves (256 queries) per workgroup, one per CU, with each wave's Q-hat
// rows in LDS (8 KiB per wave) and re-read once per chunk.
//
// QL selects the 8-wave layout.  The cube-sparse training forward keeps 4 waves (its chunk lists
// are per 128 queries) and then runs one wave per SIMD.
template <bool TRAIN, bool QP, bool F16, bool QL, bool GP, bool SQ>
__global__ __launch_bounds__(QL ? 512 : 256, (QL || (TRAIN && QP)) ? 1 : 2) void attn_fwd_kernel(FwdParams p) {
  static_assert(!F16 || QP, "the fp16 product needs a quantized P");
  constexpr bool HP = TRAIN && QP;  // O^hp needs its own product only when P is quantized
  constexpr int WAVES = QL ? 8 : 4;
  constexpr int BM = 32 * WAVES;
  // Separate objects, so the compiler can tell reads of one tile from copies into the other.
  __shared__ __attribute__((aligned(256))) uint8_t lds_k[kChunk * 256];
  __shared__ __attribute__((aligned(256))) uint8_t lds_v[kChunk * 256];
  __shared__ __attribute__((aligned(256))) uint8_t lds_q[QL ? WAVES * 32 * 256 : 256];
  __shared__ int32_t lds_sel[kMaxSel];

  const int64_t vid = xcd_work_id(blockIdx.x, p.per_xcd, p.nblocks);
  if (vid < 0) return;
  const int64_t bh = vid / p.qtiles;
  const int qt = (int)(vid % p.qtiles);
  const int64_t bb = bh / p.heads, hh = bh % p.heads;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in a scalar register
  const int lane = tid & 63;
  const int n = lane & 31;   // the lane's query within the wave
  const int hf = lane >> 5;  // lane half
  const int64_t qrow = (int64_t)qt * BM + wave * 32 + n;
  const bool qvalid = qrow < p.lq;

  int64_t n_iter = p.nchunks;
  if (p.causal) {
    const int64_t q_last = (int64_t)qt * BM + BM - 1;
    n_iter = (q_last < p.lk - 1 ? q_last : p.lk - 1) / kChunk + 1;
  }
  // Cube-sparse: this query cube's chunk list, read once into LDS.
  if (p.sel) {
    const int32_t *src = p.sel + (bh * (p.lq / kChunk) + (int64_t)qt * BM / kChunk) * p.nchunks;
    for (int i = tid; i < p.nchunks; i += WAVES * 64) lds_sel[i] = src[i];
    __syncthreads();
  }
  auto chunk_of = [&](int64_t it) -> int64_t {
    return p.sel ? clamp_chunk(__builtin_amdgcn_readfirstlane(lds_sel[it]), p.kchunks) : it;  // uniform: a scalar
  };
  auto ktile = [&](int64_t c) { return (const uint8_t *)(p.kq + (bh * p.kchunks + c) * (kChunk * kD / 8)); };
  auto vtile = [&](int64_t c) { return (const uint8_t *)(p.vt + (bh * p.kchunks + c) * (kChunk * kD / 8)); };

  // Start the first chunk's copies before the Q work so they overlap it.
  const StageOffsets so = stage_offsets<WAVES>(wave, lane);
  int64_t chunk = chunk_of(0);
  stage_k<WAVES>(ktile(chunk), lds_k, so, wave);
  stage_v<WAVES>(vtile(chunk), lds_v, so, wave);

  bf16x8 qf[8];
  load_q_frags(p, bb, hh, qrow, qvalid, hf, qf);
  // QL: the wave's 32 Q-hat rows go to its own LDS region (row n = the lane's query, columns
  // swizzled by sw_row), read back as the S^T B operand once per chunk.
  uint32_t qa = 0;
  if (QL) {
    const int sw = n & 15;
    uint8_t *qrow_lds = lds_q + wave * 8192 + n * 256;
#pragma unroll
    for (int t = 0; t < 8; ++t) *(bf16x8 *)(qrow_lds + (((2 * t + hf) ^ sw) << 4)) = qf[t];
    qa = lds_addr(lds_q) + wave * 8192 + n * 256 + 16 * (hf ^ sw);
  }

  f32x16 acc[4];
  f32x16 acc_hp[HP ? 4 : 1];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};
#pragma unroll
  for (int dt = 0; dt < (HP ? 4 : 1); ++dt) acc_hp[dt] = f32x16{};
  // Final-max variant: the running max starts at the row's final maximum, so it never moves.
  float m_run = (p.m_init && qvalid) ? p.m_init[bh * p.lq + qrow] : -__builtin_inff();
  float l_run = 0.0f;

  // LDS byte addresses of this lane's A-operand reads.  The arrays are 256-byte aligned and a
  // column's XOR swizzle only touches bits 4..7 of the offset, so the loop-dependent part of a
  // column index enters as one XOR.  K-hat row krow, column 2t + hf: `^ 32*t`.  V-hat^T row
  // d = 32*dt + n, column 4*kt + 2*hf + j: sw_row(d) = n & 15 for every dt, so the physical
  // column (4*kt + j) ^ (2*hf ^ sw) is `^ 16*(4*kt + j)`.
  uint32_t ka, va;
  {
    const int krow = perm_row(n), swk = sw_kq(krow);
    ka = lds_addr(lds_k) + krow * 256 + 16 * (hf ^ swk);
    const int swv = n & 15;
    va = lds_addr(lds_v) + n * 256 + 16 * ((2 * hf) ^ swv);
  }

  for (int64_t it = 0; it < n_iter; ++it) {
    // K-hat(chunk) has landed once this wave's V copies (issued after it) are the only ones
    // outstanding; the barrier makes every wave's copies visible.  Smooth-Q: the logit chains
    // start from delta of the lane's keys, loaded first (16 more loads the wait lets through).
    f32x16 s[4];
    if constexpr (SQ) {
      const float *dl = p.delta + (bh * p.kchunks + chunk) * kChunk + 16 * hf;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) s[kt] = delta16(dl + 32 * kt);
      if constexpr (WAVES == 4) AQ_WAIT_VMCNT(24); else AQ_WAIT_VMCNT(20);
    } else {
      if constexpr (WAVES == 4) AQ_WAIT_VMCNT(8); else AQ_WAIT_VMCNT(4);
    }
    __builtin_amdgcn_s_barrier();
    AQ_OPAQUE(ka);
    AQ_OPAQUE(va);

    // ---- S^T = K-hat Q-hat^T for the 128 keys of the chunk ------------------------------
    // (smooth-Q: the chains start from delta; otherwise from the MFMA's constant zero)
    if constexpr (QL) {
      // Q-hat column pair t is read once and feeds the four sub-tiles' chains.
      AQ_OPAQUE(qa);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const bf16x8 b = as_bf16x8(lds_read16(qa ^ (32 * t)));
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
          s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(lds_read16((ka ^ (32 * t)) + 8192 * kt)), b,
                                                          (SQ || t > 0) ? s[kt] : f32x16{}, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
        for (int t0 = 0; t0 < 8; t0 += 4) {
          bf16x8 a[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) a[t] = as_bf16x8(lds_read16((ka ^ (32 * (t0 + t))) + 8192 * kt));
#pragma unroll
          for (int t = 0; t < 4; ++t)
            s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[t], qf[t0 + t], (SQ || t0 + t > 0) ? s[kt] : f32x16{},
                                                            0, 0, 0);
        }
      }
    }
    const int64_t next = it + 1 < n_iter ? chunk_of(it + 1) : -1;
    __builtin_amdgcn_s_barrier();  // every wave is done reading K-hat(chunk)
    if (next >= 0) stage_k<WAVES>(ktile(next), lds_k, so, wave);

    // ---- masks: keys past lk (last chunk) and causal -------------------------------------
    const int64_t key0 = chunk * kChunk + 16 * hf;  // key of register 0 in sub-tile 0
    const bool tail = (chunk + 1) * kChunk > p.lk;
    const bool diag = p.causal && (chunk + 1) * kChunk - 1 > (int64_t)qt * BM + wave * 32;
    if (tail || diag) {
      const int64_t last = p.causal ? (qrow < p.lk - 1 ? qrow : p.lk - 1) : p.lk - 1;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) mask_tail(s[kt], valid_prefix(key0 + 32 * kt, last));
    }

    // ---- running max (refreshed once per chunk) -----------------------------------------
    // Block maxima of the logits first: each lane's 16 registers of a sub-tile are one P block.
    float bmax[4];
    max16x4(s, bmax);
    float cm = max3f(max3f(bmax[0], bmax[1], bmax[2]), bmax[3], bmax[3]);
    cm = pair_max(cm);
    const float m_new = max_nq(m_run, cm * p.c);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first chunk
    if (TRAIN && hf == 0 && qvalid) p.cmax[(bh * p.nchunks + it) * p.lq + qrow] = m_new;
    const float g = (GP && p.two_level) ? two_level_scale(cm, p.c, m_new) : p.gp_static;
    if (TRAIN && GP && p.pg && hf == 0 && qvalid) p.pg[(bh * p.nchunks + it) * p.lq + qrow] = g;
    m_run = m_new;
    // The rescale is skipped when no row of the wave moved its maximum (alpha == 1 exactly).
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) acc[dt] *= alpha;
      if (HP) {
#pragma unroll
        for (int dt = 0; dt < (HP ? 4 : 1); ++dt) acc_hp[dt] *= alpha;
      }
    }

    // V-hat(chunk): wait for this wave's V copies (K(next) may still be in flight).
    if (next < 0) AQ_WAIT_VMCNT(0);
    else if constexpr (WAVES == 4) AQ_WAIT_VMCNT(8);
    else AQ_WAIT_VMCNT(4);
    __builtin_amdgcn_s_barrier();

    // ---- per 32-key sub-tile: P, its sum, P-hat, and O^T += V-hat^T P-hat^T ---------------
    float psum = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      u32x4 pq[2], ph[2];
      form_p<QP, F16, HP, GP>(s[kt], bmax[kt], p.c, m_new, g, psum, pq, ph);
      u32x4 a[2][4];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) a[j][dt] = lds_read16((va ^ (16 * (4 * kt + j))) + 8192 * dt);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          if (F16) {
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a[j][dt]),
                                                             __builtin_bit_cast(f16x8, pq[j]), acc[dt], 0, 0, 0);
            if (HP)
              acc_hp[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a[j][dt]),
                                                                  __builtin_bit_cast(f16x8, ph[j]), acc_hp[dt], 0, 0, 0);
          } else {
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[j][dt]), as_bf16x8(pq[j]), acc[dt], 0, 0, 0);
            if (HP)
              acc_hp[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[j][dt]), as_bf16x8(ph[j]), acc_hp[dt], 0, 0, 0);
          }
        }
    }
    l_run = l_run * alpha + psum;
    __builtin_amdgcn_s_barrier();  // every wave is done reading V-hat(chunk)
    if (next >= 0) stage_v<WAVES>(vtile(next), lds_v, so, wave);
    chunk = next;
  }

  // ---- epilogue --------------------------------------------------------------------------
  const float l = pair_sum(l_run);
  const float inv_l = 1.0f / l;
  if (!qvalid) return;
  uint16_t *op = p.o + bb * p.so.b + hh * p.so.h + qrow * p.so.l;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d0 = 32 * dt + 8 * a + 4 * hf;
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      const bf16x4 w = {(__bf16)(acc[dt][4 * a + 0] * inv_l), (__bf16)(acc[dt][4 * a + 1] * inv_l),
                        (__bf16)(acc[dt][4 * a + 2] * inv_l), (__bf16)(acc[dt][4 * a + 3] * inv_l)};
      *(bf16x4 *)(op + d0) = w;
      if (TRAIN) {
        const f32x16 &h = HP ? acc_hp[HP ? dt : 0] : acc[dt];
        float *hp = p.o_hp + (bh * p.lq + qrow) * kD + d0;
        *(f32x4 *)hp = f32x4{h[4 * a] * inv_l, h[4 * a + 1] * inv_l, h[4 * a + 2] * inv_l, h[4 * a + 3] * inv_l};
      }
    }
  if (TRAIN && hf == 0) p.lse[bh * p.lq + qrow] = m_run + __builtin_amdgcn_logf(l);
}

// ------------------------------------------------------------------------------------------
// Ping-pong inference forward (dense)
// ------------------------------------------------------------------------------------------
//
// 8 waves (256 queries) per workgroup, one workgroup per CU: waves w and w+4 share SIMD w%4 and
// belong to the two groups g = w/4 of 128 queries.  Each group alternates a vector phase V(it)
// (running max, P-hat of chunk it on the VALUs) and a matrix phase M(it) (S of chunk it+1 and
// O^T += V-hat(it)^T P-hat(it)^T on the matrix cores); group 1 runs one phase behind group 0, so
// on every SIMD one wave's exponentials and fake quantization run beside the other wave's MFMAs.
// One workgroup barrier separates the phases.
//
// LDS: two buffers of 64 KiB, buffer it%2 holding K-hat(it+1) as four 8 KiB sub-tiles of 32 rows
// (256 B rows, sw_kq swizzle) and V-hat^T(it) as four [128 d][32 keys] sub-tiles (64 B rows,
// 16-byte columns swizzled by sw_v64, so each sub-tile is contiguous).  Group 0 reads buffer it%2
// in phase 2it+1, group 1 in phase 2it+2; it is refilled for iteration it+2 at the start of phase
// 2it+3 and waited for at the end of phase 2it+4.  K-hat(0) for the prologue's S(0) goes to
// buffer 1's K half.
//
// Why two groups on one CU rather than one wave per SIMD doing both halves: a wave hides only
// about 4-5 independent VALU operations behind each 32-cycle 32x32x16 MFMA of its own, while a
// VALU stream from a second wave on the same SIMD runs beside the first wave's MFMA chain (at
// about three quarters of its own rate when the MFMA wave has the higher priority, which
// s_setprio gives the matrix phase).  Per 128-key chunk a wave issues 64 MFMAs and some 450 VALU
// instructions (69 of them exponentials), so the VALU half only hides under a second wave.
constexpr uint32_t kLdsK = 0, kLdsV = 32768;  // byte offsets of the K-hat and V-hat^T halves

// A ds_read_b128 serves 16 lanes per cycle from 64 banks (256 bytes): the 16 rows d..d+15 of a
// read must then cover the 16 distinct 16-byte slots of 256 bytes, 4 * (d & 3) + column, so rows
// that share d & 3 get different columns.
__device__ __forceinline__ int sw_v64(int d) { return (d >> 2) & 3; }
constexpr int kPPWaves = 8;
constexpr int kPPAhead = 8;  // LDS operand reads issued ahead of their MFMA in the matrix phase

template <bool QP, bool F16, bool GP>
__global__ __launch_bounds__(kPPWaves * 64, 1) void attn_fwd_pp_kernel(FwdParams p) {
  constexpr int BM = 32 * kPPWaves;
  __shared__ __attribute__((aligned(256))) uint8_t lds[2 * 65536];

  const int64_t vid = xcd_work_id(blockIdx.x, p.per_xcd, p.nblocks);
  if (vid < 0) return;
  const int64_t bh = vid / p.qtiles;
  const int qt = (int)(vid % p.qtiles);
  const int64_t bb = bh / p.heads, hh = bh % p.heads;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int lane = tid & 63;
  const int n = lane & 31;
  const int hf = lane >> 5;
  const int64_t qrow = (int64_t)qt * BM + wave * 32 + n;
  const bool qvalid = qrow < p.lq;

  const int lk = (int)p.lk;
  int n_iter = (int)p.nchunks;
  if (p.causal) {
    const int q_last = qt * BM + BM - 1;
    n_iter = (q_last < lk - 1 ? q_last : lk - 1) / kChunk + 1;
  }
  const uint32_t lds0 = lds_addr(lds);
  const uint8_t *kbase = (const uint8_t *)(p.kq + bh * p.kchunks * (kChunk * kD / 8));
  const uint8_t *vbase = (const uint8_t *)(p.vt + bh * p.kchunks * (kChunk * kD / 8));
  // Copies (one 1 KiB piece of every sub-tile per wave): K rows 32kt + 4w + lane/16, physical
  // column lane%16; V rows d = 16w + lane/4, physical column lane%4 (logical keys 32kt +
  // 8*(column ^ sw_v64(d))).
  uint32_t k_off, v_off;
  {
    const int r = 4 * wave + (lane >> 4), d = 16 * wave + (lane >> 2);
    k_off = (uint32_t)(r * 256 + (((lane & 15) ^ sw_kq(r)) << 4));
    v_off = (uint32_t)(d * 256 + (((lane & 3) ^ sw_v64(d)) << 4));
  }
  auto copy_k = [&](int c, uint32_t buf) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
      load_lds16_sa(kbase + (int64_t)c * 32768 + kt * 8192, k_off, buf + kLdsK + kt * 8192 + 1024 * wave);
  };
  auto copy_v = [&](int c, uint32_t buf) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
      load_lds16_sa(vbase + (int64_t)c * 32768 + kt * 64, v_off, buf + kLdsV + kt * 8192 + 1024 * wave);
  };
  // Iteration j's buffer: K-hat(j+1) and V-hat(j).
  auto fill = [&](int j) {
    const uint32_t buf = lds0 + (uint32_t)(j & 1) * 65536;
    if (j + 1 < n_iter) copy_k(j + 1, buf);
    if (j < n_iter) copy_v(j, buf);
  };
  // Piece q of fill(j) as a copy the operand reads of the matrix phase may pass: q < 4 the K-hat
  // sub-tile q of chunk j+1, else the V-hat sub-tile q-4 of chunk j, with both chunks clamped to
  // the last one (fill(n_iter) then rewrites buffer n_iter%2, which nothing reads any more).
  auto fill_piece = [&](int j, int q) {
    const uint32_t buf = lds0 + (uint32_t)(j & 1) * 65536;
    const int last = n_iter - 1;
    if (q < 4) {
      const int jk = j + 1 < last ? j + 1 : last;
      load_lds16_sa_free(kbase + (int64_t)jk * 32768 + q * 8192, k_off, buf + kLdsK + q * 8192 + 1024 * wave);
    } else {
      const int jv = j < last ? j : last;
      load_lds16_sa_free(vbase + (int64_t)jv * 32768 + (q - 4) * 64, v_off, buf + kLdsV + (q - 4) * 8192 + 1024 * wave);
    }
  };

  // Prologue: K-hat(0) into buffer 1's K half, iteration 0's buffer, Q-hat.
  copy_k(0, lds0 + 65536);
  fill(0);
  bf16x8 qf[8];
  load_q_frags(p, bb, hh, qrow, qvalid, hf, qf);

  uint32_t ka, va;
  {
    const int krow = perm_row(n), swk = sw_kq(krow);
    ka = lds0 + kLdsK + krow * 256 + 16 * (hf ^ swk);
    va = lds0 + kLdsV + n * 64 + 16 * ((2 * hf) ^ sw_v64(n));
  }
  f32x16 s[4];
  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};
  float m_run = (p.m_init && qvalid) ? p.m_init[bh * p.lq + qrow] : -__builtin_inff();
  float l_run = 0.0f, alpha = 1.0f;
  u32x4 pq[4][2];

  // The first chunk's logits: column pair t outermost (each chain's sum in the same order), the
  // operand reads eight MFMAs ahead of their use; left to the compiler, each MFMA waited for its
  // own read.
  auto first_logits = [&](uint32_t kbuf) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(lds_read16(kbuf + (ka ^ (32 * t)) + 8192 * kt)), qf[t],
                                                        t == 0 ? f32x16{} : s[kt], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int g = 0; g < 32; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (g < 24) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  AQ_WAIT_VMCNT(0);
  __builtin_amdgcn_s_barrier();
  first_logits(65536);
  // Buffer 1's K half is read by every wave before iteration 1's copies go there.
  __builtin_amdgcn_s_barrier();

  // V(it): mask, running max, P-hat of chunk it (all four sub-tiles) into pq.
  auto vphase = [&](int it) {
    const bool tail = (it + 1) * kChunk > lk;
    const bool diag = p.causal && (it + 1) * kChunk - 1 > qt * BM + wave * 32;
    if (tail || diag) {
      const int key0 = it * kChunk + 16 * hf, lk1 = lk - 1, q = (int)qrow;
      const int last = p.causal ? (q < lk1 ? q : lk1) : lk1;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) mask_tail(s[kt], valid_prefix(key0 + 32 * kt, last));
    }
    float bmax[4];
    max16x4(s, bmax);
    float cm = max3f(max3f(bmax[0], bmax[1], bmax[2]), bmax[3], bmax[3]);
    cm = pair_max(cm);
    const float m_new = max_nq(m_run, cm * p.c);
    alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // applied to acc by the next matrix phase
    m_run = m_new;
    const float g = (GP && p.two_level) ? two_level_scale(cm, p.c, m_new) : p.gp_static;
    float psum = 0.0f;
    u32x4 ph[2];
    if constexpr (QP) {
      // the four blocks' scales first: their dependent chains (two transcendentals each) overlap
      ProbBlock pb[4];
      if constexpr (GP) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) pb[kt] = prob_block_static(bmax[kt], p.c, m_new, g);
      } else {
        prob_blocks4(bmax, p.c, m_new, pb);
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) form_pq<F16, false, GP>(s[kt], pb[kt], p.c, psum, pq[kt], ph);
    } else {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) form_p<QP, F16, false, GP>(s[kt], bmax[kt], p.c, m_new, g, psum, pq[kt], ph);
    }
    l_run = l_run * alpha + psum;
    // Pinned here: otherwise the compiler sinks this phase's work past the barrier into the next.
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      AQ_OPAQUE(pq[kt][0]);
      AQ_OPAQUE(pq[kt][1]);
    }
    AQ_OPAQUE(l_run);
    AQ_OPAQUE(m_run);
    AQ_OPAQUE(alpha);
  };
  // M(it): S of chunk it+1 and O^T += V-hat(it)^T P-hat(it)^T, from buffer it%2.  The last
  // iteration also computes logits, from a stale K half, and drops them: a branch would split the
  // block whose operand reads are scheduled ahead of the MFMAs.
  auto mphase = [&](int it) {
    // the rescale of the running output for this chunk's maximum (skipped when no row moved)
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) acc[dt] *= alpha;
    }
    const uint32_t buf = (uint32_t)(it & 1) * 65536;
    // One address register per K-hat column pair and per V-hat half; the sub-tile and d-tile
    // offsets then ride in the reads' immediate offset field.
    uint32_t kad[8], vad[2];
#pragma unroll
    for (int t = 0; t < 8; ++t) kad[t] = buf + (ka ^ (32 * t));
#pragma unroll
    for (int j = 0; j < 2; ++j) vad[j] = buf + (va ^ (16 * j));
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(lds_read16(kad[0] + 8192 * kt)), qf[0], f32x16{}, 0, 0, 0);
#pragma unroll
      for (int t = 1; t < 8; ++t) {
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(lds_read16(kad[t] + 8192 * kt)), qf[t], s[kt], 0, 0, 0);
        // this wave's share of fill(it+1), spread over the first half of the phase: one copy per
        // few MFMAs keeps the address unit from backing up, so a copy holds the wave about as
        // long as the MFMA in flight
        if (kt >= 1 && kt <= 2 && (t & 1)) fill_piece(it + 1, 4 * (kt - 1) + (t >> 1));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const u32x4 a = lds_read16(vad[j] + 8192 * kt + 2048 * dt);
          if (F16)
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                             __builtin_bit_cast(f16x8, pq[kt][j]), acc[dt], 0, 0, 0);
          else
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(pq[kt][j]), acc[dt], 0, 0, 0);
        }
    }
    // Operand reads kPPAhead MFMAs ahead of their use across the whole phase, not all up front.
    __builtin_amdgcn_sched_group_barrier(0x100, kPPAhead, 0);
#pragma unroll
    for (int g = 0; g < 64; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (g < 64 - kPPAhead) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) AQ_OPAQUE(s[kt]);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) AQ_OPAQUE(acc[dt]);
  };

  // Phases ph = 0 .. 2n: group 0 runs V(0) M(0) V(1) M(1) ... and idles in the last phase, group
  // 1 idles in phase 0 and then runs the same sequence, so phase 2it+g is V(it) and 2it+1+g is
  // M(it) for group g.  Every wave issues its share of iteration j's copies in phase 2j-1 (buffer
  // j%2 is free: its last reader, group 1's M(j-2), ran in phase 2j-2) and waits for them at the
  // end of phase 2j, before group 0's M(j) in phase 2j+1.
  if (grp == 1) __builtin_amdgcn_s_barrier();
  for (int it = 0; it < n_iter; ++it) {
    // Iteration it+1's copies (buffer (it+1)%2, free from phase 2it+1): each group's share among
    // the MFMAs of its M(it) (phases 2it+1 and 2it+2).  A wave stays at a copy instruction until
    // the CU's address unit takes it (1 KiB each, about 64 bytes per clock for the CU): issued all
    // at once at the start of a vector phase, the four waves of a group spent about 500 cycles on
    // their 32.  Both shares are waited for at the end of phase 2it+2.
    __builtin_amdgcn_s_setprio(0);
    vphase(it);
    if (grp == 0) AQ_WAIT_VMCNT(0);  // end of phase 2it
    __builtin_amdgcn_s_barrier();
    // the matrix phase issues first: its MFMAs keep the matrix unit busy and the vector phase
    // beside it fills the remaining issue slots
    __builtin_amdgcn_s_setprio(2);
    mphase(it);
    if (grp == 1) AQ_WAIT_VMCNT(0);  // end of phase 2it+2
    __builtin_amdgcn_s_barrier();
  }
  if (grp == 0) __builtin_amdgcn_s_barrier();

  // ---- epilogue --------------------------------------------------------------------------
  const float l = pair_sum(l_run);
  const float inv_l = 1.0f / l;
  if (!qvalid) return;
  uint16_t *op = p.o + bb * p.so.b + hh * p.so.h + qrow * p.so.l;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d0 = 32 * dt + 8 * a + 4 * hf;
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      const bf16x4 w = {(__bf16)(acc[dt][4 * a + 0] * inv_l), (__bf16)(acc[dt][4 * a + 1] * inv_l),
                        (__bf16)(acc[dt][4 * a + 2] * inv_l), (__bf16)(acc[dt][4 * a + 3] * inv_l)};
      *(bf16x4 *)(op + d0) = w;
    }
}

// ------------------------------------------------------------------------------------------
// Ping-pong cube-sparse inference forward
// ------------------------------------------------------------------------------------------
//
// attn_fwd_pp_kernel over chunk lists: one workgroup per two query cubes, wave group g holding
// cube 2*qt + g (128 queries, 32 per wave) and walking that cube's list in order with the dense
// kernel's arithmetic, so each group's output is final (no state crosses groups).  The groups'
// matrix phases read different chunks, so the buffer of phase ph holds K-hat(it+1) and V-hat(it)
// of the group whose matrix phase ph is (group (ph-1)%2, iteration it), copied by every wave
// during phase ph-1.  A missing second cube (odd n) walks the first cube's list and stores
// nothing.
constexpr uint32_t kLdsVList = 2 * 65536;  // the two cubes' lists, int16

__global__ __launch_bounds__(kPPWaves * 64, 1) void attn_fwd_vsa_pp_kernel(FwdParams p) {
  __shared__ __attribute__((aligned(256))) uint8_t lds[kLdsVList + 2 * kMaxSel * 2];

  const int64_t vid = xcd_work_id(blockIdx.x, p.per_xcd, p.nblocks);
  if (vid < 0) return;
  const int64_t bh = vid / p.qtiles;
  const int qt = (int)(vid % p.qtiles);
  const int64_t bb = bh / p.heads, hh = bh % p.heads;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, qs = wave & 3;
  const int lane = tid & 63;
  const int n = lane & 31;
  const int hf = lane >> 5;
  const int64_t ncubes = p.kchunks;
  const int64_t qrow = (int64_t)(2 * qt + grp) * kChunk + qs * 32 + n;
  const bool qvalid = qrow < p.lq;

  const int nsel = (int)p.nchunks;
  int16_t *lists = (int16_t *)(lds + kLdsVList);
  for (int i = tid; i < 2 * nsel; i += kPPWaves * 64) {
    const int g = i / nsel, pos = i - g * nsel;
    const int64_t c = 2 * qt + g < ncubes ? 2 * qt + g : ncubes - 1;
    lists[i] = (int16_t)clamp_chunk(p.sel[(bh * ncubes + c) * nsel + pos], p.kchunks);
  }
  __syncthreads();
  auto chunk_of = [&](int g, int pos) -> int64_t { return __builtin_amdgcn_readfirstlane((int)lists[g * nsel + pos]); };

  const uint32_t lds0 = lds_addr(lds);
  const uint8_t *kbase = (const uint8_t *)(p.kq + bh * p.kchunks * (kChunk * kD / 8));
  const uint8_t *vbase = (const uint8_t *)(p.vt + bh * p.kchunks * (kChunk * kD / 8));
  // Copies as in attn_fwd_pp_kernel.
  uint32_t k_off, v_off;
  {
    const int r = 4 * wave + (lane >> 4), d = 16 * wave + (lane >> 2);
    k_off = (uint32_t)(r * 256 + (((lane & 15) ^ sw_kq(r)) << 4));
    v_off = (uint32_t)(d * 256 + (((lane & 3) ^ sw_v64(d)) << 4));
  }
  auto copy_k = [&](int64_t c, uint32_t buf) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
      load_lds16_sa(kbase + c * 32768 + kt * 8192, k_off, buf + kLdsK + kt * 8192 + 1024 * wave);
  };
  auto copy_v = [&](int64_t c, uint32_t buf) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
      load_lds16_sa(vbase + c * 32768 + kt * 64, v_off, buf + kLdsV + kt * 8192 + 1024 * wave);
  };
  // The buffer of phase ph >= 1: K-hat(it+1) and V-hat(it) of group g = (ph-1)%2's iteration
  // it = (ph-1-g)/2, positions clamped to the list (a buffer no later phase reads may then get
  // a copy of a listed chunk).  It is copied during phase ph-1 by the wave group whose matrix
  // phase that is: each of its waves copies its own 1 KiB slice of every sub-tile and that of its
  // partner wave in the other group (row and d offsets 16 rows / 64 d apart: the partner's K
  // column swizzle differs, its V swizzle does not), so the vector phase issues no copies.
  uint32_t k_off2;
  {
    const int r = (4 * wave + (lane >> 4)) ^ 16;
    k_off2 = (uint32_t)(r * 256 + (((lane & 15) ^ sw_kq(r)) << 4));
  }
  const uint32_t v_off2 = v_off ^ 16384u;
  auto buffer_chunks = [&](int ph, int64_t &ck, int64_t &cv) {
    const int g = (ph - 1) & 1, it = (ph - 1 - g) >> 1, last = nsel - 1;
    ck = chunk_of(g, it + 1 < last ? it + 1 : last);
    cv = chunk_of(g, it < last ? it : last);
  };
  // Piece pc (0..15) of buffer ph's copies: slice (wave, then partner) pc / 8, sub-tile pc % 8
  // (K-hat 0..3, V-hat 4..7).
  auto fill_piece = [&](int ph, int64_t ck, int64_t cv, int pc) {
    const uint32_t buf = lds0 + (uint32_t)(ph & 1) * 65536;
    const int q = pc & 7, w = pc < 8 ? wave : wave ^ 4;
    if (q < 4)
      load_lds16_sa_free(kbase + ck * 32768 + q * 8192, pc < 8 ? k_off : k_off2, buf + kLdsK + q * 8192 + 1024 * w);
    else
      load_lds16_sa_free(vbase + cv * 32768 + (q - 4) * 64, pc < 8 ? v_off : v_off2, buf + kLdsV + (q - 4) * 8192 + 1024 * w);
  };

  // Prologue: the groups' first K-hat chunks into buffer 0's halves, Q-hat, first logits.
  copy_k(chunk_of(0, 0), lds0);
  copy_k(chunk_of(1, 0), lds0 + 32768);
  bf16x8 qf[8];
  load_q_frags(p, bb, hh, qrow, qvalid, hf, qf);

  uint32_t ka, va;
  {
    const int krow = perm_row(n), swk = sw_kq(krow);
    ka = lds0 + kLdsK + krow * 256 + 16 * (hf ^ swk);
    va = lds0 + kLdsV + n * 64 + 16 * ((2 * hf) ^ sw_v64(n));
  }
  f32x16 s[4];
  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};
  float m_run = (p.m_init && qvalid) ? p.m_init[bh * p.lq + qrow] : -__builtin_inff();
  float l_run = 0.0f, alpha = 1.0f;
  u32x4 pq[4][2];

  // The first chunk's logits: column pair t outermost (each chain's sum in the same order), the
  // operand reads eight MFMAs ahead of their use; left to the compiler, each MFMA waited for its
  // own read.
  auto first_logits = [&](uint32_t kbuf) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(lds_read16(kbuf + (ka ^ (32 * t)) + 8192 * kt)), qf[t],
                                                        t == 0 ? f32x16{} : s[kt], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int g = 0; g < 32; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (g < 24) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  AQ_WAIT_VMCNT(0);
  __syncthreads();
  first_logits(grp ? 32768u : 0u);
  __builtin_amdgcn_s_barrier();  // buffer 0 is read; phase 0 fills buffer 1

  // V(it): running max, P-hat of position it (attn_fwd_pp_kernel's vector phase).
  auto vphase = [&]() {
    float bmax[4];
    max16x4(s, bmax);
    float cm = max3f(max3f(bmax[0], bmax[1], bmax[2]), bmax[3], bmax[3]);
    cm = pair_max(cm);
    const float m_new = max_nq(m_run, cm * p.c);
    alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // applied to acc by the next matrix phase
    m_run = m_new;
    float psum = 0.0f;
    u32x4 ph[2];
    ProbBlock pb[4];
    prob_blocks4(bmax, p.c, m_new, pb);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) form_pq<true, false, false>(s[kt], pb[kt], p.c, psum, pq[kt], ph);
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      AQ_OPAQUE(pq[kt][0]);
      AQ_OPAQUE(pq[kt][1]);
    }
    AQ_OPAQUE(l_run);
    AQ_OPAQUE(m_run);
    AQ_OPAQUE(alpha);
  };
  // M(it) in phase phm: S of position it+1 and O^T += V-hat(it)^T P-hat(it)^T, from buffer phm%2
  // (the last position's next logits come from a stale K half and are dropped).
  auto mphase = [&](int phm, int64_t ck, int64_t cv) {
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) acc[dt] *= alpha;
    }
    const uint32_t buf = (uint32_t)(phm & 1) * 65536;
    uint32_t kad[8], vad[2];
#pragma unroll
    for (int t = 0; t < 8; ++t) kad[t] = buf + (ka ^ (32 * t));
#pragma unroll
    for (int j = 0; j < 2; ++j) vad[j] = buf + (va ^ (16 * j));
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(lds_read16(kad[0] + 8192 * kt)), qf[0], f32x16{}, 0, 0, 0);
#pragma unroll
      for (int t = 1; t < 8; ++t) {
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(lds_read16(kad[t] + 8192 * kt)), qf[t], s[kt], 0, 0, 0);
        // the next buffer's copies, about one per two MFMAs over the first three quarters of
        // the phase
        if (t & 1) fill_piece(phm + 1, ck, cv, 4 * kt + (t >> 1));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const u32x4 a = lds_read16(vad[j] + 8192 * kt + 2048 * dt);
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                           __builtin_bit_cast(f16x8, pq[kt][j]), acc[dt], 0, 0, 0);
        }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, kPPAhead, 0);
#pragma unroll
    for (int g = 0; g < 64; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (g < 64 - kPPAhead) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) AQ_OPAQUE(s[kt]);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) AQ_OPAQUE(acc[dt]);
  };

  // Group g's iteration it: V(it) in phase 2it+g, M(it) in phase 2it+g+1.  Phase ph+1's buffer
  // is copied during phase ph by the group whose matrix phase ph is (in phase 0, by group 1, idle
  // then) and waited for at the end of phase ph.
  if (grp == 1) {
    int64_t ck, cv;
    buffer_chunks(1, ck, cv);
#pragma unroll
    for (int pc = 0; pc < 16; ++pc) fill_piece(1, ck, cv, pc);
    AQ_WAIT_VMCNT(0);
    __builtin_amdgcn_s_barrier();
  }
  for (int it = 0; it < nsel; ++it) {
    const int phv = 2 * it + grp;
    int64_t ck, cv;
    buffer_chunks(phv + 2, ck, cv);
    __builtin_amdgcn_s_setprio(0);
    vphase();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_s_setprio(2);
    mphase(phv + 1, ck, cv);
    AQ_WAIT_VMCNT(0);
    __builtin_amdgcn_s_barrier();
  }
  if (grp == 0) __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_s_setprio(0);

  // ---- epilogue ----------------------------------------------------------------------------
  const float l = pair_sum(l_run);
  const float inv_l = 1.0f / l;
  if (!qvalid) return;
  uint16_t *op = p.o + bb * p.so.b + hh * p.so.h + qrow * p.so.l;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d0 = 32 * dt + 8 * a + 4 * hf;
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      const bf16x4 w = {(__bf16)(acc[dt][4 * a + 0] * inv_l), (__bf16)(acc[dt][4 * a + 1] * inv_l),
                        (__bf16)(acc[dt][4 * a + 2] * inv_l), (__bf16)(acc[dt][4 * a + 3] * inv_l)};
      *(bf16x4 *)(op + d0) = w;
    }
}

// ------------------------------------------------------------------------------------------
// Ping-pong training forward (dense; unit scales with every quantizer on, smooth-K allowed)
// ------------------------------------------------------------------------------------------
//
// The inference ping-pong schedule with the training outputs: the second accumulator for O^hp
// and its unquantized P operands (fp16), the chunk maxima and lse.  The two accumulators leave
// no room for the Q-hat operand in registers, and the two chunk buffers no room for Q-hat as
// bf16 in LDS, so each wave keeps its Q-hat in LDS as E2M1 codes and fp16 block scales (3 KiB)
// and decodes each column pair to fp16 before the logit MFMAs that use it; the K-hat rows are
// staged as fp16.  Under the unit scale every Q-hat and K-hat value is exact in fp16 and so is
// every product, so the logits are those of the bf16 kernels bit for bit.  The matrix phase runs
// chunk it's P-hat V-hat and P V-hat products first and chunk it+1's logits after them, so the P
// operands are dead before the logits are born.  With 96 MFMAs per chunk the matrix phase is the
// longer one, so the rescale of the running outputs moves to the vector phase.

// The lane's Q-hat (zero past lq) as codes: for column pair t (d = 16t + 8hf .. +7), code[t]
// holds the 8 E2M1 codes (byte i: elements 2i, 2i+1), scale[t] the block's E4M3 scale.  The codes
// are the codec's decisions: E2M1 of the exact quotient x / S, ties to even, sign kept.
__device__ __forceinline__ void load_q_codes(const FwdParams &p, int64_t bb, int64_t hh, int64_t qrow, bool qvalid,
                                             int hf, uint32_t (&code)[8], float (&scale)[8]) {
  const uint16_t *qp = p.q + bb * p.sq.b + hh * p.sq.h + (qvalid ? qrow : 0) * p.sq.l;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (qvalid) v = *(const u32x4 *)(qp + 16 * t + 8 * hf);
    float f[8] = {bf16lo(v.x), bf16hi(v.x), bf16lo(v.y), bf16hi(v.y), bf16lo(v.z), bf16hi(v.z), bf16lo(v.w), bf16hi(v.w)};
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = fmaxf(am, __builtin_fabsf(f[i]));
    am = pair_max(am);
    const float S = block_scale_unit(am);
    const float inv = S == 0.0f ? 0.0f : recip_e4m3(S);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = div_e4m3(f[i], S, inv);
    code[t] = e2m1_codes8(f);
    scale[t] = S;
  }
}

// LDS of the training kernel past the two chunk buffers: per wave, its lanes' Q-hat codes
// [t][lane] (4 bytes) and block scales [t][lane] (fp16), read back once per column pair and chunk.
constexpr uint32_t kLdsQc = 2 * 65536, kQcWave = 8 * 64 * 4 + 8 * 64 * 2;

__global__ __launch_bounds__(kPPWaves * 64, 1) void attn_fwd_pp_train_kernel(FwdParams p) {
  constexpr int BM = 32 * kPPWaves;
  __shared__ __attribute__((aligned(256))) uint8_t lds[kLdsQc + kPPWaves * kQcWave];

  const int64_t vid = xcd_work_id(blockIdx.x, p.per_xcd, p.nblocks);
  if (vid < 0) return;
  const int64_t bh = vid / p.qtiles;
  const int qt = (int)(vid % p.qtiles);
  const int64_t bb = bh / p.heads, hh = bh % p.heads;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int lane = tid & 63;
  const int n = lane & 31;
  const int hf = lane >> 5;
  const int64_t qrow = (int64_t)qt * BM + wave * 32 + n;
  const bool qvalid = qrow < p.lq;

  const int lk = (int)p.lk;
  int n_iter = (int)p.nchunks;
  if (p.causal) {
    const int q_last = qt * BM + BM - 1;
    n_iter = (q_last < lk - 1 ? q_last : lk - 1) / kChunk + 1;
  }
  const uint32_t lds0 = lds_addr(lds);
  const uint8_t *kbase = (const uint8_t *)(p.kq + bh * p.kchunks * (kChunk * kD / 8));
  const uint8_t *vbase = (const uint8_t *)(p.vt + bh * p.kchunks * (kChunk * kD / 8));
  // Copies, buffers and phases exactly as in attn_fwd_pp_kernel.
  uint32_t k_off, v_off;
  {
    const int r = 4 * wave + (lane >> 4), d = 16 * wave + (lane >> 2);
    k_off = (uint32_t)(r * 256 + (((lane & 15) ^ sw_kq(r)) << 4));
    v_off = (uint32_t)(d * 256 + (((lane & 3) ^ sw_v64(d)) << 4));
  }
  auto copy_k = [&](int c, uint32_t buf) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
      load_lds16_sa(kbase + (int64_t)c * 32768 + kt * 8192, k_off, buf + kLdsK + kt * 8192 + 1024 * wave);
  };
  auto copy_v = [&](int c, uint32_t buf) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
      load_lds16_sa(vbase + (int64_t)c * 32768 + kt * 64, v_off, buf + kLdsV + kt * 8192 + 1024 * wave);
  };
  auto fill = [&](int j) {
    const uint32_t buf = lds0 + (uint32_t)(j & 1) * 65536;
    if (j + 1 < n_iter) copy_k(j + 1, buf);
    if (j < n_iter) copy_v(j, buf);
  };
  // Piece q of fill(j) as a copy the operand reads of the matrix phase may pass (as in
  // attn_fwd_pp_kernel): q < 4 the K-hat sub-tile q of chunk j+1, else the V-hat sub-tile q-4 of
  // chunk j, both chunks clamped to the last one.
  auto fill_piece = [&](int j, int q) {
    const uint32_t buf = lds0 + (uint32_t)(j & 1) * 65536;
    const int last = n_iter - 1;
    if (q < 4) {
      const int jk = j + 1 < last ? j + 1 : last;
      load_lds16_sa_free(kbase + (int64_t)jk * 32768 + q * 8192, k_off, buf + kLdsK + q * 8192 + 1024 * wave);
    } else {
      const int jv = j < last ? j : last;
      load_lds16_sa_free(vbase + (int64_t)jv * 32768 + (q - 4) * 64, v_off, buf + kLdsV + (q - 4) * 8192 + 1024 * wave);
    }
  };

  copy_k(0, lds0 + 65536);
  fill(0);
  // The lane's Q-hat codes and scales into the wave's LDS region (registers are short here).
  const uint32_t qca = lds0 + kLdsQc + (uint32_t)wave * kQcWave + 4 * lane;
  const uint32_t qsa = lds0 + kLdsQc + (uint32_t)wave * kQcWave + 8 * 64 * 4 + 2 * lane;
  {
    uint32_t qc[8];
    float qs[8];
    load_q_codes(p, bb, hh, qrow, qvalid, hf, qc, qs);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      *(__attribute__((address_space(3))) uint32_t *)(uintptr_t)(qca + 256 * t) = qc[t];
      *(__attribute__((address_space(3))) _Float16 *)(uintptr_t)(qsa + 128 * t) = (_Float16)qs[t];
    }
  }

  uint32_t ka, va;
  {
    const int krow = perm_row(n), swk = sw_kq(krow);
    ka = lds0 + kLdsK + krow * 256 + 16 * (hf ^ swk);
    va = lds0 + kLdsV + n * 64 + 16 * ((2 * hf) ^ sw_v64(n));
  }
  // S^T of a chunk from buffer offset kbuf: column pair t outermost, so each Q-hat pair is decoded
  // once and feeds the four sub-tiles' chains.  Software-pipelined by hand, a scheduling barrier
  // closing each pair's step: step t issues pair t+1's K-hat and code/scale reads, then pair t's
  // four MFMAs (their operands read in step t-1), then pair t+1's decode; so each read has a
  // step of MFMAs to land in, and only two Q-hat pairs are live at a time.
  auto logits = [&](uint32_t kbuf, f32x16 (&st)[4]) {
    uint32_t kb = kbuf + ka;
    AQ_OPAQUE(kb);  // per-pair addresses formed here, not held across the loop
    auto kread = [&](int t, int kt) -> u32x4 { return lds_read16((kb ^ (32 * t)) + 8192 * kt); };
    auto qdec = [&](uint32_t code, _Float16 h) -> f16x8 {
      const f16x2 x0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(code, 1.0f, 0) * h;
      const f16x2 x1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(code, 1.0f, 1) * h;
      const f16x2 x2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(code, 1.0f, 2) * h;
      const f16x2 x3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(code, 1.0f, 3) * h;
      return f16x8{x0[0], x0[1], x1[0], x1[1], x2[0], x2[1], x3[0], x3[1]};
    };
    auto code_of = [&](int t) -> uint32_t {
      return *(const __attribute__((address_space(3))) uint32_t *)(uintptr_t)(qca + 256 * t);
    };
    auto scale_of = [&](int t) -> _Float16 {
      return *(const __attribute__((address_space(3))) _Float16 *)(uintptr_t)(qsa + 128 * t);
    };
    u32x4 kc[4], kn[4];
    f16x8 b = qdec(code_of(0), scale_of(0)), bn = b;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) kc[kt] = kread(0, kt);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      uint32_t cn = 0u;
      _Float16 hn = (_Float16)0.0f;
      if (t < 7) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) kn[kt] = kread(t + 1, kt);
        cn = code_of(t + 1);
        hn = scale_of(t + 1);
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, kc[kt]), b, t ? st[kt] : f32x16{}, 0, 0,
                                                        0);
      if (t < 7) bn = qdec(cn, hn);
      __builtin_amdgcn_sched_barrier(0);
      if (t < 7) {
        b = bn;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) kc[kt] = kn[kt];
      }
    }
  };

  f32x16 s[4], acc[4], acc_hp[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    acc[dt] = f32x16{};
    acc_hp[dt] = f32x16{};
  }
  float m_run = (p.m_init && qvalid) ? p.m_init[bh * p.lq + qrow] : -__builtin_inff();
  float l_run = 0.0f, alpha = 1.0f;
  u32x4 pq[4][2], ph[4][2];

  AQ_WAIT_VMCNT(0);
  __builtin_amdgcn_s_barrier();
  logits(65536u, s);
  __builtin_amdgcn_s_barrier();

  // V(it): mask, running max (stored as chunk it's maximum), P-hat and P of chunk it.
  auto vphase = [&](int it) {
    const bool tail = (it + 1) * kChunk > lk;
    const bool diag = p.causal && (it + 1) * kChunk - 1 > qt * BM + wave * 32;
    if (tail || diag) {
      const int key0 = it * kChunk + 16 * hf, lk1 = lk - 1, q = (int)qrow;
      const int last = p.causal ? (q < lk1 ? q : lk1) : lk1;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) mask_tail(s[kt], valid_prefix(key0 + 32 * kt, last));
    }
    float bmax[4];
    max16x4(s, bmax);
    float cm = max3f(max3f(bmax[0], bmax[1], bmax[2]), bmax[3], bmax[3]);
    cm = pair_max(cm);
    const float m_new = max_nq(m_run, cm * p.c);
    alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    if (hf == 0 && qvalid) p.cmax[(bh * p.nchunks + it) * p.lq + qrow] = m_new;
    float psum = 0.0f;
    ProbBlock pb[4];
    prob_blocks4(bmax, p.c, m_new, pb);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) form_pq<true, true, false>(s[kt], pb[kt], p.c, psum, pq[kt], ph[kt]);
    l_run = l_run * alpha + psum;
    // the running outputs' rescale (skipped when no row moved) here rather than in the matrix
    // phase, which is the longer one in this kernel
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        acc[dt] *= alpha;
        acc_hp[dt] *= alpha;
      }
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      AQ_OPAQUE(pq[kt][0]);
      AQ_OPAQUE(pq[kt][1]);
      AQ_OPAQUE(ph[kt][0]);
      AQ_OPAQUE(ph[kt][1]);
    }
    AQ_OPAQUE(l_run);
    AQ_OPAQUE(m_run);
    AQ_OPAQUE(alpha);
  };
  // M(it): O^T += V-hat(it)^T P-hat(it)^T and O^hp^T += V-hat(it)^T P(it)^T, then S of chunk it+1,
  // from buffer it%2 (the last iteration's logits come from a stale K half and are dropped).
  auto mphase = [&](int it) {
    const uint32_t buf = (uint32_t)(it & 1) * 65536;
    uint32_t vad[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) vad[j] = buf + (va ^ (16 * j));
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const f16x8 a = __builtin_bit_cast(f16x8, lds_read16(vad[j] + 8192 * kt + 2048 * dt));
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, __builtin_bit_cast(f16x8, pq[kt][j]), acc[dt], 0, 0, 0);
          acc_hp[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, __builtin_bit_cast(f16x8, ph[kt][j]), acc_hp[dt], 0, 0, 0);
          // this wave's share of fill(it+1) (buffer (it+1)%2, which no read of this phase
          // touches), one copy per eight MFMAs
          if (dt == 1) fill_piece(it + 1, 2 * kt + j);
        }
    // each V-hat read 4 reads ahead of its two MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int g = 0; g < 32; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      if (g < 28) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    // the P operands die here, before the logits' accumulators are born
    __builtin_amdgcn_sched_barrier(0);
    logits(buf, s);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) AQ_OPAQUE(s[kt]);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      AQ_OPAQUE(acc[dt]);
      AQ_OPAQUE(acc_hp[dt]);
    }
  };

  // The phases and copies of the inference kernel: iteration it+1's copies issued by each group
  // among the MFMAs of its M(it) (phases 2it+1 and 2it+2), both shares waited for at the end of
  // phase 2it+2.
  if (grp == 1) __builtin_amdgcn_s_barrier();
  for (int it = 0; it < n_iter; ++it) {
    __builtin_amdgcn_s_setprio(0);
    vphase(it);
    if (grp == 0) AQ_WAIT_VMCNT(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_s_setprio(2);
    mphase(it);
    if (grp == 1) AQ_WAIT_VMCNT(0);
    __builtin_amdgcn_s_barrier();
  }
  if (grp == 0) __builtin_amdgcn_s_barrier();

  // ---- epilogue: O, O^hp, lse --------------------------------------------------------------
  const float l = pair_sum(l_run);
  const float inv_l = 1.0f / l;
  if (!qvalid) return;
  uint16_t *op = p.o + bb * p.so.b + hh * p.so.h + qrow * p.so.l;
  float *hp = p.o_hp + (bh * p.lq + qrow) * kD;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d0 = 32 * dt + 8 * a + 4 * hf;
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      const bf16x4 w = {(__bf16)(acc[dt][4 * a + 0] * inv_l), (__bf16)(acc[dt][4 * a + 1] * inv_l),
                        (__bf16)(acc[dt][4 * a + 2] * inv_l), (__bf16)(acc[dt][4 * a + 3] * inv_l)};
      *(bf16x4 *)(op + d0) = w;
      *(f32x4 *)(hp + d0) = f32x4{acc_hp[dt][4 * a] * inv_l, acc_hp[dt][4 * a + 1] * inv_l,
                                  acc_hp[dt][4 * a + 2] * inv_l, acc_hp[dt][4 * a + 3] * inv_l};
    }
  if (hf == 0) p.lse[bh * p.lq + qrow] = m_run + __builtin_amdgcn_logf(l);
}

// ------------------------------------------------------------------------------------------
// Ping-pong cube-sparse training forward
// ------------------------------------------------------------------------------------------
//
// attn_fwd_pp_train_kernel over chunk lists: one workgroup per two query cubes, wave group g
// holding cube 2*qt + g (128 queries, 32 per wave) and walking that cube's list in order, so each
// group's running maximum, outputs and statistics are its own and final.  The groups' matrix
// phases read different chunks, so (as in attn_fwd_vsa_pp_kernel) the buffer of phase ph holds
// K-hat(it+1) and V-hat(it) of the group whose matrix phase ph is (group (ph-1)%2, iteration it),
// copied by every wave during phase ph-1.  A missing second cube (odd n) walks the first cube's
// list and stores nothing.
constexpr uint32_t kLdsVtList = kLdsQc + kPPWaves * kQcWave;  // the two cubes' lists, int16

__global__ __launch_bounds__(kPPWaves * 64, 1) void attn_fwd_vsa_pp_train_kernel(FwdParams p) {
  __shared__ __attribute__((aligned(256))) uint8_t lds[kLdsVtList + 2 * kMaxSel * 2];

  const int64_t vid = xcd_work_id(blockIdx.x, p.per_xcd, p.nblocks);
  if (vid < 0) return;
  const int64_t bh = vid / p.qtiles;
  const int qt = (int)(vid % p.qtiles);
  const int64_t bb = bh / p.heads, hh = bh % p.heads;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, qs = wave & 3;
  const int lane = tid & 63;
  const int n = lane & 31;
  const int hf = lane >> 5;
  const int64_t ncubes = p.kchunks;
  const int64_t qrow = (int64_t)(2 * qt + grp) * kChunk + qs * 32 + n;
  const bool qvalid = qrow < p.lq;

  const int nsel = (int)p.nchunks;
  int16_t *lists = (int16_t *)(lds + kLdsVtList);
  for (int i = tid; i < 2 * nsel; i += kPPWaves * 64) {
    const int g = i / nsel, pos = i - g * nsel;
    const int64_t c = 2 * qt + g < ncubes ? 2 * qt + g : ncubes - 1;
    lists[i] = (int16_t)clamp_chunk(p.sel[(bh * ncubes + c) * nsel + pos], p.kchunks);
  }
  __syncthreads();
  auto chunk_of = [&](int g, int pos) -> int64_t { return __builtin_amdgcn_readfirstlane((int)lists[g * nsel + pos]); };

  const uint32_t lds0 = lds_addr(lds);
  const uint8_t *kbase = (const uint8_t *)(p.kq + bh * p.kchunks * (kChunk * kD / 8));
  const uint8_t *vbase = (const uint8_t *)(p.vt + bh * p.kchunks * (kChunk * kD / 8));
  // Copies as in attn_fwd_pp_kernel.
  uint32_t k_off, v_off;
  {
    const int r = 4 * wave + (lane >> 4), d = 16 * wave + (lane >> 2);
    k_off = (uint32_t)(r * 256 + (((lane & 15) ^ sw_kq(r)) << 4));
    v_off = (uint32_t)(d * 256 + (((lane & 3) ^ sw_v64(d)) << 4));
  }
  auto copy_k = [&](int64_t c, uint32_t buf) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
      load_lds16_sa(kbase + c * 32768 + kt * 8192, k_off, buf + kLdsK + kt * 8192 + 1024 * wave);
  };
  auto copy_v = [&](int64_t c, uint32_t buf) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
      load_lds16_sa(vbase + c * 32768 + kt * 64, v_off, buf + kLdsV + kt * 8192 + 1024 * wave);
  };
  // The buffer of phase ph >= 1 (K-hat(it+1) and V-hat(it) of group (ph-1)%2's iteration it,
  // positions clamped), copied during phase ph-1 by the group whose matrix phase that is, each
  // wave its own slice and its partner's, as in the inference kernel.
  uint32_t k_off2;
  {
    const int r = (4 * wave + (lane >> 4)) ^ 16;
    k_off2 = (uint32_t)(r * 256 + (((lane & 15) ^ sw_kq(r)) << 4));
  }
  const uint32_t v_off2 = v_off ^ 16384u;
  auto buffer_chunks = [&](int ph, int64_t &ck, int64_t &cv) {
    const int g = (ph - 1) & 1, it = (ph - 1 - g) >> 1, last = nsel - 1;
    ck = chunk_of(g, it + 1 < last ? it + 1 : last);
    cv = chunk_of(g, it < last ? it : last);
  };
  auto fill_piece = [&](int ph, int64_t ck, int64_t cv, int pc) {
    const uint32_t buf = lds0 + (uint32_t)(ph & 1) * 65536;
    const int q = pc & 7, w = pc < 8 ? wave : wave ^ 4;
    if (q < 4)
      load_lds16_sa_free(kbase + ck * 32768 + q * 8192, pc < 8 ? k_off : k_off2, buf + kLdsK + q * 8192 + 1024 * w);
    else
      load_lds16_sa_free(vbase + cv * 32768 + (q - 4) * 64, pc < 8 ? v_off : v_off2, buf + kLdsV + (q - 4) * 8192 + 1024 * w);
  };

  // Prologue: the groups' first K-hat chunks into buffer 0's halves, Q-hat codes, first logits.
  copy_k(chunk_of(0, 0), lds0);
  copy_k(chunk_of(1, 0), lds0 + 32768);
  const uint32_t qca = lds0 + kLdsQc + (uint32_t)wave * kQcWave + 4 * lane;
  const uint32_t qsa = lds0 + kLdsQc + (uint32_t)wave * kQcWave + 8 * 64 * 4 + 2 * lane;
  {
    uint32_t qc[8];
    float qsc[8];
    load_q_codes(p, bb, hh, qrow, qvalid, hf, qc, qsc);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      *(__attribute__((address_space(3))) uint32_t *)(uintptr_t)(qca + 256 * t) = qc[t];
      *(__attribute__((address_space(3))) _Float16 *)(uintptr_t)(qsa + 128 * t) = (_Float16)qsc[t];
    }
  }
  uint32_t ka, va;
  {
    const int krow = perm_row(n), swk = sw_kq(krow);
    ka = lds0 + kLdsK + krow * 256 + 16 * (hf ^ swk);
    va = lds0 + kLdsV + n * 64 + 16 * ((2 * hf) ^ sw_v64(n));
  }
  // S^T of a chunk from buffer offset kbuf (attn_fwd_pp_train_kernel's arrangement).
  // S^T of a chunk from buffer offset kbuf: column pair t outermost, so each Q-hat pair is decoded
  // once and feeds the four sub-tiles' chains.  Software-pipelined by hand, a scheduling barrier
  // closing each pair's step: step t issues pair t+1's K-hat and code/scale reads, then pair t's
  // four MFMAs (their operands read in step t-1), then pair t+1's decode; so each read has a
  // step of MFMAs to land in, and only two Q-hat pairs are live at a time.
  auto logits = [&](uint32_t kbuf, f32x16 (&st)[4]) {
    uint32_t kb = kbuf + ka;
    AQ_OPAQUE(kb);  // per-pair addresses formed here, not held across the loop
    auto kread = [&](int t, int kt) -> u32x4 { return lds_read16((kb ^ (32 * t)) + 8192 * kt); };
    auto qdec = [&](uint32_t code, _Float16 h) -> f16x8 {
      const f16x2 x0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(code, 1.0f, 0) * h;
      const f16x2 x1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(code, 1.0f, 1) * h;
      const f16x2 x2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(code, 1.0f, 2) * h;
      const f16x2 x3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(code, 1.0f, 3) * h;
      return f16x8{x0[0], x0[1], x1[0], x1[1], x2[0], x2[1], x3[0], x3[1]};
    };
    auto code_of = [&](int t) -> uint32_t {
      return *(const __attribute__((address_space(3))) uint32_t *)(uintptr_t)(qca + 256 * t);
    };
    auto scale_of = [&](int t) -> _Float16 {
      return *(const __attribute__((address_space(3))) _Float16 *)(uintptr_t)(qsa + 128 * t);
    };
    u32x4 kc[4], kn[4];
    f16x8 b = qdec(code_of(0), scale_of(0)), bn = b;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) kc[kt] = kread(0, kt);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      uint32_t cn = 0u;
      _Float16 hn = (_Float16)0.0f;
      if (t < 7) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) kn[kt] = kread(t + 1, kt);
        cn = code_of(t + 1);
        hn = scale_of(t + 1);
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, kc[kt]), b, t ? st[kt] : f32x16{}, 0, 0,
                                                        0);
      if (t < 7) bn = qdec(cn, hn);
      __builtin_amdgcn_sched_barrier(0);
      if (t < 7) {
        b = bn;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) kc[kt] = kn[kt];
      }
    }
  };

  f32x16 s[4], acc[4], acc_hp[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    acc[dt] = f32x16{};
    acc_hp[dt] = f32x16{};
  }
  float m_run = -__builtin_inff();
  float l_run = 0.0f, alpha = 1.0f;
  u32x4 pq[4][2], ph[4][2];

  AQ_WAIT_VMCNT(0);
  __syncthreads();
  logits(grp ? 32768u : 0u, s);
  __builtin_amdgcn_s_barrier();  // buffer 0 is read; phase 0 fills buffer 1

  // V(it): running max (stored as position it's maximum), P-hat and P of position it.
  auto vphase = [&](int it) {
    float bmax[4];
    max16x4(s, bmax);
    float cm = max3f(max3f(bmax[0], bmax[1], bmax[2]), bmax[3], bmax[3]);
    cm = pair_max(cm);
    const float m_new = max_nq(m_run, cm * p.c);
    alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    if (hf == 0 && qvalid) p.cmax[(bh * p.nchunks + it) * p.lq + qrow] = m_new;
    float psum = 0.0f;
    ProbBlock pb[4];
    prob_blocks4(bmax, p.c, m_new, pb);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) form_pq<true, true, false>(s[kt], pb[kt], p.c, psum, pq[kt], ph[kt]);
    l_run = l_run * alpha + psum;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        acc[dt] *= alpha;
        acc_hp[dt] *= alpha;
      }
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      AQ_OPAQUE(pq[kt][0]);
      AQ_OPAQUE(pq[kt][1]);
      AQ_OPAQUE(ph[kt][0]);
      AQ_OPAQUE(ph[kt][1]);
    }
    AQ_OPAQUE(l_run);
    AQ_OPAQUE(m_run);
    AQ_OPAQUE(alpha);
  };
  // M(it) in phase phm: O^T += V-hat(it)^T P-hat(it)^T and O^hp^T += V-hat(it)^T P(it)^T, then S
  // of position it+1, from buffer phm%2 (the last position's next logits come from a stale K half
  // and are dropped).
  auto mphase = [&](int phm, int64_t ck, int64_t cv) {
    const uint32_t buf = (uint32_t)(phm & 1) * 65536;
    uint32_t vad[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) vad[j] = buf + (va ^ (16 * j));
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const f16x8 a = __builtin_bit_cast(f16x8, lds_read16(vad[j] + 8192 * kt + 2048 * dt));
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, __builtin_bit_cast(f16x8, pq[kt][j]), acc[dt], 0, 0, 0);
          acc_hp[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, __builtin_bit_cast(f16x8, ph[kt][j]), acc_hp[dt], 0, 0, 0);
          // the next buffer's copies, one per four MFMAs of the P.V products
          if (dt & 1) fill_piece(phm + 1, ck, cv, 4 * kt + 2 * j + (dt >> 1));
        }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int g = 0; g < 32; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      if (g < 28) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    logits(buf, s);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) AQ_OPAQUE(s[kt]);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      AQ_OPAQUE(acc[dt]);
      AQ_OPAQUE(acc_hp[dt]);
    }
  };

  // Group g's iteration it: V(it) in phase 2it+g, M(it) in phase 2it+g+1.  Phase ph+1's buffer
  // is copied during phase ph by the group whose matrix phase ph is (in phase 0, by group 1) and
  // waited for at the end of phase ph.
  if (grp == 1) {
    int64_t ck, cv;
    buffer_chunks(1, ck, cv);
#pragma unroll
    for (int pc = 0; pc < 16; ++pc) fill_piece(1, ck, cv, pc);
    AQ_WAIT_VMCNT(0);
    __builtin_amdgcn_s_barrier();
  }
  for (int it = 0; it < nsel; ++it) {
    const int phv = 2 * it + grp;
    int64_t ck, cv;
    buffer_chunks(phv + 2, ck, cv);
    __builtin_amdgcn_s_setprio(0);
    vphase(it);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_s_setprio(2);
    mphase(phv + 1, ck, cv);
    AQ_WAIT_VMCNT(0);
    __builtin_amdgcn_s_barrier();
  }
  if (grp == 0) __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_s_setprio(0);

  // ---- epilogue: O, O^hp, lse --------------------------------------------------------------
  const float l = pair_sum(l_run);
  const float inv_l = 1.0f / l;
  if (!qvalid) return;
  uint16_t *op = p.o + bb * p.so.b + hh * p.so.h + qrow * p.so.l;
  float *hp = p.o_hp + (bh * p.lq + qrow) * kD;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d0 = 32 * dt + 8 * a + 4 * hf;
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      const bf16x4 w = {(__bf16)(acc[dt][4 * a + 0] * inv_l), (__bf16)(acc[dt][4 * a + 1] * inv_l),
                        (__bf16)(acc[dt][4 * a + 2] * inv_l), (__bf16)(acc[dt][4 * a + 3] * inv_l)};
      *(bf16x4 *)(op + d0) = w;
      *(f32x4 *)(hp + d0) = f32x4{acc_hp[dt][4 * a] * inv_l, acc_hp[dt][4 * a + 1] * inv_l,
                                  acc_hp[dt][4 * a + 2] * inv_l, acc_hp[dt][4 * a + 3] * inv_l};
    }
  if (hf == 0) p.lse[bh * p.lq + qrow] = m_run + __builtin_amdgcn_logf(l);
}

// ------------------------------------------------------------------------------------------
// Row-max pass of the final-max variant
// ------------------------------------------------------------------------------------------
//
// m_out[bh, q] = c * (the largest logit of row q over its keys: all of them, the causal prefix, or
// the selected cubes), the statistics the reference-order reading relates every P to.  The logits
// are formed with the forward kernels' MFMA arrangement (same operands, same accumulation order),
// so the forward's chunk maxima are bitwise at most this value and its running max, seeded with
// it, never moves.  4 waves of 32 queries per workgroup; K-hat chunks staged through LDS.
__global__ __launch_bounds__(256, 2) void rowmax_kernel(FwdParams p) {
  constexpr int WAVES = 4;
  constexpr int BM = 32 * WAVES;
  __shared__ __attribute__((aligned(256))) uint8_t lds_k[kChunk * 256];
  __shared__ int32_t lds_sel[kMaxSel];

  const int64_t vid = xcd_work_id(blockIdx.x, p.per_xcd, p.nblocks);
  if (vid < 0) return;
  const int64_t bh = vid / p.qtiles;
  const int qt = (int)(vid % p.qtiles);
  const int64_t bb = bh / p.heads, hh = bh % p.heads;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, n = lane & 31, hf = lane >> 5;
  const int64_t qrow = (int64_t)qt * BM + wave * 32 + n;
  const bool qvalid = qrow < p.lq;

  int64_t n_iter = p.nchunks;
  if (p.causal) {
    const int64_t q_last = (int64_t)qt * BM + BM - 1;
    n_iter = (q_last < p.lk - 1 ? q_last : p.lk - 1) / kChunk + 1;
  }
  if (p.sel) {
    const int32_t *src = p.sel + (bh * (p.lq / kChunk) + (int64_t)qt * BM / kChunk) * p.nchunks;
    for (int i = tid; i < p.nchunks; i += WAVES * 64) lds_sel[i] = src[i];
    __syncthreads();
  }
  auto chunk_of = [&](int64_t it) -> int64_t {
    return p.sel ? clamp_chunk(__builtin_amdgcn_readfirstlane(lds_sel[it]), p.kchunks) : it;
  };
  auto ktile = [&](int64_t c) { return (const uint8_t *)(p.kq + (bh * p.kchunks + c) * (kChunk * kD / 8)); };
  const StageOffsets so = stage_offsets<WAVES>(wave, lane);
  int64_t chunk = chunk_of(0);
  stage_k<WAVES>(ktile(chunk), lds_k, so, wave);

  bf16x8 qf[8];
  load_q_frags(p, bb, hh, qrow, qvalid, hf, qf);
  uint32_t ka;
  {
    const int krow = perm_row(n), swk = sw_kq(krow);
    ka = lds_addr(lds_k) + krow * 256 + 16 * (hf ^ swk);
  }
  float mx = -__builtin_inff();
  for (int64_t it = 0; it < n_iter; ++it) {
    // (smooth-Q: the chains start from delta, loaded after the K copies the wait is for)
    f32x16 s[4];
    if (p.delta) {
      const float *dl = p.delta + (bh * p.kchunks + chunk) * kChunk + 16 * hf;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) s[kt] = delta16(dl + 32 * kt);
      AQ_WAIT_VMCNT(16);
    } else {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) s[kt] = f32x16{};
      AQ_WAIT_VMCNT(0);
    }
    __builtin_amdgcn_s_barrier();
    AQ_OPAQUE(ka);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int t0 = 0; t0 < 8; t0 += 4) {
        bf16x8 a[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) a[t] = as_bf16x8(lds_read16((ka ^ (32 * (t0 + t))) + 8192 * kt));
#pragma unroll
        for (int t = 0; t < 4; ++t) s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[t], qf[t0 + t], s[kt], 0, 0, 0);
      }
    }
    const int64_t next = it + 1 < n_iter ? chunk_of(it + 1) : -1;
    __builtin_amdgcn_s_barrier();  // every wave is done reading K-hat(chunk)
    if (next >= 0) stage_k<WAVES>(ktile(next), lds_k, so, wave);
    const int64_t key0 = chunk * kChunk + 16 * hf;
    const bool tail = (chunk + 1) * kChunk > p.lk;
    const bool diag = p.causal && (chunk + 1) * kChunk - 1 > (int64_t)qt * BM + wave * 32;
    if (tail || diag) {
      const int64_t last = p.causal ? (qrow < p.lk - 1 ? qrow : p.lk - 1) : p.lk - 1;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) mask_tail(s[kt], valid_prefix(key0 + 32 * kt, last));
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
    chunk = next;
  }
  mx = pair_max(mx);
  if (qvalid && hf == 0) p.m_out[bh * p.lq + qrow] = mx * p.c;
}

}  // namespace

// fp16 P-hat V-hat product: both operands fake-quantized under unit global scales (a static scale
// makes the values inexact in fp16; they are rounded to bf16 instead), or both rounded to E4M3FN
// (the FP8 P.V product, which requires a quantized P).
static bool use_f16_unit(unsigned flags) {
  return (flags & kFlagV) && (flags & kFlagP) && !(flags & (kFlagGsfQkv | kFlagsPGlobal));
}
static bool use_f16(unsigned flags) { return use_f16_unit(flags) || (flags & kFlagPvFp8); }
// Training calls that attn_fwd_pp_train_kernel (dense) and attn_fwd_vsa_pp_train_kernel
// (cube-sparse) serve: every quantizer on under unit scales (Q-hat, K-hat exact in fp16), smooth-K
// allowed; not the final-max pass (it reads bf16 K-hat rows) nor smooth-Q.
static bool pp_train_ok(const AttnArgs &a) {
  const bool train = a.o_hp && a.lse && a.cmax;
  return train && (a.flags & kFlagQ) && (a.flags & kFlagK) && use_f16_unit(a.flags) &&
         !(a.flags & (kFlagFinalMax | kFlagSmoothQ));
}

// The forward kernel of a call, by its mode: training (QL layout for dense calls), ping-pong dense
// inference, or the single-group kernel (cube-sparse or smooth-Q inference); qp / f16 / gp as in
// form_p.
template <bool GP, bool SQ>
static void launch_fwd_kernel(const FwdParams &p, dim3 grid, dim3 block, bool train, bool ql, bool pipe, bool qp,
                              bool f16, const char *nm, const char *nm_train, hipStream_t stream) {
  if (GP && f16) {  // the FP8 P.V product: E4M3FN operands, exact in fp16
    if (ql) AQ_LAUNCH(nm_train, (attn_fwd_kernel<true, true, true, true, GP, SQ>), grid, block, 0, stream, p);
    else if (train) AQ_LAUNCH(nm_train, (attn_fwd_kernel<true, true, true, false, GP, SQ>), grid, block, 0, stream, p);
    else if (pipe && !SQ) AQ_LAUNCH(nm, (attn_fwd_pp_kernel<true, true, GP>), grid, block, 0, stream, p);
    else AQ_LAUNCH(nm, (attn_fwd_kernel<false, true, true, false, GP, SQ>), grid, block, 0, stream, p);
    return;
  }
  if (GP) {  // P quantized under a global scale: bf16 product
    if (ql) AQ_LAUNCH(nm_train, (attn_fwd_kernel<true, true, false, true, GP, SQ>), grid, block, 0, stream, p);
    else if (train) AQ_LAUNCH(nm_train, (attn_fwd_kernel<true, true, false, false, GP, SQ>), grid, block, 0, stream, p);
    else if (pipe && !SQ) AQ_LAUNCH(nm, (attn_fwd_pp_kernel<true, false, GP>), grid, block, 0, stream, p);
    else AQ_LAUNCH(nm, (attn_fwd_kernel<false, true, false, false, GP, SQ>), grid, block, 0, stream, p);
    return;
  }
  if (ql) {
    if (f16) AQ_LAUNCH(nm_train, (attn_fwd_kernel<true, true, true, true, false, SQ>), grid, block, 0, stream, p);
    else AQ_LAUNCH(nm_train, (attn_fwd_kernel<true, true, false, true, false, SQ>), grid, block, 0, stream, p);
  } else if (train) {
    if (f16) AQ_LAUNCH(nm_train, (attn_fwd_kernel<true, true, true, false, false, SQ>), grid, block, 0, stream, p);
    else if (qp) AQ_LAUNCH(nm_train, (attn_fwd_kernel<true, true, false, false, false, SQ>), grid, block, 0, stream, p);
    else AQ_LAUNCH(nm_train, (attn_fwd_kernel<true, false, false, false, false, SQ>), grid, block, 0, stream, p);
  } else if (pipe && !SQ) {
    if (f16) AQ_LAUNCH(nm, (attn_fwd_pp_kernel<true, true, false>), grid, block, 0, stream, p);
    else if (qp) AQ_LAUNCH(nm, (attn_fwd_pp_kernel<true, false, false>), grid, block, 0, stream, p);
    else AQ_LAUNCH(nm, (attn_fwd_pp_kernel<false, false, false>), grid, block, 0, stream, p);
  } else {
    if (f16) AQ_LAUNCH(nm, (attn_fwd_kernel<false, true, true, false, false, SQ>), grid, block, 0, stream, p);
    else if (qp) AQ_LAUNCH(nm, (attn_fwd_kernel<false, true, false, false, false, SQ>), grid, block, 0, stream, p);
    else AQ_LAUNCH(nm, (attn_fwd_kernel<false, false, false, false, false, SQ>), grid, block, 0, stream, p);
  }
}

// Workgroup tiling of a forward-type kernel with `waves` 32-query waves per workgroup.
static void set_tiling(FwdParams &p, const AttnArgs &a, int waves) {
  p.qtiles = (int)((a.lq + 32 * waves - 1) / (32 * waves));
  p.nblocks = (int64_t)a.batch * a.heads * p.qtiles;
  p.per_xcd = (p.nblocks + 7) / 8;
}

hipError_t launch_attn_fwd_sel(const AttnArgs &a, const int32_t *sel, int64_t nsel, hipStream_t stream) {
  constexpr int WAVES = 4;
  if (sel && (nsel > kMaxSel || nsel < 1)) return hipErrorInvalidValue;
  const Workspace w = workspace_layout(sel ? 2 : 0, a.batch, a.heads, a.lq, a.lk);
  const VariantPtrs vp = variant_ptrs(a, w);
  uint8_t *ws = (uint8_t *)a.workspace;
  FwdParams p{};
  p.q = (const uint16_t *)a.q;
  p.sq = a.sq;
  p.o = (uint16_t *)a.o;
  p.so = a.so;
  p.kq = (const u32x4 *)(ws + w.kq);
  p.vt = (const u32x4 *)(ws + w.vt);
  p.lse = a.lse;
  p.cmax = a.cmax;
  p.o_hp = a.o_hp;
  p.sel = sel;
  p.heads = a.heads;
  p.lq = a.lq;
  p.lk = a.lk;
  p.kchunks = (a.lk + kChunk - 1) / kChunk;
  p.nchunks = sel ? nsel : p.kchunks;
  p.c = (float)((double)a.scale * 1.4426950408889634);
  p.causal = a.causal;
  p.quant_q = (a.flags & kFlagQ) != 0;
  p.gq = vp.gq;
  p.qmean = vp.qmean;
  p.delta = vp.delta;
  const bool qp = (a.flags & kFlagP) != 0, f16 = use_f16(a.flags);
  const bool gp = qp && (a.flags & kFlagsPGlobal);
  p.gp_static = (a.flags & kFlagGsfP) ? kPScaleStatic : 1.0f;
  // Training outputs come as a set (lse, chunk maxima, O^hp).
  const bool train = a.o_hp && a.lse && a.cmax;
  if (!train && (a.o_hp || a.lse || a.cmax)) return hipErrorInvalidValue;
  // Two-level P: the chunk-maximum array holds a second block of the same shape, P's global
  // scale of every (row, chunk), for the backward.
  p.two_level = (a.flags & kFlagTwoLevelP) != 0;
  if (train && p.two_level) p.pg = a.cmax + (int64_t)a.batch * a.heads * p.nchunks * a.lq;

  if (a.flags & kFlagFinalMax) {
    // Row maxima first; the forward's running max starts there.
    FwdParams r = p;
    r.m_out = (float *)(ws + w.mfin);
    set_tiling(r, a, WAVES);
    AQ_LAUNCH("rowmax", rowmax_kernel, dim3((unsigned)(r.per_xcd * 8)), dim3(WAVES * 64), 0, stream, r);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    p.m_init = r.m_out;
  }

  const bool pp_train = pp_train_ok(a) && !sel;  // attn_fwd_pp_train_kernel
  const bool ql = train && qp && !sel && !pp_train;  // see attn_fwd_kernel
  const bool pipe = !train && !sel && !p.delta;  // attn_fwd_pp_kernel (not under smooth-Q)
  const int waves = ql ? 8 : (pipe || pp_train) ? kPPWaves : WAVES;
  set_tiling(p, a, waves);
  const dim3 grid((unsigned)(p.per_xcd * 8)), block(waves * 64);
  const char *nm_train = sel ? "vsa_fwd_train" : "attn_fwd_train", *nm = sel ? "vsa_fwd" : "attn_fwd";
  if (pp_train) {
    AQ_LAUNCH(nm_train, attn_fwd_pp_train_kernel, grid, block, 0, stream, p);
    return hipGetLastError();
  }
  // Cube-sparse training under unit scales: the ping-pong training kernel over the lists, two
  // query cubes per workgroup.
  if (sel && pp_train_ok(a)) {
    FwdParams v = p;
    v.qtiles = (int)((a.lq / kChunk + 1) / 2);
    v.nblocks = (int64_t)a.batch * a.heads * v.qtiles;
    v.per_xcd = (v.nblocks + 7) / 8;
    AQ_LAUNCH(nm_train, attn_fwd_vsa_pp_train_kernel, dim3((unsigned)(v.per_xcd * 8)), dim3(kPPWaves * 64), 0,
              stream, v);
    return hipGetLastError();
  }
  // Cube-sparse inference under unit scales with P and V quantized: the ping-pong kernel over the
  // lists, two query cubes per workgroup.
  if (sel && !train && !p.delta && qp && use_f16_unit(a.flags)) {
    FwdParams v = p;
    v.qtiles = (int)((a.lq / kChunk + 1) / 2);
    v.nblocks = (int64_t)a.batch * a.heads * v.qtiles;
    v.per_xcd = (v.nblocks + 7) / 8;
    AQ_LAUNCH(nm, attn_fwd_vsa_pp_kernel, dim3((unsigned)(v.per_xcd * 8)), dim3(kPPWaves * 64), 0, stream, v);
    return hipGetLastError();
  }
  const bool sq = p.delta != nullptr;
  if (gp && sq) launch_fwd_kernel<true, true>(p, grid, block, train, ql, pipe, qp, f16, nm, nm_train, stream);
  else if (gp) launch_fwd_kernel<true, false>(p, grid, block, train, ql, pipe, qp, f16, nm, nm_train, stream);
  else if (sq) launch_fwd_kernel<false, true>(p, grid, block, train, ql, pipe, qp, f16, nm, nm_train, stream);
  else launch_fwd_kernel<false, false>(p, grid, block, train, ql, pipe, qp, f16, nm, nm_train, stream);
  return hipGetLastError();
}

// The variants' per-call quantities, then K-hat rows and V-hat tiles for keys [0, lk) of every
// head, into the workspace of `op` (0: dense forward, 2: cube-sparse forward).
hipError_t launch_kv_prepass(const AttnArgs &a, int op, hipStream_t stream, bool overlap) {
  const Workspace w = workspace_layout(op, a.batch, a.heads, a.lq, a.lk);
  uint8_t *ws = (uint8_t *)a.workspace;
  hipError_t e = launch_variant_prep(a, w, stream);
  if (e != hipSuccess) return e;
  const VariantPtrs vp0 = variant_ptrs(a, w);
  const bool kq = (a.flags & kFlagK) != 0 && !vp0.gk && !vp0.kmean;
  const bool vq = (a.flags & kFlagV) != 0 && !vp0.gv && !(a.flags & kFlagPvFp8);
  if (kq && vq) {
    // the common case: both operands under unit scales, one streamed launch
    e = launch_kv_stream(a.k, a.sk, a.v, a.sv, a.batch, a.heads, a.lk, 0, (int64_t)a.batch * a.heads, ws + w.kq,
                         pp_train_ok(a), ws + w.vt, use_f16_unit(a.flags), stream);
    return e != hipSuccess ? e : launch_qk_delta(a, w, stream);
  }
  SideFork f{stream, -1};
  if (overlap && (e = side_fork(stream, f)) != hipSuccess) return e;
  const VariantPtrs vp = variant_ptrs(a, w);
  // (fp16 K-hat rows for the ping-pong training kernel, bf16 for every other forward kernel)
  e = launch_tile_prepass(a.k, a.sk, a.batch, a.heads, a.lk, (a.flags & kFlagK) ? kQuantD : kQuantNone, ws + w.kq,
                          nullptr, vp.gk, vp.kmean, stream, pp_train_ok(a) ? kOutF16 : kOutBf16);
  if (e == hipSuccess) e = launch_qk_delta(a, w, stream);
  const TileQuant qv = use_f16_unit(a.flags) ? kQuantRowsF16 : ((a.flags & kFlagV) ? kQuantRows : kQuantNone);
  if (e == hipSuccess)
    e = launch_tile_prepass(a.v, a.sv, a.batch, a.heads, a.lk, qv, nullptr, ws + w.vt, vp.gv, nullptr, f.stream,
                            (a.flags & kFlagPvFp8) ? kOutFp8F16 : kOutBf16);
  const hipError_t j = side_join(stream, f);
  return e != hipSuccess ? e : j;
}

hipError_t launch_attn_fwd(const AttnArgs &a, hipStream_t stream) {
  hipError_t e = launch_kv_prepass(a, 0, stream, true);
  if (e != hipSuccess) return e;
  return launch_attn_fwd_sel(a, nullptr, 0, stream);
}

}  // namespace aq
