// attn_bwd.hip - straight-through backward of NVFP4 fake-quant attention on gfx950.
//
// "vsqa-preview-1.3b metadata.json", dense precision record: backward "consistent STE with
// auxiliary output"; "attn_qat_train" API page: use_qat_qkv_backward, fake_quant_p_bwd,
// use_high_prec_o.  Fake-quant nodes pass gradients through unchanged and the running maxima are
// constants.  In base-2 logit units y = c * <q-hat, k-hat> (c = softmax_scale * log2 e), with the
// forward's lse2 and chunk maxima m_c:
//   A     = exp2(y - lse2)                        unquantized probabilities
//   A-hat = fq(exp2(y - m_c)) * exp2(m_c - lse2)   the probabilities the forward multiplied V with
//   D_i = <dO_i, o_hp_i>,  dP = dO V-hat^T,  dS = A * (dP - D)
//   dV = A-hat^T dO,  dQ = scale dS K-hat,  dK = scale dS^T Q-hat.
//
// Work split (deterministic, no atomics):
//   dvec_kernel   D_i.
//   bwd_dq        one workgroup per (head, 128 queries), looping over 128-key chunks; S^T, dP^T and
//                 dQ^T keep one query per lane exactly like the forward, and A needs no fake quant.
//   bwd_dkdv      one workgroup per (head, 128-key chunk); each wave owns 32 keys and loops over
//                 64-query tiles.  S^T is recomputed with the forward's MFMA arrangement (same
//                 A rows, B columns and k-slot order) so P and P-hat match the forward bit for
//                 bit; dV and dK contract over queries, so A-hat and dS are moved to one key per
//                 lane by an exact MFMA against a one-hot matrix before the gradient MFMAs.
#include "attn_common.hpp"
#include "launch.hpp"
#include "timing.hpp"

namespace aq {
namespace {

constexpr int kD = kHeadDim;

// D_i = <dO_i, o_hp_i>: 16 lanes per row, 8 elements per lane.
__global__ __launch_bounds__(256) void dvec_kernel(const uint16_t *__restrict__ d_o, Strides s, const float *__restrict__ o_hp,
                                                   float *__restrict__ dvec, int heads, int64_t lq, int64_t rows) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid >> 4;
  const int part = (int)(gid & 15);
  float acc = 0.0f;
  if (row < rows) {
    const int64_t bh = row / lq, i = row % lq;
    const int64_t b = bh / heads, h = bh % heads;
    const u32x4 v = *(const u32x4 *)(d_o + b * s.b + h * s.h + i * s.l + part * 8);
    const f32x4 o0 = *(const f32x4 *)(o_hp + row * kD + part * 8);
    const f32x4 o1 = *(const f32x4 *)(o_hp + row * kD + part * 8 + 4);
    acc = bf16lo(v.x) * o0[0] + bf16hi(v.x) * o0[1] + bf16lo(v.y) * o0[2] + bf16hi(v.y) * o0[3] +
          bf16lo(v.z) * o1[0] + bf16hi(v.z) * o1[1] + bf16lo(v.w) * o1[2] + bf16hi(v.w) * o1[3];
  }
  for (int off = 1; off < 16; off <<= 1) acc += __shfl_xor(acc, off);
  if (row < rows && part == 0) dvec[row] = acc;
}

struct BwdParams {
  const u32x4 *qq;    // Q-hat rows   [BH, Cq*128, 128]
  const u32x4 *kq;    // K-hat rows   [BH, Ck*128, 128]
  const u32x4 *vq;    // V-hat rows   [BH, Ck*128, 128]
  const uint16_t *d_o;
  Strides sdo;
  const float *lse;   // [BH, lq]
  const float *cmax;  // [BH, Ck, lq]
  const float *dvec;  // [BH, lq]
  uint16_t *dq, *dk, *dv;
  Strides sdq, sdk, sdv;
  int heads;
  int64_t lq, lk, Cq, Ck;
  int64_t nwork, per_xcd;
  float c, scale;
  bool causal, quant_p;
  // Cube-sparse fine stage (null for dense): sel [BH, n, nsel] selected key cubes of every query
  // cube, ascending; slot_t [BH, n key cubes, n query cubes] position of the key cube in that
  // query cube's list, or -1.  Chunk maxima are then [BH, nsel, lq], one per selected cube.
  const int32_t *sel;
  const int16_t *slot_t;
  int64_t nsel;
  // Two-level P: [BH, Ck or nsel, lq] P's global scale per (query, chunk) as the forward used it,
  // laid out like the chunk maxima; null otherwise.
  const float *pg;
  // Smooth-Q: delta [BH, Ck*128] added to every logit, and the queries' mean [BH, 128], which the
  // key gradients see added back to Q-hat; null otherwise.
  const float *delta, *qmean;
  // GP kernels: P's global scale when it is not the two-level one (448*6, or 1), and whether P-hat is
  // rounded to FP8 E4M3FN (the FP8 P.V product), as the forward did.
  float gp_static;
  bool pv_fp8;
  // Dense dQ and dK/dV (set per launch): work ids below nfull are whole units on blocks
  // [0, full_blocks) (XCD-ordered, per_xcd per XCD); each of the remaining units is split into
  // `split` pieces, one block each after full_blocks, whose fp32 sums go to part for the reduction
  // kernel: dQ units (head, 128 queries) along their key chunks, part [piece][128 queries][128 d];
  // dK/dV units (head, key chunk) along their query tiles, part [piece][dK, dV][128 keys][128 d].
  // split = 0: no pieces.
  int64_t nfull, full_blocks;
  int split;
  float *part;
};

// ---------------------------------------------------------------------------------------------
// dQ: workgroup = (head, 128 queries), 8 waves, loop over 128-key chunks.  Wave w owns queries
// 32*(w%4) .. +31 (their Q-hat and dO in registers, the B operands of S^T and dP^T) and keys
// 64*(w/4) .. +63 of every chunk; the two waves that share queries add their partial dQ through
// LDS at the end.  Two waves per SIMD.
//
// LDS: two chunk buffers of 64 KiB, each K-hat rows [128][256 B] then V-hat rows (A operands of
// S^T and dP^T, sw_kd swizzle).  The A operand of dQ^T (K-hat^T: 8 consecutive keys of one d per
// lane half) comes from the same K-hat rows through transposed reads.  Chunk c+1 is copied
// asynchronously while chunk c is computed; one barrier per chunk.
// ---------------------------------------------------------------------------------------------
constexpr int kDqThreads = 512;
constexpr int kDqLds = 2 * 65536;

// Swizzle of the dQ kernel's K-hat/V-hat rows.  A-operand reads in perm_row order: 16 lanes read
// rows {0..3, 16..19, 4..7, 20..23} (+8 for the next 16), told apart by bits 0, 1, 2 and 4 of the
// row.  Transposed reads: 4 consecutive rows (bits 0, 1) each supply 32 contiguous bytes, so bits
// 0 and 1 must pick the 64-byte quarter (the two high bits of the 16-byte column).
__device__ __forceinline__ int sw_kd(int r) { return ((r >> 2) & 1) | ((r >> 3) & 2) | ((r & 3) << 2); }

template <bool SPARSE, bool SQ>
__global__ __launch_bounds__(kDqThreads, 1) void bwd_dq_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(256))) uint8_t lds[kDqLds];
  const uint32_t lds0 = lds_addr(lds);
  const int64_t vid = xcd_work_id(blockIdx.x, p.per_xcd, p.nwork);
  if (vid < 0) return;
  const int64_t bh = vid / p.Cq;
  const int64_t qc = vid % p.Cq;
  const int64_t bb = bh / p.heads, hh = bh % p.heads;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 31, hf = lane >> 5;
  const int qg = wave & 3, kh = wave >> 2;
  const int qrow = (int)(qc * kChunk) + qg * 32 + n;
  const bool qvalid = qrow < p.lq;

  int64_t n_iter = SPARSE ? p.nsel : p.Ck;
  if (p.causal) {
    const int64_t q_last = qc * kChunk + kChunk - 1;
    n_iter = (q_last < p.lk - 1 ? q_last : p.lk - 1) / kChunk + 1;
  }
  // Key chunk of iteration `it`: the it-th selected cube, or chunk `it` (a uniform scalar).
  const int32_t *sel_row = SPARSE ? p.sel + (bh * p.Cq + qc) * p.nsel : nullptr;
  auto chunk_at = [&](int64_t it) -> int64_t { return SPARSE ? clamp_chunk(sel_row[it], p.Ck) : it; };
  // Chunk copies: per lane 4 K-hat and 4 V-hat pieces of 16 bytes.
  uint32_t c_voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (i * 8 + wave) * 4 + (lane >> 4);
    c_voff[i] = (uint32_t)(r * 256 + (((lane & 15) ^ sw_kd(r)) << 4));
  }
  auto stage_chunk = [&](int64_t ch, int buf) {
    const u32x4 *ks = p.kq + (bh * p.Ck + ch) * (kChunk * kD / 8);
    const u32x4 *vs = p.vq + (bh * p.Ck + ch) * (kChunk * kD / 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      load_lds16_s(ks, c_voff[i], lds + buf * 65536 + (i * 8 + wave) * 1024);
      load_lds16_s(vs, c_voff[i], lds + buf * 65536 + 32768 + (i * 8 + wave) * 1024);
    }
  };
  stage_chunk(chunk_at(0), 0);

  bf16x8 qf[8], of[8];
  {
    const u32x4 *qsrc = p.qq + (bh * p.Cq * kChunk + qc * kChunk + qg * 32 + n) * (kD / 8);
    const uint16_t *osrc = p.d_o + bb * p.sdo.b + hh * p.sdo.h + (int64_t)(qvalid ? qrow : 0) * p.sdo.l;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      qf[t] = as_bf16x8(qsrc[2 * t + hf]);
      u32x4 v = {0u, 0u, 0u, 0u};
      if (qvalid) v = *(const u32x4 *)(osrc + 16 * t + 8 * hf);
      of[t] = as_bf16x8(v);
    }
  }
  const float lse2 = qvalid ? p.lse[bh * p.lq + qrow] : 0.0f;
  const float Di = qvalid ? p.dvec[bh * p.lq + qrow] : 0.0f;
  // largest key this query sees (-1: an out-of-range query row sees none)
  const int last = !qvalid ? -1 : (p.causal && qrow < p.lk - 1 ? qrow : (int)p.lk - 1);

  // S^T / dP^T A operand: row 64*kh + 32*k2 + perm_row(n), 16-byte column 2t + hf (XOR term of the
  // swizzle in bits 5..7, so column pair t is `^ 32*t`; k2 adds 8 KiB, V-hat 32 KiB).
  int a_off;
  {
    const int r = 64 * kh + perm_row(n), sw = sw_kd(r);
    a_off = r * 256 + 16 * ((hf ^ sw) & 1) + 32 * (sw >> 1);
  }
  // Transposed reads (see ds_read_tr16): lane (group g = (lane/16)%2, h = lane/32, e = (lane/4)%4,
  // j = lane%4) reads key row 64*kh + 32*k2 + 16*h + 8*jj + 4*a + e, d columns 32*dt + 16*g + 4*j
  // .. +3, for dQ^T k-slot group jj (8 keys) and half a.  The row's swizzle is 4*e + 2*h + a, so the
  // 16-byte column is 4*(dt^e) + ((2*g + j/2) ^ (2*h + a)).
  int t_off;
  {
    const int e = (lane >> 2) & 3, j = lane & 3, g = (lane >> 4) & 1;
    const int lo = (2 * g + (j >> 1)) ^ (2 * hf);
    t_off = (64 * kh + 16 * hf + e) * 256 + 64 * e + 16 * lo + 8 * (j & 1);
  }

  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};

  for (int64_t it = 0; it < n_iter; ++it) {
    const int buf = (int)(it & 1);
    const int64_t ch = chunk_at(it);
    AQ_WAIT_VMCNT(0);  // this wave's copies of chunk ch
    __syncthreads();   // everyone's copies landed; the other buffer is free
    if (it + 1 < n_iter) stage_chunk(chunk_at(it + 1), buf ^ 1);
    uint32_t ka = lds0 + buf * 65536 + a_off, ta = lds0 + buf * 65536 + t_off;
    AQ_OPAQUE(ka);
    AQ_OPAQUE(ta);
    const bool tail = (ch + 1) * kChunk > p.lk;
    const bool diag = p.causal && (ch + 1) * kChunk - 1 > qc * kChunk + qg * 32;
    // Both 32-key halves' logits and dP first, then both halves' dS, then both halves' dQ
    // products: the second half's MFMAs are independent of the first half's vector work.
    f32x16 s[2], dp[2];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      // smooth-Q: the logit chain starts from delta of the lane's 16 keys, as the forward's does
      dp[k2] = f32x16{};
      if constexpr (SQ) s[k2] = delta16(p.delta + (bh * p.Ck + ch) * kChunk + 64 * kh + 32 * k2 + 16 * hf);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t at = (ka ^ (32 * t)) + k2 * 8192;
        s[k2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(lds_read16(at)), qf[t],
                                                        (SQ || t > 0) ? s[k2] : f32x16{}, 0, 0, 0);
        dp[k2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(lds_read16(at + 32768)), of[t], dp[k2], 0, 0, 0);
      }
    }
    bf16x8 d0[2], d1[2];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      if (tail || diag || !qvalid) {
        const int key0 = (int)(ch * kChunk) + 64 * kh + 32 * k2 + 16 * hf;
        mask_tail(s[k2], valid_prefix(key0, last));
      }
      float ds[16];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const float A = __builtin_amdgcn_exp2f(__builtin_fmaf(s[k2][rr], p.c, -lse2));
        ds[rr] = A * (dp[k2][rr] - Di);
      }
      d0[k2] = pack8_cvt(ds);
      d1[k2] = pack8_cvt(ds + 8);
    }
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        // k-slot group jj = 0 (keys 16h + 0..7, register pack d0) and jj = 1 (keys 16h + 8..15)
        const uint32_t b0 = (ta ^ (dt << 6)) + k2 * 8192, b1 = (ta ^ ((dt << 6) | 16)) + k2 * 8192;
        const uint2 x0 = ds_read_tr16_at(b0), x1 = ds_read_tr16_at(b1 + 1024);
        const uint2 y0 = ds_read_tr16_at(b0 + 2048), y1 = ds_read_tr16_at(b1 + 3072);
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(u32x4{x0.x, x0.y, x1.x, x1.y}), d0[k2], acc[dt], 0, 0, 0);
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(u32x4{y0.x, y0.y, y1.x, y1.y}), d1[k2], acc[dt], 0, 0, 0);
      }
  }

  // The two waves of a query group add their partial sums; wave kh = 0 stores.
  AQ_WAIT_VMCNT(0);
  __syncthreads();
  float *xch = (float *)(lds + qg * 16384);
  if (kh == 1) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *(f32x4 *)(xch + ((dt * 4 + a) * 64 + lane) * 4) =
            f32x4{acc[dt][4 * a], acc[dt][4 * a + 1], acc[dt][4 * a + 2], acc[dt][4 * a + 3]};
  }
  __syncthreads();
  if (kh == 1 || !qvalid) return;
  uint16_t *op = p.dq + bb * p.sdq.b + hh * p.sdq.h + (int64_t)qrow * p.sdq.l;
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const f32x4 o = *(const f32x4 *)(xch + ((dt * 4 + a) * 64 + lane) * 4);
      const int d0 = 32 * dt + 8 * a + 4 * hf;
      *(bf16x4 *)(op + d0) = bf16x4{(__bf16)((acc[dt][4 * a] + o[0]) * p.scale), (__bf16)((acc[dt][4 * a + 1] + o[1]) * p.scale),
                                    (__bf16)((acc[dt][4 * a + 2] + o[2]) * p.scale), (__bf16)((acc[dt][4 * a + 3] + o[3]) * p.scale)};
    }
}

// ---------------------------------------------------------------------------------------------
// dQ, software-pipelined form (every call but smooth-Q): workgroup = (head, 128 queries), 4 waves,
// two workgroups per CU.  Wave w holds Q-hat and dO of queries 32w .. +31 in registers and walks
// every 32-key sub-tile of the head's key sequence (chunk list) itself.  Iteration s does the
// vector work of sub-tile s (A = exp2(y - lse2), dS = A (dP - D), packed to bf16) interleaved with
// the MFMAs of dQ^T += K-hat^T dS^T for sub-tile s-1 and of S^T, dP^T for sub-tile s+1, none of
// which depends on it: per sub-tile a wave issues 24 MFMAs and about 72 vector instructions, few
// enough for its own MFMAs to hide them.  The workgroup barrier of each iteration only publishes
// the copies.
//
// LDS: five slots of 16 KiB, each one sub-tile's K-hat rows [32][256 B] then V-hat rows [32][256 B]
// (sw_kd swizzle).  Sub-tile s is read in iterations s-1 (S^T, dP^T) and s+1 (K-hat^T for dQ^T);
// sub-tile s+3 is copied into the slot of s-2 at the start of iteration s and waited for at the
// start of iteration s+2.
// ---------------------------------------------------------------------------------------------
constexpr int kDqsWaves = 4;
constexpr int kDqsSlots = 5;
constexpr int kDqsSlot = 16384;

template <bool SPARSE>
__global__ __launch_bounds__(kDqsWaves * 64, 2) void bwd_dq_sp_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(256))) uint8_t lds[kDqsSlots * kDqsSlot];
  const uint32_t lds0 = lds_addr(lds);
  // A whole unit, or piece `piece` (>= 0) of a split one (dense only).
  int64_t vid, piece = -1;
  if ((int64_t)blockIdx.x < p.full_blocks) {
    vid = xcd_work_id(blockIdx.x, p.per_xcd, p.nfull);
    if (vid < 0) return;
  } else {
    piece = (int64_t)blockIdx.x - p.full_blocks;
    vid = p.nfull + piece / p.split;
  }
  const int64_t bh = vid / p.Cq;
  const int64_t qc = vid % p.Cq;
  const int64_t bb = bh / p.heads, hh = bh % p.heads;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, n = lane & 31, hf = lane >> 5;
  const int qrow = (int)(qc * kChunk) + wave * 32 + n;
  const bool qvalid = qrow < p.lq;

  int64_t n_chunks = SPARSE ? p.nsel : p.Ck;
  if (p.causal) {
    const int64_t q_last = qc * kChunk + kChunk - 1;
    n_chunks = (q_last < p.lk - 1 ? q_last : p.lk - 1) / kChunk + 1;
  }
  // piece j of `split`: key chunks (list positions) [n_chunks * j / split, n_chunks * (j + 1) / split)
  int64_t c_lo = 0;
  if (piece >= 0) {
    const int64_t j = piece % p.split, hi = n_chunks * (j + 1) / p.split;
    c_lo = n_chunks * j / p.split;
    n_chunks = hi - c_lo;
  }
  const int nsteps = (int)(4 * n_chunks);
  const int32_t *sel_row = SPARSE ? p.sel + (bh * p.Cq + qc) * p.nsel : nullptr;
  // Head-local key of row 0 of sub-tile s (a uniform scalar).
  auto step_key = [&](int s) -> int64_t {
    const int64_t ch = SPARSE ? clamp_chunk(sel_row[c_lo + (s >> 2)], p.Ck) : c_lo + (int64_t)(s >> 2);
    return ch * kChunk + 32 * (s & 3);
  };
  const uint8_t *kbase = (const uint8_t *)(p.kq + bh * p.Ck * kChunk * (kD / 8));
  const uint8_t *vbase = (const uint8_t *)(p.vq + bh * p.Ck * kChunk * (kD / 8));
  // Copies of one sub-tile by the four waves: wave w copies rows 16i + 4w + lane/16 (i = 0, 1) of
  // K-hat and of V-hat, physical column lane%16.
  uint32_t c_off[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (i * 4 + wave) * 4 + (lane >> 4);
    c_off[i] = (uint32_t)(r * 256 + (((lane & 15) ^ sw_kd(r)) << 4));
  }
  auto slot_of = [&](int s) -> uint32_t { return lds0 + (uint32_t)(s % kDqsSlots) * kDqsSlot; };
  auto copy_step = [&](int s) {
    const int64_t row0 = step_key(s);
    const uint32_t dst = slot_of(s) + (uint32_t)wave * 1024;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      load_lds16_sa(kbase + row0 * 256, c_off[i], dst + i * 4096);
      load_lds16_sa(vbase + row0 * 256, c_off[i], dst + 8192 + i * 4096);
    }
  };

  for (int s = 0; s < 3 && s < nsteps; ++s) copy_step(s);
  bf16x8 qf[8], of[8];
  {
    const u32x4 *qsrc = p.qq + (bh * p.Cq * kChunk + qc * kChunk + wave * 32 + n) * (kD / 8);
    const uint16_t *osrc = p.d_o + bb * p.sdo.b + hh * p.sdo.h + (int64_t)(qvalid ? qrow : 0) * p.sdo.l;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      qf[t] = as_bf16x8(qsrc[2 * t + hf]);
      u32x4 v = {0u, 0u, 0u, 0u};
      if (qvalid) v = *(const u32x4 *)(osrc + 16 * t + 8 * hf);
      of[t] = as_bf16x8(v);
    }
  }
  const float lse2 = qvalid ? p.lse[bh * p.lq + qrow] : 0.0f;
  const float Di = qvalid ? p.dvec[bh * p.lq + qrow] : 0.0f;
  const int last = !qvalid ? -1 : (p.causal && qrow < p.lk - 1 ? qrow : (int)p.lk - 1);

  // Lane offsets inside a slot (slots are 16 KiB aligned, so the XOR terms, bits 4..7, act on the
  // offsets alone): the S^T / dP^T A operand at column pair t is `a_off ^ 32t`; the transposed
  // reads of K-hat^T for dQ^T d tile dt are `t_off ^ 64dt` and `(t_off ^ (64dt | 16)) + 1024`.
  uint32_t a_off, t_off;
  {
    const int r = perm_row(n), sw = sw_kd(r);
    a_off = (uint32_t)(r * 256 + 16 * ((hf ^ sw) & 1) + 32 * (sw >> 1));
    const int e = (lane >> 2) & 3, j = lane & 3, g2 = (lane >> 4) & 1;
    const int lo = (2 * g2 + (j >> 1)) ^ (2 * hf);
    t_off = (uint32_t)((16 * hf + e) * 256 + 64 * e + 16 * lo + 8 * (j & 1));
  }

  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};

  // S^T and dP^T of sub-tile s.
  auto logits = [&](int s, f32x16 &sv, f32x16 &dpv) {
    const uint32_t a = slot_of(s) + a_off;
    sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(lds_read16(a)), qf[0], f32x16{}, 0, 0, 0);
    dpv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(lds_read16(a + 8192)), of[0], f32x16{}, 0, 0, 0);
#pragma unroll
    for (int t = 1; t < 8; ++t) {
      const uint32_t at = a ^ (32u * t);
      sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(lds_read16(at)), qf[t], sv, 0, 0, 0);
      dpv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(lds_read16(at + 8192)), of[t], dpv, 0, 0, 0);
    }
  };
  // dQ^T += K-hat^T dS^T of sub-tile s (dS in d0 / d1).
  auto dq_products = [&](int s, const bf16x8 &d0, const bf16x8 &d1) {
    const uint32_t b = slot_of(s) + t_off;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const uint32_t b0 = b ^ (uint32_t)(dt << 6), b1 = (b ^ (uint32_t)((dt << 6) | 16)) + 1024;
      const uint2 x0 = ds_read_tr16_at(b0), x1 = ds_read_tr16_at(b1);
      const uint2 y0 = ds_read_tr16_at(b0 + 2048), y1 = ds_read_tr16_at(b1 + 2048);
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(u32x4{x0.x, x0.y, x1.x, x1.y}), d0, acc[dt], 0, 0, 0);
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(u32x4{y0.x, y0.y, y1.x, y1.y}), d1, acc[dt], 0, 0, 0);
    }
  };
  // Keys past lk, causal keys past the query, and query rows past lq (every key) are masked.
  auto mask_step = [&](int s, f32x16 &sv) {
    const int64_t k0 = step_key(s);
    const bool tail = k0 + 32 > p.lk;
    const bool diag = p.causal && k0 + 31 > qc * kChunk + wave * 32;
    if (tail || diag || !qvalid) mask_tail(sv, valid_prefix(k0 + 16 * hf, (int64_t)last));
  };
  // dS of one sub-tile, packed to bf16.
  auto dscores = [&](const f32x16 &sv, const f32x16 &dpv, bf16x8 &d0, bf16x8 &d1) {
    float ds[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const float A = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[rr], p.c, -lse2));
      ds[rr] = A * (dpv[rr] - Di);
    }
    d0 = pack8_cvt(ds);
    d1 = pack8_cvt(ds + 8);
  };

  // Iteration 0 runs the dQ products of "sub-tile -1" with dS = 0 from the slot sub-tile 4 will use:
  // zero it, or bits left in LDS by an earlier kernel (a NaN or Inf pattern) would turn 0 * x into
  // NaN.  Sub-tile 4's copy is issued in iteration 1, after that read.
  {
    u32x4 *z = (u32x4 *)(lds + (kDqsSlots - 1) * kDqsSlot) + tid;
#pragma unroll
    for (int i = 0; i < kDqsSlot / (16 * kDqsWaves * 64); ++i) z[i * kDqsWaves * 64] = u32x4{0u, 0u, 0u, 0u};
  }
  AQ_WAIT_VMCNT(0);
  __syncthreads();
  f32x16 sA, dpA, sB, dpB;
  bf16x8 dA0 = {}, dA1 = {}, dB0, dB1;  // dS of sub-tile -1 is zero: its products add nothing
  logits(0, sA, dpA);
  // One iteration: wait for sub-tile s+1, refill, then the interleaved work of sub-tile s.
  // (cur: S/dP of sub-tile s in, S/dP of s+1 out; dprev: dS of s-1 in, dnext: dS of s out.)
  auto iteration = [&](int s, f32x16 &s_cur, f32x16 &dp_cur, f32x16 &s_nxt, f32x16 &dp_nxt, const bf16x8 &dp0,
                       const bf16x8 &dp1, bf16x8 &dn0, bf16x8 &dn1) {
    if (s >= 1 && s + 2 < nsteps) AQ_WAIT_VMCNT(4);
    else AQ_WAIT_VMCNT(0);
    __builtin_amdgcn_s_barrier();
    if (s + 3 < nsteps) copy_step(s + 3);
    mask_step(s, s_cur);
    AQ_OPAQUE(s_cur);
    // MFMAs: dQ of s-1 (8, two transposed reads each), S/dP of s+1 (16, one read each); between
    // them the vector work of s.  Software-pipelined by hand in 8 steps, a scheduling barrier
    // closing each: step t issues the operand reads of step t+1, then the S^T and dP^T MFMAs of
    // column pair t and dQ^T MFMA t (d tile t/2, dS half t%2), whose operands step t-1 read, and
    // dS of rows 2t and 2t+1; so every read has a step of MFMAs to land in (left to the compiler,
    // each read sat just before its MFMA).  Same products in the same order as logits,
    // dq_products and dscores.
    const uint32_t a = slot_of(s + 1) + a_off;
    const uint32_t b = slot_of(s - 1 + kDqsSlots) + t_off;
    u32x4 ks[2], kp[2];
    uint2 t0[2], t1[2];
    auto reads = [&](int t) {
      const uint32_t at = a ^ (32u * t);
      ks[t & 1] = lds_read16(at);
      kp[t & 1] = lds_read16(at + 8192);
      const int dt = t >> 1;
      const uint32_t h = (uint32_t)(t & 1) * 2048;
      t0[t & 1] = ds_read_tr16_at((b ^ (uint32_t)(dt << 6)) + h);
      t1[t & 1] = ds_read_tr16_at((b ^ (uint32_t)((dt << 6) | 16)) + 1024 + h);
    };
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    uint32_t dsw[8];
    reads(0);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (t + 1 < 8) reads(t + 1);
      const int c = t & 1;
      s_nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ks[c]), qf[t], t == 0 ? f32x16{} : s_nxt, 0, 0, 0);
      dp_nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kp[c]), of[t], t == 0 ? f32x16{} : dp_nxt, 0, 0, 0);
      acc[t >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(u32x4{t0[c].x, t0[c].y, t1[c].x, t1[c].y}),
                                                            c ? dp1 : dp0, acc[t >> 1], 0, 0, 0);
      float ds[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const float A = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[2 * t + r], p.c, -lse2));
        ds[r] = A * (dp_cur[2 * t + r] - Di);
      }
      dsw[t] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)ds[0], (__bf16)ds[1]});
      AQ_OPAQUE(dsw[t]);  // formed in this step, not sunk to its use after the loop
      __builtin_amdgcn_sched_barrier(0);
    }
    dn0 = __builtin_bit_cast(bf16x8, u32x4{dsw[0], dsw[1], dsw[2], dsw[3]});
    dn1 = __builtin_bit_cast(bf16x8, u32x4{dsw[4], dsw[5], dsw[6], dsw[7]});
    AQ_OPAQUE(dn0);
    AQ_OPAQUE(dn1);
  };
  int s = 0;
  for (; s + 1 < nsteps; s += 2) {
    iteration(s, sA, dpA, sB, dpB, dA0, dA1, dB0, dB1);
    iteration(s + 1, sB, dpB, sA, dpA, dB0, dB1, dA0, dA1);
  }
  if (s < nsteps) {
    iteration(s, sA, dpA, sB, dpB, dA0, dA1, dB0, dB1);
    dq_products(s, dB0, dB1);
  } else if (nsteps > 0) {
    dq_products(s - 1, dA0, dA1);
  }

  if (piece >= 0) {
    // a piece: its fp32 sums (before the scale) for dq_reduce_kernel
    float *dst = p.part + piece * (kChunk * kD) + (wave * 32 + n) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *(f32x4 *)(dst + 32 * dt + 8 * a + 4 * hf) =
            f32x4{acc[dt][4 * a], acc[dt][4 * a + 1], acc[dt][4 * a + 2], acc[dt][4 * a + 3]};
    return;
  }
  if (!qvalid) return;
  uint16_t *op = p.dq + bb * p.sdq.b + hh * p.sdq.h + (int64_t)qrow * p.sdq.l;
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d0i = 32 * dt + 8 * a + 4 * hf;
      *(bf16x4 *)(op + d0i) = bf16x4{(__bf16)(acc[dt][4 * a] * p.scale), (__bf16)(acc[dt][4 * a + 1] * p.scale),
                                     (__bf16)(acc[dt][4 * a + 2] * p.scale), (__bf16)(acc[dt][4 * a + 3] * p.scale)};
    }
}

// dQ of the split units: the pieces' fp32 sums added in piece order (deterministic), scaled,
// rounded to bf16.  One lane per 4 consecutive d of one query.
__global__ __launch_bounds__(256) void dq_reduce_kernel(BwdParams p, int64_t total) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= total) return;
  const int d4 = (int)(gid & 31), row = (int)((gid >> 5) & 127);
  const int64_t u = gid >> 12;
  const int64_t vid = p.nfull + u;
  const int64_t bh = vid / p.Cq, qc = vid % p.Cq;
  const int64_t q = qc * kChunk + row;
  if (q >= p.lq) return;
  const float *src = p.part + u * p.split * (kChunk * kD) + row * kD + 4 * d4;
  f32x4 acc = *(const f32x4 *)src;
  for (int j = 1; j < p.split; ++j) {
    const f32x4 x = *(const f32x4 *)(src + (int64_t)j * kChunk * kD);
    acc = f32x4{acc[0] + x[0], acc[1] + x[1], acc[2] + x[2], acc[3] + x[3]};
  }
  const int64_t bb = bh / p.heads, hh = bh % p.heads;
  uint16_t *out = p.dq + bb * p.sdq.b + hh * p.sdq.h + q * p.sdq.l;
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  *(bf16x4 *)(out + 4 * d4) = bf16x4{(__bf16)(acc[0] * p.scale), (__bf16)(acc[1] * p.scale),
                                      (__bf16)(acc[2] * p.scale), (__bf16)(acc[3] * p.scale)};
}

// ---------------------------------------------------------------------------------------------
// dK, dV: workgroup = (head, 128-key chunk), 8 waves, loop over 64-query tiles.  Wave w owns keys
// 32*(w%4) .. +31 of the chunk and queries 32*(w/4) .. +31 of every tile; the two waves that share
// keys add their partial dK/dV through LDS at the end.  Two waves per SIMD, so one wave's
// exponentials and fake quantization overlap the other's MFMAs.
//
// LDS (bytes):
//   [0, 32K)         K-hat rows of the chunk (A operand of S^T, perm_row order, sw_kq swizzle)
//   [32K, 64K)       V-hat rows of the chunk (A operand of dP^T)
//   [64K, 128K)      two tile buffers, each Q-hat rows [64][256 B] then dO rows [64][256 B]
//                    (B operands of S^T and dP^T; read transposed as the A operands of dK^T and
//                    dV^T), sw_qr swizzle
//   [128K, 128K+1.5K) two statistic buffers, each chunk max, lse and D of the tile's 64 queries
// Tile qb+1 is copied asynchronously into the other buffer while tile qb is computed; one barrier
// per tile.
// ---------------------------------------------------------------------------------------------
constexpr int kQT = 64;  // queries per tile
constexpr int kDkdvThreads = 512;
constexpr int kLdsR = 65536, kLdsStat = 131072;
constexpr int kLdsOneHot = kLdsStat + 2 * 1024;  // two one-hot B operands, 16 bytes per lane
constexpr int kMaxCubes = 4096;                   // cube-sparse: longest query-cube list
constexpr int kLdsList = kLdsOneHot + 2048;       // that list (+ its length), int32
constexpr int kLdsDelta = kLdsList + 4 * (kMaxCubes + 1);  // smooth-Q: delta of the chunk's 128 keys
constexpr int kDkdvLds = kLdsDelta + 4 * kChunk;

// Lane layout of the S^T B operand: lane n takes query pi(n) of its wave's 32 (bits 2 and 3 of n
// exchanged).  After the one-hot transposition the 8 k-slots of each lane half are then 8
// consecutive queries, so the matching A operand is one transposed LDS read pair.
__device__ __forceinline__ int pi_q(int n) { return (n & 19) | ((n & 4) << 1) | ((n & 8) >> 1); }

// Per-lane constants of the dK/dV kernel.  Byte offsets whose swizzled 16-byte column depends on
// a loop index t carry the lane's XOR term in bits 5..7, so column pair t is `off ^ (32 * t)`.
struct DkdvLane {
  int k_off;     // K-hat/V-hat A-operand row kg*32 + perm_row(n), column hf
  int r_off;     // Q-hat/dO B-operand row qloc, column hf
  int tr_off;    // transposed reads, query group a = 0; bits 6..7 hold e (d tile dt enters as ^ 64*dt)
  int qloc;      // tile-local query of this lane's S^T column
  uint32_t q_voff[2], o_voff[2];  // copy offsets of this lane's two Q-hat and dO rows of a tile
  int o_row[2];  // those rows, tile-local
  int key_base;  // head-local key of register 0
};

// Copies of tile qb into buffer `buf`: Q-hat rows from the workspace, dO rows from the caller's
// tensor (rows past lq repeat row lq-1; every product they feed is masked), and the three
// per-query statistics (entries past lq repeat entry lq-1), plus P's two-level scales when there
// are any; cm_row is the chunk-max row of the key chunk for these queries.  Per lane: 4 copies of
// 16 bytes, plus one 4-byte copy in waves 0..2 (and in wave 3 under two-level P).
__device__ __forceinline__ void dkdv_stage_tile(const BwdParams &p, const DkdvLane &ln, int64_t bh, int64_t bb,
                                                int64_t hh, int64_t cm_row, int64_t qb, uint8_t *lds, int buf,
                                                int wave, int lane) {
  uint8_t *rq = lds + kLdsR + buf * 32768, *ro = rq + 16384;
  const u32x4 *qsrc = p.qq + (bh * p.Cq * kChunk + qb * kQT) * (kD / 8);
  const uint16_t *osrc = p.d_o + bb * p.sdo.b + hh * p.sdo.h + qb * kQT * p.sdo.l;
  const int64_t rem = p.lq - 1 - qb * kQT;  // last valid tile-local row
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    load_lds16_s(qsrc, ln.q_voff[i], rq + (i * 8 + wave) * 1024);
    uint32_t ov = ln.o_voff[i];
    if (rem < kQT - 1 && ln.o_row[i] > rem)  // tail tile: repeat the last valid row
      ov = (uint32_t)(rem * p.sdo.l * 2) + (ln.o_voff[i] - (uint32_t)(ln.o_row[i] * p.sdo.l * 2));
    load_lds16_s(osrc, ov, ro + (i * 8 + wave) * 1024);
  }
  if (wave < 3 || (wave == 3 && p.pg)) {
    const float *src = (wave == 0   ? p.cmax + cm_row * p.lq
                        : wave == 3 ? p.pg + cm_row * p.lq
                                    : (wave == 1 ? p.lse : p.dvec) + bh * p.lq) +
                       qb * kQT;
    const int q = lane < rem ? lane : (int)(rem < 0 ? 0 : rem);
    load_lds4_s(src, (uint32_t)q * 4u, lds + kLdsStat + buf * 1024 + wave * 256);
  }
}

// One 64-query tile for one wave (BUF: which tile buffer holds it).
template <int BUF, bool GP, bool SQ>
__device__ __forceinline__ void dkdv_tile(const BwdParams &p, uint32_t lds0, DkdvLane ln, int64_t qb, bool tail,
                                          f32x16 *dk, f32x16 *dv, float &csum) {
  // LDS byte addresses; lds0 is 256-byte aligned, so the swizzle XORs act on the offsets alone.
  uint32_t ka = lds0 + ln.k_off, ra = lds0 + kLdsR + ln.r_off, ta0 = lds0 + kLdsR + ln.tr_off;
  AQ_OPAQUE(ka);
  AQ_OPAQUE(ra);
  AQ_OPAQUE(ta0);
  constexpr uint32_t kQ = BUF * 32768, kO = BUF * 32768 + 16384;  // buffer offsets from kLdsR

  // Smooth-Q: the logit chain starts from delta of the lane's 16 keys, as the forward's does.
  f32x16 s = f32x16{}, dp = f32x16{};
  if (SQ) {
    const uint32_t da = lds0 + kLdsDelta + 4 * (ln.key_base % kChunk);
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const u32x4 v = lds_read16(da + 16 * r4);
      s[4 * r4 + 0] = u2f(v.x);
      s[4 * r4 + 1] = u2f(v.y);
      s[4 * r4 + 2] = u2f(v.z);
      s[4 * r4 + 3] = u2f(v.w);
    }
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t kt_ = ka ^ (32 * t), rt = ra ^ (32 * t);
    const bf16x8 ak = as_bf16x8(lds_read16(kt_));
    const bf16x8 bq = as_bf16x8(lds_read16(rt + kQ));
    const bf16x8 av = as_bf16x8(lds_read16(kt_ + 32768));
    const bf16x8 bo = as_bf16x8(lds_read16(rt + kO));
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, bq, s, 0, 0, 0);
    dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bo, dp, 0, 0, 0);
  }
  const uint32_t sta = lds0 + kLdsStat + BUF * 1024 + 4 * ln.qloc;
  const float mc = lds_read_f32(sta), lse2 = lds_read_f32(sta + 256), Di = lds_read_f32(sta + 512);
  const int qrow = (int)(qb * kQT) + ln.qloc;
  const int lq = (int)p.lq;
  if (tail || qrow >= lq || (p.causal && ln.key_base + 15 > qrow)) {
    const int last = qrow >= lq ? -1 : (p.causal && qrow < (int)p.lk - 1 ? qrow : (int)p.lk - 1);
    mask_tail(s, valid_prefix(ln.key_base, last));
  }
  // A = exp2(y - m_c) exp2(m_c - lse2); dS = A (dP - D); A-hat = fq(exp2(y - m_c)) exp2(m_c - lse2),
  // with the P block's codes formed exactly as the forward formed them (prob_block).
  float bm = s[0];
#pragma unroll
  for (int rr = 1; rr < 16; ++rr) bm = fmaxf(bm, s[rr]);
  const float w = __builtin_amdgcn_exp2f(mc - lse2);
  float ah[16], ds[16];
  if (p.quant_p) {
    const float g = (GP && p.pg) ? lds_read_f32(sta + 768) : p.gp_static;
    const ProbBlock pb = GP ? prob_block_static(bm, p.c, mc, g) : prob_block(bm, p.c, mc);
    const float sw = pb.Sd * w, swD = sw * Di;  // A = r * Sd * w
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      ah[rr] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rr], p.c, -pb.mb));  // P / Sd
      ds[rr] = ah[rr] * __builtin_fmaf(sw, dp[rr], -swD);
    }
    const uint32_t c0 = e2m1_codes8(ah), c1 = e2m1_codes8(ah + 8);
    if (GP) {
      // P-hat as the forward used it (rounded to bf16), then the normalisation
      e2m1_decode8(c0, pb.S, ah);
      e2m1_decode8(c1, pb.S, ah + 8);
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const float b = bf16lo(f32_to_bf16_rne(ah[rr]));
        ah[rr] = (p.pv_fp8 ? round_e4m3(b) : b) * w;
      }
    } else {
      e2m1_decode8(c0, pb.S * w, ah);
      e2m1_decode8(c1, pb.S * w, ah + 8);
    }
  } else {
    const float wD = w * Di;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      ah[rr] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rr], p.c, -mc));
      ds[rr] = ah[rr] * __builtin_fmaf(w, dp[rr], -wD);
      ah[rr] *= w;
    }
  }
  // Move A-hat and dS to one key per lane: D[query][key] = sum_k X[query][k] onehot[k][key].
  const uint32_t oh = lds0 + kLdsOneHot + 16 * (threadIdx.x & 63);
  const bf16x8 one0 = as_bf16x8(lds_read16(oh)), one1 = as_bf16x8(lds_read16(oh + 1024));
  f32x16 ta = f32x16{}, ts = f32x16{};
  ta = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pack8_cvt(ah), one0, ta, 0, 0, 0);
  ta = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pack8_cvt(ah + 8), one1, ta, 0, 0, 0);
  ts = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pack8_cvt(ds), one0, ts, 0, 0, 0);
  ts = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pack8_cvt(ds + 8), one1, ts, 0, 0, 0);
  // ta/ts register 8*s2 + kk of lane (key j, half h) holds query 16*s2 + 8*h + kk of the wave's 32.
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    float fa[8], fs[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      fa[kk] = ta[8 * s2 + kk];
      fs[kk] = ts[8 * s2 + kk];
      if (SQ) csum += fs[kk];  // smooth-Q: this key's dS summed over the queries (the dK MFMA's values)
    }
    const bf16x8 ba = pack8_exact(fa), bs = pack8_exact(fs);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      // query groups a = 0, 1: rows +0 / +4 (1024 bytes) with column-pair bit 4 flipped
      const uint32_t a0 = ta0 ^ (dt << 6), a1 = ta0 ^ ((dt << 6) | 16);
      const uint32_t s2o = s2 * 4096;
      const uint2 o0 = ds_read_tr16_at(a0 + kO + s2o), o1 = ds_read_tr16_at(a1 + kO + s2o + 1024);
      const uint2 q0 = ds_read_tr16_at(a0 + kQ + s2o), q1 = ds_read_tr16_at(a1 + kQ + s2o + 1024);
      dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(u32x4{o0.x, o0.y, o1.x, o1.y}), ba, dv[dt], 0, 0, 0);
      dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(u32x4{q0.x, q0.y, q1.x, q1.y}), bs, dk[dt], 0, 0, 0);
    }
  }
}

template <bool SPARSE, bool GP, bool SQ>
__global__ __launch_bounds__(kDkdvThreads, 1) void bwd_dkdv_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(256))) uint8_t lds[kDkdvLds];
  const uint32_t lds0 = lds_addr(lds);
  // A whole unit, or piece `piece` (>= 0) of a split one.
  int64_t vid, piece = -1;
  if ((int64_t)blockIdx.x < p.full_blocks) {
    vid = xcd_work_id(blockIdx.x, p.per_xcd, p.nfull);
    if (vid < 0) return;
  } else {
    piece = (int64_t)blockIdx.x - p.full_blocks;
    vid = p.nfull + piece / p.split;
  }
  const int64_t bh = vid / p.Ck;
  const int64_t kc = vid % p.Ck;
  const int64_t bb = bh / p.heads, hh = bh % p.heads;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 31, hf = lane >> 5;
  const int kg = wave & 3, qh = wave >> 2;
  const int64_t nqt = (p.lq + kQT - 1) / kQT;
  int64_t qt0 = p.causal ? (kc * kChunk) / kQT : 0;

  // Cube-sparse: the query cubes that selected this key cube, ascending, with the key cube's
  // position in each one's list (packed qc | slot << 16), compacted by wave 0.
  int32_t *lds_list = (int32_t *)(lds + kLdsList);
  int64_t ntiles = nqt - qt0;
  if (!SPARSE && piece >= 0) {
    // piece j of `split`: query tiles [ntiles * j / split, ntiles * (j + 1) / split)
    const int64_t j = piece % p.split, lo = ntiles * j / p.split, hi = ntiles * (j + 1) / p.split;
    qt0 += lo;
    ntiles = hi - lo;
  }
  if constexpr (SPARSE) {
    if (wave == 0) {
      const int16_t *col = p.slot_t + (bh * p.Ck + kc) * p.Cq;
      int cnt = 0;
      for (int64_t base = 0; base < p.Cq; base += 64) {
        const int64_t qcube = base + lane;
        const int sl = qcube < p.Cq ? (int)col[qcube] : -1;
        const uint64_t m = __builtin_amdgcn_ballot_w64(sl >= 0);
        const int pos = cnt + (int)__builtin_popcountll(m & ((1ull << lane) - 1ull));
        if (sl >= 0) lds_list[pos] = (int32_t)qcube | (sl << 16);
        cnt += (int)__builtin_popcountll(m);
      }
      if (lane == 0) lds_list[kMaxCubes] = cnt;
    }
    __syncthreads();
    ntiles = 2 * (int64_t)lds_list[kMaxCubes];
  }
  // Tile t: query tile and chunk-max row.
  auto tile_qb = [&](int64_t t) -> int64_t {
    return SPARSE ? 2 * (int64_t)(lds_list[t >> 1] & 0xffff) + (t & 1) : qt0 + t;
  };
  auto tile_cm = [&](int64_t t) -> int64_t {
    return SPARSE ? bh * p.nsel + (lds_list[t >> 1] >> 16) : bh * p.Ck + kc;
  };

  DkdvLane ln;
  {
    const int krow = kg * 32 + perm_row(n), swk = sw_kq(krow);
    ln.k_off = krow * 256 + 16 * ((hf ^ swk) & 1) + 32 * (swk >> 1);
    ln.qloc = 32 * qh + pi_q(n);
    const int swq = sw_qr(ln.qloc);
    ln.r_off = ln.qloc * 256 + 16 * ((hf ^ swq) & 1) + 32 * (swq >> 1);
    // Transposed read (ds_read_b64_tr_b16): in each 16-lane group, lane 4e+j supplies 4 elements
    // of row (base + e) and lane i receives element i%4 from lanes 4e + i/4, e = 0..3.  Lane
    // (group g = (lane/16)%2, h = lane/32, e = (lane/4)%4, j = lane%4) reads tile row
    // 32*qh + 16*s2 + 8*h + 4*a + e, d columns 32*dt + 16*g + 4*j .. +3.  That row's swizzle is
    // 4*e + 2*h + a, so the 16-byte column is 4*(dt^e) + ((2*g + j/2) ^ (2*h + a)).
    const int e = (lane >> 2) & 3, j = lane & 3, g = (lane >> 4) & 1;
    const int lo = (2 * g + (j >> 1)) ^ (2 * hf);
    ln.tr_off = (32 * qh + 8 * hf + e) * 256 + 64 * e + 16 * lo + 8 * (j & 1);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = (i * 8 + wave) * 4 + (lane >> 4);
      const int jc = (lane & 15) ^ sw_qr(r);
      ln.o_row[i] = r;
      ln.q_voff[i] = (uint32_t)(r * 256 + jc * 16);
      ln.o_voff[i] = (uint32_t)(r * p.sdo.l * 2 + jc * 16);
    }
  }
  ln.key_base = (int)(kc * kChunk) + kg * 32 + 16 * hf;

  // This chunk's K-hat and V-hat rows, the one-hot operands, then the first tile.
  {
    const u32x4 *ks = p.kq + (bh * p.Ck + kc) * (kChunk * kD / 8);
    const u32x4 *vs = p.vq + (bh * p.Ck + kc) * (kChunk * kD / 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (i * 8 + wave) * 4 + (lane >> 4);
      const uint32_t off = (uint32_t)(r * 256 + (((lane & 15) ^ sw_kq(r)) << 4));
      load_lds16_s(ks, off, lds + (i * 8 + wave) * 1024);
      load_lds16_s(vs, off, lds + 32768 + (i * 8 + wave) * 1024);
    }
    if (wave == 0) {
      *(bf16x8 *)(lds + kLdsOneHot + lane * 16) = onehot_b(lane, 0);
      *(bf16x8 *)(lds + kLdsOneHot + 1024 + lane * 16) = onehot_b(lane, 1);
    }
    if (SQ && wave == 1 && lane < 32)
      *(f32x4 *)(lds + kLdsDelta + lane * 16) = *(const f32x4 *)(p.delta + (bh * p.Ck + kc) * kChunk + 4 * lane);
  }
  if (ntiles > 0) dkdv_stage_tile(p, ln, bh, bb, hh, tile_cm(0), tile_qb(0), lds, 0, wave, lane);

  const bool tail = (kc + 1) * kChunk > p.lk;
  f32x16 dk[4], dv[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    dk[dt] = f32x16{};
    dv[dt] = f32x16{};
  }
  float csum = 0.0f;

  // Tiles in pairs (buffer 0, then buffer 1), then an odd last tile in buffer 0.
  int64_t t = 0;
  for (; t + 1 < ntiles; t += 2) {
    AQ_WAIT_VMCNT(0);  // this wave's copies of tile t
    __syncthreads();   // everyone's copies landed; buffer 1 is free
    dkdv_stage_tile(p, ln, bh, bb, hh, tile_cm(t + 1), tile_qb(t + 1), lds, 1, wave, lane);
    dkdv_tile<0, GP, SQ>(p, lds0, ln, tile_qb(t), tail, dk, dv, csum);
    AQ_WAIT_VMCNT(0);
    __syncthreads();  // buffer 0 is free
    if (t + 2 < ntiles) dkdv_stage_tile(p, ln, bh, bb, hh, tile_cm(t + 2), tile_qb(t + 2), lds, 0, wave, lane);
    dkdv_tile<1, GP, SQ>(p, lds0, ln, tile_qb(t + 1), tail, dk, dv, csum);
  }
  if (t < ntiles) {
    AQ_WAIT_VMCNT(0);
    __syncthreads();
    dkdv_tile<0, GP, SQ>(p, lds0, ln, tile_qb(t), tail, dk, dv, csum);
  }

  // The two waves of a key group add their partial sums: wave qh = 0 finishes dK, qh = 1 dV.
  // Partner partials go through LDS as [key group][tensor][dt][register/4][lane] float4.
  AQ_WAIT_VMCNT(0);  // no copy may still be landing in the LDS reused below
  __syncthreads();
  {
    f32x16 *give = qh == 0 ? dv : dk;
    float *dst = (float *)(lds + (kg * 2 + (qh == 0 ? 1 : 0)) * 16384);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *(f32x4 *)(dst + ((dt * 4 + a) * 64 + lane) * 4) =
            f32x4{give[dt][4 * a], give[dt][4 * a + 1], give[dt][4 * a + 2], give[dt][4 * a + 3]};
  }
  if (SQ) {
    // smooth-Q: this key's dS summed over all queries (both lane halves, then both query waves)
    csum += __shfl_xor(csum, 32, 64);
    if (qh == 1 && hf == 0) ((float *)(lds + kLdsStat))[kg * 32 + n] = csum;
  }
  __syncthreads();
  const int64_t key = kc * kChunk + kg * 32 + n;
  f32x16 *mine = qh == 0 ? dk : dv;
  if (SQ && qh == 0) {
    // dK_j += (sum_i dS_ij) * mean: the key gradients see the restored query q-hat + mean
    const float cs = csum + ((const float *)(lds + kLdsStat))[kg * 32 + n];
    const float *qm = p.qmean + bh * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const f32x4 m = *(const f32x4 *)(qm + 32 * dt + 8 * a + 4 * hf);
#pragma unroll
        for (int i = 0; i < 4; ++i) dk[dt][4 * a + i] = __builtin_fmaf(cs, m[i], dk[dt][4 * a + i]);
      }
  }
  const float *src = (const float *)(lds + (kg * 2 + (qh == 0 ? 0 : 1)) * 16384);
  if (!SPARSE && piece >= 0) {
    // a piece: its fp32 sums (before the dK scale) for dkdv_reduce_kernel
    float *dst = p.part + (piece * 2 + qh) * (kChunk * kD) + (kg * 32 + n) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const f32x4 o = *(const f32x4 *)(src + ((dt * 4 + a) * 64 + lane) * 4);
        *(f32x4 *)(dst + 32 * dt + 8 * a + 4 * hf) =
            f32x4{mine[dt][4 * a] + o[0], mine[dt][4 * a + 1] + o[1], mine[dt][4 * a + 2] + o[2], mine[dt][4 * a + 3] + o[3]};
      }
    return;
  }
  const float mul = qh == 0 ? p.scale : 1.0f;
  if (key >= p.lk) return;
  uint16_t *out = qh == 0 ? p.dk + bb * p.sdk.b + hh * p.sdk.h + key * p.sdk.l
                          : p.dv + bb * p.sdv.b + hh * p.sdv.h + key * p.sdv.l;
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const f32x4 o = *(const f32x4 *)(src + ((dt * 4 + a) * 64 + lane) * 4);
      const int d0 = 32 * dt + 8 * a + 4 * hf;
      *(bf16x4 *)(out + d0) = bf16x4{(__bf16)((mine[dt][4 * a] + o[0]) * mul), (__bf16)((mine[dt][4 * a + 1] + o[1]) * mul),
                                     (__bf16)((mine[dt][4 * a + 2] + o[2]) * mul), (__bf16)((mine[dt][4 * a + 3] + o[3]) * mul)};
    }
}

// ---------------------------------------------------------------------------------------------
// Ping-pong dK/dV (dense calls without a global P scale or smooth-Q)
// ---------------------------------------------------------------------------------------------
// bwd_dkdv_kernel's work and arithmetic (same units, pieces, operands and per-element operations),
// scheduled as the forward's ping-pong kernels are.  Wave group g (waves 4g .. 4g+3, one per SIMD,
// key group kg = wave % 4) owns query half g of every 64-query tile, and the two groups run one
// phase apart, each alternating
//   matrix phase M(t): the one-hot transposition of tile t-1's dS, dK/dV += the products of tile
//                      t-1 (transposed Q-hat and dO reads against the key-major A-hat and dS; the
//                      dV MFMAs first, while dS's transposition completes), then S^T and dP^T of
//                      tile t;
//   vector phase V(t): masks, P-hat and dS of tile t, A-hat's one-hot transposition;
// so on every SIMD one group's MFMAs run beside the other group's vector work, with one workgroup
// barrier per phase (group 0 runs M(0) V(0) M(1) ... V(T-1) M(T) and idles last, group 1 idles
// first; M(0) adds zero operands, M(T)'s S^T and dP^T are dropped).  A group reads only its own 32
// rows of a tile buffer, so the halves are independent: the group in its matrix phase copies the
// other group's next tile half (16 KiB of Q-hat and dO rows and its three statistics) among its
// MFMAs, into the half that group finished reading in its last matrix phase, and waits for the
// copies before the phase's closing barrier.
// LDS (bytes):
//   [0, 64K)         K-hat and V-hat rows of the chunk (as in bwd_dkdv_kernel)
//   [64K, 128K)      two tile buffers, Q-hat rows [64][256 B] then dO rows [64][256 B], sw_qr
//   [128K, +3K)      statistics [buffer][group][chunk max, lse, D][64 floats] (entries 32..63 of
//                    a group repeat 0..31)
//   [128K+3K, +2K)   the two one-hot B operands
constexpr int kPPStat = 131072;
constexpr int kPPOneHot = kPPStat + 2 * 1536;
constexpr int kDkdvPPLds = kPPOneHot + 2048;
constexpr int kPPList = kDkdvPPLds;  // cube-sparse: the list of (query cube, position), int32

// SPARSE: the cube-sparse mode of bwd_dkdv_kernel (the query cubes that selected this key cube,
// two tiles each, listed by wave 0 in LDS).
template <bool SPARSE>
__global__ __launch_bounds__(kDkdvThreads, 1) void bwd_dkdv_pp_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(256))) uint8_t lds[kDkdvPPLds + (SPARSE ? 4 * (kMaxCubes + 1) : 0)];
  const uint32_t lds0 = lds_addr(lds);
  int64_t vid, piece = -1;
  if ((int64_t)blockIdx.x < p.full_blocks) {
    vid = xcd_work_id(blockIdx.x, p.per_xcd, p.nfull);
    if (vid < 0) return;
  } else {
    piece = (int64_t)blockIdx.x - p.full_blocks;
    vid = p.nfull + piece / p.split;
  }
  const int64_t bh = vid / p.Ck;
  const int64_t kc = vid % p.Ck;
  const int64_t bb = bh / p.heads, hh = bh % p.heads;
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 31, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave & 3, grp = wave >> 2, other = grp ^ 1;
  const int64_t nqt = (p.lq + kQT - 1) / kQT;
  int64_t qt0 = p.causal ? (kc * kChunk) / kQT : 0;
  int64_t ntiles = nqt - qt0;
  if (!SPARSE && piece >= 0) {
    const int64_t j = piece % p.split, lo = ntiles * j / p.split, hi = ntiles * (j + 1) / p.split;
    qt0 += lo;
    ntiles = hi - lo;
  }
  int32_t *lds_list = (int32_t *)(lds + kPPList);
  if constexpr (SPARSE) {
    if (wave == 0) {
      const int16_t *col = p.slot_t + (bh * p.Ck + kc) * p.Cq;
      int cnt = 0;
      for (int64_t base = 0; base < p.Cq; base += 64) {
        const int64_t qcube = base + lane;
        const int sl = qcube < p.Cq ? (int)col[qcube] : -1;
        const uint64_t m = __builtin_amdgcn_ballot_w64(sl >= 0);
        const int pos = cnt + (int)__builtin_popcountll(m & ((1ull << lane) - 1ull));
        if (sl >= 0) lds_list[pos] = (int32_t)qcube | (sl << 16);
        cnt += (int)__builtin_popcountll(m);
      }
      if (lane == 0) lds_list[kMaxCubes] = cnt;
    }
    __syncthreads();
    ntiles = 2 * (int64_t)lds_list[kMaxCubes];
  }
  const int T = (int)ntiles;
  // Tile t: its query tile, and the row of the chunk maxima its queries use.
  auto tile_qb = [&](int t) -> int64_t {
    if constexpr (SPARSE) return 2 * (int64_t)(__builtin_amdgcn_readfirstlane(lds_list[t >> 1]) & 0xffff) + (t & 1);
    return qt0 + t;
  };
  auto tile_cm = [&](int t) -> int64_t {
    if constexpr (SPARSE) return bh * p.nsel + (__builtin_amdgcn_readfirstlane(lds_list[t >> 1]) >> 16);
    return bh * p.Ck + kc;
  };

  DkdvLane ln;
  {
    const int krow = kg * 32 + perm_row(n), swk = sw_kq(krow);
    ln.k_off = krow * 256 + 16 * ((hf ^ swk) & 1) + 32 * (swk >> 1);
    ln.qloc = 32 * grp + pi_q(n);
    const int swq = sw_qr(ln.qloc);
    ln.r_off = ln.qloc * 256 + 16 * ((hf ^ swq) & 1) + 32 * (swq >> 1);
    const int e = (lane >> 2) & 3, j = lane & 3, g = (lane >> 4) & 1;
    const int lo = (2 * g + (j >> 1)) ^ (2 * hf);
    ln.tr_off = (32 * grp + 8 * hf + e) * 256 + 64 * e + 16 * lo + 8 * (j & 1);
  }
  ln.key_base = (int)(kc * kChunk) + kg * 32 + 16 * hf;
  // Copy `what` (0..3: Q-hat / dO rows of step i = what/2; 4: a statistic) of the other group's
  // half of tile t into buffer t%2: this wave's rows 32*other + 4*(kg + 4i) + lane/16, and
  // statistic min(kg, 2) (wave 3 rewrites D with the same values).  dO rows and statistics past
  // lq repeat the last valid one.  Offsets are formed here, not held across the loop.
  const int stat_k = kg < 2 ? kg : 2;
  const float *stat_src0 = stat_k == 0 ? p.cmax + (bh * p.Ck + kc) * p.lq : (stat_k == 1 ? p.lse : p.dvec) + bh * p.lq;
  auto copy_piece = [&](int t, int what) {
    const int64_t qb = tile_qb(t);
    const int rem = (int)(p.lq - 1 - qb * kQT);
    const uint32_t rq = lds0 + kLdsR + (uint32_t)(t & 1) * 32768;
    if (what < 4) {
      const int i = what >> 1;
      const int r = 32 * other + 4 * (kg + 4 * i) + (lane >> 4);
      const uint32_t jc16 = (uint32_t)(((lane & 15) ^ sw_qr(r)) << 4);
      const uint32_t dst = rq + (uint32_t)(8 * other + kg + 4 * i) * 1024;
      if ((what & 1) == 0) {
        load_lds16_sa_free(p.qq + (bh * p.Cq * kChunk + qb * kQT) * (kD / 8), (uint32_t)r * 256u + jc16, dst);
      } else {
        const int rr = r < rem ? r : rem;
        load_lds16_sa_free(p.d_o + bb * p.sdo.b + hh * p.sdo.h + qb * kQT * p.sdo.l,
                           (uint32_t)(rr * p.sdo.l * 2) + jc16, dst + 16384);
      }
    } else {
      const int q = 32 * other + (lane & 31);
      const int qe = q < rem ? q : rem;
      const float *stat_src = SPARSE && stat_k == 0 ? p.cmax + tile_cm(t) * p.lq : stat_src0;
      load_lds4_sa_free(stat_src + qb * kQT, (uint32_t)qe * 4u,
                        lds0 + kPPStat + (uint32_t)(t & 1) * 1536 + other * 768 + stat_k * 256);
    }
  };

  // This chunk's K-hat and V-hat rows, the one-hot operands, and group 0's half of tile 0.
  {
    const u32x4 *ks = p.kq + (bh * p.Ck + kc) * (kChunk * kD / 8);
    const u32x4 *vs = p.vq + (bh * p.Ck + kc) * (kChunk * kD / 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (i * 8 + wave) * 4 + (lane >> 4);
      const uint32_t off = (uint32_t)(r * 256 + (((lane & 15) ^ sw_kq(r)) << 4));
      load_lds16_s(ks, off, lds + (i * 8 + wave) * 1024);
      load_lds16_s(vs, off, lds + 32768 + (i * 8 + wave) * 1024);
    }
    if (wave == 0) {
      *(bf16x8 *)(lds + kPPOneHot + lane * 16) = onehot_b(lane, 0);
      *(bf16x8 *)(lds + kPPOneHot + 1024 + lane * 16) = onehot_b(lane, 1);
    }
    if (T > 0 && grp == 1) {
#pragma unroll
      for (int w = 0; w < 5; ++w) copy_piece(0, w);
    }
  }
  AQ_WAIT_VMCNT(0);
  __syncthreads();
  // The wave's K-hat A operands stay in registers for the whole loop.
  bf16x8 kfr[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) kfr[u] = as_bf16x8(lds_read16((lds0 + ln.k_off) ^ (32 * u)));

  const bool tail = (kc + 1) * kChunk > p.lk;
  f32x16 dk[4], dv[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    dk[dt] = f32x16{};
    dv[dt] = f32x16{};
  }
  f32x16 s = f32x16{}, dp = f32x16{};
  // The last vector phase's A-hat, key-major, and dS, still query-major (packed to bf16; the
  // matrix phase moves it to one key per lane); zero before the first.
  bf16x8 ba[2], pd[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    ba[h] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
    pd[h] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  }

  // M(t) as above (t = 0: zero operands against tile 0; t = T: S^T and dP^T of tile T-1 again,
  // dropped); copies of the other group's tile t+grp among the first MFMAs.  Operands are read
  // two dK/dV steps or one S^T / dP^T step (two MFMAs) ahead of their use.
  auto mphase = [&](int t) {
    const int t2 = t >= 1 ? t - 1 : 0, t1 = t < T ? t : T - 1;
    uint32_t ta0 = lds0 + kLdsR + (uint32_t)(t2 & 1) * 32768 + ln.tr_off;
    uint32_t va = lds0 + 32768 + ln.k_off, ra = lds0 + kLdsR + (uint32_t)(t1 & 1) * 32768 + ln.r_off;
    AQ_OPAQUE(va);  // per-step addresses formed in the phase, not held across the loop
    const int tc = t + grp < T ? t + grp : T - 1;  // past the last tile: tile T-1 again (same bytes)
    u32x4 op[3];                // one dK/dV A operand (two transposed reads), by step % 3
    u32x4 bq[2], av[2], bo[2];  // S^T / dP^T operands, by step parity
    // dK/dV steps 0..7: dV of (s2, dt) = (g/4, g%4); 8..15: dK of the same
    auto load_m2 = [&](int g, int b) {
      const int s2 = (g >> 2) & 1, dt = g & 3;
      const uint32_t a0 = ta0 ^ (dt << 6), a1 = ta0 ^ ((dt << 6) | 16);
      const uint32_t off = (g < 8 ? 16384u : 0u) + s2 * 4096;
      const uint2 x0 = ds_read_tr16_at(a0 + off), x1 = ds_read_tr16_at(a1 + off + 1024);
      op[b] = u32x4{x0.x, x0.y, x1.x, x1.y};
    };
    auto load_m1 = [&](int u, int b) {
      const uint32_t rt = ra ^ (32 * u);
      bq[b] = lds_read16(rt);
      av[b] = lds_read16(va ^ (32 * u));
      bo[b] = lds_read16(rt + 16384);
    };
    // dS of tile t-1 to one key per lane (exact in bf16): its MFMAs finish during the dV MFMAs
    f32x16 ts = f32x16{};
    {
      const uint32_t oh = lds0 + kPPOneHot + 16 * lane;
      ts = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pd[0], as_bf16x8(lds_read16(oh)), ts, 0, 0, 0);
      ts = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pd[1], as_bf16x8(lds_read16(oh + 1024)), ts, 0, 0, 0);
    }
    bf16x8 bs[2];
    load_m2(0, 0);
    load_m2(1, 1);
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      if (g < 14) load_m2(g + 2, (g + 2) % 3);
      else if (g == 14) load_m1(0, 0);
      const int s2 = (g >> 2) & 1, dt = g & 3;
      if (g < 8) {
        dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(op[g % 3]), ba[s2], dv[dt], 0, 0, 0);
      } else {
        dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(op[g % 3]), bs[s2], dk[dt], 0, 0, 0);
      }
      if (g < 5) copy_piece(tc, g);
      if (g == 5) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float fs[8];
#pragma unroll
          for (int kk = 0; kk < 8; ++kk) fs[kk] = ts[8 * h + kk];
          bs[h] = pack8_exact(fs);
        }
      }
    }
    s = f32x16{};
    dp = f32x16{};
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (u < 7) load_m1(u + 1, (u + 1) & 1);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr[u], as_bf16x8(bq[u & 1]), s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av[u & 1]), as_bf16x8(bo[u & 1]), dp, 0, 0, 0);
    }
    // the one-hot reads and dS's two MFMAs, dK/dV steps 0 and 1's reads; per dK/dV MFMA the
    // reads two steps ahead (the second last: S^T / dP^T step 0's three); per S^T / dP^T step its
    // next step's three reads after its MFMAs (2 + 1)
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < 14) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      else if (i == 14) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (j < 14 && (j & 1) == 0) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      else if (j < 14) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    AQ_OPAQUE(s);
    AQ_OPAQUE(dp);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      AQ_OPAQUE(dk[dt]);
      AQ_OPAQUE(dv[dt]);
    }
  };

  // V(t): P-hat and dS of tile t exactly as bwd_dkdv_kernel forms them; A-hat moved to one key per
  // lane.
  auto vphase = [&](int t) {
    const int64_t qb = tile_qb(t);
    const uint32_t sta = lds0 + kPPStat + (uint32_t)(t & 1) * 1536 + grp * 768 + 4 * pi_q(n);
    const float mc = lds_read_f32(sta), lse2 = lds_read_f32(sta + 256), Di = lds_read_f32(sta + 512);
    const int qrow = (int)(qb * kQT) + ln.qloc;
    const int lq = (int)p.lq;
    if (tail || qrow >= lq || (p.causal && ln.key_base + 15 > qrow)) {
      const int last = qrow >= lq ? -1 : (p.causal && qrow < (int)p.lk - 1 ? qrow : (int)p.lk - 1);
      mask_tail(s, valid_prefix(ln.key_base, last));
    }
    float bm = s[0];
#pragma unroll
    for (int rr = 1; rr < 16; ++rr) bm = fmaxf(bm, s[rr]);
    const float w = __builtin_amdgcn_exp2f(mc - lse2);
    float ah[16], ds[16];
    if (p.quant_p) {
      const ProbBlock pb = prob_block(bm, p.c, mc);
      const float sw = pb.Sd * w, swD = sw * Di;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        ah[rr] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rr], p.c, -pb.mb));
        ds[rr] = ah[rr] * __builtin_fmaf(sw, dp[rr], -swD);
      }
      const uint32_t c0 = e2m1_codes8(ah), c1 = e2m1_codes8(ah + 8);
      e2m1_decode8(c0, pb.S * w, ah);
      e2m1_decode8(c1, pb.S * w, ah + 8);
    } else {
      const float wD = w * Di;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        ah[rr] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rr], p.c, -mc));
        ds[rr] = ah[rr] * __builtin_fmaf(w, dp[rr], -wD);
        ah[rr] *= w;
      }
    }
    const uint32_t oh = lds0 + kPPOneHot + 16 * lane;
    const bf16x8 one0 = as_bf16x8(lds_read16(oh)), one1 = as_bf16x8(lds_read16(oh + 1024));
    pd[0] = pack8_cvt(ds);
    pd[1] = pack8_cvt(ds + 8);
    f32x16 ta = f32x16{};
    ta = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pack8_cvt(ah), one0, ta, 0, 0, 0);
    ta = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pack8_cvt(ah + 8), one1, ta, 0, 0, 0);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      float fa[8];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) fa[kk] = ta[8 * s2 + kk];
      ba[s2] = pack8_exact(fa);
      AQ_OPAQUE(ba[s2]);
      AQ_OPAQUE(pd[s2]);
    }
  };

  if (T > 0) {
    if (grp == 1) __syncthreads();  // group 1 idles in the first phase
    for (int t = 0; t <= T; ++t) {
      __builtin_amdgcn_s_setprio(2);
      mphase(t);
      AQ_WAIT_VMCNT(0);  // this wave's copies for the other group
      __syncthreads();
      if (t < T) {
        __builtin_amdgcn_s_setprio(0);
        vphase(t);
        __syncthreads();
      }
    }
    __builtin_amdgcn_s_setprio(0);
    if (grp == 0) __syncthreads();  // group 0 idles in the last phase
  }

  // The two waves of a key group add their partial sums (as bwd_dkdv_kernel): group 0 finishes
  // dK, group 1 dV.
  AQ_WAIT_VMCNT(0);
  __syncthreads();
  {
    f32x16 *give = grp == 0 ? dv : dk;
    float *dst = (float *)(lds + (kg * 2 + (grp == 0 ? 1 : 0)) * 16384);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *(f32x4 *)(dst + ((dt * 4 + a) * 64 + lane) * 4) =
            f32x4{give[dt][4 * a], give[dt][4 * a + 1], give[dt][4 * a + 2], give[dt][4 * a + 3]};
  }
  __syncthreads();
  const int64_t key = kc * kChunk + kg * 32 + n;
  f32x16 *mine = grp == 0 ? dk : dv;
  const float *src = (const float *)(lds + (kg * 2 + (grp == 0 ? 0 : 1)) * 16384);
  if (piece >= 0) {
    float *dst = p.part + (piece * 2 + grp) * (kChunk * kD) + (kg * 32 + n) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const f32x4 o = *(const f32x4 *)(src + ((dt * 4 + a) * 64 + lane) * 4);
        *(f32x4 *)(dst + 32 * dt + 8 * a + 4 * hf) =
            f32x4{mine[dt][4 * a] + o[0], mine[dt][4 * a + 1] + o[1], mine[dt][4 * a + 2] + o[2], mine[dt][4 * a + 3] + o[3]};
      }
    return;
  }
  const float mul = grp == 0 ? p.scale : 1.0f;
  if (key >= p.lk) return;
  uint16_t *out = grp == 0 ? p.dk + bb * p.sdk.b + hh * p.sdk.h + key * p.sdk.l
                           : p.dv + bb * p.sdv.b + hh * p.sdv.h + key * p.sdv.l;
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const f32x4 o = *(const f32x4 *)(src + ((dt * 4 + a) * 64 + lane) * 4);
      const int d0 = 32 * dt + 8 * a + 4 * hf;
      *(bf16x4 *)(out + d0) = bf16x4{(__bf16)((mine[dt][4 * a] + o[0]) * mul), (__bf16)((mine[dt][4 * a + 1] + o[1]) * mul),
                                     (__bf16)((mine[dt][4 * a + 2] + o[2]) * mul), (__bf16)((mine[dt][4 * a + 3] + o[3]) * mul)};
    }
}

// dK and dV of the split units: the pieces' fp32 sums added in piece order (deterministic), dK
// scaled, rounded to bf16.  One lane per 4 consecutive d of one key of one tensor.
__global__ __launch_bounds__(256) void dkdv_reduce_kernel(BwdParams p, int64_t total) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= total) return;
  const int d4 = (int)(gid & 31), key_local = (int)((gid >> 5) & 127), tensor = (int)((gid >> 12) & 1);
  const int64_t u = gid >> 13;
  const int64_t vid = p.nfull + u;
  const int64_t bh = vid / p.Ck, kc = vid % p.Ck;
  const int64_t key = kc * kChunk + key_local;
  if (key >= p.lk) return;
  const float *src = p.part + (u * p.split * 2 + tensor) * (kChunk * kD) + key_local * kD + 4 * d4;
  f32x4 acc = *(const f32x4 *)src;
  for (int j = 1; j < p.split; ++j) {
    const f32x4 x = *(const f32x4 *)(src + (int64_t)j * 2 * kChunk * kD);
    acc = f32x4{acc[0] + x[0], acc[1] + x[1], acc[2] + x[2], acc[3] + x[3]};
  }
  const float mul = tensor == 0 ? p.scale : 1.0f;
  const int64_t bb = bh / p.heads, hh = bh % p.heads;
  uint16_t *out = tensor == 0 ? p.dk + bb * p.sdk.b + hh * p.sdk.h + key * p.sdk.l
                              : p.dv + bb * p.sdv.b + hh * p.sdv.h + key * p.sdv.l;
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  *(bf16x4 *)(out + 4 * d4) =
      bf16x4{(__bf16)(acc[0] * mul), (__bf16)(acc[1] * mul), (__bf16)(acc[2] * mul), (__bf16)(acc[3] * mul)};
}

}  // namespace

namespace {

// How many of `units` equally long work units to split, and into how many pieces, so that the
// last round of `slots` concurrent workgroups ends sooner: the last `units % slots` units become
// `split` pieces each (2..8, at most max_parts, at most max_pieces pieces in all), taking the
// split with the fewest rounds of pieces per piece length (the smallest on ties).
struct SplitPlan {
  int64_t nfull = 0, pieces = 0;
  int split = 0;
};
SplitPlan plan_split(int64_t units, int64_t slots, int64_t max_parts, int64_t max_pieces) {
  SplitPlan r;
  r.nfull = units;
  const int64_t tail = slots > 0 ? units % slots : 0;
  if (tail == 0) return r;
  int64_t best_num = 1, best_den = 1;  // the tail's length in rounds now: one
  for (int64_t parts = 2; parts <= 8 && parts <= max_parts && tail * parts <= max_pieces; ++parts) {
    const int64_t rounds = (tail * parts + slots - 1) / slots;  // rounds of pieces, each 1/parts long
    if (rounds * best_den < best_num * parts) {
      best_num = rounds;
      best_den = parts;
      r.split = (int)parts;
    }
  }
  if (r.split) {
    r.nfull = units - tail;
    r.pieces = tail * r.split;
  }
  return r;
}

// Compute units of the current device (one dK/dV workgroup each at a time), cached per device.
int cu_count() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// slot_t[bh][kc][qc] = position of key cube kc in query cube qc's selection, or -1: one lane per
// entry, a linear search of the (short) selection row.
__global__ __launch_bounds__(256) void vsa_slot_kernel(const int32_t *__restrict__ sel, int16_t *__restrict__ slot_t,
                                                       int64_t n, int64_t nsel, int64_t total) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= total) return;
  const int64_t qc = gid % n, kc = (gid / n) % n, bh = gid / (n * n);
  const int32_t *row = sel + (bh * n + qc) * nsel;
  int s = -1;
  for (int64_t t = 0; t < nsel; ++t)
    if (row[t] == (int32_t)kc) s = (int)t;
  slot_t[gid] = (int16_t)s;
}

template <bool SQ>
static void launch_dkdv(const BwdParams &p, bool sparse, bool gp, dim3 grid, hipStream_t stream) {
  const char *nm = sparse ? "vsa_bwd_dkdv" : "bwd_dkdv";
  if (!sparse && !gp && !SQ) AQ_LAUNCH(nm, bwd_dkdv_pp_kernel<false>, grid, dim3(kDkdvThreads), 0, stream, p);
  else if (sparse && !gp && !SQ) AQ_LAUNCH(nm, bwd_dkdv_pp_kernel<true>, grid, dim3(kDkdvThreads), 0, stream, p);
  else if (sparse && gp) AQ_LAUNCH(nm, (bwd_dkdv_kernel<true, true, SQ>), grid, dim3(kDkdvThreads), 0, stream, p);
  else if (sparse) AQ_LAUNCH(nm, (bwd_dkdv_kernel<true, false, SQ>), grid, dim3(kDkdvThreads), 0, stream, p);
  else if (gp) AQ_LAUNCH(nm, (bwd_dkdv_kernel<false, true, SQ>), grid, dim3(kDkdvThreads), 0, stream, p);
  else AQ_LAUNCH(nm, (bwd_dkdv_kernel<false, false, SQ>), grid, dim3(kDkdvThreads), 0, stream, p);
}

// Shared by the dense and the cube-sparse backward: operand prepasses, D, dQ, dK/dV.
hipError_t launch_bwd_common(const AttnArgs &a, const BwdArgs &b, const Workspace &w, const int32_t *sel,
                             const int16_t *slot_t, int64_t nsel, hipStream_t stream) {
  uint8_t *ws = (uint8_t *)a.workspace;
  const TileQuant qd_q = (a.flags & kFlagQ) ? kQuantD : kQuantNone;
  const TileQuant qd_k = (a.flags & kFlagK) ? kQuantD : kQuantNone;
  const TileQuant qr_v = (a.flags & kFlagV) ? kQuantRows : kQuantNone;
  hipError_t e;
  // The forward's operands again (same scales and smoothing, recomputed from the same tensors).
  if ((e = launch_variant_prep(a, w, stream))) return e;
  const VariantPtrs vp = variant_ptrs(a, w);
  if ((e = launch_tile_prepass(a.q, a.sq, a.batch, a.heads, a.lq, qd_q, ws + w.qq, nullptr, vp.gq, vp.qmean, stream)))
    return e;
  if ((e = launch_tile_prepass(a.k, a.sk, a.batch, a.heads, a.lk, qd_k, ws + w.kq, nullptr, vp.gk, vp.kmean, stream)))
    return e;
  if ((e = launch_qk_delta(a, w, stream))) return e;
  if ((e = launch_tile_prepass(a.v, a.sv, a.batch, a.heads, a.lk, qr_v, ws + w.vq, nullptr, vp.gv, nullptr, stream,
                               (a.flags & kFlagPvFp8) ? kOutFp8Bf16 : kOutBf16)))
    return e;

  const int64_t bh = (int64_t)a.batch * a.heads;
  const int64_t rows = bh * a.lq;
  AQ_LAUNCH("dvec", dvec_kernel, dim3((unsigned)((rows * 16 + 255) / 256)), dim3(256), 0, stream,
                     (const uint16_t *)b.d_o, b.sdo, (const float *)a.o_hp, (float *)(ws + w.dvec), a.heads, a.lq,
                     rows);
  if ((e = hipGetLastError())) return e;

  BwdParams p{};
  p.qq = (const u32x4 *)(ws + w.qq);
  p.kq = (const u32x4 *)(ws + w.kq);
  p.vq = (const u32x4 *)(ws + w.vq);
  p.d_o = (const uint16_t *)b.d_o;
  p.sdo = b.sdo;
  p.lse = a.lse;
  p.cmax = a.cmax;
  p.dvec = (const float *)(ws + w.dvec);
  p.dq = (uint16_t *)b.dq;
  p.dk = (uint16_t *)b.dk;
  p.dv = (uint16_t *)b.dv;
  p.sdq = b.sdq;
  p.sdk = b.sdk;
  p.sdv = b.sdv;
  p.heads = a.heads;
  p.lq = a.lq;
  p.lk = a.lk;
  p.Cq = (a.lq + kChunk - 1) / kChunk;
  p.Ck = (a.lk + kChunk - 1) / kChunk;
  p.c = (float)((double)a.scale * 1.4426950408889634);
  p.scale = a.scale;
  p.causal = a.causal;
  p.quant_p = (a.flags & 8u) != 0;
  p.sel = sel;
  p.slot_t = slot_t;
  p.nsel = nsel;
  if ((a.flags & kFlagTwoLevelP) && p.quant_p) p.pg = a.cmax + bh * (sel ? nsel : p.Ck) * a.lq;
  p.delta = vp.delta;
  p.qmean = vp.qmean;

  // dQ units (head, 128 queries), two workgroups per CU.  The software-pipelined kernel splits
  // the units of a partly filled last round along their key chunks (list positions) when all
  // units are equally long: non-causal dense calls, and cube-sparse calls (topk cubes each).
  p.nwork = bh * p.Cq;
  p.nfull = p.nwork;
  p.split = 0;
  p.part = (float *)(ws + w.part);
  SplitPlan dq_plan;
  dq_plan.nfull = p.nwork;
  if (!a.causal && !p.delta)  // (the cube-sparse units all walk topk cubes)
    dq_plan = plan_split(p.nwork, 2 * (int64_t)cu_count(), sel ? nsel : p.Ck, (int64_t)(w.part_bytes / kDqPieceBytes));
  p.nfull = dq_plan.nfull;
  p.split = dq_plan.split;
  p.per_xcd = (p.nfull + 7) / 8;
  p.full_blocks = p.per_xcd * 8;
  const dim3 dq_grid((unsigned)(p.full_blocks + dq_plan.pieces));
  if (sel && p.delta) AQ_LAUNCH("vsa_bwd_dq", (bwd_dq_kernel<true, true>), dq_grid, dim3(kDqThreads), 0, stream, p);
  else if (sel) AQ_LAUNCH("vsa_bwd_dq", (bwd_dq_sp_kernel<true>), dq_grid, dim3(kDqsWaves * 64), 0, stream, p);
  else if (p.delta) AQ_LAUNCH("bwd_dq", (bwd_dq_kernel<false, true>), dq_grid, dim3(kDqThreads), 0, stream, p);
  else AQ_LAUNCH("bwd_dq", (bwd_dq_sp_kernel<false>), dq_grid, dim3(kDqsWaves * 64), 0, stream, p);
  if ((e = hipGetLastError())) return e;
  if (dq_plan.pieces > 0) {
    const int64_t total = (p.nwork - p.nfull) * kChunk * (kD / 4);
    AQ_LAUNCH("dq_reduce", dq_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, p, total);
    if ((e = hipGetLastError())) return e;
  }

  // dK/dV units (head, key chunk), one workgroup per CU at a time.  Dense non-causal calls whose
  // last round would leave CUs idle split each of its units into pieces along the query tiles
  // (all units are equally long there), so that round ends sooner.
  p.nwork = bh * p.Ck;
  SplitPlan kv_plan;
  kv_plan.nfull = p.nwork;
  if (!sel && !a.causal)
    kv_plan = plan_split(p.nwork, cu_count(), (a.lq + kQT - 1) / kQT, (int64_t)(w.part_bytes / kDkdvPieceBytes));
  p.nfull = kv_plan.nfull;
  p.split = kv_plan.split;
  const int64_t pieces = kv_plan.pieces;
  p.per_xcd = (p.nfull + 7) / 8;
  p.full_blocks = p.per_xcd * 8;
  const dim3 dkdv_grid((unsigned)(p.full_blocks + pieces));
  const bool gp = p.quant_p && (a.flags & kFlagsPGlobal);
  p.gp_static = (a.flags & kFlagGsfP) ? kPScaleStatic : 1.0f;
  p.pv_fp8 = (a.flags & kFlagPvFp8) != 0;
  if (p.delta) launch_dkdv<true>(p, sel != nullptr, gp, dkdv_grid, stream);
  else launch_dkdv<false>(p, sel != nullptr, gp, dkdv_grid, stream);
  if ((e = hipGetLastError())) return e;
  if (pieces > 0) {
    const int64_t total = (p.nwork - p.nfull) * 2 * kChunk * (kD / 4);
    AQ_LAUNCH("dkdv_reduce", dkdv_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, p,
              total);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd(const AttnArgs &a, const BwdArgs &b, hipStream_t stream) {
  return launch_bwd_common(a, b, workspace_layout(1, a.batch, a.heads, a.lq, a.lk), nullptr, nullptr, 0, stream);
}

hipError_t launch_vsa_bwd(const AttnArgs &a, const BwdArgs &b, const int32_t *sel, int n_cubes, int topk,
                          hipStream_t stream) {
  if (n_cubes > kMaxCubes || a.lq != a.lk || a.lk != (int64_t)n_cubes * kChunk) return hipErrorInvalidValue;
  const Workspace w = workspace_layout(3, a.batch, a.heads, a.lq, a.lk);
  int16_t *slot = (int16_t *)((uint8_t *)a.workspace + w.slot);
  const int64_t total = (int64_t)a.batch * a.heads * n_cubes * n_cubes;
  AQ_LAUNCH("vsa_slot", vsa_slot_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, sel, slot,
                     (int64_t)n_cubes, (int64_t)topk, total);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_bwd_common(a, b, w, sel, slot, topk, stream);
}

}  // namespace aq
