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
  const u32x4 *qt;    // Q-hat tiles  [BH, Cq, 128, 128]
  const u32x4 *dot;   // dO tiles     [BH, Cq, 128, 128]
  const u32x4 *kq;    // K-hat rows   [BH, Ck*128, 128]
  const u32x4 *kt;    // K-hat tiles  [BH, Ck, 128, 128]
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
};

// ---------------------------------------------------------------------------------------------
// dQ: workgroup = (head, 128 queries), 4 waves x 32 queries; loop over 128-key chunks in two
// 64-key halves.  LDS: K-hat rows, V-hat rows (A operands of S^T and dP^T, perm_row order) and the
// K-hat tile (A operand of dQ^T), 96 KiB.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(BwdParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint8_t *lds_k = lds, *lds_v = lds + 32768, *lds_kt = lds + 65536;
  const int64_t vid = xcd_work_id(blockIdx.x, p.per_xcd, p.nwork);
  if (vid < 0) return;
  const int64_t bh = vid / p.Cq;
  const int64_t qc = vid % p.Cq;
  const int64_t bb = bh / p.heads, hh = bh % p.heads;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 31, hf = lane >> 5;
  const int64_t qrow = qc * kChunk + wave * 32 + n;
  const bool qvalid = qrow < p.lq;

  bf16x8 qf[8], of[8];
  {
    const u32x4 *qsrc = p.qq + (bh * p.Cq * kChunk + qc * kChunk + wave * 32 + n) * (kD / 8);
    const uint16_t *osrc = p.d_o + bb * p.sdo.b + hh * p.sdo.h + (qvalid ? qrow : 0) * p.sdo.l;
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
  const int64_t last = !qvalid ? -1 : (p.causal && qrow < p.lk - 1 ? qrow : p.lk - 1);
  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};
  const int krow = perm_row(n);

  int64_t n_iter = p.Ck;
  if (p.causal) {
    const int64_t q_last = qc * kChunk + kChunk - 1;
    n_iter = (q_last < p.lk - 1 ? q_last : p.lk - 1) / kChunk + 1;
  }
  // The next chunk's three tiles stream into registers while the current one is computed.
  u32x4 stg[24];
  auto load_chunk = [&](int64_t ch) {
    const u32x4 *ks = p.kq + (bh * p.Ck + ch) * (kChunk * kD / 8);
    const u32x4 *vs = p.vq + (bh * p.Ck + ch) * (kChunk * kD / 8);
    const u32x4 *ts = p.kt + (bh * p.Ck + ch) * (kChunk * kD / 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int id = i * 256 + tid;
      stg[i] = ks[id];
      stg[8 + i] = vs[id];
      stg[16 + i] = ts[id];
    }
  };
  load_chunk(0);
  for (int64_t ch = 0; ch < n_iter; ++ch) {
    __syncthreads();  // every wave is done reading the previous chunk
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int id = i * 256 + tid, r = id >> 4, j = id & 15;
      *(u32x4 *)(lds_k + kq_off(r, j)) = stg[i];
      *(u32x4 *)(lds_v + kq_off(r, j)) = stg[8 + i];
      *(u32x4 *)(lds_kt + row_off(r, j)) = stg[16 + i];
    }
    __syncthreads();
    if (ch + 1 < n_iter) load_chunk(ch + 1);
    const bool tail = (ch + 1) * kChunk > p.lk;
    const bool diag = p.causal && (ch + 1) * kChunk - 1 > qc * kChunk + wave * 32;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      bf16x8 dsb[2][2];
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const int kt = 2 * kh + k2;
        const int r = 32 * kt + krow;
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const bf16x8 ak = as_bf16x8(*(const u32x4 *)(lds_k + kq_off(r, 2 * t + hf)));
          const bf16x8 av = as_bf16x8(*(const u32x4 *)(lds_v + kq_off(r, 2 * t + hf)));
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qf[t], s, 0, 0, 0);
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, of[t], dp, 0, 0, 0);
        }
        if (tail || diag || !qvalid) {
          const int64_t key0 = ch * kChunk + 32 * kt + 16 * hf;
          mask_tail(s, valid_prefix(key0, last));
        }
        float ds[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const float A = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rr], p.c, -lse2));
          ds[rr] = A * (dp[rr] - Di);
        }
        dsb[k2][0] = pack8_cvt(ds);
        dsb[k2][1] = pack8_cvt(ds + 8);
      }
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            const int kt = 2 * kh + k2;
            const bf16x8 a = as_bf16x8(*(const u32x4 *)(lds_kt + row_off(32 * dt + n, 4 * kt + 2 * hf + j)));
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsb[k2][j], acc[dt], 0, 0, 0);
          }
    }
  }
  if (!qvalid) return;
  uint16_t *op = p.dq + bb * p.sdq.b + hh * p.sdq.h + qrow * p.sdq.l;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d0 = 32 * dt + 8 * a + 4 * hf;
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      *(bf16x4 *)(op + d0) = bf16x4{(__bf16)(acc[dt][4 * a] * p.scale), (__bf16)(acc[dt][4 * a + 1] * p.scale),
                                    (__bf16)(acc[dt][4 * a + 2] * p.scale), (__bf16)(acc[dt][4 * a + 3] * p.scale)};
    }
}

// ---------------------------------------------------------------------------------------------
// dK, dV: workgroup = (head, 128-key chunk), 4 waves x 32 keys, loop over 64-query tiles.
// LDS: per tile Q-hat rows and dO rows [64][256 B] (B operands of S^T and dP^T), Q-hat^T and
// dO^T [128 d][128 B] (A operands of dK^T and dV^T), 64 KiB; plus the chunk's K-hat and V-hat
// rows (A operands of S^T and dP^T), 64 KiB.
// ---------------------------------------------------------------------------------------------
constexpr int kQT = 64;  // queries per tile

// Byte offset of the 8-byte group g (4 queries) of row d in a [128 d][64 q] tile.  The 8-byte
// slots of each 128-byte row are XOR-swizzled by d/2, so the 32 lanes reading the same group of
// 32 consecutive rows (two rows per 256-byte bank window) use 32 distinct slots.
__device__ __forceinline__ int qt_swz(int d) { return (d >> 1) & 15; }
__device__ __forceinline__ int qt_off(int d, int g) { return d * 128 + ((g ^ qt_swz(d)) << 3); }

// Per-lane statistics of one 64-query tile (two 32-query blocks).
struct TileStats {
  float mc[2], lse[2], dv[2];
};

__device__ __forceinline__ void load_stats(const BwdParams &p, int64_t bh, int64_t kc, int64_t qb, int n,
                                           TileStats &st) {
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int64_t qrow = qb * kQT + 32 * nt + n;
    const bool ok = qrow < p.lq;
    st.mc[nt] = ok ? p.cmax[(bh * p.Ck + kc) * p.lq + qrow] : 0.0f;
    st.lse[nt] = ok ? p.lse[bh * p.lq + qrow] : 0.0f;
    st.dv[nt] = ok ? p.dvec[bh * p.lq + qrow] : 0.0f;
  }
}

// One 64-query tile in registers, 16 x 16 bytes per lane: Q-hat rows, dO rows (64 rows x 256 B
// each), then the Q-hat and dO tiles (128 d-rows x 128 B each).
__device__ __forceinline__ void load_tile(const BwdParams &p, int64_t bh, int64_t bb, int64_t hh, int64_t qb,
                                          int tid, u32x4 *stg) {
  const u32x4 *qs = p.qq + (bh * p.Cq * kChunk + qb * kQT) * (kD / 8);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = i * 256 + tid, r = id >> 4, j = id & 15;
    const int64_t qrow = qb * kQT + r;
    stg[i] = qs[id];
    stg[4 + i] = u32x4{0u, 0u, 0u, 0u};
    if (qrow < p.lq) stg[4 + i] = *(const u32x4 *)(p.d_o + bb * p.sdo.b + hh * p.sdo.h + qrow * p.sdo.l + 8 * j);
  }
  const int64_t tc = (qb * kQT) / kChunk, toff = (qb * kQT) % kChunk;
  const uint8_t *qts = (const uint8_t *)(p.qt + (bh * p.Cq + tc) * (kChunk * kD / 8));
  const uint8_t *ots = (const uint8_t *)(p.dot + (bh * p.Cq + tc) * (kChunk * kD / 8));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = i * 256 + tid, d = id >> 3, j = id & 7;
    const int64_t src = (int64_t)d * 256 + toff * 2 + j * 16;
    stg[8 + i] = *(const u32x4 *)(qts + src);
    stg[12 + i] = *(const u32x4 *)(ots + src);
  }
}

__device__ __forceinline__ void store_tile(uint8_t *lds_q, uint8_t *lds_o, uint8_t *lds_qt, uint8_t *lds_ot, int tid,
                                           const u32x4 *stg) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = i * 256 + tid, r = id >> 4, j = id & 15;
    *(u32x4 *)(lds_q + row_off(r, j)) = stg[i];
    *(u32x4 *)(lds_o + row_off(r, j)) = stg[4 + i];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // 16-byte chunk j holds 8-byte groups 2j, 2j+1; under the swizzle they land in chunk
    // j ^ (f/2), with the two halves exchanged when f is odd.
    const int id = i * 256 + tid, d = id >> 3, j = id & 7, f = qt_swz(d);
    const int dst = d * 128 + ((j ^ (f >> 1)) << 4);
    const u32x4 a = stg[8 + i], b = stg[12 + i];
    *(u32x4 *)(lds_qt + dst) = (f & 1) ? u32x4{a.z, a.w, a.x, a.y} : a;
    *(u32x4 *)(lds_ot + dst) = (f & 1) ? u32x4{b.z, b.w, b.x, b.y} : b;
  }
}

__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint8_t *lds_q = lds, *lds_o = lds + 16384, *lds_qt = lds + 32768, *lds_ot = lds + 49152;
  uint8_t *lds_k = lds + 65536, *lds_v = lds + 98304;  // this chunk's K-hat and V-hat rows
  const int64_t vid = xcd_work_id(blockIdx.x, p.per_xcd, p.nwork);
  if (vid < 0) return;
  const int64_t bh = vid / p.Ck;
  const int64_t kc = vid % p.Ck;
  const int64_t bb = bh / p.heads, hh = bh % p.heads;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 31, hf = lane >> 5;
  const int64_t nqt = (p.lq + kQT - 1) / kQT;
  const int64_t qt0 = p.causal ? (kc * kChunk) / kQT : 0;

  // Prefetch the first tile and its statistics before the per-wave set-up.
  TileStats st;
  u32x4 stg[16];
  load_stats(p, bh, kc, qt0, n, st);
  load_tile(p, bh, bb, hh, qt0, tid, stg);

  // This chunk's K-hat and V-hat rows (A operands of S^T and dP^T, read in perm_row order).
  {
    const u32x4 *ks = p.kq + (bh * p.Ck + kc) * (kChunk * kD / 8);
    const u32x4 *vs = p.vq + (bh * p.Ck + kc) * (kChunk * kD / 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int id = i * 256 + tid, r = id >> 4, j = id & 15;
      *(u32x4 *)(lds_k + kq_off(r, j)) = ks[id];
      *(u32x4 *)(lds_v + kq_off(r, j)) = vs[id];
    }
  }
  const int krow = wave * 32 + perm_row(n);
  const bf16x8 one0 = onehot_b(lane, 0), one1 = onehot_b(lane, 1);
  f32x16 dk[4], dv[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    dk[dt] = f32x16{};
    dv[dt] = f32x16{};
  }
  const int64_t key_base = kc * kChunk + wave * 32 + 16 * hf;  // key of register 0 (S^T layout)
  const bool tail = (kc + 1) * kChunk > p.lk;

  for (int64_t qb = qt0; qb < nqt; ++qb) {
    __syncthreads();  // every wave is done reading the previous tile
    store_tile(lds_q, lds_o, lds_qt, lds_ot, tid, stg);
    const TileStats cur = st;
    __syncthreads();
    if (qb + 1 < nqt) {  // the next tile streams in while this one is computed
      load_stats(p, bh, kc, qb + 1, n, st);
      load_tile(p, bh, bb, hh, qb + 1, tid, stg);
    }

#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int64_t qrow = qb * kQT + 32 * nt + n;
      const bool qvalid = qrow < p.lq;
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const bf16x8 ak = as_bf16x8(*(const u32x4 *)(lds_k + kq_off(krow, 2 * t + hf)));
        const bf16x8 bq = as_bf16x8(*(const u32x4 *)(lds_q + row_off(32 * nt + n, 2 * t + hf)));
        const bf16x8 av = as_bf16x8(*(const u32x4 *)(lds_v + kq_off(krow, 2 * t + hf)));
        const bf16x8 bo = as_bf16x8(*(const u32x4 *)(lds_o + row_off(32 * nt + n, 2 * t + hf)));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, bq, s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bo, dp, 0, 0, 0);
      }
      const float mc = cur.mc[nt], lse2 = cur.lse[nt], Di = cur.dv[nt];
      if (tail || !qvalid || (p.causal && key_base + 15 > qrow)) {
        const int64_t last = !qvalid ? -1 : (p.causal && qrow < p.lk - 1 ? qrow : p.lk - 1);
        mask_tail(s, valid_prefix(key_base, last));
      }
      // P exactly as the forward formed it, its fake quantization, and the weights.
      float Ah[16], ds[16];
      float bm = s[0];
#pragma unroll
      for (int rr = 1; rr < 16; ++rr) bm = fmaxf(bm, s[rr]);
      const float w = __builtin_amdgcn_exp2f(mc - lse2);
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        Ah[rr] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rr], p.c, -mc));
        ds[rr] = (Ah[rr] * w) * (dp[rr] - Di);
      }
      if (p.quant_p) {
        const float am = __builtin_amdgcn_exp2f(__builtin_fmaf(bm, p.c, -mc));  // as the forward
        const float S = block_scale_unit(am);
        const float inv = S == 0.0f ? 0.0f : recip_e4m3(S);
        fq_prob_oct(Ah, S, inv);
        fq_prob_oct(Ah + 8, S, inv);
      }
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) Ah[rr] *= w;
      // Move A-hat and dS to one key per lane: D[query][key] = sum_k X[query][k] onehot[k][key].
      f32x16 ta = f32x16{}, ts = f32x16{};
      ta = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pack8_cvt(Ah), one0, ta, 0, 0, 0);
      ta = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pack8_cvt(Ah + 8), one1, ta, 0, 0, 0);
      ts = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pack8_cvt(ds), one0, ts, 0, 0, 0);
      ts = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pack8_cvt(ds + 8), one1, ts, 0, 0, 0);
      // ta/ts register r of lane (key j, half h) holds query 8*(r/4) + 4*h + r%4 of this 32-query
      // block; k-slot (h, jj) of step s2 is register 8*s2 + jj, i.e. queries 16*s2 + 4h + {0..3}
      // and 16*s2 + 8 + 4h + {0..3}.
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        float fa[8], fs[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          fa[jj] = ta[8 * s2 + jj];
          fs[jj] = ts[8 * s2 + jj];
        }
        const bf16x8 ba = pack8_exact(fa), bs = pack8_exact(fs);
        const int g0 = (32 * nt + 16 * s2 + 4 * hf) >> 2;  // 4-query group index
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const int d = 32 * dt + n;
          const uint2 o0 = *(const uint2 *)(lds_ot + qt_off(d, g0));
          const uint2 o1 = *(const uint2 *)(lds_ot + qt_off(d, g0 + 2));
          const uint2 q0 = *(const uint2 *)(lds_qt + qt_off(d, g0));
          const uint2 q1 = *(const uint2 *)(lds_qt + qt_off(d, g0 + 2));
          dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(u32x4{o0.x, o0.y, o1.x, o1.y}), ba, dv[dt], 0, 0, 0);
          dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(u32x4{q0.x, q0.y, q1.x, q1.y}), bs, dk[dt], 0, 0, 0);
        }
      }
    }
  }

  // dK^T / dV^T: lane holds key j = n of the wave's 32 (natural order), rows d.
  const int64_t key = kc * kChunk + wave * 32 + n;
  if (key >= p.lk) return;
  uint16_t *kp = p.dk + bb * p.sdk.b + hh * p.sdk.h + key * p.sdk.l;
  uint16_t *vp = p.dv + bb * p.sdv.b + hh * p.sdv.h + key * p.sdv.l;
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d0 = 32 * dt + 8 * a + 4 * hf;
      *(bf16x4 *)(kp + d0) = bf16x4{(__bf16)(dk[dt][4 * a] * p.scale), (__bf16)(dk[dt][4 * a + 1] * p.scale),
                                    (__bf16)(dk[dt][4 * a + 2] * p.scale), (__bf16)(dk[dt][4 * a + 3] * p.scale)};
      *(bf16x4 *)(vp + d0) = bf16x4{(__bf16)dv[dt][4 * a], (__bf16)dv[dt][4 * a + 1], (__bf16)dv[dt][4 * a + 2],
                                    (__bf16)dv[dt][4 * a + 3]};
    }
}

}  // namespace

hipError_t launch_attn_bwd(const AttnArgs &a, const BwdArgs &b, hipStream_t stream) {
  const Workspace w = workspace_layout(1, a.batch, a.heads, a.lq, a.lk);
  uint8_t *ws = (uint8_t *)a.workspace;
  const TileQuant qd_q = (a.flags & 1u) ? kQuantD : kQuantNone;
  const TileQuant qd_k = (a.flags & 2u) ? kQuantD : kQuantNone;
  const TileQuant qr_v = (a.flags & 4u) ? kQuantRows : kQuantNone;
  hipError_t e;
  if ((e = launch_tile_prepass(a.q, a.sq, a.batch, a.heads, a.lq, qd_q, ws + w.qq, ws + w.qt, stream))) return e;
  if ((e = launch_tile_prepass(a.k, a.sk, a.batch, a.heads, a.lk, qd_k, ws + w.kq, ws + w.kt, stream))) return e;
  if ((e = launch_tile_prepass(a.v, a.sv, a.batch, a.heads, a.lk, qr_v, ws + w.vq, nullptr, stream))) return e;
  if ((e = launch_tile_prepass(b.d_o, b.sdo, a.batch, a.heads, a.lq, kQuantNone, nullptr, ws + w.dot, stream))) return e;

  const int64_t bh = (int64_t)a.batch * a.heads;
  const int64_t rows = bh * a.lq;
  AQ_LAUNCH("dvec", dvec_kernel, dim3((unsigned)((rows * 16 + 255) / 256)), dim3(256), 0, stream,
                     (const uint16_t *)b.d_o, b.sdo, (const float *)a.o_hp, (float *)(ws + w.dvec), a.heads, a.lq,
                     rows);
  if ((e = hipGetLastError())) return e;

  BwdParams p{};
  p.qq = (const u32x4 *)(ws + w.qq);
  p.qt = (const u32x4 *)(ws + w.qt);
  p.dot = (const u32x4 *)(ws + w.dot);
  p.kq = (const u32x4 *)(ws + w.kq);
  p.kt = (const u32x4 *)(ws + w.kt);
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

  // Dynamic LDS above 64 KiB must be allowed per kernel.
  if ((e = hipFuncSetAttribute((const void *)bwd_dq_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, 98304)))
    return e;
  if ((e = hipFuncSetAttribute((const void *)bwd_dkdv_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, 131072)))
    return e;
  p.nwork = bh * p.Cq;
  p.per_xcd = (p.nwork + 7) / 8;
  AQ_LAUNCH("bwd_dq", bwd_dq_kernel, dim3((unsigned)(p.per_xcd * 8)), dim3(256), 98304, stream, p);
  if ((e = hipGetLastError())) return e;

  p.nwork = bh * p.Ck;
  p.per_xcd = (p.nwork + 7) / 8;
  AQ_LAUNCH("bwd_dkdv", bwd_dkdv_kernel, dim3((unsigned)(p.per_xcd * 8)), dim3(256), 131072, stream, p);
  return hipGetLastError();
}

}  // namespace aq
