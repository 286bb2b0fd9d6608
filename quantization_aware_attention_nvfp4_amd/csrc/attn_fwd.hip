// attn_fwd.hip - NVFP4 fake-quantized attention forward on gfx950 (MI355X).
//
// Method ("vsqa-preview-1.3b metadata.json", attention.precision: "NVFP4 fake-quant with BF16
// matmul", quant_p, quant_v, unit global scales; "attn_qat_train" API page: attn_qat_train with
// use_high_prec_o): Q-hat and K-hat are fake-quantized along D, V-hat along keys, and the softmax
// probabilities P along keys, all in 16-element blocks with E4M3 scales and E2M1 values; both
// matmuls run on BF16 MFMA with fp32 accumulation inside an online softmax whose running maximum
// is refreshed once per 128-key chunk.
//
// Kernels:
//   kq_prepass  K-hat  -> workspace kq [B*H, C*128, 128] bf16 (row-major, zero padded keys)
//   vt_prepass  V-hat  -> workspace vt [B*H, C, 128 d, 128 keys] bf16 (each chunk d-major)
//   attn_fwd    one workgroup per (head, tile of 32*WAVES queries); each wave owns 32 queries.
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
#include "aq_device.hpp"
#include "launch.hpp"

namespace aq {
namespace {

constexpr int kD = kHeadDim;

// ------------------------------------------------------------------------------------------
// Prepass kernels
// ------------------------------------------------------------------------------------------

// K-hat: one lane per 8 d-values of a key row; lanes 2i, 2i+1 hold one 16-element block.
__global__ __launch_bounds__(256) void kq_prepass(const uint16_t *__restrict__ k, Strides sk,
                                                  u32x4 *__restrict__ kq, int heads, int64_t lk,
                                                  int64_t lk_pad, int64_t total16, bool quant) {
  for (int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x; id < total16;
       id += (int64_t)gridDim.x * 256) {
    const int part = (int)(id & 15);             // which 8-value group of the row
    const int64_t row = (id >> 4) % lk_pad;      // key
    const int64_t bh = (id >> 4) / lk_pad;
    const int64_t b = bh / heads, h = bh % heads;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < lk) v = *(const u32x4 *)(k + b * sk.b + h * sk.h + row * sk.l + part * 8);
    if (quant) {
      float f[8] = {bf16lo(v.x), bf16hi(v.x), bf16lo(v.y), bf16hi(v.y),
                    bf16lo(v.z), bf16hi(v.z), bf16lo(v.w), bf16hi(v.w)};
      float am = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) am = fmaxf(am, __builtin_fabsf(f[i]));
      am = fmaxf(am, xor1(am));
      const float S = block_scale_unit(am);
      const float inv = S == 0.0f ? 0.0f : recip_e4m3(S);
      v.x = pack_exact_bf16(fq_unit(f[0], S, inv), fq_unit(f[1], S, inv));
      v.y = pack_exact_bf16(fq_unit(f[2], S, inv), fq_unit(f[3], S, inv));
      v.z = pack_exact_bf16(fq_unit(f[4], S, inv), fq_unit(f[5], S, inv));
      v.w = pack_exact_bf16(fq_unit(f[6], S, inv), fq_unit(f[7], S, inv));
    }
    kq[id] = v;
  }
}

// V-hat, transposed per chunk: one workgroup per (head, 128-key chunk).  The chunk is staged in
// LDS as [key][d]; lane (d, half) quantizes the four 16-key blocks of column d in its half of the
// chunk and writes them as 32 contiguous bytes of row d of the transposed tile.
__global__ __launch_bounds__(256) void vt_prepass(const uint16_t *__restrict__ v, Strides sv,
                                                  uint16_t *__restrict__ vt, int heads, int64_t lk,
                                                  int64_t nchunks, bool quant) {
  __shared__ uint16_t tile[kChunk][kD];
  const int64_t bh = blockIdx.x / nchunks;
  const int64_t c = blockIdx.x % nchunks;
  const int64_t b = bh / heads, h = bh % heads;
  const uint16_t *src = v + b * sv.b + h * sv.h;
  for (int i = threadIdx.x; i < kChunk * kD / 8; i += 256) {
    const int row = i / (kD / 8), part = i % (kD / 8);
    const int64_t key = c * kChunk + row;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (key < lk) x = *(const u32x4 *)(src + key * sv.l + part * 8);
    *(u32x4 *)&tile[row][part * 8] = x;
  }
  __syncthreads();
  const int d = threadIdx.x & (kD - 1);
  const int half = threadIdx.x >> 7;
  uint16_t *dst = vt + ((bh * nchunks + c) * kD + d) * kChunk;
  for (int blk = 0; blk < 4; ++blk) {
    const int k0 = half * 64 + blk * 16;
    float f[16];
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      f[i] = bf16lo(tile[k0 + i][d]);
      am = fmaxf(am, __builtin_fabsf(f[i]));
    }
    uint32_t w[8];
    if (quant) {
      const float S = block_scale_unit(am);
      const float inv = S == 0.0f ? 0.0f : recip_e4m3(S);
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = pack_exact_bf16(fq_unit(f[2 * i], S, inv), fq_unit(f[2 * i + 1], S, inv));
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = pack_exact_bf16(f[2 * i], f[2 * i + 1]);
    }
    *(u32x4 *)(dst + k0) = u32x4{w[0], w[1], w[2], w[3]};
    *(u32x4 *)(dst + k0 + 8) = u32x4{w[4], w[5], w[6], w[7]};
  }
}

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
  bool causal, quant_q, quant_p;
};

// Swizzled byte offset of 16-byte column j of row r in a 256-byte-row LDS tile.
__device__ __forceinline__ int kq_off(int r, int j) { return r * 256 + ((j ^ ((r & 3) | ((r >> 2) & 4))) << 4); }
__device__ __forceinline__ int vt_off(int r, int j) { return r * 256 + ((j ^ (r & 7)) << 4); }

// Accumulator register r of lane half h holds row 8*(r/4) + 4*h + r%4 of a 32x32 tile.
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

template <int WAVES, bool TRAIN>
__global__ __launch_bounds__(WAVES * 64) void attn_fwd_kernel(FwdParams p) {
  constexpr int BM = 32 * WAVES;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kChunk * 256];
  uint8_t *lds_k = lds;
  uint8_t *lds_v = lds + kChunk * 256;

  // XCD-aware tile order: workgroup i runs on XCD i % 8; give each XCD a contiguous range of
  // (head, query-tile) ids so the workgroups sharing a head's K/V share that XCD's L2.
  const int64_t bid = blockIdx.x;
  const int64_t vid = (bid & 7) * p.per_xcd + (bid >> 3);
  if (vid >= p.nblocks) return;
  const int64_t bh = vid / p.qtiles;
  const int qt = (int)(vid % p.qtiles);
  const int64_t bb = bh / p.heads, hh = bh % p.heads;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;   // the lane's query within the wave
  const int hf = lane >> 5;  // lane half
  const int64_t qrow = (int64_t)qt * BM + wave * 32 + n;
  const bool qvalid = qrow < p.lq;

  // ---- Q-hat fragment: B operand of S^T, d = 16t + 8hf + (0..7) -------------------------
  bf16x8 qf[8];
  {
    const uint16_t *qp = p.q + bb * p.sq.b + hh * p.sq.h + (qvalid ? qrow : 0) * p.sq.l;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (qvalid) v = *(const u32x4 *)(qp + 16 * t + 8 * hf);
      if (p.quant_q) {
        float f[8] = {bf16lo(v.x), bf16hi(v.x), bf16lo(v.y), bf16hi(v.y),
                      bf16lo(v.z), bf16hi(v.z), bf16lo(v.w), bf16hi(v.w)};
        float am = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) am = fmaxf(am, __builtin_fabsf(f[i]));
        am = fmaxf(am, xor32(am));
        const float S = block_scale_unit(am);
        const float inv = S == 0.0f ? 0.0f : recip_e4m3(S);
        v.x = pack_exact_bf16(fq_unit(f[0], S, inv), fq_unit(f[1], S, inv));
        v.y = pack_exact_bf16(fq_unit(f[2], S, inv), fq_unit(f[3], S, inv));
        v.z = pack_exact_bf16(fq_unit(f[4], S, inv), fq_unit(f[5], S, inv));
        v.w = pack_exact_bf16(fq_unit(f[6], S, inv), fq_unit(f[7], S, inv));
      }
      qf[t] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x16 acc[4];
  f32x16 acc_hp[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    acc[dt] = f32x16{};
    acc_hp[dt] = f32x16{};
  }
  float m_run = -__builtin_inff();
  float l_run = 0.0f;
  constexpr bool train = TRAIN;

  // The K row this lane feeds as A-operand row i = n: key(i) within a 32-key sub-tile.
  const int krow = 16 * ((n >> 2) & 1) + 4 * (n >> 3) + (n & 3);
  const int64_t q_last = (int64_t)qt * BM + BM - 1;  // last query of the workgroup's tile
  int64_t n_iter = p.nchunks;
  if (p.causal) {
    const int64_t last_needed = (q_last < p.lk - 1 ? q_last : p.lk - 1) / kChunk;
    n_iter = last_needed + 1;
  }

  for (int64_t it = 0; it < n_iter; ++it) {
    const int64_t chunk = p.sel ? (int64_t)p.sel[(bh * (p.lq / kChunk) + (int64_t)qt * BM / kChunk) * p.nchunks + it] : it;
    // ---- stage K-hat and V-hat^T chunk into LDS ----------------------------------------
    __syncthreads();
    {
      const u32x4 *ksrc = p.kq + (bh * p.kchunks + chunk) * (kChunk * kD / 8);
      const u32x4 *vsrc = p.vt + (bh * p.kchunks + chunk) * (kChunk * kD / 8);
      constexpr int kPer = kChunk * kD / 8 / (WAVES * 64);
      u32x4 kv[kPer], vv[kPer];
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        kv[i] = ksrc[i * WAVES * 64 + tid];
        vv[i] = vsrc[i * WAVES * 64 + tid];
      }
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int id = i * WAVES * 64 + tid;
        const int r = id >> 4, j = id & 15;
        *(u32x4 *)(lds_k + kq_off(r, j)) = kv[i];
        *(u32x4 *)(lds_v + vt_off(r, j)) = vv[i];
      }
    }
    __syncthreads();

    // ---- S^T = K-hat Q-hat^T for the 128 keys of the chunk ------------------------------
    f32x16 s[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      s[kt] = f32x16{};
      const int r = 32 * kt + krow;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4 *)(lds_k + kq_off(r, 2 * t + hf)));
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], s[kt], 0, 0, 0);
      }
    }

    // ---- masks: keys past lk (last chunk) and causal -------------------------------------
    const int64_t key0 = chunk * kChunk + 16 * hf;  // key of register 0 in sub-tile 0
    const bool tail = (chunk + 1) * kChunk > p.lk;
    const bool diag = p.causal && (chunk + 1) * kChunk - 1 > (int64_t)qt * BM + wave * 32;
    if (tail || diag) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t key = key0 + 32 * kt + r;
          if (key >= p.lk || (p.causal && key > qrow)) s[kt][r] = -__builtin_inff();
        }
    }

    // ---- running max (refreshed once per chunk) -----------------------------------------
    float cm = -__builtin_inff();
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) cm = fmaxf(cm, s[kt][r]);
    cm = fmaxf(cm, xor32(cm));
    const float m_new = fmaxf(m_run, cm * p.c);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first chunk

    // ---- P, its sum, and P-hat in bf16 B-operands -----------------------------------------
    bf16x8 pq[4][2], ph[4][2];
    float psum = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      float P[16];
      float am = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        P[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][r], p.c, -m_new));
        psum += P[r];
        am = fmaxf(am, P[r]);
      }
      if (train) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          uint32_t w[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) w[i] = f32_to_bf16_rne(P[8 * j + 2 * i]) | (f32_to_bf16_rne(P[8 * j + 2 * i + 1]) << 16);
          ph[kt][j] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
        }
      }
      if (p.quant_p) {
        const float S = block_scale_unit(am);
        const float inv = S == 0.0f ? 0.0f : recip_e4m3(S);
#pragma unroll
        for (int r = 0; r < 16; ++r) P[r] = fq_unit(P[r], S, inv);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          uint32_t w[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) w[i] = pack_exact_bf16(P[8 * j + 2 * i], P[8 * j + 2 * i + 1]);
          pq[kt][j] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
        }
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          uint32_t w[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) w[i] = f32_to_bf16_rne(P[8 * j + 2 * i]) | (f32_to_bf16_rne(P[8 * j + 2 * i + 1]) << 16);
          pq[kt][j] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
        }
      }
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (p.cmax && hf == 0 && qvalid) p.cmax[(bh * p.nchunks + it) * p.lq + qrow] = m_new;

    // ---- O^T = alpha O^T + V-hat^T P-hat^T ------------------------------------------------
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      acc[dt] *= alpha;
      if (train) acc_hp[dt] *= alpha;
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4 *)(lds_v + vt_off(32 * dt + n, 4 * kt + 2 * hf + j)));
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pq[kt][j], acc[dt], 0, 0, 0);
          if (train) acc_hp[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, ph[kt][j], acc_hp[dt], 0, 0, 0);
        }
  }

  // ---- epilogue --------------------------------------------------------------------------
  const float l = l_run + xor32(l_run);
  const float inv_l = 1.0f / l;
  if (!qvalid) return;
  uint16_t *op = p.o + bb * p.so.b + hh * p.so.h + qrow * p.so.l;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d0 = 32 * dt + 8 * a + 4 * hf;
      const uint32_t w0 = f32_to_bf16_rne(acc[dt][4 * a + 0] * inv_l) | (f32_to_bf16_rne(acc[dt][4 * a + 1] * inv_l) << 16);
      const uint32_t w1 = f32_to_bf16_rne(acc[dt][4 * a + 2] * inv_l) | (f32_to_bf16_rne(acc[dt][4 * a + 3] * inv_l) << 16);
      *(uint2 *)(op + d0) = make_uint2(w0, w1);
      if (train) {
        float *hp = p.o_hp + (bh * p.lq + qrow) * kD + d0;
        *(f32x4 *)hp = f32x4{acc_hp[dt][4 * a] * inv_l, acc_hp[dt][4 * a + 1] * inv_l,
                             acc_hp[dt][4 * a + 2] * inv_l, acc_hp[dt][4 * a + 3] * inv_l};
      }
    }
  if (p.lse && hf == 0) p.lse[bh * p.lq + qrow] = m_run + __builtin_amdgcn_logf(l);
}

}  // namespace

hipError_t launch_kv_prepass(const AttnArgs &a, hipStream_t stream) {
  const Workspace w = workspace_layout(0, a.batch, a.heads, a.lq, a.lk);
  const int64_t C = (a.lk + kChunk - 1) / kChunk;
  const int64_t bh = (int64_t)a.batch * a.heads;
  uint8_t *ws = (uint8_t *)a.workspace;
  const int64_t total16 = bh * C * kChunk * (kD / 8);
  int64_t grid = (total16 + 255) / 256;
  if (grid > 16384) grid = 16384;
  hipLaunchKernelGGL(kq_prepass, dim3((unsigned)grid), dim3(256), 0, stream,
                     (const uint16_t *)a.k, a.sk, (u32x4 *)(ws + w.kq), a.heads, a.lk, C * kChunk,
                     total16, (a.flags & 2u) != 0);
  hipLaunchKernelGGL(vt_prepass, dim3((unsigned)(bh * C)), dim3(256), 0, stream,
                     (const uint16_t *)a.v, a.sv, (uint16_t *)(ws + w.vt), a.heads, a.lk, C,
                     (a.flags & 4u) != 0);
  return hipGetLastError();
}

hipError_t launch_attn_fwd_sel(const AttnArgs &a, const int32_t *sel, int64_t nsel, hipStream_t stream) {
  constexpr int WAVES = 4;
  const Workspace w = workspace_layout(0, a.batch, a.heads, a.lq, a.lk);
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
  p.qtiles = (int)((a.lq + 32 * WAVES - 1) / (32 * WAVES));
  p.nblocks = (int64_t)a.batch * a.heads * p.qtiles;
  p.per_xcd = (p.nblocks + 7) / 8;
  p.c = (float)((double)a.scale * 1.4426950408889634);
  p.causal = a.causal;
  p.quant_q = (a.flags & 1u) != 0;
  p.quant_p = (a.flags & 8u) != 0;
  if (a.o_hp)
    hipLaunchKernelGGL((attn_fwd_kernel<WAVES, true>), dim3((unsigned)(p.per_xcd * 8)), dim3(WAVES * 64), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<WAVES, false>), dim3((unsigned)(p.per_xcd * 8)), dim3(WAVES * 64), 0,
                       stream, p);
  return hipGetLastError();
}

hipError_t launch_attn_fwd(const AttnArgs &a, hipStream_t stream) {
  hipError_t e = launch_kv_prepass(a, stream);
  if (e != hipSuccess) return e;
  return launch_attn_fwd_sel(a, nullptr, 0, stream);
}

}  // namespace aq
