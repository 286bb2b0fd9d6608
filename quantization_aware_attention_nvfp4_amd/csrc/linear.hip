// linear.hip - the NVFP4 QAD linear on gfx950 ("nvfp4_qad.py": nvfp4_gemm, _NVFP4STE and the
// calibrating path of NVFP4QADLinearMethod.apply).
//
// Forward: y = fq(x, g_x) fq(W, g_W)^T + bias with g_W = 448*6 / amax|W| (weight_global_sf) and
// g_x unit or static (input_global_sf); the blocks of 16 run along the input features.  The
// pages run it as an FP4 GEMM; here the fake-quantized operands (bf16, exact under the unit scale)
// feed a BF16 MFMA GEMM, the "fake-quant + BF16 GEMM" reading.  Backward (the straight-through
// estimator): grad_x = grad W, grad_W = grad^T x, grad_b = column sums of grad, full precision.
//
// GEMM: C[P][Q] = sum_k L[p][k] R[q][k] (+ bias[q]) with L, R bf16, k contiguous, K a multiple of
// 64.  One workgroup computes a 256 x 256 tile with 8 waves, two per SIMD so that one issues MFMAs
// while the other waits on LDS, in a 4 (p) x 2 (q) grid of 64 x 128 blocks (eight 32 x 32
// accumulators each).  K advances 64 at a time (128-byte rows: the asynchronous global -> LDS
// copies read whole cache lines) through a ring of five 32 KiB LDS slots, one operand of one step
// each, so that each step's operands are requested one to two steps ahead.
// The MFMA's A operand is R (rows q), its B operand L (rows p): a lane's accumulator registers then
// hold one p and four runs of four consecutive q, stored as 8-byte pieces of C's rows.
#include "aq_device.hpp"
#include "attn_common.hpp"
#include "launch.hpp"
#include "timing.hpp"

namespace aq {
namespace {

constexpr int kTile = 256, kBK = 64, kSlots = 5;
// 8 waves, two per SIMD, in a 4 (p) x 2 (q) grid; a wave owns 64 p x 128 q (kNA q tiles by kNB p
// tiles of 32 x 32).
constexpr int kWavesP = 4, kWavesQ = 2, kGemmWaves = kWavesP * kWavesQ;
constexpr int kNA = kTile / kWavesQ / 32, kNB = kTile / kWavesP / 32;
constexpr int kRowBytes = kBK * 2;            // one tile row of one K step: 128 bytes (a cache line)
constexpr int kOpBytes = kTile * kRowBytes;   // one operand of one K step: 32 KiB, one LDS slot
constexpr int kGroup = 8;                     // p-tiles per group of the tile order
constexpr int kCopies = kOpBytes / 1024 / kGemmWaves;  // 1 KiB copies per wave and operand per step

// 16-byte column g (k / 8, 0..7) of tile row r sits at physical column g ^ sw_g(r): a ds_read_b128
// serves 16 lanes per cycle from 256 bytes, i.e. two 128-byte rows, so the 16 rows r0..r0+15 of
// one read must cover 16 distinct slots 8 * (r & 1) + column.
__device__ __forceinline__ int sw_g(int r) { return (r >> 1) & 7; }

struct GemmParams {
  const uint16_t *L, *R;
  uint16_t *C;
  const uint16_t *bias;  // [Q] bf16, or null
  int64_t ldl, ldr, ldc;  // row strides in elements
  int64_t P, Q, K;
  int64_t np, nq;         // tiles along P and Q
  int64_t ntiles, per_xcd;
};

__global__ __launch_bounds__(kGemmWaves * 64, 1) void gemm_tn_kernel(GemmParams g) {
  __shared__ __attribute__((aligned(256))) uint8_t lds[kSlots * kOpBytes];  // a ring of operand slots
  const int64_t vid = xcd_work_id(blockIdx.x, g.per_xcd, g.ntiles);
  if (vid < 0) return;
  // Tile order: groups of kGroup p-tiles walked q-tile by q-tile, so the workgroups that run
  // together on one XCD share a few L and R tiles in its L2.
  const int64_t per_group = (int64_t)kGroup * g.nq;
  const int64_t grp = vid / per_group, in = vid % per_group;
  const int64_t gp0 = grp * kGroup;
  const int64_t gsize = g.np - gp0 < kGroup ? g.np - gp0 : kGroup;
  const int64_t pt = gp0 + in % gsize, qt = in / gsize;
  const int64_t p0 = pt * kTile, q0 = qt * kTile;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, n = lane & 31, hf = lane >> 5;
  const int wp = wave % kWavesP, wq = wave / kWavesP;  // p rows 64*wp, q rows 128*wq of the tile

  // Copies: instruction i of wave w fills tile rows 8*(kCopies*w + i) + lane/8, physical column
  // lane%8 (each instruction reads whole 128-byte lines).
  uint32_t loff[kCopies], roff[kCopies];
#pragma unroll
  for (int i = 0; i < kCopies; ++i) {
    const int r = 8 * (kCopies * wave + i) + (lane >> 3), c = (lane & 7) ^ sw_g(r);
    const int64_t pr = p0 + r < g.P ? r : g.P - 1 - p0;  // rows past the edge read the last row
    const int64_t qr = q0 + r < g.Q ? r : g.Q - 1 - q0;
    loff[i] = (uint32_t)((pr * g.ldl + 8 * c) * 2);
    roff[i] = (uint32_t)((qr * g.ldr + 8 * c) * 2);
  }
  const uint8_t *lbase = (const uint8_t *)(g.L + p0 * g.ldl);
  const uint8_t *rbase = (const uint8_t *)(g.R + q0 * g.ldr);
  const uint32_t lds0 = lds_addr(lds);

  // LDS read addresses: A (R rows) tile t rows 128*wq + 32t + n, B (L rows) tile t rows
  // 64*wp + 32t + n; 16-byte column 2*kk + hf of sub-step kk.  Rows r and r + 32t share sw_g
  // (bits 1-3 of r), so one base per operand serves all its tiles.
  const int ra = 32 * kNA * wq + n, rb = 32 * kNB * wp + n;
  const uint32_t aoff = ra * kRowBytes, boff = rb * kRowBytes;
  const int swa = sw_g(ra), swb = sw_g(rb);

  f32x16 acc[kNA][kNB];  // [q tile][p tile]
#pragma unroll
  for (int a = 0; a < kNA; ++a)
#pragma unroll
    for (int b = 0; b < kNB; ++b) acc[a][b] = f32x16{};

  // The operands of the K steps go through a ring of kSlots LDS slots as units u = 0, 1, 2, ...:
  // unit 2j is L of step j, unit 2j + 1 is R of step j, and unit u fills slot u % kSlots.  In the
  // last of step j's four sub-steps every wave waits for its reads of step j and its copies of
  // step j + 1, then meets the others at one barrier; step j's slots are then free and receive
  // units 2j + 5 and 2j + 6, and the first operands of step j + 1 are read while step j's last
  // MFMAs run.  Each sub-step reads the next one's operands while its own MFMAs run.
  static_assert(kSlots == 5 && kCopies == 4 && kNA == 4 && kNB == 2, "the waits below count units of 4 copies");
  const int nk = (int)(g.K / kBK);
  const int nunits = 2 * nk;
  bf16x8 av[2][kNA], bv[2][kNB];
  auto read_a = [&](uint32_t slot, int kk, int r, int t) {
    av[r][t] = as_bf16x8(lds_read16(slot + aoff + 32 * t * kRowBytes + 16 * ((2 * kk + hf) ^ swa)));
  };
  auto read_b = [&](uint32_t slot, int kk, int r, int t) {
    bv[r][t] = as_bf16x8(lds_read16(slot + boff + 32 * t * kRowBytes + 16 * ((2 * kk + hf) ^ swb)));
  };
  auto mfma = [&](int r, int a, int b) {
    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[r][a], bv[r][b], acc[a][b], 0, 0, 0);
  };
  auto slot_addr = [&](int u) { return lds0 + (uint32_t)(u % kSlots) * kOpBytes; };
  auto copy = [&](int u, int i) {  // copy instruction i of unit u
    const int64_t k0 = (int64_t)(u >> 1) * kBK;
    const uint32_t dst = slot_addr(u) + 1024 * (kCopies * wave + i);
    if (u & 1) load_lds16_sa(rbase + 2 * k0, roff[i], dst);
    else load_lds16_sa(lbase + 2 * k0, loff[i], dst);
  };
#pragma unroll
  for (int u = 0; u < kSlots; ++u)
    if (u < nunits)
#pragma unroll
      for (int i = 0; i < kCopies; ++i) copy(u, i);
  // units 0 and 1; units 2 .. 4 may stay outstanding
  if (nunits >= 5) AQ_WAIT_VMCNT(12);
  else if (nunits == 4) AQ_WAIT_VMCNT(8);
  else AQ_WAIT_VMCNT(0);
  __builtin_amdgcn_s_barrier();
  uint32_t ls = slot_addr(0), rs = slot_addr(1);  // slots of step j's L and R
#pragma unroll
  for (int t = 0; t < kNA; ++t) read_a(rs, 0, 0, t);
#pragma unroll
  for (int t = 0; t < kNB; ++t) read_b(ls, 0, 0, t);
  for (int j = 0; j < nk; ++j) {
    // sub-steps 0 .. 2: MFMAs of kk with the operands in r = kk & 1, reads of kk + 1
#pragma unroll
    for (int kk = 0; kk < 3; ++kk) {
      const int r = kk & 1;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int a = 0; a < kNA; ++a) {
        read_a(rs, kk + 1, r ^ 1, a);
        if (a < kNB) read_b(ls, kk + 1, r ^ 1, a);
#pragma unroll
        for (int b = 0; b < kNB; ++b) mfma(r, a, b);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // sub-step 3 (operands in r = 1): two MFMAs keep the matrix unit busy across the waits and
    // the barrier
    mfma(1, 0, 0);
    mfma(1, 0, 1);
    __builtin_amdgcn_sched_barrier(0);
    const int u0 = 2 * j + 2;  // step j + 1's units
    const uint32_t nls = slot_addr(u0), nrs = slot_addr(u0 + 1);
    if (j + 1 < nk) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave is done reading step j
      if (u0 + 2 < nunits) AQ_WAIT_VMCNT(4);                // unit u0 + 2 may stay outstanding
      else AQ_WAIT_VMCNT(0);
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int t = 0; t < kNA; ++t) read_a(nrs, 0, 0, t);
#pragma unroll
      for (int t = 0; t < kNB; ++t) read_b(nls, 0, 0, t);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int a = 1; a < kNA; ++a) {
#pragma unroll
      for (int b = 0; b < kNB; ++b) mfma(1, a, b);
      // units 2j + 5 and 2j + 6 into step j's slots, spread between the MFMAs
      if (a == 1) {
        if (u0 + 3 < nunits)
#pragma unroll
          for (int i = 0; i < kCopies; ++i) copy(u0 + 3, i);
      } else if (a == 2) {
        if (u0 + 4 < nunits)
#pragma unroll
          for (int i = 0; i < kCopies; ++i) copy(u0 + 4, i);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    ls = nls;
    rs = nrs;
  }

  // Epilogue: lane holds p = p0 + 64 wp + 32 b + n and, per run u, q = q0 + 128 wq + 32 a + 8u +
  // 4 hf + (0..3).
#pragma unroll
  for (int b = 0; b < kNB; ++b) {
    const int64_t p = p0 + 32 * kNB * wp + 32 * b + n;
    if (p >= g.P) continue;
    uint16_t *crow = g.C + p * g.ldc;
#pragma unroll
    for (int a = 0; a < kNA; ++a)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t q = q0 + 32 * kNA * wq + 32 * a + 8 * u + 4 * hf;
        float v[4] = {acc[a][b][4 * u], acc[a][b][4 * u + 1], acc[a][b][4 * u + 2], acc[a][b][4 * u + 3]};
        if (q + 3 < g.Q) {
          if (g.bias) {
            const uint2 bw = *(const uint2 *)(g.bias + q);
            v[0] += bf16lo(bw.x); v[1] += bf16hi(bw.x); v[2] += bf16lo(bw.y); v[3] += bf16hi(bw.y);
          }
          *(uint2 *)(crow + q) = uint2{f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16),
                                       f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16)};
        } else {
          for (int e = 0; e < 4; ++e)
            if (q + e < g.Q) {
              const float bv = g.bias ? bf16lo(g.bias[q + e]) : 0.0f;
              crow[q + e] = (uint16_t)f32_to_bf16_rne(v[e] + bv);
            }
        }
      }
  }
}

// out[c][r] = in[r][c] for a row-major [R, C] bf16 matrix (row stride ldi, C and ldi multiples of
// 8), into [C, Rp] with rows r >= R zero (Rp = R rounded up to a multiple of 64), through 64 x 64
// tiles in LDS with 16-byte global loads and stores; a workgroup takes RT row tiles of one column
// tile.  With COLSUM the column sums over the workgroup's 64 * RT rows go to part[chunk][c] (fp32:
// a lane adds its 8 rows of each tile in order, then the 8 lanes of one column are combined by a
// fixed butterfly); without WRITE only those sums are produced.
constexpr int kRowTiles = 4, kColChunk = 64 * kRowTiles;
template <bool COLSUM, bool WRITE>
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t *__restrict__ in, int64_t ldi, int64_t R,
                                                        int64_t C, uint16_t *__restrict__ out, int64_t Rp,
                                                        int64_t ntc, float *__restrict__ part) {
  constexpr int kLd = 72;  // LDS row stride in elements (144 bytes: rows stay 16-byte aligned)
  __shared__ __attribute__((aligned(16))) uint16_t t[64 * kLd];
  const int64_t chunk = blockIdx.x / ntc, tc = blockIdx.x % ntc;
  const int tid = threadIdx.x;
  float sum[2] = {0.0f, 0.0f};
  for (int s = 0; s < kRowTiles; ++s) {
    const int64_t tr = chunk * kRowTiles + s;
    if (tr * 64 >= Rp) break;
    if (s) __syncthreads();  // the previous tile's reads are done
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int idx = tid + 256 * j, rr = idx >> 3, cg = idx & 7;
      const int64_t r = tr * 64 + rr, c = tc * 64 + 8 * cg;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (r < R && c < C) v = *(const u32x4 *)(in + r * ldi + c);
      *(u32x4 *)(t + rr * kLd + 8 * cg) = v;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int idx = tid + 256 * j, oc = idx >> 3, rg = idx & 7;  // output row oc, rows 8rg .. 8rg+7
      const int64_t c = tc * 64 + oc;
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = t[(8 * rg + e) * kLd + oc];
      if (WRITE && c < C)
        *(u32x4 *)(out + c * Rp + tr * 64 + 8 * rg) =
            u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
      if (COLSUM)
#pragma unroll
        for (int e = 0; e < 8; ++e) sum[j] += bf16lo(h[e]);
    }
  }
  if (COLSUM) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float v = sum[j];
      v += __shfl_xor(v, 1, 64);
      v += __shfl_xor(v, 2, 64);
      v += __shfl_xor(v, 4, 64);
      const int idx = tid + 256 * j, oc = idx >> 3;
      const int64_t c = tc * 64 + oc;
      if ((idx & 7) == 0 && c < C) part[chunk * C + c] = v;
    }
  }
}

// gb[n] = bf16 of the sum of part[chunk][n] over the chunks: four lane groups each add a contiguous
// quarter of the chunks in order, and the quarters are added in order.
__global__ __launch_bounds__(256) void colsum_final_kernel(const float *__restrict__ part, int64_t nchunk, int64_t N,
                                                           uint16_t *__restrict__ gb) {
  __shared__ float q[4][64];
  const int c = threadIdx.x & 63, grp = threadIdx.x >> 6;
  const int64_t n = (int64_t)blockIdx.x * 64 + c;
  const int64_t per = (nchunk + 3) / 4, c0 = grp * per, c1 = c0 + per < nchunk ? c0 + per : nchunk;
  float s = 0.0f;
  if (n < N) {
#pragma unroll 8
    for (int64_t i = c0; i < c1; ++i) s += part[i * N + n];
  }
  q[grp][c] = s;
  __syncthreads();
  if (grp == 0 && n < N) gb[n] = (uint16_t)f32_to_bf16_rne(((q[0][c] + q[1][c]) + q[2][c]) + q[3][c]);
}

// *amax = max(*amax, max|x|) over n elements (calibration), an atomic maximum per workgroup on the
// float's bits (NaN counts as 0).
__global__ __launch_bounds__(256) void observe_amax_kernel(const uint16_t *__restrict__ x, int64_t n,
                                                           uint32_t *__restrict__ amax) {
  __shared__ float red[4];
  float m = 0.0f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    m = fmaxf(m, __builtin_fabsf(bf16lo(x[i])));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) atomicMax(amax, f2u(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))));
}

}  // namespace

hipError_t launch_gemm_tn(const void *L, int64_t ldl, const void *R, int64_t ldr, void *C, int64_t ldc,
                          const void *bias, int64_t P, int64_t Q, int64_t K, hipStream_t stream) {
  GemmParams g{};
  g.L = (const uint16_t *)L;
  g.R = (const uint16_t *)R;
  g.C = (uint16_t *)C;
  g.bias = (const uint16_t *)bias;
  g.ldl = ldl;
  g.ldr = ldr;
  g.ldc = ldc;
  g.P = P;
  g.Q = Q;
  g.K = K;
  g.np = (P + kTile - 1) / kTile;
  g.nq = (Q + kTile - 1) / kTile;
  g.ntiles = g.np * g.nq;
  g.per_xcd = (g.ntiles + 7) / 8;
  AQ_LAUNCH("gemm_tn", gemm_tn_kernel, dim3((unsigned)(g.per_xcd * 8)), dim3(kGemmWaves * 64), 0, stream, g);
  return hipGetLastError();
}

hipError_t launch_transpose(const void *in, int64_t ldi, int64_t R, int64_t C, void *out, int64_t Rp,
                            hipStream_t stream) {
  const int64_t nch = (Rp + kColChunk - 1) / kColChunk, ntc = (C + 63) / 64;
  AQ_LAUNCH("transpose", (transpose_kernel<false, true>), dim3((unsigned)(nch * ntc)), dim3(256), 0, stream,
            (const uint16_t *)in, ldi, R, C, (uint16_t *)out, Rp, ntc, (float *)nullptr);
  return hipGetLastError();
}

static hipError_t launch_colsum_final(const float *part, int64_t M, int64_t N, void *gb, hipStream_t stream) {
  AQ_LAUNCH("colsum_final", colsum_final_kernel, dim3((unsigned)((N + 63) / 64)), dim3(256), 0, stream, part,
            colsum_chunks(M), N, (uint16_t *)gb);
  return hipGetLastError();
}

hipError_t launch_transpose_colsum(const void *g, int64_t M, int64_t N, void *gt, int64_t Mp, void *gb, float *part,
                                   hipStream_t stream) {
  const int64_t nch = colsum_chunks(M), ntc = (N + 63) / 64;
  AQ_LAUNCH("transpose_colsum", (transpose_kernel<true, true>), dim3((unsigned)(nch * ntc)), dim3(256), 0, stream,
            (const uint16_t *)g, N, M, N, (uint16_t *)gt, Mp, ntc, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_colsum_final(part, M, N, gb, stream);
}

hipError_t launch_colsum(const void *g, int64_t M, int64_t N, void *gb, float *part, hipStream_t stream) {
  const int64_t nch = colsum_chunks(M), ntc = (N + 63) / 64;
  AQ_LAUNCH("colsum_partial", (transpose_kernel<true, false>), dim3((unsigned)(nch * ntc)), dim3(256), 0, stream,
            (const uint16_t *)g, N, M, N, (uint16_t *)nullptr, (M + 63) / 64 * 64, ntc, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_colsum_final(part, M, N, gb, stream);
}

int64_t colsum_chunks(int64_t M) { return (M + kColChunk - 1) / kColChunk; }

hipError_t launch_observe_amax(const void *x, int64_t n, float *amax, hipStream_t stream) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  AQ_LAUNCH("observe_amax", observe_amax_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const uint16_t *)x,
            n, (uint32_t *)amax);
  return hipGetLastError();
}

}  // namespace aq
