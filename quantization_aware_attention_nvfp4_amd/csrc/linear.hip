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
// 64.  One workgroup computes a 256 x 256 tile with 4 waves in a 2 x 2 grid (128 x 128 each, the
// sixteen 32 x 32 accumulators in the AGPRs); K advances 64 at a time through two LDS buffers of
// 32 KiB for each operand, filled by asynchronous global -> LDS copies one step ahead.  The MFMA's
// A operand is R (rows q), its B operand L (rows p): a lane's accumulator registers then hold one
// p and four runs of four consecutive q, stored as 8-byte pieces of C's rows.
#include "aq_device.hpp"
#include "attn_common.hpp"
#include "launch.hpp"
#include "timing.hpp"

namespace aq {
namespace {

constexpr int kTile = 256, kBK = 64, kGemmWaves = 4;
constexpr int kRowBytes = kBK * 2;            // one tile row of one K step: 128 bytes
constexpr int kOpBytes = kTile * kRowBytes;   // one operand tile: 32 KiB
constexpr int kGroup = 4;                     // p-tiles per group of the tile order

// 16-byte column g (k / 8) of tile row r sits at physical column g ^ sw_g(r): a ds_read_b128
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
  __shared__ __attribute__((aligned(256))) uint8_t lds[2 * 2 * kOpBytes];  // [buf][L, R]
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
  const int wp = wave & 1, wq = wave >> 1;  // the wave's 128 x 128 block: p rows 128*wp, q rows 128*wq

  // Copies: instruction i of wave w fills tile rows 8*(8w + i) + lane/8, physical column lane%8.
  uint32_t loff[8], roff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 8 * (8 * wave + i) + (lane >> 3), c = (lane & 7) ^ sw_g(r);
    const int64_t pr = p0 + r < g.P ? r : g.P - 1 - p0;  // rows past the edge read the last row
    const int64_t qr = q0 + r < g.Q ? r : g.Q - 1 - q0;
    loff[i] = (uint32_t)((pr * g.ldl + 8 * c) * 2);
    roff[i] = (uint32_t)((qr * g.ldr + 8 * c) * 2);
  }
  const uint8_t *lbase = (const uint8_t *)(g.L + p0 * g.ldl);
  const uint8_t *rbase = (const uint8_t *)(g.R + q0 * g.ldr);
  const uint32_t lds0 = lds_addr(lds);
  auto stage = [&](int64_t k0, int buf) {
    const uint32_t dst = lds0 + buf * 2 * kOpBytes + 1024 * 8 * wave;
#pragma unroll
    for (int i = 0; i < 8; ++i) load_lds16_sa(lbase + 2 * k0, loff[i], dst + 1024 * i);
#pragma unroll
    for (int i = 0; i < 8; ++i) load_lds16_sa(rbase + 2 * k0, roff[i], dst + kOpBytes + 1024 * i);
  };

  // LDS read addresses: A (R rows) tile t rows 128*wq + 32t + n, B (L rows) tile t rows
  // 128*wp + 32t + n; 16-byte column 2*kk + hf of the K step.  Rows r and r + 32t share sw_g
  // (bits 1-3 of r), so one base per operand serves all four tiles.
  const int ra = 128 * wq + n, rb = 128 * wp + n;
  const uint32_t abase = lds0 + kOpBytes + ra * kRowBytes, bbase = lds0 + rb * kRowBytes;
  const int swa = sw_g(ra), swb = sw_g(rb);

  f32x16 acc[4][4];  // [q tile][p tile]
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x16{};

  const int64_t nk = g.K / kBK;
  stage(0, 0);
  for (int64_t kb = 0; kb < nk; ++kb) {
    const int buf = (int)(kb & 1);
    AQ_WAIT_VMCNT(0);              // this wave's copies of step kb
    __builtin_amdgcn_s_barrier();  // everyone's copies landed; step kb-1's buffer is free
    if (kb + 1 < nk) stage((kb + 1) * kBK, buf ^ 1);
    const uint32_t ab = abase + buf * 2 * kOpBytes, bb = bbase + buf * 2 * kOpBytes;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int gcol = 2 * kk + hf;
      bf16x8 av[4], bv[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        av[t] = as_bf16x8(lds_read16(ab + 32 * t * kRowBytes + 16 * (gcol ^ swa)));
        bv[t] = as_bf16x8(lds_read16(bb + 32 * t * kRowBytes + 16 * (gcol ^ swb)));
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[a], bv[b], acc[a][b], 0, 0, 0);
    }
  }

  // Epilogue: lane holds p = p0 + 128 wp + 32 b + n and, per run u, q = q0 + 128 wq + 32 a + 8u +
  // 4 hf + (0..3).
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int64_t p = p0 + 128 * wp + 32 * b + n;
    if (p >= g.P) continue;
    uint16_t *crow = g.C + p * g.ldc;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t q = q0 + 128 * wq + 32 * a + 8 * u + 4 * hf;
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

// out[c][r] = in[r][c] for a row-major [R, C] bf16 matrix (row stride ldi), into [C, Rp] with
// rows r >= R zero (Rp = R rounded up to a multiple of 64).  64 x 64 tiles through LDS.
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t *__restrict__ in, int64_t ldi, int64_t R,
                                                        int64_t C, uint16_t *__restrict__ out, int64_t Rp,
                                                        int64_t ntc) {
  __shared__ uint16_t t[64][65];
  const int64_t tr = blockIdx.x / ntc, tc = blockIdx.x % ntc;
  const int tid = threadIdx.x;
  for (int i = tid; i < 64 * 64; i += 256) {
    const int rr = i >> 6, cc = i & 63;
    const int64_t r = tr * 64 + rr, c = tc * 64 + cc;
    t[rr][cc] = (r < R && c < C) ? in[r * ldi + c] : (uint16_t)0;
  }
  __syncthreads();
  for (int i = tid; i < 64 * 64; i += 256) {
    const int cc = i >> 6, rr = i & 63;
    const int64_t r = tr * 64 + rr, c = tc * 64 + cc;
    if (c < C && r < Rp) out[c * Rp + r] = t[rr][cc];
  }
}

// Column sums of g [M][N] in two deterministic stages: colsum_partial_kernel sums row chunk c
// (kColChunk rows) of 64 columns into part[c][n] (four lane groups of rows, added in order);
// colsum_final_kernel adds the chunks in order and rounds to bf16.
constexpr int kColChunk = 256;
__global__ __launch_bounds__(256) void colsum_partial_kernel(const uint16_t *__restrict__ g, int64_t M, int64_t N,
                                                             int64_t ncb, float *__restrict__ part) {
  __shared__ float acc[4][64];
  const int64_t cb = blockIdx.x % ncb, chunk = blockIdx.x / ncb;
  const int c = threadIdx.x & 63, grp = threadIdx.x >> 6;
  const int64_t n = cb * 64 + c, m0 = chunk * kColChunk, m1 = m0 + kColChunk < M ? m0 + kColChunk : M;
  float s = 0.0f;
  if (n < N)
    for (int64_t m = m0 + grp; m < m1; m += 4) s += bf16lo(g[m * N + n]);
  acc[grp][c] = s;
  __syncthreads();
  if (grp == 0 && n < N) part[chunk * N + n] = ((acc[0][c] + acc[1][c]) + acc[2][c]) + acc[3][c];
}
__global__ __launch_bounds__(256) void colsum_final_kernel(const float *__restrict__ part, int64_t nchunk, int64_t N,
                                                           uint16_t *__restrict__ gb) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  float s = 0.0f;
  for (int64_t c = 0; c < nchunk; ++c) s += part[c * N + n];
  gb[n] = (uint16_t)f32_to_bf16_rne(s);
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
  const int64_t ntr = (Rp + 63) / 64, ntc = (C + 63) / 64;
  AQ_LAUNCH("transpose", transpose_kernel, dim3((unsigned)(ntr * ntc)), dim3(256), 0, stream, (const uint16_t *)in,
            ldi, R, C, (uint16_t *)out, Rp, ntc);
  return hipGetLastError();
}

// part: nchunk * N fp32 of scratch, nchunk = ceil(M / kColChunk).
hipError_t launch_colsum(const void *g, int64_t M, int64_t N, void *gb, float *part, hipStream_t stream) {
  const int64_t ncb = (N + 63) / 64, nchunk = (M + kColChunk - 1) / kColChunk;
  AQ_LAUNCH("colsum_partial", colsum_partial_kernel, dim3((unsigned)(ncb * nchunk)), dim3(256), 0, stream,
            (const uint16_t *)g, M, N, ncb, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  AQ_LAUNCH("colsum_final", colsum_final_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, stream, part, nchunk,
            N, (uint16_t *)gb);
  return hipGetLastError();
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
