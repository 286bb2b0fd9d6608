// launch.hpp - host-side launchers of the gfx950 kernels and the workspace layout they share.
// Called only by abi.cpp after argument validation; each returns hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace aq {

constexpr int kHeadDimHost = 128;
constexpr int kChunkHost = 128;
constexpr int kMaxCubesHost = 4096;  // cube-sparse: most cubes per head (longest per-key-cube list)
constexpr int kMaxSelHost = 1024;    // cube-sparse: most selected cubes per query cube

// Flag bits of a call (the ABI's AQ_* values): the four quantizers and the variants.
constexpr unsigned kFlagQ = 1u, kFlagK = 2u, kFlagV = 4u, kFlagP = 8u;
constexpr unsigned kFlagFinalMax = 16u, kFlagGsfQkv = 32u, kFlagGsfP = 64u, kFlagSmoothK = 128u;
constexpr unsigned kFlagTwoLevelP = 256u, kFlagSmoothQ = 512u, kFlagPvFp8 = 1024u;
// P's blocks take a global scale (the static-scale kernels) under these flags: 448*6, the two-level
// scale, or 1 under the FP8 P.V product alone.
constexpr unsigned kFlagsPGlobal = kFlagGsfP | kFlagTwoLevelP | kFlagPvFp8;
// Rows of the smooth-K partial sums: one per slab of this many keys.
constexpr int kMeanSlab = 256;

struct Strides {
  int64_t b, h, l;
};

// Arguments of one attention call (forward, or the forward half of the backward).
struct AttnArgs {
  const void *q, *k, *v;
  void *o;
  int batch, heads;
  int64_t lq, lk;
  Strides sq, sk, sv, so;
  float scale;
  bool causal;
  unsigned flags;
  float *lse;   // [B*H, lq] base-2 log-sum-exp, or null
  float *cmax;  // [B*H, C, lq] base-2 running maxima, or null
  float *o_hp;  // [B*H, lq, 128] fp32, or null
  void *workspace;
};

struct BwdArgs {
  const void *d_o;
  void *dq, *dk, *dv;
  Strides sdo, sdq, sdk, sdv;
};

struct VsaArgs {
  void *o_coarse;
  int32_t *sel;
  int n_cubes, topk;
};

// Workspace regions, each 256-byte aligned.  Row tensors are [B*H, C*128, 128] bf16 with rows
// padded by zeros to a multiple of 128; tile tensors are [B*H, C, 128 d, 128 rows] bf16 (each
// 128-row chunk stored d-major).
//   op 0 (forward):  kq (K-hat rows), vt (V-hat tiles)
//   op 1 (backward): kq, vq (V-hat rows), qq (Q-hat rows), dvec [B*H, lq] fp32 (D_i = <dO_i, o_hp_i>)
//   op 2 (cube-sparse forward): kq, vt, pool [3, B*H, n, 128] bf16 (cube means of Q, K, V),
//                    selw [B*H, n, min(n, kMaxSelHost)] int32 (selection when the caller passes
//                    none; a call's topk entries per query cube)
//   op 3 (cube-sparse backward): the op 1 regions, plus slot [B*H, n, n] int16 (position of every
//                    key cube in every query cube's selection, or -1)
//   every op: scal (global scales g_q, g_k, g_v, g_p as fp32, then three uint32 abs-max
//                    accumulators), kmean [B*H, 128] fp32 (smooth-K key means), kpart
//                    [B*H, ceil(lk / kMeanSlab), 128] fp64 (their partial sums)
//   ops 0 and 2: mfin [B*H, lq] fp32 (final row maxima, base-2 units, for the final-max variant)
struct Workspace {
  size_t kq, vt, vq, qq, dvec, part, part_bytes, pool, selw, slot, scal, kmean, kpart, mfin, qmean, qpart, delta, total;
};

// Dense backward: fp32 partial sums of the work units split to fill the last round of
// workgroups (a dQ piece 64 KiB, a dK/dV piece 128 KiB), at most kSplitBytes.
constexpr size_t kSplitBytes = (size_t)96 << 20;
constexpr size_t kDkdvPieceBytes = (size_t)2 * 128 * 128 * 4;
constexpr size_t kDqPieceBytes = (size_t)128 * 128 * 4;

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline Workspace workspace_layout(int op, int batch, int heads, int64_t lq, int64_t lk) {
  const size_t bh = (size_t)batch * heads;
  const size_t Ck = (size_t)((lk + kChunkHost - 1) / kChunkHost);
  const size_t Cq = (size_t)((lq + kChunkHost - 1) / kChunkHost);
  const size_t kbytes = bh * Ck * kChunkHost * kHeadDimHost * 2;
  const size_t qbytes = bh * Cq * kChunkHost * kHeadDimHost * 2;
  Workspace w{};
  size_t off = 0;
  auto take = [&off](size_t n) {
    const size_t at = off;
    off = align256(off + n);
    return at;
  };
  w.kq = take(kbytes);
  if (op == 0 || op == 2) w.vt = take(kbytes);
  if (op == 1 || op == 3) {
    w.vq = take(kbytes);
    w.qq = take(qbytes);
    w.dvec = take(bh * (size_t)lq * 4);
  }
  if (op == 1 || op == 3) {
    // at most 8 pieces per work unit
    const size_t units = bh * (Ck > Cq ? Ck : Cq);
    const size_t most = 8 * units * kDkdvPieceBytes;
    w.part_bytes = most < kSplitBytes ? most : kSplitBytes;
    w.part = take(w.part_bytes);
  }
  if (op == 3) {
    const size_t n = (size_t)(lk / kChunkHost);
    w.slot = take(bh * n * n * 2);
  }
  if (op == 2) {
    const size_t n = (size_t)(lk / kChunkHost);
    w.pool = take(3 * bh * n * kHeadDimHost * 2);
    // a selection list has topk <= min(n, kMaxSel) entries per query cube
    w.selw = take(bh * n * (n < (size_t)kMaxSelHost ? n : (size_t)kMaxSelHost) * 4);
  }
  w.scal = take(256);
  w.kmean = take(bh * kHeadDimHost * 4);
  w.kpart = take(bh * (size_t)((lk + kMeanSlab - 1) / kMeanSlab) * kHeadDimHost * 8);
  if (op == 0 || op == 2) w.mfin = take(bh * (size_t)lq * 4);
  // smooth-Q: the queries' means, their fp64 partial sums, and delta = <mean, k-hat> per key row
  w.qmean = take(bh * kHeadDimHost * 4);
  w.qpart = take(bh * (size_t)((lq + kMeanSlab - 1) / kMeanSlab) * kHeadDimHost * 8);
  w.delta = take(bh * Ck * kChunkHost * 4);
  w.total = off;
  return w;
}

inline size_t workspace_bytes(int op, int batch, int heads, int64_t lq, int64_t lk) {
  return workspace_layout(op, batch, heads, lq, lk).total;
}

// fake quantization of [outer, axis, inner] bf16 along axis; g == nullptr: unit global scale.
hipError_t launch_fq(const void *x, void *y, int64_t outer, int64_t axis, int64_t inner,
                     const float *g, hipStream_t stream);
// *g_out = 2688 / max(max|x|, 1e-12).
hipError_t launch_static_scale(const void *x, int64_t n, float *g_out, hipStream_t stream);
// *g_out = 2688 / max(*amax, 1e-12) (NaN read as 0), both device scalars.
hipError_t launch_scale_from_amax(const float *amax, float *g_out, hipStream_t stream);

// One 128-row chunk of a strided [B, L, H, 128] bf16 tensor per workgroup: optional fake
// quantization (kQuantNone, kQuantD along d per row, kQuantRows along rows per column; kQuantRowsF16
// the same with fp16 output values), then a
// row-major copy and/or a d-major tile copy into the workspace.  g: device fp32 global scale, or
// null for the unit scale; mean: [B*H, 128] fp32 subtracted per channel before quantization (the
// smooth-K variant), or null; out: the values as they are (bf16), rounded to FP8 E4M3FN (the
// FP8 P.V product) and kept as bf16 or as fp16, or as fp16 unchanged (for unit-scale NVFP4 values,
// which fp16 holds exactly); all after kQuantNone / kQuantD / kQuantRows only.
enum TileQuant { kQuantNone = 0, kQuantD = 1, kQuantRows = 2, kQuantRowsF16 = 3 };
enum TileOut { kOutBf16 = 0, kOutFp8Bf16 = 1, kOutFp8F16 = 2, kOutF16 = 3 };
hipError_t launch_tile_prepass(const void *src, Strides s, int batch, int heads, int64_t L,
                               TileQuant quant, void *rows_out, void *tiles_out, const float *g,
                               const float *mean, hipStream_t stream, TileOut out = kOutBf16);

// Under unit scales without smoothing: K-hat rows (quantized along d; fp16 or bf16 values) and
// V-hat d-major tiles (quantized along rows; fp16 or bf16 values) of the heads [bh0, bh0 + nbh)
// of the flattened batch*heads, in one streamed launch (the layouts and values of
// launch_tile_prepass with kQuantD / kOutF16|kOutBf16 for K and kQuantRows(F16) / kOutBf16 for V).
hipError_t launch_kv_stream(const void *k, Strides sk, const void *v, Strides sv, int batch, int heads, int64_t L,
                            int64_t bh0, int64_t nbh, void *krows, bool kf16, void *vtiles, bool vf16,
                            hipStream_t stream);

// The per-call quantities of the variants, into the workspace regions scal / kmean / kpart: the
// smooth-K key means (a.flags & kFlagSmoothK), then the static global scales of Q, K (of the
// smoothed keys) and V (kFlagGsfQkv) and of P (kFlagGsfP).  A no-op without those flags.
hipError_t launch_variant_prep(const AttnArgs &a, const Workspace &w, hipStream_t stream);
// Pointers into those regions for a call's flags (null when the variant is off).
struct VariantPtrs {
  const float *gq, *gk, *gv, *gp, *kmean, *qmean, *delta;
};
VariantPtrs variant_ptrs(const AttnArgs &a, const Workspace &w);
// Smooth-Q: delta [B*H, Ck*128] = <query mean, K-hat row> for the K-hat rows in the workspace
// (run after the K prepass).  No-op without the flag.
hipError_t launch_qk_delta(const AttnArgs &a, const Workspace &w, hipStream_t stream);

// The variants' per-call quantities, then K-hat rows and V-hat tiles of every head into the
// workspace of op 0 (dense forward) or 2 (cube-sparse forward).
// The side stream of the current device (side_stream.hip).  side_fork: work enqueued on f.stream
// from here on starts after everything already queued on `main`; f.stream is `main` itself when no
// side stream is available.  side_join: `main` waits for that work.  Between the two, calls on the
// same device from other host threads wait.
struct SideFork {
  hipStream_t stream;
  int dev;
};
hipError_t side_fork(hipStream_t main, SideFork &f);
hipError_t side_join(hipStream_t main, SideFork &f);
// The K and V prepasses (after the variants' statistics, which both use); with `overlap`, the V
// prepass runs on the side stream beside the K prepass, joined before this returns.
hipError_t launch_kv_prepass(const AttnArgs &a, int op, hipStream_t stream, bool overlap = false);
// Forward kernel only (operands already in the workspace); sel: cube-sparse chunk lists
// [B*H, lq/128, nsel] or null for dense attention.
hipError_t launch_attn_fwd_sel(const AttnArgs &a, const int32_t *sel, int64_t nsel, hipStream_t stream);
hipError_t launch_attn_fwd(const AttnArgs &a, hipStream_t stream);
// The current device's address of the library's fixed forward scratch (AQ_NOALLOC_SCRATCH_BYTES,
// looked up once per device; noalloc.hip).
hipError_t noalloc_scratch(void **out);
hipError_t launch_attn_bwd(const AttnArgs &a, const BwdArgs &b, hipStream_t stream);
hipError_t launch_vsa_fwd(const AttnArgs &a, const VsaArgs &s, hipStream_t stream);
// Straight-through backward of the cube-sparse fine stage; sel [B*H, n, topk] is the forward's
// selection (ascending, distinct), a.cmax holds [B*H, topk, lq] chunk maxima.
hipError_t launch_vsa_bwd(const AttnArgs &a, const BwdArgs &b, const int32_t *sel, int n_cubes, int topk,
                          hipStream_t stream);

// ---- NVFP4 QAD linear (linear.hip) ----
// C[P][Q] = sum_k L[p][k] R[q][k] (+ bias[q]); bf16, k contiguous, K a multiple of 64, row strides
// in elements.
hipError_t launch_gemm_tn(const void *L, int64_t ldl, const void *R, int64_t ldr, void *C, int64_t ldc,
                          const void *bias, int64_t P, int64_t Q, int64_t K, hipStream_t stream);
// out [C][Rp] = in [R][C]^T with rows r >= R of the result's columns zero (C and ldi multiples
// of 8, Rp a multiple of 64).
hipError_t launch_transpose(const void *in, int64_t ldi, int64_t R, int64_t C, void *out, int64_t Rp,
                            hipStream_t stream);
// gb [N] = bf16 column sums of g [M][N] (N a multiple of 8); part: colsum_chunks(M) * N fp32 of
// scratch.
hipError_t launch_colsum(const void *g, int64_t M, int64_t N, void *gb, float *part, hipStream_t stream);
// Both of the above for g in one pass: gt [N][Mp] = g^T and gb = its column sums, bit-identical to
// launch_colsum's.
hipError_t launch_transpose_colsum(const void *g, int64_t M, int64_t N, void *gt, int64_t Mp, void *gb, float *part,
                                   hipStream_t stream);
int64_t colsum_chunks(int64_t M);
// *amax = max(*amax, max|x|) over n bf16 values.
hipError_t launch_observe_amax(const void *x, int64_t n, float *amax, hipStream_t stream);

// Workspace of the linear: op 0 (forward) x-hat [M, K] and W-hat [N, K] bf16, the weight's global
// scale; op 1 (backward) W^T [K, N], grad^T [N, Mp], x^T [K, Mp] bf16 (Mp = M rounded up to 64)
// and the column-sum partials.
struct LinearWorkspace {
  size_t xq, wq, gw, wt, gt, xt, part, total;
};
inline LinearWorkspace linear_workspace(int op, int64_t m, int64_t n, int64_t k) {
  LinearWorkspace w{};
  size_t off = 0;
  auto take = [&off](size_t b) {
    const size_t at = off;
    off = align256(off + b);
    return at;
  };
  const size_t mp = (size_t)((m + 63) / 64 * 64);
  if (op == 0) {
    w.xq = take((size_t)m * k * 2);
    w.wq = take((size_t)n * k * 2);
    w.gw = take(256);
  } else {
    w.wt = take((size_t)k * n * 2);
    w.gt = take((size_t)n * mp * 2);
    w.xt = take((size_t)k * mp * 2);
    w.part = take((size_t)colsum_chunks(m) * n * 4);
  }
  w.total = off;
  return w;
}

}  // namespace aq
