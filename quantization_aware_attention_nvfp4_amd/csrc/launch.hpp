// launch.hpp - host-side launchers of the gfx950 kernels and the workspace layout they share.
// Called only by abi.cpp after argument validation; each returns hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace aq {

constexpr int kHeadDimHost = 128;
constexpr int kChunkHost = 128;

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

// Workspace regions, each 256-byte aligned, in this order:
//   kq    [B*H, C*128, 128] bf16   K-hat, keys padded with zeros to a multiple of 128
//   vt    [B*H, C, 128 d, 128 keys] bf16   V-hat, each 128-key chunk stored d-major
//   (op 1) dvec [B*H, lq] fp32      D_i = <dO_i, o_hp_i>
//   (op 1) dqacc [B*H, lq, 128] fp32  dQ accumulator
//   (op 2) pool  [3, B*H, n, 128] bf16 cube means of Q, K, V
//   (op 2) selw  [B*H, n, n] int32   selection when the caller passes none
struct Workspace {
  size_t kq, vt, dvec, dqacc, pool, selw, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline Workspace workspace_layout(int op, int batch, int heads, int64_t lq, int64_t lk) {
  const size_t bh = (size_t)batch * heads;
  const size_t C = (size_t)((lk + kChunkHost - 1) / kChunkHost);
  Workspace w{};
  size_t off = 0;
  w.kq = off;
  off = align256(off + bh * C * kChunkHost * kHeadDimHost * 2);
  w.vt = off;
  off = align256(off + bh * C * kChunkHost * kHeadDimHost * 2);
  if (op == 1) {
    w.dvec = off;
    off = align256(off + bh * (size_t)lq * 4);
    w.dqacc = off;
    off = align256(off + bh * (size_t)lq * kHeadDimHost * 4);
  }
  if (op == 2) {
    const size_t n = (size_t)(lk / kChunkHost);
    w.pool = off;
    off = align256(off + 3 * bh * n * kHeadDimHost * 2);
    w.selw = off;
    off = align256(off + bh * n * n * 4);
  }
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

// K-hat / V-hat into the workspace (kq, vt regions) for keys [0, lk) of every head.
hipError_t launch_kv_prepass(const AttnArgs &a, hipStream_t stream);

hipError_t launch_attn_fwd(const AttnArgs &a, hipStream_t stream);
hipError_t launch_attn_bwd(const AttnArgs &a, const BwdArgs &b, hipStream_t stream);
hipError_t launch_vsa_fwd(const AttnArgs &a, const VsaArgs &s, hipStream_t stream);

}  // namespace aq
