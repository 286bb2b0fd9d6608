// attn_common.hpp - lane mappings and LDS addressing shared by the attention kernels.
//
// v_mfma_f32_32x32x16_bf16: lane l supplies row l%32 of A and column l%32 of B, each with the 8
// k-slots 8*(l/32) .. 8*(l/32)+7; accumulator element (row i, column j) sits in lane
// j + 32*((i/4)%2), register 4*(i/8) + i%4 (checked on the GPU).
#pragma once

#include "aq_device.hpp"

namespace aq {

// A key (or query) tile is fed as A rows in the order row i -> local index
// 16*((i/4)%2) + 4*(i/8) + i%4, so that accumulator register r of lane half h holds local index
// 16*h + r: each lane then owns 16 consecutive local indices of one column.
__device__ __forceinline__ int perm_row(int i) { return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3); }

// XOR swizzles of the 16-byte columns of a 256-byte-row LDS tile, so that 16 lanes reading the
// same logical column of 16 different rows hit 16 different 16-byte bank groups.
// sw_kq serves A-operand reads in perm_row order (lanes 0..15 read rows {0..3, 16..19, 4..7,
// 20..23} + 8k), sw_row reads of consecutive rows.
__device__ __forceinline__ int sw_kq(int r) { return (r & 3) | ((r >> 2) & 4) | ((r & 4) << 1); }
__device__ __forceinline__ int sw_row(int r) { return r & 15; }
__device__ __forceinline__ int kq_off(int r, int j) { return r * 256 + ((j ^ sw_kq(r)) << 4); }
__device__ __forceinline__ int row_off(int r, int j) { return r * 256 + ((j ^ sw_row(r)) << 4); }
// sw_qr serves both reads of the backward's query tiles: 16 lanes reading one column of 16
// consecutive rows (all 16 values of the 4 bits), and transposed reads in which 4 consecutive rows
// (r%4 = 0..3) each supply 32 contiguous bytes (r%4 picks the 64-byte quarter of the row).
__device__ __forceinline__ int sw_qr(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int qr_off(int r, int j) { return r * 256 + ((j ^ sw_qr(r)) << 4); }

// One-hot B operand of a 32x32x16 MFMA that moves A's k-slot values into column j: lane (column
// j = l%32, half h) holds 1 in slot jj where j == 16h + 8*step + jj.
__device__ __forceinline__ bf16x8 onehot_b(int lane, int step) {
  const int j = lane & 31, h = lane >> 5;
  bf16x8 b;
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) b[jj] = (__bf16)((j == 16 * h + 8 * step + jj) ? 1.0f : 0.0f);
  return b;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Eight fp32 values -> bf16x8 with round-to-nearest-even.
__device__ __forceinline__ bf16x8 pack8_rne(const float *f) {
  u32x4 w;
  w.x = f32_to_bf16_rne(f[0]) | (f32_to_bf16_rne(f[1]) << 16);
  w.y = f32_to_bf16_rne(f[2]) | (f32_to_bf16_rne(f[3]) << 16);
  w.z = f32_to_bf16_rne(f[4]) | (f32_to_bf16_rne(f[5]) << 16);
  w.w = f32_to_bf16_rne(f[6]) | (f32_to_bf16_rne(f[7]) << 16);
  return as_bf16x8(w);
}
// Eight fp32 values -> bf16x8 through the hardware packed conversion (v_cvt_pk_bf16_f32,
// round to nearest even; exact for values that are already bf16).
__device__ __forceinline__ bf16x8 pack8_cvt(const float *f) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)f[i];
  return r;
}
// Eight fp32 values that are exact in bf16 -> bf16x8.
__device__ __forceinline__ bf16x8 pack8_exact(const float *f) { return pack8_cvt(f); }

// Asynchronous 16-byte global -> LDS copy: lane l of the wave writes LDS bytes
// [lds_base + 16*l, +16) (checked on the GPU); lds_base must be the same in every lane.
// Written as inline assembly (M0 = LDS base, then global_load_lds_dwordx4) so the compiler does
// not treat every later LDS read as dependent on the copy and drain all copies before it; the
// callers order copies and reads themselves with AQ_WAIT_VMCNT and s_barrier.  The compiler's
// own vmcnt waits stay correct: vector memory operations complete in order, so extra copies in
// flight can only make it wait longer, never shorter.
__device__ __forceinline__ void load_lds16(const void *gsrc, uint8_t *lds_base) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0v), "v"(gsrc) : "memory", "m0");
}

// A wave-uniform pointer moved to scalar registers.
__device__ __forceinline__ const void *uniform_ptr(const void *p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Same copy from a wave-uniform base plus a 32-bit per-lane byte offset (the saddr form: the
// per-lane address costs one VGPR instead of two).
__device__ __forceinline__ void load_lds16_s(const void *sbase, uint32_t voff, uint8_t *lds_base) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0v), "v"(voff), "s"(uniform_ptr(sbase))
               : "memory", "m0");
}
// Same, with the LDS destination given as a wave-uniform LDS byte address (kept in a scalar
// register, so no vector register carries it across a loop).
__device__ __forceinline__ void load_lds16_sa(const void *sbase, uint32_t voff, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_off), "v"(voff), "s"(uniform_ptr(sbase))
               : "memory", "m0");
}
// load_lds16_sa without the "memory" clobber, for copies issued among a phase's LDS operand reads:
// the compiler may then move those reads across the copy.  Only for a destination that no read
// between the copy and its s_waitcnt + barrier touches (the other buffer of a double buffer).
__device__ __forceinline__ void load_lds16_sa_free(const void *sbase, uint32_t voff, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_off), "v"(voff), "s"(uniform_ptr(sbase))
               : "m0");
}
// The 4-byte copy in the same form (LDS destination in a scalar register, no "memory" clobber).
__device__ __forceinline__ void load_lds4_sa_free(const void *sbase, uint32_t voff, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds_off), "v"(voff), "s"(uniform_ptr(sbase))
               : "m0");
}
__device__ __forceinline__ void load_lds4_s(const void *sbase, uint32_t voff, uint8_t *lds_base) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" ::"s"(m0v), "v"(voff), "s"(uniform_ptr(sbase))
               : "memory", "m0");
}

// Asynchronous 4-byte global -> LDS copy: lane l writes LDS bytes [lds_base + 4*l, +4).
__device__ __forceinline__ void load_lds4(const void *gsrc, uint8_t *lds_base) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(m0v), "v"(gsrc) : "memory", "m0");
}

// LDS reads at an integer LDS byte address (a constant added to the address folds into the
// instruction's offset field).
typedef const u32x4 __attribute__((address_space(3))) *lds_u32x4_ptr;
typedef const float __attribute__((address_space(3))) *lds_f32_ptr;
__device__ __forceinline__ u32x4 lds_read16(uint32_t addr) { return *(lds_u32x4_ptr)(uintptr_t)addr; }
__device__ __forceinline__ float lds_read_f32(uint32_t addr) { return *(lds_f32_ptr)(uintptr_t)addr; }
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)p;
}

// Transposed LDS read (ds_read_b64_tr_b16, gfx950).  Each lane supplies the address of 4
// consecutive 16-bit elements; within every group of 16 lanes, lane i receives element i%4 of the
// four lanes 4e + i/4, e = 0..3, in that order (checked on the GPU).  So if lane 4e+j points at
// columns c0+4j .. c0+4j+3 of row r0+e, lane i gets column c0+i of rows r0 .. r0+3.
typedef short v4i16 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 ds_read_tr16(const uint8_t *lds_addr) {
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)lds_addr);
  return __builtin_bit_cast(uint2, r);
}
__device__ __forceinline__ uint2 ds_read_tr16_at(uint32_t addr) {
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)(uintptr_t)addr);
  return __builtin_bit_cast(uint2, r);
}

// Stage a 32 KiB tile ([128 rows][256 bytes] in global memory) into LDS with the XOR swizzle
// `sw` applied, using 8 asynchronous 16-byte copies per lane of a 256-lane workgroup.  LDS
// instruction i of wave w covers rows 16i + 4w .. +3, physical column = lane%16; the lane fetches
// the logical column that the swizzle maps there.
template <int (*SW)(int)>
__device__ __forceinline__ void stage_tile_async(const uint8_t *gtile, uint8_t *lds_tile, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 16 * i + 4 * wave + (lane >> 4);
    const int pc = lane & 15;
    const int j = pc ^ SW(r);
    load_lds16(gtile + r * 256 + j * 16, lds_tile + (i * 256 + 64 * wave) * 16);
  }
}

// Makes v opaque to the optimiser at this point, so values derived from it after this point are
// recomputed there instead of being hoisted out of the enclosing loop (and held in registers).
#define AQ_OPAQUE(v) asm volatile("" : "+v"(v))

// Wait until at most N of this wave's vector-memory operations are outstanding.
#define AQ_WAIT_VMCNT(N) asm volatile("s_waitcnt vmcnt(" #N ")" ::: "memory")

// Number of leading registers, out of the 16 consecutive keys key0 .. key0+15 a lane holds, whose
// key is at most `last` (the largest key the lane's query may see; -1 for none).
__device__ __forceinline__ int valid_prefix(int64_t key0, int64_t last) {
  const int64_t rel = last - key0;
  return rel < 0 ? 0 : (rel >= 15 ? 16 : (int)rel + 1);
}

__device__ __forceinline__ int valid_prefix(int key0, int last) {
  const int rel = last - key0;
  return rel < 0 ? 0 : (rel >= 15 ? 16 : rel + 1);
}

// Set registers at and past `nvalid` to -inf (selects with constant indices, no branches).
__device__ __forceinline__ void mask_tail(f32x16 &s, int nvalid) {
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = r < nvalid ? s[r] : -__builtin_inff();
}

// The largest of three values in one v_max3_f32.  Logits are never NaN; written with fmaxf, the
// compiler would first copy each MFMA result through a quieting v_max (it cannot know they are
// canonical), a third more instructions for a block maximum.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// The largest of each of four blocks of 16 logits: eight v_max3_f32 per block, the four chains
// interleaved so that consecutive instructions are independent.
__device__ __forceinline__ void max16x4(const f32x16 (&x)[4], float (&m)[4]) {
#pragma unroll
  for (int b = 0; b < 4; ++b) m[b] = max3f(x[b][0], x[b][1], x[b][2]);
#pragma unroll
  for (int i = 3; i < 15; i += 2)
#pragma unroll
    for (int b = 0; b < 4; ++b) m[b] = max3f(m[b], x[b][i], x[b][i + 1]);
#pragma unroll
  for (int b = 0; b < 4; ++b) m[b] = max3f(m[b], x[b][15], x[b][15]);
}

// Smooth-Q: 16 consecutive fp32 values (delta of a lane's 16 keys), the initial accumulator of a
// logit chain.
__device__ __forceinline__ f32x16 delta16(const float *d) {
  f32x16 r;
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    const f32x4 v = *(const f32x4 *)(d + 4 * r4);
#pragma unroll
    for (int i = 0; i < 4; ++i) r[4 * r4 + i] = v[i];
  }
  return r;
}

// A cube-sparse chunk index, read from a selection list, clamped into [0, n): a list that is not
// the forward's (out-of-range entries) then gives meaningless numbers, never an access outside the
// K-hat/V-hat workspace.
__device__ __forceinline__ int64_t clamp_chunk(int64_t c, int64_t n) { return c < 0 ? 0 : (c >= n ? n - 1 : c); }

// XCD-aware order: workgroup i runs on XCD i % 8; give each XCD a contiguous range of work ids so
// workgroups that share a head's operands share that XCD's L2.  Returns -1 for the padding
// workgroups of the last partial range.
__device__ __forceinline__ int64_t xcd_work_id(int64_t bid, int64_t per_xcd, int64_t nwork) {
  const int64_t vid = (bid & 7) * per_xcd + (bid >> 3);
  return vid < nwork ? vid : -1;
}

}  // namespace aq
