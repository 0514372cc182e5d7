// Device helpers for the gfx950 MFMA attention kernels.
//
// Matrix core instruction: v_mfma_f32_32x32x16_{bf16,f16}, D[32x32] += A[32x16] B[16x32]
// on one 64-lane wavefront.  Operand layout (A and B alike): lane l holds 8 consecutive
// k-elements of row/column (l % 32), k-group (l / 32).  Accumulator layout: lane l holds
// column (l % 32) and register r holds row 8*(r/4) + 4*(l/32) + (r%4).
//
// Two LDS tile layouts, both for 64 x 64 tiles of 16-bit elements (8 KiB):
//   * row-major ("RM"): element (row, c) at row*128 + 16*((c/8) ^ swz(row)) + 2*(c%8).
//     A 128-byte row covers half of the 64 banks, so bank group = (row parity, stored
//     chunk).  swz maps row bits (r0, r1, r2, r3) to chunk-XOR bits
//     (r2 ^ r3, r0 ^ r2, r1), which makes both read shapes conflict free:
//       - ds_read_b128 of one chunk over 16 aligned consecutive rows (16 lanes per LDS
//         cycle): for either parity the 8 rows take 8 distinct swz values;
//       - ds_read_b64_tr_b16 over 4 aligned consecutive rows x 4 aligned chunks (32 lanes
//         per cycle): rows r and r + 2 share a parity and differ in swz bit 2, so they land
//         on the two disjoint aligned 4-chunk groups.
//     Stores write 8 distinct chunks of one row and rows of both parities per cycle.
//     An A operand whose contraction index is the column (e.g. K for K Q^T) is one
//     ds_read_b128 per lane.
//   * transposed ("TR"): element (row, c) stored in LDS row c, so that an A operand
//     whose contraction index is the tile row (e.g. V^T for V^T P^T) is contiguous.
//     Within each group of 16 tile rows, row 8a + 4h + x (a, h in {0,1}, x in 0..3) is
//     stored at position 8h + 4a + x.  With that order, the 8 elements a lane of
//     k-group h reads for contraction step t of key block kb are exactly the tile rows
//     held by accumulator registers 8t..8t+7 of a lane of the same k-group, so an
//     accumulator (S^T, P^T, dS) feeds the next MFMA as a B operand straight from
//     registers.  Chunks are swizzled by swz(c) as in RM.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gqa_internal.h"

namespace gqa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

enum { kDtF32 = 0, kDtBF16 = 1, kDtF16 = 2 };

template <int DT>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c);

template <>
__device__ __forceinline__ f32x16 mfma32<kDtBF16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x16 mfma32<kDtF16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Round two floats to the 16-bit element type (nearest even) and pack: a in the low half.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b);

template <>
__device__ __forceinline__ uint32_t pack2<kDtBF16>(float a, float b) {
  bf16x2 r = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, r);
}

template <>
__device__ __forceinline__ uint32_t pack2<kDtF16>(float a, float b) {
  f16x2 r = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, r);
}

// Residual of a rounded pair: pack2(a - round(a), b - round(b)), so that hi + lo carries
// about twice the element type's mantissa (used where many products pile onto one sum).
template <int DT>
__device__ __forceinline__ uint32_t pack2_residual(float a, float b, uint32_t hi);

template <>
__device__ __forceinline__ uint32_t pack2_residual<kDtBF16>(float a, float b, uint32_t hi) {
  const float ha = __builtin_bit_cast(float, hi << 16), hb = __builtin_bit_cast(float, hi & 0xffff0000u);
  return pack2<kDtBF16>(a - ha, b - hb);
}

template <>
__device__ __forceinline__ uint32_t pack2_residual<kDtF16>(float a, float b, uint32_t hi) {
  const f16x2 h = __builtin_bit_cast(f16x2, hi);
  return pack2<kDtF16>(a - (float)h[0], b - (float)h[1]);
}

// 16-bit element (low half of w if hi == 0) to float.
template <int DT>
__device__ __forceinline__ float elem_to_f32(uint32_t w, int hi);

template <>
__device__ __forceinline__ float elem_to_f32<kDtBF16>(uint32_t w, int hi) {
  return __builtin_bit_cast(float, hi ? (w & 0xffff0000u) : (w << 16));
}

template <>
__device__ __forceinline__ float elem_to_f32<kDtF16>(uint32_t w, int hi) {
  uint16_t bits = (uint16_t)(hi ? (w >> 16) : (w & 0xffffu));
  return (float)__builtin_bit_cast(_Float16, bits);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// NaN-propagating maximum: lowers to v_maximum3_f32 with no canonicalising moves.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// acc + a.lo + a.hi for a packed pair of 16-bit values (v_dot2 with (1, 1)).
template <int DT>
__device__ __forceinline__ float add_pair(uint32_t a, float acc);

template <>
__device__ __forceinline__ float add_pair<kDtBF16>(uint32_t a, float acc) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), ones, acc, false);
}

template <>
__device__ __forceinline__ float add_pair<kDtF16>(uint32_t a, float acc) {
  const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), ones, acc, false);
}

// Value the lane (l ^ 32) holds, combined with ours: returns {ours, theirs} reduced by op.
__device__ __forceinline__ float max_across_halves(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto pr = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)pr[0]), __builtin_bit_cast(float, (uint32_t)pr[1]));
}

__device__ __forceinline__ float sum_across_halves(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto pr = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)pr[0]) + __builtin_bit_cast(float, (uint32_t)pr[1]);
}

__device__ __forceinline__ bool wave_any(bool c) { return __builtin_amdgcn_ballot_w64(c) != 0; }

// ---- LDS layouts (byte offsets inside one 8 KiB tile) ----
__device__ __forceinline__ int swz(int row) {
  return (((row >> 2) ^ (row >> 3)) & 1) | (((row ^ (row >> 2)) & 1) << 1) | ((row & 2) << 1);
}

__device__ __forceinline__ int rm_off(int row, int chunk) { return row * 128 + ((chunk ^ swz(row)) << 4); }

// TR layout: byte offset of the 16-byte chunk `chunk` (0..7) of LDS row `c`.
__device__ __forceinline__ int tr_chunk_off(int c, int chunk) { return c * 128 + ((chunk ^ swz(c)) << 4); }

// A-operand reads.  RM: rows blk*32 + (l%32), contraction chunk 2*ks + (l/32).
__device__ __forceinline__ u32x4 lds_rm_operand(const char* tile, int blk, int ks, int l32, int hl) {
  return *(const u32x4*)(tile + rm_off(blk * 32 + l32, ks * 2 + hl));
}
// TR: LDS row (output row) blk*32 + (l%32); contraction tile rows 32*kb + 16*t + ..., the
// 16-byte chunk 4*kb + 2*t + (l/32).
__device__ __forceinline__ u32x4 lds_tr_operand(const char* tile, int blk, int kb, int t, int l32, int hl) {
  const int c = blk * 32 + l32;
  return *(const u32x4*)(tile + tr_chunk_off(c, kb * 4 + t * 2 + hl));
}

// Transposed A operand from a row-major tile with ds_read_b64_tr_b16.  Within each group of
// 16 lanes that instruction returns to lane i element (i & 3) of the 4-element row that lane
// 4e + (i >> 2) addressed, for e = 0..3.  If lane j of the group addresses row r0 + (j >> 2),
// columns c0 + 4 (j & 3) .. + 3, lane i therefore receives rows r0 .. r0 + 3 of column c0 + i:
// a column segment, which is what an operand contracting over tile rows needs.
// Output: the A operand for output rows (tile columns) blk*32 + (l%32) and contraction rows
// 32*kb + 16*t + {4h..4h+3, 8+4h..8+4h+3} (h = l/32), the order of the TR layout above.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 lds_rm_transposed_operand(const char* tile, int blk, int kb, int t, int lane) {
  const int h = lane >> 5;
  const int c0 = blk * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int r0 = kb * 32 + 16 * t + 4 * h + ((lane & 15) >> 2);
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const char* pa = tile + rm_off(r0, c0 >> 3) + (c0 & 7) * 2;
  const char* pb = tile + rm_off(r0 + 8, c0 >> 3) + (c0 & 7) * 2;
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(__attribute__((address_space(3))) char*)pa);
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(__attribute__((address_space(3))) char*)pb);
  const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  return u32x4{ua[0], ua[1], ub[0], ub[1]};
}

// ---- staging of a 64 x 64 tile from global memory ----
// One "unit" = 4 consecutive tile rows r0..r0+3 (r0 % 4 == 0) times one 16-byte column
// chunk dc (8 elements).  128 units cover a tile; a thread loads its unit into registers
// (rows >= S read as zero), then writes it as RM and/or TR.
struct Unit {
  u32x4 x[4];
};

__device__ __forceinline__ void unit_load(Unit& u, const uint16_t* slab, int row0, int dc, int S) {
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int row = row0 + n;
    if (row < S) {
      u.x[n] = *(const u32x4*)(slab + (size_t)row * kHeadDim + dc * 8);
    } else {
      u.x[n] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

__device__ __forceinline__ void unit_store_rm(char* tile, const Unit& u, int r0, int dc) {
#pragma unroll
  for (int n = 0; n < 4; ++n) *(u32x4*)(tile + rm_off(r0 + n, dc)) = u.x[n];
}

__device__ __forceinline__ void unit_store_tr(char* tile, const Unit& u, int r0, int dc) {
  const int q4 = r0 >> 2;                 // which group of 4 rows
  const int chunk = (q4 >> 2) * 2 + (q4 & 1);  // 16-row group * 2 + h
  const int a = (q4 >> 1) & 1;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = dc * 8 + e;
    const int w = e >> 1;
    uint32_t lo, hi;
    if (e & 1) {
      lo = (u.x[0][w] >> 16) | (u.x[1][w] & 0xffff0000u);
      hi = (u.x[2][w] >> 16) | (u.x[3][w] & 0xffff0000u);
    } else {
      lo = (u.x[0][w] & 0xffffu) | (u.x[1][w] << 16);
      hi = (u.x[2][w] & 0xffffu) | (u.x[3][w] << 16);
    }
    *(u32x2*)(tile + tr_chunk_off(c, chunk) + a * 8) = u32x2{lo, hi};
  }
}

// ---- buffer loads ----
// A buffer resource over a [rows][64] slab of 16-bit elements: raw loads at or past the end
// of the slab return zero, so ragged tiles need no bounds branches.  Offsets are bytes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slab_rsrc(const void* base, int rows) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, rows * kHeadDim * 2, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

__device__ __forceinline__ void unit_load_buf(Unit& u, __amdgpu_buffer_rsrc_t r, int row0, int dc) {
#pragma unroll
  for (int n = 0; n < 4; ++n) u.x[n] = buf_load16(r, (row0 + n) * (kHeadDim * 2) + dc * 16);
}

// Row-major-only staging: register n holds row row0 + (n ^ flip), flip = 1 for odd units, so
// that one store instruction writes rows of both parities (both halves of the banks).
__device__ __forceinline__ void unit_load_buf_rm(Unit& u, __amdgpu_buffer_rsrc_t r, int row0, int dc, int flip) {
#pragma unroll
  for (int n = 0; n < 4; ++n) u.x[n] = buf_load16(r, (row0 + (n ^ flip)) * (kHeadDim * 2) + dc * 16);
}

__device__ __forceinline__ void unit_store_rm_flip(char* tile, const Unit& u, int r0, int dc, int flip) {
#pragma unroll
  for (int n = 0; n < 4; ++n) *(u32x4*)(tile + rm_off(r0 + (n ^ flip), dc)) = u.x[n];
}

// Row of the accumulator register r of this lane, inside a 32-row block.
__device__ __forceinline__ int acc_row(int r, int hl) { return 8 * (r >> 2) + 4 * hl + (r & 3); }

// ---- rotary position embedding ----
// m cos and m sin of the angle of a dimension pair at position pos, for a pair turning rev
// revolutions per position: pos * rev is formed in fp64 (within an fp64 ulp for any int
// position) and its whole revolutions dropped there, so the remaining f in [-1/2, 1/2]
// revolution is accurate to fp32 rounding at any position.  The hardware sine and cosine
// take their argument in revolutions; on [-1/2, 1/2] they are within 1.3e-7 of the exact
// values (measured on gfx950 over 2^24 evenly spaced points), about 2 fp32 ulps.  R^T (the
// backward) flips the sine.
__device__ __forceinline__ void rope_cs(int pos, double rev, float mscale, bool inverse, float& mc, float& ms) {
  const double t = (double)pos * rev;
  const float f = (float)(t - __builtin_rint(t));
  const float s = __builtin_amdgcn_sinf(f), c = __builtin_amdgcn_cosf(f);
  mc = mscale * c;
  ms = inverse ? -(mscale * s) : mscale * s;
}

// The pair (x0, x1) rotated by the angle whose m cos and m sin are mc and ms.
__device__ __forceinline__ void rope_pair(float& x0, float& x1, float mc, float ms) {
  const float y0 = __builtin_fmaf(x0, mc, -(x1 * ms));
  const float y1 = __builtin_fmaf(x0, ms, x1 * mc);
  x0 = y0;
  x1 = y1;
}

// Rotate back (m R^T at position pos) the two pairs held in 4 consecutive fp32 gradient
// values that start at pair index pi.
__device__ __forceinline__ f32x4 rope_back4(f32x4 v, int pos, const RopeSpec& r, int pi) {
  float x0 = v[0], x1 = v[1], x2 = v[2], x3 = v[3];
  float mc, ms;
  rope_cs(pos, r.rev[pi], r.mscale, true, mc, ms);
  rope_pair(x0, x1, mc, ms);
  rope_cs(pos, r.rev[pi + 1], r.mscale, true, mc, ms);
  rope_pair(x2, x3, mc, ms);
  return f32x4{x0, x1, x2, x3};
}

// Rotate the 4 pairs packed in w (8 16-bit elements) at position pos; rev[j] is the
// frequency of the j-th pair.
template <int DT>
__device__ __forceinline__ u32x4 rope_chunk16(u32x4 w, int pos, const double (&rev)[4], float mscale, bool inverse) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float mc, ms;
    rope_cs(pos, rev[j], mscale, inverse, mc, ms);
    float x0 = elem_to_f32<DT>(w[j], 0), x1 = elem_to_f32<DT>(w[j], 1);
    rope_pair(x0, x1, mc, ms);
    w[j] = pack2<DT>(x0, x1);
  }
  return w;
}

// Which (row block, head group) a forward workgroup serves (bf16 and FP8 forwards alike:
// Params has n_qblk, B, H, hpw, xcd_hg, xcd_kv).  Longest row blocks first in both
// orders.  Workgroup j runs on XCD j mod 8; in the plain order consecutive workgroups take
// consecutive head groups, so an XCD serves every eighth head group and a kv head's K/V
// tiles pass through two XCDs' L2 caches.  With xcd_hg > 0 (B * H / hpw a multiple of 8,
// each XCD's share of whole kv heads) XCD x serves head groups x * xcd_hg .. + xcd_hg - 1,
// one row block of each after the other: fewer kv heads per L2 at any time.
template <class Params>
__device__ __forceinline__ void fwd_block_order(const Params& p, int j, int& qblk, int& rest) {
  if (p.xcd_hg > 0 && p.xcd_kv > 0) {
    const int x = j & 7, pos = j >> 3;
    const int per_kv = p.n_qblk * p.xcd_kv;  // workgroups of one kv head
    const int kvi = pos / per_kv, r = pos % per_kv;
    qblk = p.n_qblk - 1 - r / p.xcd_kv;
    rest = x * p.xcd_hg + kvi * p.xcd_kv + r % p.xcd_kv;
  } else if (p.xcd_hg > 0) {
    const int x = j & 7, pos = j >> 3;
    qblk = p.n_qblk - 1 - pos / p.xcd_hg;
    rest = x * p.xcd_hg + pos % p.xcd_hg;
  } else {
    const int per_q = p.B * (p.H / p.hpw);
    qblk = p.n_qblk - 1 - j / per_q;
    rest = j % per_q;
  }
}

}  // namespace gqa
