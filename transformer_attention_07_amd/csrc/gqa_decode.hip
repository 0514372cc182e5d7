// Decode attention on gfx950: a few query rows per head (the newest Sq positions) against a
// long key/value cache of Skv keys, with the causal window-and-sinks visibility of the
// prefill kernels.  This is the cache-based generation the model card's FlashAttention
// Inference and Text Generation examples describe ("SnapKitty Transformer 8B").
//
// Bound.  Every visible K/V row of a kv head is read once for all of its H/G query heads
// and Sq rows: at most 16 x 8 rows share a 64-key tile, i.e. at most ~8 k flop per byte
// read, against a ridge near 300 for bf16 MFMA.  The pass is HBM-bound; the products
// still run on MFMA (they are dense contractions over the head dimension and the keys)
// so that the exps and the LDS traffic, not the arithmetic, are what remains per byte.
//
// Work decomposition (split-KV).  The keys visible to at least one row (sink tiles, then
// the window) form one list of 64-key tiles.  A workgroup of 4 waves serves one (batch,
// kv head, chunk of up to 128 rows) and one of `nsplit` splits; each wave is an
// independent partial that takes every (4 nsplit)-th tile of the list.  A wave streams
// its tiles through its own two K/V buffers in LDS (direct loads, no registers, rows past
// the cache read zero) and keeps an exact online softmax per row: the tile maximum, a
// rescale of O and the row sum.  It writes its unnormalised O, maximum and sum; the merge
// kernel combines the partials of each row with the log-sum-exp rule and writes O and lse.
// Nothing is shared between waves, so there is no workgroup barrier; the buffers are
// private to a wave and their loads are waited for with the wave's own counters.
//
// Per wave and tile, as in the prefill forward: S^T = K Q^T on v_mfma_f32_32x32x16 with the
// rows as the B operand held in registers (lane = row, so row statistics are in-lane plus
// one exchange between the two 32-lane halves), P^T rounded to the 16-bit type feeds
// O^T += V^T P^T from registers, and V^T comes from the row-major V tile through
// ds_read_b64_tr_b16.  The K and V operands of a tile are read once and shared by the
// (up to four) 32-row blocks.
#include "gqa_device.h"
#include "gqa_internal.h"

namespace gqa {
namespace {

constexpr float kLn2 = 0.69314718055994530942f;

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Direct-to-LDS staging of a 64-row tile by one wave: instruction j (0..7) writes lane i's
// 16 bytes to LDS bytes 1024 j + 16 i (rows 8j .. 8j+7), so the lane fetches the global
// chunk that the row's swizzle places in that slot.  Byte offset inside the tile's rows.
__device__ __forceinline__ int stage_voff(int j, int lane) {
  const int r = 8 * j + (lane >> 3);
  return r * 128 + (((lane & 7) ^ swz(r)) << 4);
}

// s_waitcnt: vector-memory count VM (0..63), LDS/scalar count LG (0..15), export count
// untouched.
template <int VM, int LG>
__device__ __forceinline__ void wait_counts() {
  static_assert(VM >= 0 && VM < 64 && LG >= 0 && LG < 16, "counter fields");
  __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (LG << 8) | (((VM >> 4) & 3) << 14));
}

// One 64-key tile (K and V row-major in LDS, rows k0 ..) against NB 32-row blocks of query
// rows held as B operands: S^T = K Q^T, the online-softmax update (exact maximum, rescale of
// O and of the row sum), O^T += V^T P^T.  `full`: every pair of the tile is visible, no mask.
template <int DT, int NB>
__device__ __forceinline__ void decode_tile(const char* kt, const char* vt, int k0, bool full,
                                            const u32x4 (&qf)[NB][4], const int (&pos)[NB],
                                            f32x16 (&o)[NB][2], float (&m)[NB], float (&l)[NB],
                                            const int (&koff)[4], const int (&voff)[2][2], int hl, float c2,
                                            int Skv, int W, int NS) {
  u32x4 ka[2][4];     // K operands [half][contraction step]
  u32x4 va[2][2][2];  // V^T operands [half][d block][step t]
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) ka[kb][ks] = *(const u32x4*)(kt + kb * 4096 + koff[ks]);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const char* base = vt + (kb * 32 + 16 * t) * 128;
        const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(__attribute__((address_space(3))) char*)(base + voff[db][0]));
        const s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(__attribute__((address_space(3))) char*)(base + voff[db][1]));
        const u32x2 ux = __builtin_bit_cast(u32x2, x), uy = __builtin_bit_cast(u32x2, y);
        va[kb][db][t] = u32x4{ux[0], ux[1], uy[0], uy[1]};
      }
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    f32x16 s[2];  // S^T of the two 32-key halves: register r is key k0 + 32 kb + 4 hl + rr(r)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = mfma32<DT>(ka[kb][0], qf[cb][0], f32x16{});
#pragma unroll
      for (int ks = 1; ks < 4; ++ks) s[kb] = mfma32<DT>(ka[kb][ks], qf[cb][ks], s[kb]);
    }
    if (!full) {
      const int i_pos = pos[cb];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = k0 + kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
          const bool vis = (j <= i_pos) & (j < Skv) & ((W == 0) | (j > i_pos - W) | (j < NS));
          s[kb][r] = vis ? s[kb][r] : -INFINITY;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = vmax(mx, s[kb][r]);
    mx = max_across_halves(mx) * c2;
    const float mnew = vmax(m[cb], mx);
    // a row with no visible key yet keeps maximum -inf: no rescale, and P = exp2(-inf) = 0
    const float alpha = mnew == -INFINITY ? 1.f : exp2_fast(m[cb] - mnew);
    const float nm = mnew == -INFINITY ? 0.f : -mnew;
    u32x4 pf[2][2];  // P^T as B operands [half][step t]
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = exp2_fast(__builtin_fmaf(s[kb][8 * t + e], c2, nm));
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          pf[kb][t][w] = pack2<DT>(pv[2 * w], pv[2 * w + 1]);
          ls += pv[2 * w] + pv[2 * w + 1];
        }
      }
    l[cb] = l[cb] * alpha + ls;
    m[cb] = mnew;
#pragma unroll
    for (int db = 0; db < 2; ++db) o[cb][db] *= alpha;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int db = 0; db < 2; ++db) o[cb][db] = mfma32<DT>(va[kb][db][t], pf[kb][t], o[cb][db]);
  }
}

template <int DT, int NRB>
__global__ __launch_bounds__(256, 1) void decode_split_kernel(DecodeParams p) {
  // Two buffers per wave, each buffer a distinct LDS object so that the compiler can tell
  // the buffer being read from the one the direct loads are filling.
  __shared__ __attribute__((aligned(1024))) char k_st0[kDecodeWaves][8192];
  __shared__ __attribute__((aligned(1024))) char k_st1[kDecodeWaves][8192];
  __shared__ __attribute__((aligned(1024))) char v_st0[kDecodeWaves][8192];
  __shared__ __attribute__((aligned(1024))) char v_st1[kDecodeWaves][8192];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  const int wg = (int)blockIdx.x;
  const int split = wg % p.nsplit;
  const int set = wg / p.nsplit;  // (b * G + g) * nrc + rc
  const int rc = set % p.nrc;
  const int bg = set / p.nrc;
  const int b = bg / p.G, g = bg % p.G;
  const int n_part = p.n_part;  // 4 * nsplit: every wave is a partial
  const int part = split * kDecodeWaves + wave;
  const int Skv = p.Skv, Sq = p.Sq;
  const int W = p.mask.window, NS = p.mask.sinks;
  const float c2 = p.scale_log2;

  // this wave's tiles: entries part, part + n_part, ... of the visible-tile list
  const int nt = p.tiles.count();
  const int my_nt = nt > part ? (nt - 1 - part) / n_part + 1 : 0;

  // Rows: lane l32 of block cb is row r = rc * 128 + 32 cb + l32 (query head g*hpg + r/Sq,
  // row r % Sq at position Skv - Sq + r % Sq); past the last row, position -1 (sees nothing).
  u32x4 qf[NRB][4];  // Q^T as B operands [row block][contraction step]
  int pos[NRB];
#pragma unroll
  for (int cb = 0; cb < NRB; ++cb) {
    const int r = rc * kDecodeRows + cb * 32 + l32;
    const bool ok = r < p.rows;
    const int hh = ok ? r / Sq : 0, t = ok ? r % Sq : 0;
    pos[cb] = ok ? Skv - Sq + t : -1;
    const uint16_t* qrow = (const uint16_t*)p.q + ((size_t)(b * p.H + g * p.hpg + hh) * Sq + t) * kHeadDim;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qf[cb][ks] = ok ? *(const u32x4*)(qrow + ks * 16 + hl * 8) : u32x4{0u, 0u, 0u, 0u};
  }
  // every row of the chunk exists (no padding lanes)
  const bool rows_full = rc * kDecodeRows + NRB * 32 <= p.rows;

  int koff[4];     // K operand: LDS row l32 of the half, chunk 2 ks + hl
  int voff[2][2];  // transposed V read [d block][second row group]
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) koff[ks] = rm_off(l32, ks * 2 + hl);
  {
    const int r0 = 4 * hl + ((lane & 15) >> 2);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int c0 = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      voff[db][0] = rm_off(r0, c0 >> 3) + (c0 & 7) * 2;
      voff[db][1] = rm_off(r0 + 8, c0 >> 3) + (c0 & 7) * 2;
    }
  }
  int soff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) soff[j] = stage_voff(j, lane);

  const size_t slab = (size_t)bg * Skv * kHeadDim;
  const __amdgpu_buffer_rsrc_t krs = slab_rsrc((const uint16_t*)p.k + slab, Skv);
  const __amdgpu_buffer_rsrc_t vrs = slab_rsrc((const uint16_t*)p.v + slab, Skv);
  // first row of this wave's tile i; past its last tile, row Skv: every load is out of
  // range and fills zeros, so the staging stays unconditional
  auto tile_row = [&](int i) __attribute__((always_inline)) {
    return i < my_nt ? p.tiles.tile(part + i * n_part) * kTile : Skv;
  };
  // 16 direct loads: the K tile, then the V tile
  auto stage = [&](char* kt, char* vt, int row0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(kt + 1024 * j), 16, row0 * 128 + soff[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(vt + 1024 * j), 16, row0 * 128 + soff[j], 0, 0, 0);
  };

  f32x16 o[NRB][2];  // O^T accumulators [row block][d block]
  float m[NRB];      // running maximum of c2 * s (log2 units)
  float l[NRB];      // running sum over this lane's half of the keys
#pragma unroll
  for (int cb = 0; cb < NRB; ++cb) {
    o[cb][0] = o[cb][1] = f32x16{};
    m[cb] = -INFINITY;
    l[cb] = 0.f;
  }

  auto compute = [&](const char* kt, const char* vt, int i) __attribute__((always_inline)) {
    const int k0 = p.tiles.tile(part + i * n_part) * kTile;
    // every row of the chunk sees every key of the tile: rows at Skv - Sq .. Skv - 1
    const bool full = __builtin_amdgcn_readfirstlane(
                          (int)rows_full & (int)(k0 + 63 <= Skv - Sq) &
                          ((int)(W == 0) | (int)(k0 > Skv - 1 - W) | (int)(k0 + 63 < NS))) != 0;
    decode_tile<DT, NRB>(kt, vt, k0, full, qf, pos, o, m, l, koff, voff, hl, c2, Skv, W, NS);
  };

  // Double-buffered stream over this wave's tiles, unrolled by two so that both buffers are
  // fixed at compile time: the next tile's 16 loads go into the other buffers, the wait
  // leaves exactly those in flight, and the LDS reads of the current buffers are waited
  // for before the next iteration's loads overwrite them.
  stage(k_st0[wave], v_st0[wave], tile_row(0));
  auto body = [&](auto par, int i) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    stage(P ? k_st0[wave] : k_st1[wave], P ? v_st0[wave] : v_st1[wave], tile_row(i + 1));
    wait_counts<16, 15>();
    asm volatile("" ::: "memory");
    compute(P ? k_st1[wave] : k_st0[wave], P ? v_st1[wave] : v_st0[wave], i);
    asm volatile("" ::: "memory");
    wait_counts<63, 0>();
  };
  for (int i = 0; i < my_nt; i += 2) {
    body(std::integral_constant<int, 0>{}, i);
    if (i + 1 >= my_nt) break;
    body(std::integral_constant<int, 1>{}, i + 1);
  }
  // no direct load may still be writing this wave's LDS when the wave ends
  wait_counts<0, 0>();
  asm volatile("" ::: "memory");

  // partial state of this wave: O^T lane column = row, registers = d db*32 + 8 (r/4) + 4 hl + r%4
  const size_t pidx = (size_t)set * n_part + part;
#pragma unroll
  for (int cb = 0; cb < NRB; ++cb) {
    const float lt = sum_across_halves(l[cb]);
    const int rr = cb * 32 + l32;
    if (rc * kDecodeRows + rr >= p.rows) continue;
    float* po = p.part_o + (pidx * kDecodeRows + rr) * kHeadDim;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = db * 32 + 8 * r4 + 4 * hl;
        *(f32x4*)(po + d0) = f32x4{o[cb][db][4 * r4], o[cb][db][4 * r4 + 1], o[cb][db][4 * r4 + 2],
                                   o[cb][db][4 * r4 + 3]};
      }
    if (hl == 0) {
      float* pml = p.part_ml + pidx * 2 * kDecodeRows;
      pml[rr] = m[cb];
      pml[kDecodeRows + rr] = lt;
    }
  }
}

// Chunks of more than 32 rows: one wave per 32-row block, and the workgroup's waves share
// each tile.  The workgroup is one partial (split) over every nsplit-th tile of the list;
// the tiles pass through a ring of kSharedStages LDS buffers filled by all waves together
// (each issues the direct loads j with j % NRB == wave), one barrier per tile.
constexpr int kSharedStages = 4;

template <int DT, int NRB>
__global__ __launch_bounds__(64 * NRB, 2) void decode_shared_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(1024))) char k_sh0[8192];
  __shared__ __attribute__((aligned(1024))) char k_sh1[8192];
  __shared__ __attribute__((aligned(1024))) char k_sh2[8192];
  __shared__ __attribute__((aligned(1024))) char k_sh3[8192];
  __shared__ __attribute__((aligned(1024))) char v_sh0[8192];
  __shared__ __attribute__((aligned(1024))) char v_sh1[8192];
  __shared__ __attribute__((aligned(1024))) char v_sh2[8192];
  __shared__ __attribute__((aligned(1024))) char v_sh3[8192];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // = row block
  const int l32 = lane & 31, hl = lane >> 5;
  const int wg = (int)blockIdx.x;
  const int split = wg % p.nsplit;
  const int set = wg / p.nsplit;  // (b * G + g) * nrc + rc
  const int rc = set % p.nrc;
  const int bg = set / p.nrc;
  const int b = bg / p.G, g = bg % p.G;
  const int n_part = p.n_part;  // nsplit: every workgroup is a partial
  const int part = split;
  const int Skv = p.Skv, Sq = p.Sq;
  const int W = p.mask.window, NS = p.mask.sinks;
  const float c2 = p.scale_log2;
  const int nt = p.tiles.count();
  const int my_nt = nt > part ? (nt - 1 - part) / n_part + 1 : 0;

  // this wave's rows: r = rc * 128 + 32 wave + l32
  u32x4 qf[1][4];
  int pos[1];
  {
    const int r = rc * kDecodeRows + wave * 32 + l32;
    const bool ok = r < p.rows;
    const int hh = ok ? r / Sq : 0, t = ok ? r % Sq : 0;
    pos[0] = ok ? Skv - Sq + t : -1;
    const uint16_t* qrow = (const uint16_t*)p.q + ((size_t)(b * p.H + g * p.hpg + hh) * Sq + t) * kHeadDim;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qf[0][ks] = ok ? *(const u32x4*)(qrow + ks * 16 + hl * 8) : u32x4{0u, 0u, 0u, 0u};
  }
  const bool rows_full = rc * kDecodeRows + NRB * 32 <= p.rows;

  int koff[4], voff[2][2], soff[8];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) koff[ks] = rm_off(l32, ks * 2 + hl);
  {
    const int r0 = 4 * hl + ((lane & 15) >> 2);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int c0 = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      voff[db][0] = rm_off(r0, c0 >> 3) + (c0 & 7) * 2;
      voff[db][1] = rm_off(r0 + 8, c0 >> 3) + (c0 & 7) * 2;
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) soff[j] = stage_voff(j, lane);

  const size_t slab = (size_t)bg * Skv * kHeadDim;
  const __amdgpu_buffer_rsrc_t krs = slab_rsrc((const uint16_t*)p.k + slab, Skv);
  const __amdgpu_buffer_rsrc_t vrs = slab_rsrc((const uint16_t*)p.v + slab, Skv);
  auto tile_row = [&](int i) __attribute__((always_inline)) {
    return i < my_nt ? p.tiles.tile(part + i * n_part) * kTile : Skv;
  };
  // this wave's share of the tile's 16 direct loads (8 K, 8 V)
  auto stage = [&](char* kt, char* vt, int row0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j % NRB == wave) {
        if (j < 8)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(kt + 1024 * j), 16, row0 * 128 + soff[j], 0, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(vt + 1024 * (j - 8)), 16,
                                                   row0 * 128 + soff[j - 8], 0, 0, 0);
      }
  };
  // loads per tile of the wave with the fewest: waiting until at most twice that many are
  // outstanding guarantees that this wave's loads of the oldest staged tile have landed
  constexpr int kMinPerTile = 16 / NRB;

  f32x16 o[1][2];
  float m[1], l[1];
  o[0][0] = o[0][1] = f32x16{};
  m[0] = -INFINITY;
  l[0] = 0.f;

  char* kb[kSharedStages] = {k_sh0, k_sh1, k_sh2, k_sh3};
  char* vb[kSharedStages] = {v_sh0, v_sh1, v_sh2, v_sh3};
#pragma unroll
  for (int u = 0; u < kSharedStages - 1; ++u) stage(kb[u], vb[u], tile_row(u));
  // Tile i: wait for this wave's loads of tile i, barrier (every wave's loads of tile i have
  // landed and every wave is done with tile i - 1), load tile i + 3 into tile i - 1's buffer,
  // compute tile i.
  auto body = [&](auto par, int i) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    constexpr int F = (P + kSharedStages - 1) % kSharedStages;
    asm volatile("" ::: "memory");
    wait_counts<2 * kMinPerTile, 0>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    stage(kb[F], vb[F], tile_row(i + kSharedStages - 1));
    const int k0 = tile_row(i);
    const bool full = __builtin_amdgcn_readfirstlane(
                          (int)rows_full & (int)(k0 + 63 <= Skv - Sq) &
                          ((int)(W == 0) | (int)(k0 > Skv - 1 - W) | (int)(k0 + 63 < NS))) != 0;
    decode_tile<DT, 1>(kb[P], vb[P], k0, full, qf, pos, o, m, l, koff, voff, hl, c2, Skv, W, NS);
  };
  for (int i = 0; i < my_nt; i += kSharedStages) {
    body(std::integral_constant<int, 0>{}, i);
    if (i + 1 >= my_nt) break;
    body(std::integral_constant<int, 1>{}, i + 1);
    if (i + 2 >= my_nt) break;
    body(std::integral_constant<int, 2>{}, i + 2);
    if (i + 3 >= my_nt) break;
    body(std::integral_constant<int, 3>{}, i + 3);
  }
  // no direct load may still be writing this workgroup's LDS when its waves end
  wait_counts<0, 0>();
  asm volatile("" ::: "memory");

  const size_t pidx = (size_t)set * n_part + part;
  const float lt = sum_across_halves(l[0]);
  const int rr = wave * 32 + l32;
  if (rc * kDecodeRows + rr >= p.rows) return;
  float* po = p.part_o + (pidx * kDecodeRows + rr) * kHeadDim;
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d0 = db * 32 + 8 * r4 + 4 * hl;
      *(f32x4*)(po + d0) = f32x4{o[0][db][4 * r4], o[0][db][4 * r4 + 1], o[0][db][4 * r4 + 2], o[0][db][4 * r4 + 3]};
    }
  if (hl == 0) {
    float* pml = p.part_ml + pidx * 2 * kDecodeRows;
    pml[rr] = m[0];
    pml[kDecodeRows + rr] = lt;
  }
}

// One wave per output row (b, h, t): lane = d.  O = sum_p w_p O_p / sum_p w_p l_p with
// w_p = 2^(m_p - max_p m_p); lse = (max_p m_p + log2 sum_p w_p l_p) ln 2.
template <int DT>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams p) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);  // over B * H * Sq
  if (row >= (long long)p.B * p.H * p.Sq) return;
  const int t = (int)(row % p.Sq);
  const long long bh = row / p.Sq;
  const int h = (int)(bh % p.H), b = (int)(bh / p.H);
  const int g = h / p.hpg, hh = h % p.hpg;
  const int r = hh * p.Sq + t, rc = r / kDecodeRows, rr = r % kDecodeRows;
  const int set = (b * p.G + g) * p.nrc + rc;
  const int n_part = p.n_part;
  const float* ml = p.part_ml + (size_t)set * n_part * 2 * kDecodeRows + rr;
  const float* po = p.part_o + ((size_t)set * n_part * kDecodeRows + rr) * kHeadDim + lane;
  // unrolled so that the partials' loads are in flight together
  float mstar = -INFINITY;
#pragma unroll 8
  for (int i = 0; i < n_part; ++i) mstar = vmax(mstar, ml[(size_t)i * 2 * kDecodeRows]);
  float L = 0.f, acc = 0.f;
#pragma unroll 8
  for (int i = 0; i < n_part; ++i) {
    const float mi = ml[(size_t)i * 2 * kDecodeRows];
    const float w = mi == -INFINITY ? 0.f : exp2_fast(mi - mstar);
    L += w * ml[(size_t)i * 2 * kDecodeRows + kDecodeRows];
    acc += w * po[(size_t)i * kDecodeRows * kHeadDim];
  }
  const float out = acc / L;
  ((uint16_t*)p.o)[row * kHeadDim + lane] = (uint16_t)(pack2<DT>(out, 0.f) & 0xFFFFu);
  if (lane == 0) p.lse[row] = (mstar + log2f(L)) * kLn2;
}

template <int DT>
hipError_t launch_split(const DecodeParams& p, int nrb, dim3 grid, hipStream_t s) {
  void* args[] = {(void*)&p};
  if (p.shared_tiles) {
    switch (nrb) {
      case 2: return hipLaunchKernel((const void*)decode_shared_kernel<DT, 2>, grid, dim3(128), args, 0, s);
      case 3: return hipLaunchKernel((const void*)decode_shared_kernel<DT, 3>, grid, dim3(192), args, 0, s);
      default: return hipLaunchKernel((const void*)decode_shared_kernel<DT, 4>, grid, dim3(256), args, 0, s);
    }
  }
  // chunks of at most 32 rows (one row block) run the wave-private kernel
  return hipLaunchKernel((const void*)decode_split_kernel<DT, 1>, grid, dim3(64 * kDecodeWaves), args, 0, s);
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int dtype, hipStream_t s) {
  const int nrb = (imin(p.rows, kDecodeRows) + 31) / 32;  // 32-row blocks of the fullest chunk
  const dim3 grid1((unsigned)((long long)p.B * p.G * p.nrc * p.nsplit));
  hipError_t e = dtype == kDtBF16 ? launch_split<kDtBF16>(p, nrb, grid1, s) : launch_split<kDtF16>(p, nrb, grid1, s);
  if (e != hipSuccess) return e;
  const dim3 grid2((unsigned)(((long long)p.B * p.H * p.Sq + 3) / 4)), block2(256);
  void* args[] = {(void*)&p};
  if (dtype == kDtBF16) return hipLaunchKernel((const void*)decode_merge_kernel<kDtBF16>, grid2, block2, args, 0, s);
  return hipLaunchKernel((const void*)decode_merge_kernel<kDtF16>, grid2, block2, args, 0, s);
}

}  // namespace gqa
