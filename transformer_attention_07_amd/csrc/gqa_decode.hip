// Decode attention on gfx950: a few query rows per head (the newest Sq positions) against a
// long key/value cache of Skv keys, with the causal window-and-sinks visibility of the
// prefill kernels.  This is the cache-based generation the model card's FlashAttention
// Inference and Text Generation examples describe ("SnapKitty Transformer 8B").
//
// Bound.  Every visible K/V row of a kv head is read once for all of its H/G query heads
// and Sq rows: at most 128 rows share a 64-key tile, i.e. at most 128 flop per byte read
// (256 flop per row and key against 256 bytes of K and V per key), against a ridge near
// 300 for bf16 MFMA.  The pass is HBM-bound, but at 128 rows its products and exps are
// close to half of the stream's time, so they run on MFMA (dense contractions over the
// head dimension and the keys) and overlap the loads.
//
// Work decomposition (split-KV).  The keys visible to at least one row (sink tiles, then
// the window) form one list of 64-key tiles, dealt round-robin to the partials of each
// (batch, kv head, chunk of up to 128 rows); a merge kernel combines the partials of each
// row with the log-sum-exp rule and writes O and lse.
//  * Chunks of at most 32 rows: a workgroup of 4 waves, each wave an independent partial
//    over every (4 nsplit)-th tile, streaming them through its own two K/V buffers in LDS
//    (direct loads, rows past the cache read zero) and waiting with its own counters: no
//    workgroup barrier.
//  * Larger chunks: one wave per 32-row block, the workgroup one partial; its waves fill a
//    5-stage LDS ring together and share every tile, one barrier per tile, and work in the
//    prefill forward's unit pipeline (a unit's softmax beside the previous unit's P V and
//    the next unit's scores).
// Both keep an online softmax with the prefill forward's lazy maximum (a tile is
// exponentiated against the running maximum unless a lane's partial row sum leaves its
// guard) and write their unnormalised O, maximum and sum.
//
// Per wave and tile, as in the prefill forward: S^T = K Q^T on v_mfma_f32_32x32x16 with the
// rows as the B operand held in registers (lane = row, so row statistics are in-lane plus
// one exchange between the two 32-lane halves), P^T rounded to the 16-bit type feeds
// O^T += V^T P^T from registers, and V^T comes from the row-major V tile through
// ds_read_b64_tr_b16.  The K and V operands of a tile are read once per wave and shared by
// its row blocks.
#include <type_traits>

#include "gqa_device.h"
#include "gqa_internal.h"

namespace gqa {
namespace {

constexpr float kLn2 = 0.69314718055994530942f;
// Lazy maximum (see decode_tile): a tile is redone against its own maximum when a lane's
// partial row sum exceeds this, and the running maximum is raised when the tile's exceeds
// it by more than kDecodeRescale (log2 units).
constexpr float kDecodeSumGuard = 65536.0f;
constexpr float kDecodeRescale = 8.0f;

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

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

// One direct load of 16 bytes per lane into LDS at dst + 16 lane.  (A plain function: the
// builtin called straight from a generic lambda makes the host pass drop the kernel's
// launch stub without a diagnostic.)
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t rs, lds_char* dst, int off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)dst, 16, off, 0, 0, 0);
}

// One 64-key tile (K and V row-major in LDS, rows k0 ..) against NB 32-row blocks of query
// rows held as B operands: S^T = K Q^T, the online-softmax update (exact maximum, rescale of
// O and of the row sum), O^T += V^T P^T.  `full`: every pair of the tile is visible, no mask.
template <int DT, int NB>
__device__ __forceinline__ void decode_tile(const lds_char* kt, const lds_char* vt, int k0, bool full,
                                            const u32x4 (&qf)[NB][4], const int (&pos)[NB],
                                            f32x16 (&o)[NB][2], float (&m)[NB], float (&l)[NB],
                                            const int (&koff)[4], const int (&voff)[2][2], int hl, float c2,
                                            int Skv, int W, int NS) {
  u32x4 ka[2][4];     // K operands [half][contraction step]
  u32x4 va[2][2][2];  // V^T operands [half][d block][step t]
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) ka[kb][ks] = *(const lds_u32x4*)(kt + kb * 4096 + koff[ks]);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const lds_char* base = vt + (kb * 32 + 16 * t) * 128;
        const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + voff[db][0]));
        const s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + voff[db][1]));
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
    // Lazy maximum, as in the prefill forward: the tile is exponentiated against the running
    // maximum m, which only keeps exp2 in range.  When a lane's partial row sum leaves
    // (0, kSumGuard] (some P > 2^16 / 64, an overflow) or a row inside the sequence has no
    // maximum yet, the tile takes the exact path: its maximum, the running maximum raised
    // when it grew by more than 2^8 (with O and the sum rescaled), and exponentiated again.
    u32x4 pf[2][2];  // P^T as B operands [half][step t]
    float ls = 0.f;
    auto exponentiate = [&](float nm) __attribute__((always_inline)) {
      ls = 0.f;
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
    };
    exponentiate(m[cb] == -INFINITY ? 0.f : -m[cb]);
    const bool need = !(ls <= kDecodeSumGuard) | ((m[cb] == -INFINITY) & (pos[cb] >= 0));
    if (__builtin_expect(wave_any(need), 0)) {
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = vmax(mx, s[kb][r]);
      mx = max_across_halves(mx) * c2;
      // raise the maximum when it grew by more than 2^8 (or the row had none)
      const float mnew = (mx > m[cb] + kDecodeRescale) ? mx : m[cb];
      // a row with no visible key yet keeps maximum -inf: no rescale, and P = exp2(-inf) = 0
      const float alpha = mnew == -INFINITY || m[cb] == -INFINITY ? 1.f : exp2_fast(m[cb] - mnew);
      asm volatile("" ::: "memory");  // keep the rescale inside this rare branch
      l[cb] *= alpha;
#pragma unroll
      for (int db = 0; db < 2; ++db) o[cb][db] *= alpha;
      m[cb] = mnew;
      exponentiate(mnew == -INFINITY ? 0.f : -mnew);
    }
    l[cb] += ls;
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
  auto stage = [&](lds_char* kt, lds_char* vt, int row0) __attribute__((always_inline)) {
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

  auto compute = [&](const lds_char* kt, const lds_char* vt, int i) __attribute__((always_inline)) {
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
  lds_char* const k0b = (lds_char*)k_st0[wave];
  lds_char* const k1b = (lds_char*)k_st1[wave];
  lds_char* const v0b = (lds_char*)v_st0[wave];
  lds_char* const v1b = (lds_char*)v_st1[wave];
  stage(k0b, v0b, tile_row(0));
  auto body = [&](auto par, int i) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    stage(P ? k0b : k1b, P ? v0b : v1b, tile_row(i + 1));
    wait_counts<16, 15>();
    asm volatile("" ::: "memory");
    compute(P ? k1b : k0b, P ? v1b : v0b, i);
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
constexpr int kSharedStages = 5;

// The ring's buffers, each a distinct LDS object selected at compile time, so that every
// LDS address is a known constant (typed LDS pointers from here on: no generic pointer is
// ever cast back to LDS).  A stage holds a tile's K (bytes 0..8191) and V (8192..16383):
// one object per stage keeps the direct loads in flight within the compiler's count of
// LDS objects it tells apart (more objects and it waits for every load before some reads).
__shared__ __attribute__((aligned(1024))) char g_dec_t0[16384];
__shared__ __attribute__((aligned(1024))) char g_dec_t1[16384];
__shared__ __attribute__((aligned(1024))) char g_dec_t2[16384];
__shared__ __attribute__((aligned(1024))) char g_dec_t3[16384];
__shared__ __attribute__((aligned(1024))) char g_dec_t4[16384];
// f(integral_constant<int, U>) for U = B .. E - 1, in order
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

template <int U>
__device__ __forceinline__ lds_char* ring_k() {
  static_assert(U >= 0 && U < kSharedStages, "ring slot");
  if constexpr (U == 0) return (lds_char*)g_dec_t0;
  else if constexpr (U == 1) return (lds_char*)g_dec_t1;
  else if constexpr (U == 2) return (lds_char*)g_dec_t2;
  else if constexpr (U == 3) return (lds_char*)g_dec_t3;
  else return (lds_char*)g_dec_t4;
}
template <int U>
__device__ __forceinline__ lds_char* ring_v() {
  return ring_k<U>() + 8192;
}

// The running maximum of a row before its first visible key: a finite value below every
// score (log2 units), so that the first visible key exponentiates to +inf and the row-sum
// guard takes the exact path; masked keys (-inf) still give 0.  A partial that never sees
// a key keeps it, and its merge weight 2^(-1e38 - m) is 0.
constexpr float kDecodeNoMax = -1.0e38f;

// One wave's 32 query rows (lane column l32 = row) in the shared-tile kernel, worked in
// units of one 32-key half of a tile: S^T = K Q^T on MFMA, the online softmax with the lazy
// maximum, O^T += V^T P^T.  Row r of the wave sits at position pos (-1: no row).
template <int DT>
struct DecWave {
  int hl;
  int pos;
  float c2;
  u32x4 qf[4];     // the rows as B operands [contraction step]
  f32x16 o[2];     // O^T accumulators [d block]
  float mrow;      // running maximum (log2 units), kDecodeNoMax before any key
  float lrow;      // running sum (this lane's half of the keys)
  float nmuse;     // -mrow
  int koff[4];     // lane's byte offset of the K operand, step ks (half 0)
  int voff[2][2];  // lane's byte offset of the transposed V read [d block][second row group]

  __device__ __forceinline__ void load_k(const lds_char* kt, int kb, u32x4 (&a)[4]) const {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) a[ks] = *(const lds_u32x4*)(kt + kb * 4096 + koff[ks]);
  }
  __device__ __forceinline__ void scores(const u32x4 (&a)[4], f32x16& s) const {
    s = mfma32<DT>(a[0], qf[0], f32x16{});
#pragma unroll
    for (int ks = 1; ks < 4; ++ks) s = mfma32<DT>(a[ks], qf[ks], s);
  }
  __device__ __forceinline__ void load_v(const lds_char* vt, int kb, u32x4 (&a)[2][2]) const {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const lds_char* base = vt + (kb * 32 + 16 * t) * 128;
        const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + voff[db][0]));
        const s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + voff[db][1]));
        const u32x2 ux = __builtin_bit_cast(u32x2, x), uy = __builtin_bit_cast(u32x2, y);
        a[db][t] = u32x4{ux[0], ux[1], uy[0], uy[1]};
      }
  }
  __device__ __forceinline__ void accumulate(const u32x4 (&a)[2][2], const u32x4 (&pf)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < 2; ++db) o[db] = mfma32<DT>(a[db][t], pf[t], o[db]);
  }
  // hide the keys of half [k, k + 31] this lane's row does not see: register r holds key
  // k + 4 hl + 8 (r / 4) + r % 4
  __device__ __forceinline__ void mask(f32x16& s, int k, int Skv, int W, int NS) const {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = k + 8 * (r >> 2) + 4 * hl + (r & 3);
      const bool vis = (j <= pos) & (j < Skv) & ((W == 0) | (j > pos - W) | (j < NS));
      s[r] = vis ? s[r] : -INFINITY;
    }
  }
  // raise the running maximum when the unit's exceeds it by more than kDecodeRescale (rare)
  __device__ __forceinline__ void decide(const f32x16& s) {
    float a = vmax(s[0], s[1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) a = vmax(vmax(a, s[r]), s[r + 1]);
    const float mx = max_across_halves(a) * c2;
    if (__builtin_expect(wave_any(mx > mrow + kDecodeRescale), 0)) {
      const float mnew = vmax(mrow, mx);  // finite: mrow starts at kDecodeNoMax
      const float alpha = exp2_fast(mrow - mnew);
      mrow = mnew;
      nmuse = -mnew;
      lrow *= alpha;
      asm volatile("" ::: "memory");  // keep the rescale inside this rare branch
#pragma unroll
      for (int db = 0; db < 2; ++db) o[db] *= alpha;
    }
  }
  __device__ __forceinline__ void probs(const f32x16& s, u32x4 (&pf)[2], float& ls) const {
    float lsum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = exp2_fast(__builtin_fmaf(s[8 * t + e], c2, nmuse));
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        pf[t][w] = pack2<DT>(pv[2 * w], pv[2 * w + 1]);
        lsum += pv[2 * w] + pv[2 * w + 1];
      }
    }
    ls = lsum;
  }
  // Lazy maximum, as in the prefill forward: the unit is exponentiated against the running
  // maximum, which only keeps exp2 in range; a lane's partial row sum above the guard (an
  // exponent above log2(guard / 16), the row's first visible key included) sends it
  // through the exact path.
  __device__ __forceinline__ void softmax(const f32x16& s, u32x4 (&pf)[2]) {
    float ls;
    probs(s, pf, ls);
    if (__builtin_expect(wave_any(!(ls <= kDecodeSumGuard)), 0)) {
      decide(s);
      probs(s, pf, ls);
    }
    lrow += ls;
  }
};

template <int DT, int NRB>
__global__ __launch_bounds__(64 * NRB, NRB > 2 ? 2 : 1) void decode_shared_kernel(DecodeParams p) {

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
  const int nt = p.tiles.count();
  const int my_nt = nt > part ? (nt - 1 - part) / n_part + 1 : 0;

  DecWave<DT> D;
  D.hl = hl;
  D.c2 = p.scale_log2;
  {
    // this wave's rows: r = rc * 128 + 32 wave + l32
    const int r = rc * kDecodeRows + wave * 32 + l32;
    const bool ok = r < p.rows;
    const int hh = ok ? r / Sq : 0, t = ok ? r % Sq : 0;
    D.pos = ok ? Skv - Sq + t : -1;
    const uint16_t* qrow = (const uint16_t*)p.q + ((size_t)(b * p.H + g * p.hpg + hh) * Sq + t) * kHeadDim;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      D.qf[ks] = ok ? *(const u32x4*)(qrow + ks * 16 + hl * 8) : u32x4{0u, 0u, 0u, 0u};
  }
  const bool rows_full = rc * kDecodeRows + NRB * 32 <= p.rows;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) D.koff[ks] = rm_off(l32, ks * 2 + hl);
  {
    const int r0 = 4 * hl + ((lane & 15) >> 2);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int c0 = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      D.voff[db][0] = rm_off(r0, c0 >> 3) + (c0 & 7) * 2;
      D.voff[db][1] = rm_off(r0 + 8, c0 >> 3) + (c0 & 7) * 2;
    }
  }
  // global offsets of this wave's direct loads inside a tile's rows: load wave + NRB u of
  // the K rows and the same of the V rows (NRB dividing 16), else all eight
  constexpr int kOwn = 16 % NRB == 0 ? 8 / NRB : 8;
  int soff[kOwn];
#pragma unroll
  for (int u = 0; u < kOwn; ++u) soff[u] = stage_voff(16 % NRB == 0 ? wave + NRB * u : u, lane);
  D.o[0] = D.o[1] = f32x16{};
  D.mrow = kDecodeNoMax;
  D.nmuse = -kDecodeNoMax;
  D.lrow = 0.f;

  const size_t slab = (size_t)bg * Skv * kHeadDim;
  const __amdgpu_buffer_rsrc_t krs = slab_rsrc((const uint16_t*)p.k + slab, Skv);
  const __amdgpu_buffer_rsrc_t vrs = slab_rsrc((const uint16_t*)p.v + slab, Skv);
  // rows of this workgroup's tile i; past its last tile, row Skv: loads read zeros
  auto tile_row = [&](int i) __attribute__((always_inline)) {
    return i < my_nt ? p.tiles.tile(part + i * n_part) * kTile : Skv;
  };
  // every row of the chunk sees every key of half [k, k + 31]
  auto half_full = [&](int k) __attribute__((always_inline)) {
    return __builtin_amdgcn_readfirstlane((int)rows_full & (int)(k + 31 <= Skv - Sq) &
                                          ((int)(W == 0) | (int)(k > Skv - 1 - W) | (int)(k + 31 < NS))) != 0;
  };
  // this wave's share of the tile's 16 direct loads (8 K, 8 V): loads wave + NRB u.  Each
  // load sits at a compile-time LDS offset (one branch per wave index), so the compiler
  // knows which buffer every load in flight writes.
  auto stage = [&](lds_char* kt, lds_char* vt, int row0) __attribute__((always_inline)) {
    if constexpr (16 % NRB == 0) {
      static_for<0, NRB>([&](auto wv) __attribute__((always_inline)) {
        constexpr int WV = decltype(wv)::value;
        if (wave == WV) {
#pragma unroll
          for (int u = 0; u < kOwn; ++u) lds_load16(krs, kt + 1024 * (WV + NRB * u), row0 * 128 + soff[u]);
#pragma unroll
          for (int u = 0; u < kOwn; ++u) lds_load16(vrs, vt + 1024 * (WV + NRB * u), row0 * 128 + soff[u]);
        }
      });
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (j % NRB == wave) {
          if (j < 8)
            lds_load16(krs, kt + 1024 * j, row0 * 128 + soff[j]);
          else
            lds_load16(vrs, vt + 1024 * (j - 8), row0 * 128 + soff[j - 8]);
        }
    }
  };
  // loads per tile of the wave with the fewest: waiting until at most two tiles' worth are
  // outstanding guarantees that this wave's loads of the oldest of three have landed
  constexpr int kMinPerTile = 16 / NRB;

  // Software pipeline over units (one 32-key half): a unit's softmax runs while the
  // matrix cores compute the previous unit's P V and the next unit's scores, three
  // independent pieces the compiler interleaves inside the wave.  Tile i's two units
  // read the scores of (i, 1) and (i + 1, 0), so tile i + 1 must have landed when tile
  // i starts: iteration i waits for this wave's loads of tile i + 1, then a barrier (every
  // wave's loads of tile i + 1 have landed; every wave is done with tile i - 1, whose
  // second V half the previous unit read), and at its end loads tile i + 4 into tile
  // i - 1's buffer.  Three tiles are in flight during the wait.
  static_for<0, kSharedStages - 1>([&](auto u) __attribute__((always_inline)) {
    constexpr int U = decltype(u)::value;
    stage(ring_k<U>(), ring_v<U>(), tile_row(U));
  });
  f32x16 sx, sy;               // S^T of the units at half 0 / half 1
  u32x4 ka0[4], ka1[4];        // K operands of half 0 / half 1
  u32x4 va0[2][2], va1[2][2];  // V^T operands of half 0 / half 1
  u32x4 px[2], py[2];          // P^T of the units from sx / sy
  wait_counts<(kSharedStages - 2) * kMinPerTile, 0>();  // tile 0
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  D.load_k(ring_k<0>(), 0, ka0);
  D.scores(ka0, sx);
  D.load_k(ring_k<0>(), 1, ka1);
  // the first unit's P V (of no earlier unit) adds zero
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    py[t] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int db = 0; db < 2; ++db) va1[db][t] = u32x4{0u, 0u, 0u, 0u};
  }

  // Step i: the wait, barrier and loads run on every step of the last round too (past the
  // end they load zeros, with no memory traffic), so that every path through the loop has
  // the same loads in flight; only the units are skipped past the last tile.  The loads go
  // at the step's end, after its LDS reads (issued right before them, they made the
  // compiler wait for every load in flight ahead of one of the reads).
  auto body = [&](auto par, int i) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    constexpr int P1 = (P + 1) % kSharedStages;                  // tile i + 1
    constexpr int F = (P + kSharedStages - 1) % kSharedStages;   // tile i - 1, receives i + 4
    asm volatile("" ::: "memory");
    wait_counts<(kSharedStages - 3) * kMinPerTile, 0>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (i >= my_nt) {
      stage(ring_k<F>(), ring_v<F>(), tile_row(i + kSharedStages - 1));
      return;
    }
    const int k0 = tile_row(i);
    // (i, 0) from sx; P V of (i - 1, 1); scores of (i, 1)
    if (__builtin_expect(!half_full(k0), 0)) D.mask(sx, k0, Skv, W, NS);
    D.accumulate(va1, py);
    D.scores(ka1, sy);
    D.load_k(ring_k<P1>(), 0, ka0);
    D.load_v(ring_v<P>(), 0, va0);
    D.softmax(sx, px);
    // (i, 1) from sy; P V of (i, 0); scores of (i + 1, 0)
    if (__builtin_expect(!half_full(k0 + 32), 0)) D.mask(sy, k0 + 32, Skv, W, NS);
    D.accumulate(va0, px);
    D.scores(ka0, sx);
    D.load_k(ring_k<P1>(), 1, ka1);
    D.load_v(ring_v<P>(), 1, va1);
    D.softmax(sy, py);
    stage(ring_k<F>(), ring_v<F>(), tile_row(i + kSharedStages - 1));
  };
  for (int i = 0; i < my_nt; i += kSharedStages)
    static_for<0, kSharedStages>([&](auto u) __attribute__((always_inline)) { body(u, i + decltype(u)::value); });
  D.accumulate(va1, py);  // P V of the last unit
  // no direct load may still be writing this workgroup's LDS when its waves end
  wait_counts<0, 0>();
  asm volatile("" ::: "memory");

  const size_t pidx = (size_t)set * n_part + part;
  const float lt = sum_across_halves(D.lrow);
  const int rr = wave * 32 + l32;
  if (rc * kDecodeRows + rr >= p.rows) return;
  float* po = p.part_o + (pidx * kDecodeRows + rr) * kHeadDim;
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d0 = db * 32 + 8 * r4 + 4 * hl;
      *(f32x4*)(po + d0) = f32x4{D.o[db][4 * r4], D.o[db][4 * r4 + 1], D.o[db][4 * r4 + 2], D.o[db][4 * r4 + 3]};
    }
  if (hl == 0) {
    float* pml = p.part_ml + pidx * 2 * kDecodeRows;
    pml[rr] = D.mrow;
    pml[kDecodeRows + rr] = lt;
  }
}

// One wave per output row (b, h, t): lane = d.  O = sum_p w_p O_p / sum_p w_p l_p with
// w_p = 2^(m_p - max_p m_p); lse = (max_p m_p + log2 sum_p w_p l_p) ln 2.  The partials
// go in groups of kMergeGroup: lane j loads the maximum and sum of partial c + j while
// every lane loads its element of all the group's O rows, all in one round trip (the
// work is a few KB per row, so latency, not bandwidth, sets its time); the weights reach
// every lane through readlane.  Between groups the running maximum, sum and O are
// rescaled as in the online softmax.
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
  constexpr int kMergeGroup = 32;
  float mrun = -INFINITY, L = 0.f, acc = 0.f;
  for (int c = 0; c < n_part; c += kMergeGroup) {
    const int cnt = imin(kMergeGroup, n_part - c);
    const bool mine = lane < cnt;
    const float mi = mine ? ml[(size_t)(c + lane) * 2 * kDecodeRows] : -INFINITY;
    const float li = mine ? ml[(size_t)(c + lane) * 2 * kDecodeRows + kDecodeRows] : 0.f;
    float ov[kMergeGroup];
#pragma unroll
    for (int u = 0; u < kMergeGroup; ++u) ov[u] = u < cnt ? po[(size_t)(c + u) * kDecodeRows * kHeadDim] : 0.f;
    float mg = mi;
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) mg = vmax(mg, __shfl_xor(mg, s, 64));
    const float mnew = vmax(mrun, mg);
    // a partial (or the groups so far) with no visible key has maximum -inf (the
    // shared-tile kernel's: -1e38) and weight 0
    const float keep = mrun == -INFINITY ? 0.f : exp2_fast(mrun - mnew);
    const float w = mi == -INFINITY ? 0.f : exp2_fast(mi - mnew);
    float wl = w * li;
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) wl += __shfl_xor(wl, s, 64);
    L = L * keep + wl;
    acc *= keep;
    const int wbits = __builtin_bit_cast(int, w);
#pragma unroll
    for (int u = 0; u < kMergeGroup; ++u)
      acc += __builtin_bit_cast(float, __builtin_amdgcn_readlane(wbits, u)) * ov[u];
    mrun = mnew;
  }
  const float out = acc / L;
  ((uint16_t*)p.o)[row * kHeadDim + lane] = (uint16_t)(pack2<DT>(out, 0.f) & 0xFFFFu);
  if (lane == 0) p.lse[row] = (mrun + log2f(L)) * kLn2;
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
