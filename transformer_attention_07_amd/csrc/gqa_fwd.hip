// Forward pass of causal grouped-query attention on gfx950 matrix cores (bf16 / f16).
//
// Work decomposition.  One workgroup = 4 wavefronts over one batch b and one kv head g,
// two workgroups per CU (two waves per SIMD).  Wave w owns a 64-row query tile of query
// head h (hpw heads x qpw row tiles per workgroup; all heads belong to kv group g, so every
// wave reads the same K/V tiles).  The workgroup walks the key tiles that hold at least
// one visible key: sink tiles, then the window/causal range; everything between is never
// loaded.  K and V tiles arrive by direct loads into LDS (buffer_load ... lds, no staging
// registers; rows past the end of the sequence read zero), triple-buffered with one
// barrier per tile.
//
// Per wave, S^T = K Q^T runs on v_mfma_f32_32x32x16 with the wave's Q tile held in
// registers as the B operand, so each accumulator lane holds one query column: row
// statistics are in-lane plus one exchange between the two 32-lane halves.  The loop is a
// software pipeline over units of one 32-key half and one 32-row column block: while the
// VALU exponentiates one unit, the matrix cores compute the previous unit's
// O^T += V^T P^T and the next unit's scores, so the compiler can interleave the two inside
// the wave.  Operands are read from LDS a unit or two ahead of their MFMAs.  V^T operands
// come from the row-major V tile through ds_read_b64_tr_b16 transposed reads, and P^T
// straight from the S^T accumulator registers (see gqa_device.h).
//
// Online softmax in fp32: exp2 with scale*log2(e) folded into one FMA and row sums of the
// unrounded P in fp32 (so lse keeps fp32 accuracy).  The running maximum only keeps exp2
// in range, so a unit is exponentiated against it without computing the unit's own
// maximum; a lane's partial row sum above 2^16 (a row's first visible key always gives
// one, against the finite starting maximum) sends the unit through the exact path: take
// its maximum, raise the running maximum when it grew by more than 2^8, rescale O and the
// sums, exponentiate again.  P thus stays below 2^16,
// which the rounded operands and fp32 sums carry at full relative precision.  Units that
// are not fully visible are masked with one compare per element against per-lane bounds.
//
// The online softmax with running max and sum and the fused score/softmax/PV loop follow
// the "SnapKitty Transformer 8B" model card's FlashAttention Kernel section; the tiling,
// operand orientation and staging here are this library's own for CDNA4.
#include <type_traits>

#include "gqa_device.h"

namespace gqa {

namespace {

constexpr float kRescaleThreshold = 8.0f;  // log2 units
// A unit's exponentials are taken against the running maximum without looking at the
// unit's own maximum; if a lane's partial row sum exceeds this (some P > 2^16 / 16, or an
// overflow), the unit is redone after a proper maximum decision.
constexpr float kSumGuard = 65536.0f;
// The running maximum of a row that has seen no visible key yet: a finite value below every
// score (log2 units) the kernel meets, so that its first visible key gives exp2 of about
// 10^38 = inf, which the row-sum guard sends through the exact path; masked keys (-inf)
// still give 0.  (Scores below -10^38 in log2 units, i.e. past fp32's range at the default
// scale, would need the old explicit test.)
constexpr float kNoMax = -1.0e38f;
constexpr float kLn2 = 0.69314718055994530942f;

// Per-wave state and the pieces of one key tile.  The loop works in units of one 32-key
// half and one 32-row column block (a 32 x 32 block of scores).
template <int DT>
struct FwdWave {
  int lane, l32, hl;
  int q0, q1;
  MaskSpec m;
  float c2;
  u32x4 qf[2][4];   // Q tile as B operands [column block][contraction step]
  f32x16 o[2][2];   // O^T accumulators [d block][column block]
  float mrow[2];    // running maximum (log2 units) per column block; kNoMax before any key
  float lrow[2];    // running sum (this lane's half of the keys)
  float nmuse[2];   // -mrow
  int lim_hi;       // a key half [k, k + 31] is fully visible to all 64 rows iff
  int win_lo;       //   k + 31 <= lim_hi && (k >= win_lo || k + 31 < m.sinks)
  int koff[4];      // lane's byte offset of the K operand, contraction step ks (block 0)
  int voff[2][2];   // lane's byte offset of the transposed V read [d block][second row group]

  __device__ __forceinline__ void init_offsets() {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) koff[ks] = rm_off(l32, ks * 2 + hl);
    const int r0 = 4 * hl + ((lane & 15) >> 2);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int c0 = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      voff[db][0] = rm_off(r0, c0 >> 3) + (c0 & 7) * 2;
      voff[db][1] = rm_off(r0 + 8, c0 >> 3) + (c0 & 7) * 2;
    }
  }

  // K operands of key half kb of the tile in `kl` (row-major LDS tile); the swizzle depends
  // on row bits 0..3 only, so the half offset is an additive constant
  __device__ __forceinline__ void load_k(const char* kl, int kb, u32x4 (&a)[4]) const {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) a[ks] = *(const u32x4*)(kl + kb * 4096 + koff[ks]);
  }
  // S^T of column block CB: K Q^T[CB] from loaded K operands
  template <int CB>
  __device__ __forceinline__ void scores(const u32x4 (&a)[4], f32x16& s) const {
    s = mfma32<DT>(a[0], qf[CB][0], f32x16{});
#pragma unroll
    for (int ks = 1; ks < 4; ++ks) s = mfma32<DT>(a[ks], qf[CB][ks], s);
  }

  // V^T operands of key half kb of the tile in `vl` (row-major tile read transposed: rows
  // 32 kb + 16 t + {0..3, 8..11} + 4 h, see lds_rm_transposed_operand) [d block][step t]
  __device__ __forceinline__ void load_v(const char* vl, int kb, u32x4 (&a)[2][2]) const {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const char* base = vl + (kb * 32 + 16 * t) * 128;
        const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(__attribute__((address_space(3))) char*)(base + voff[db][0]));
        const s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(__attribute__((address_space(3))) char*)(base + voff[db][1]));
        const u32x2 ux = __builtin_bit_cast(u32x2, x), uy = __builtin_bit_cast(u32x2, y);
        a[db][t] = u32x4{ux[0], ux[1], uy[0], uy[1]};
      }
  }
  // O^T[db][CB] += V^T[db] P^T[CB] from loaded V operands
  template <int CB>
  __device__ __forceinline__ void accumulate(const u32x4 (&a)[2][2], const u32x4 (&pf)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < 2; ++db) o[db][CB] = mfma32<DT>(a[db][t], pf[t], o[db][CB]);
  }

  // wave-uniform (a scalar branch): bitwise tests, then readfirstlane
  __device__ __forceinline__ bool half_full(int k) const {
    return __builtin_amdgcn_readfirstlane((int)(k + 31 <= lim_hi) & ((int)(k >= win_lo) | (int)(k + 31 < m.sinks))) != 0;
  }

  // hide the keys of half [k0, k0 + 31] that column block CB's rows do not see.  Register r
  // of this lane holds key k0 + 4*hl + rr(r) with rr(r) = 8*(r/4) + r%4 a compile-time
  // constant, so every test is one compare of rr against a per-lane bound.
  template <int CB>
  __device__ __forceinline__ void mask(f32x16& s, int k0) const {
    const int base = k0 + 4 * hl;
    const int kmax = m.S - 1 - base;  // rr <= kmax: key inside the sequence
    const int i = q0 + CB * 32 + l32;
    const int causal_hi = m.causal ? i - base : kmax;       // rr <= causal_hi: not in the future
    const int hi = causal_hi < kmax ? causal_hi : kmax;
    const int wlo = m.window > 0 ? i - m.window + 1 - base : -(1 << 30);  // rr >= wlo: in window
    const int sink_hi = m.sinks - 1 - base;                  // rr <= sink_hi: a sink
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rr = 8 * (r >> 2) + (r & 3);
      const bool ok = (rr <= hi) && (rr >= wlo || rr <= sink_hi);
      s[r] = ok ? s[r] : -INFINITY;
    }
  }

  // Running-maximum update of column block CB from one (masked) unit of scores: when some
  // row's maximum grew by more than the threshold, every row takes its new maximum and O
  // and the sums of the block are rescaled (rare).
  template <int CB>
  __device__ __forceinline__ void decide(const f32x16& s) {
    float a = vmax(s[0], s[1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) a = vmax(vmax(a, s[r]), s[r + 1]);
    uint32_t u = __builtin_bit_cast(uint32_t, a);
    auto pr = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const float mx = vmax(__builtin_bit_cast(float, (uint32_t)pr[0]), __builtin_bit_cast(float, (uint32_t)pr[1])) * c2;
    if (__builtin_expect(wave_any(mx > mrow[CB] + kRescaleThreshold), 0)) {
      const float mnew = vmax(mrow[CB], mx);  // finite: mrow starts at kNoMax
      const float alpha = exp2_fast(mrow[CB] - mnew);
      mrow[CB] = mnew;
      nmuse[CB] = -mnew;
      lrow[CB] *= alpha;
      // keep this block a real branch: O *= 1 is an identity, and hoisting the multiplies
      // out of the (rare) branch would put them on every step
      asm volatile("" ::: "memory");
#pragma unroll
      for (int db = 0; db < 2; ++db) o[db][CB] *= alpha;
    }
  }

  // P^T of one unit at the current maximum, packed into B operands [t]
  template <int CB>
  __device__ __forceinline__ void probs(const f32x16& s, u32x4 (&pf)[2], float& ls) const {
    float lsum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = exp2_fast(__builtin_fmaf(s[8 * t + e], c2, nmuse[CB]));
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        pf[t][w] = pack2<DT>(pv[2 * w], pv[2 * w + 1]);
        lsum += pv[2 * w] + pv[2 * w + 1];
      }
    }
    ls = lsum;
  }

  // Softmax of one (masked) unit against the running maximum.  The maximum only serves to
  // keep exp2 in range, so it is left alone unless a lane's partial row sum shows an
  // exponent above log2(kSumGuard / 16) (which includes a row's first visible key, against
  // kNoMax); then the unit's maximum is taken (decide, which raises it and rescales O and
  // the row sums) and the unit is exponentiated again.  P therefore stays below 2^16: the
  // rounded operands and fp32 sums keep their relative precision at any magnitude.
  template <int CB>
  __device__ __forceinline__ void softmax(const f32x16& s, u32x4 (&pf)[2]) {
    float ls;
    probs<CB>(s, pf, ls);
    const bool need = !(ls <= kSumGuard);
    if (__builtin_expect(wave_any(need), 0)) {
      decide<CB>(s);
      probs<CB>(s, pf, ls);
    }
    lrow[CB] += ls;
  }
};

// Direct-to-LDS staging: buffer_load_dwordx4 ... lds writes lane i's 16 bytes to M0 + 16 i,
// so each lane picks the global chunk that belongs in its LDS slot.  Instruction j (0..7)
// fills LDS rows 8j..8j+7 of a tile; this returns the lane's byte offset inside the tile's
// global rows for instruction j.
__device__ __forceinline__ int direct_voff(int j, int lane) {
  const int r = 8 * j + (lane >> 3);
  return r * 128 + (((lane & 7) ^ swz(r)) << 4);
}

typedef __attribute__((address_space(3))) void lds_void;

// Workgroup barrier for LDS filled only by direct loads: wait until at most VM of this
// wave's vector-memory operations are outstanding and its LDS reads have returned, then
// s_barrier.  (__syncthreads would also drain the younger direct loads, which are meant to
// stay in flight across the barrier.)  The empty asm keeps the compiler from moving LDS
// accesses across it.
template <int VM>
__device__ __forceinline__ void lds_barrier() {
  static_assert(VM >= 0 && VM < 16, "vmcnt field");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0070 | VM);  // vmcnt(VM) expcnt(7) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wave `wave` stages LDS rows 16*wave .. 16*wave + 15 of the tile starting at global row
// `row0` (rows at or past the end of the slab read as zero).
__device__ __forceinline__ void stage_rows(__amdgpu_buffer_rsrc_t rs, char* tile, int row0, const int (&voff)[2],
                                           int wave) {
#pragma unroll
  for (int u = 0; u < 2; ++u)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(tile + 1024 * (2 * wave + u)), 16,
                                             row0 * 128 + voff[u], 0, 0, 0);
}

template <int DT, bool ROPE>
__global__ __launch_bounds__(256, 2) void fwd_mfma_kernel(FwdParams p) {
  __shared__ __attribute__((aligned(1024))) char k_lds0[8192];
  __shared__ __attribute__((aligned(1024))) char k_lds1[8192];
  __shared__ __attribute__((aligned(1024))) char k_lds2[8192];
  __shared__ __attribute__((aligned(1024))) char v_lds0[8192];
  __shared__ __attribute__((aligned(1024))) char v_lds1[8192];
  __shared__ __attribute__((aligned(1024))) char v_lds2[8192];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int nhq = p.H / p.hpw;
  int qblk, rest;  // row block and head group (b * nhq + head block) of this workgroup
  fwd_block_order(p, (int)blockIdx.x, qblk, rest);
  const int b = rest / nhq;
  const int h = (rest % nhq) * p.hpw + (wave % p.hpw);
  const int g = h / (p.H / p.G);
  const int S = p.S;
  const int Q0 = qblk * kTile * p.qpw;
  const int Q1 = imin(Q0 + kTile * p.qpw, S) - 1;

  FwdWave<DT> W;
  W.lane = lane;
  W.l32 = lane & 31;
  W.hl = lane >> 5;
  W.q0 = Q0 + (wave / p.hpw) * kTile;
  W.q1 = imin(W.q0 + kTile - 1, S - 1);
  W.m = p.mask;
  W.c2 = p.scale_log2;
  W.init_offsets();
  const bool active = W.q0 < S;
  const __amdgpu_buffer_rsrc_t qrs = slab_rsrc((const uint16_t*)p.q + (size_t)(b * p.H + h) * S * kHeadDim, S);
  const __amdgpu_buffer_rsrc_t krs = slab_rsrc((const uint16_t*)p.k + (size_t)(b * p.G + g) * S * kHeadDim, S);
  const __amdgpu_buffer_rsrc_t vrs = slab_rsrc((const uint16_t*)p.v + (size_t)(b * p.G + g) * S * kHeadDim, S);

  const TileRanges tr = key_tiles_for_rows(W.m, Q0, Q1);
  const int nt = tr.count();
  const int voff[2] = {direct_voff(2 * wave, lane), direct_voff(2 * wave + 1, lane)};
  // rows of key tile n; past the last tile, row S: every load is out of range and fills zeros
  auto tile_row = [&](int n) __attribute__((always_inline)) { return n < nt ? tr.tile(n) * kTile : S; };

  stage_rows(krs, k_lds0, tile_row(0), voff, wave);
  stage_rows(vrs, v_lds0, tile_row(0), voff, wave);
  stage_rows(krs, k_lds1, tile_row(1), voff, wave);

#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      W.qf[cb][ks] = buf_load16(qrs, (W.q0 + cb * 32 + W.l32) * 128 + ks * 32 + W.hl * 16);
  if constexpr (ROPE) {
    // Rotary embedding of the wave's Q tile in registers: this lane holds pairs
    // 8 ks + 4 hl .. + 3 of rows q0 + cb * 32 + l32 (rows past S are zeros and stay so).
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        double rev[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) rev[j] = W.hl ? p.rope.rev[8 * ks + 4 + j] : p.rope.rev[8 * ks + j];
        W.qf[cb][ks] = rope_chunk16<DT>(W.qf[cb][ks], W.q0 + cb * 32 + W.l32, rev, p.rope.mscale, false);
      }
  }
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) W.o[db][cb] = f32x16{};
  W.mrow[0] = W.mrow[1] = kNoMax;
  W.lrow[0] = W.lrow[1] = 0.f;
  W.nmuse[0] = W.nmuse[1] = -kNoMax;
  W.lim_hi = __builtin_amdgcn_readfirstlane(W.m.causal ? imin(W.q0, S - 1) : S - 1);
  W.win_lo = __builtin_amdgcn_readfirstlane(W.m.window > 0 ? W.q1 - W.m.window + 1 : -(1 << 30));

  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // Software pipeline over units (one 32-key half, one 32-row column block): a unit's
  // softmax runs while the matrix cores compute the previous unit's P V and the next
  // unit's scores, all three independent of one another.  Between two softmax ends
  // (where the rare rescale branch sits) nothing else breaks the code, so the compiler
  // interleaves the softmax's vector instructions with those eight MFMAs inside the wave.
  // Tile n's units are (half 0, block 0), (0, 1), (1, 0), (1, 1); operands are read from
  // LDS a unit or two ahead, into two sets of registers per operand: K half 0 / half 1 and
  // V half 0 / half 1, scores and P alternating between two sets.  Tile n reads K_n,
  // K_{n+1} (the next tile's first scores) and V_n.  K and V tiles are triple-buffered
  // (buffer n % 3) and the loop is unrolled by three, so every buffer is fixed at compile
  // time.  One barrier per tile: right after it, the direct loads of K_{n+2} and V_{n+1}
  // go into the buffers of K_{n-1} and V_{n-2}, which no wave reads any more; they have
  // the whole tile to land and the next barrier drains them, so nothing is in flight
  // across the loop's back edge.  Loads past the last tile read zeros (no traffic), which
  // keeps the steps unconditional.  The (rare) mask of a unit that is not fully visible
  // sits at the unit's start, ahead of its matrix products, so it splits nothing.
  f32x16 sx, sy;               // S^T of the units softmaxed at block 0 / block 1
  u32x4 ka0[4], ka1[4];        // K operands of key half 0 / half 1
  u32x4 va0[2][2], va1[2][2];  // V^T operands of key half 0 / half 1
  u32x4 px[2], py[2];          // P^T of the units softmaxed from sx / sy
  W.load_k(k_lds0, 0, ka0);
  W.template scores<0>(ka0, sx);
  // the first unit's P V (of no earlier unit) adds zero
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    py[t] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int db = 0; db < 2; ++db) va1[db][t] = u32x4{0u, 0u, 0u, 0u};
  }

  auto tile = [&](auto par, int n) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    char* kn = P == 0 ? k_lds0 : P == 1 ? k_lds1 : k_lds2;    // K_n
    char* kn1 = P == 0 ? k_lds1 : P == 1 ? k_lds2 : k_lds0;   // K_{n+1}
    char* kn2 = P == 0 ? k_lds2 : P == 1 ? k_lds0 : k_lds1;   // receives K_{n+2}
    char* vn = P == 0 ? v_lds0 : P == 1 ? v_lds1 : v_lds2;    // V_n
    char* vn1 = P == 0 ? v_lds1 : P == 1 ? v_lds2 : v_lds0;   // receives V_{n+1}
    const int k0 = tr.tile(n) * kTile;
    stage_rows(krs, kn2, tile_row(n + 2), voff, wave);
    stage_rows(vrs, vn1, tile_row(n + 1), voff, wave);
    // (half 0, block 0) from sx; P V of (n - 1, half 1, block 1); scores of (half 0, block 1)
    if (__builtin_expect(!W.half_full(k0), 0)) W.template mask<0>(sx, k0);
    W.template accumulate<1>(va1, py);
    W.template scores<1>(ka0, sy);
    W.load_k(kn, 1, ka1);
    W.load_v(vn, 0, va0);
    W.template softmax<0>(sx, px);
    // (half 0, block 1) from sy; P V of (half 0, block 0); scores of (half 1, block 0)
    if (__builtin_expect(!W.half_full(k0), 0)) W.template mask<1>(sy, k0);
    W.template accumulate<0>(va0, px);
    W.template scores<0>(ka1, sx);
    W.template softmax<1>(sy, py);
    // (half 1, block 0) from sx; P V of (half 0, block 1); scores of (half 1, block 1)
    if (__builtin_expect(!W.half_full(k0 + 32), 0)) W.template mask<0>(sx, k0 + 32);
    W.template accumulate<1>(va0, py);
    W.template scores<1>(ka1, sy);
    W.load_k(kn1, 0, ka0);
    W.load_v(vn, 1, va1);
    W.template softmax<0>(sx, px);
    // (half 1, block 1) from sy; P V of (half 1, block 0); scores of (n + 1, half 0, block 0)
    if (__builtin_expect(!W.half_full(k0 + 32), 0)) W.template mask<1>(sy, k0 + 32);
    W.template accumulate<0>(va1, px);
    W.template scores<0>(ka0, sx);
    W.template softmax<1>(sy, py);
    lds_barrier<0>();  // this tile's loads have landed; its buffers are read no more
  };
  for (int n = 0; n < nt; n += 3) {
    tile(std::integral_constant<int, 0>{}, n);
    if (n + 1 >= nt) break;
    tile(std::integral_constant<int, 1>{}, n + 1);
    if (n + 2 >= nt) break;
    tile(std::integral_constant<int, 2>{}, n + 2);
  }
  W.template accumulate<1>(va1, py);  // P V of the last unit

  if constexpr (ROPE) {
    // the rotated Q tile for the backward, stored once the tile loop is done so that these
    // writes spread over the run instead of joining every workgroup's first loads
    if (p.q_rot != nullptr) {
      const __amdgpu_buffer_rsrc_t qrot =
          slab_rsrc((const uint16_t*)p.q_rot + (size_t)(b * p.H + h) * S * kHeadDim, S);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)  // stores past the slab's end are dropped
          __builtin_amdgcn_raw_buffer_store_b128(W.qf[cb][ks], qrot,
                                                 (W.q0 + cb * 32 + W.l32) * 128 + ks * 32 + W.hl * 16, 0, 0);
    }
  }
  if (!active) return;
  uint16_t* oslab = (uint16_t*)p.o + (size_t)(b * p.H + h) * S * kHeadDim;
  uint16_t* olo_slab = p.o_lo ? (uint16_t*)p.o_lo + (size_t)(b * p.H + h) * S * kHeadDim : nullptr;
  float* lse_row = p.lse + (size_t)(b * p.H + h) * S;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const float l = sum_across_halves(W.lrow[cb]);
    const int i = W.q0 + cb * 32 + W.l32;
    if (i >= S) continue;
    const float inv = 1.0f / l;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = db * 32 + 8 * r4 + 4 * W.hl;
        const float x0 = W.o[db][cb][4 * r4 + 0] * inv, x1 = W.o[db][cb][4 * r4 + 1] * inv;
        const float x2 = W.o[db][cb][4 * r4 + 2] * inv, x3 = W.o[db][cb][4 * r4 + 3] * inv;
        const u32x2 w = {pack2<DT>(x0, x1), pack2<DT>(x2, x3)};
        *(u32x2*)(oslab + (size_t)i * kHeadDim + d0) = w;
        if (olo_slab != nullptr) {
          const u32x2 r = {pack2_residual<DT>(x0, x1, w[0]), pack2_residual<DT>(x2, x3, w[1])};
          *(u32x2*)(olo_slab + (size_t)i * kHeadDim + d0) = r;
        }
      }
    if (W.hl == 0) lse_row[i] = (W.mrow[cb] + log2f(l)) * kLn2;
  }
}

}  // namespace

hipError_t launch_fwd_mfma(const FwdParams& p, int dtype, hipStream_t s) {
  const long long nblk = (long long)p.n_qblk * p.B * (p.H / p.hpw);
  dim3 grid((unsigned)nblk), block(256);
  void* args[] = {(void*)&p};
  const void* fn;
  if (p.rope.enabled)
    fn = dtype == kDtBF16 ? (const void*)fwd_mfma_kernel<kDtBF16, true> : (const void*)fwd_mfma_kernel<kDtF16, true>;
  else
    fn = dtype == kDtBF16 ? (const void*)fwd_mfma_kernel<kDtBF16, false> : (const void*)fwd_mfma_kernel<kDtF16, false>;
  return hipLaunchKernel(fn, grid, block, args, 0, s);
}

}  // namespace gqa
