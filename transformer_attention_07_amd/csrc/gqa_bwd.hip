// Backward pass of causal grouped-query attention on gfx950 matrix cores (bf16 / f16
// inputs, fp32 gradients).  Loss convention L = <O, dO>.
//
//   preprocess : delta_i = sum_c dO_ic O_ic                       (HBM-bound, fp32)
//   dK/dV      : per (b, g, 128-key block), 4 waves x 32 keys (two workgroups, two waves
//                per SIMD, per CU, so one's barrier waits are covered by the other).  For
//                every query head of the group and every query tile that sees the block:
//                  S  = Q K^T        P = exp(scale*S - lse)   (recomputed from the saved lse)
//                  delta - dP = dO (-V)^T + delta  (V enters negated, the accumulator
//                                                    starts at delta)
//                  dS = P * (dP - delta) = -P * (delta - dP)
//                  dV^T += dO^T P    dK^T += Q^T dS           (scale applied at the end)
//                The sum over the H/G heads of the group stays in registers: no atomics.
//                Q and dO tiles and the lse / delta rows arrive by direct loads into LDS
//                (double-buffered, one barrier per tile); the transposed operands dO^T
//                and Q^T come from the row-major tiles through ds_read_b64_tr_b16.
//   dQ         : per (b, h, 64-row tile), the forward's decomposition (two waves per
//                SIMD).  For every key tile it sees: S^T = K Q^T, dP^T - delta = V dO^T +
//                (-delta) (the accumulator starts at the lane's -delta), dS^T = P^T (dP^T -
//                delta), dQ^T += K^T dS^T.  K and V tiles arrive by direct loads into LDS.
//                Deterministic (each dQ element has one writer).
//
// Every staging buffer is its own LDS object and both loops are unrolled by two, so the
// buffer a step reads is known at compile time to differ from the one the direct loads of
// the next step fill; the loads then stay in flight across the step's compute.
//
// The recompute of P from the saved log-sum-exp and dS = P * (dO V^T - D) follow the
// FlashAttention-3 backward entry of the "SnapKitty Transformer 8B" model card
// (Protected Inventions); that entry reduces dQ with atomics across query tiles, which
// this library replaces by the separate deterministic dQ pass.
#include <type_traits>

#include "gqa_device.h"

namespace gqa {

namespace {

constexpr float kLog2e = 1.44269504088896340736f;

// ------------------------------------------------------------------------------------
// delta = rowsum(dO * O), with O = rounded O + its residual when the forward kept it
// ------------------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(256) void bwd_preprocess_kernel(BwdParams p) {
  constexpr int kEpl = (DT == kDtF32) ? 4 : 8;  // elements per 16-byte lane load
  constexpr int kLpr = kHeadDim / kEpl;          // lanes per row (16 or 8)
  constexpr int kRowsPerBlock = 256 / kLpr;
  const long long rows = (long long)p.B * p.H * p.S;
  const long long row = (long long)blockIdx.x * kRowsPerBlock + threadIdx.x / kLpr;
  const int part = threadIdx.x % kLpr;
  float acc = 0.f;
  if (row < rows) {
    const size_t off = (size_t)row * kHeadDim + part * kEpl;
    if constexpr (DT == kDtF32) {
      const f32x4 a = *(const f32x4*)((const float*)p.o + off);
      const f32x4 b = *(const f32x4*)((const float*)p.d_o + off);
      acc = a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
    } else {
      const u32x4 a = *(const u32x4*)((const uint16_t*)p.o + off);
      const u32x4 b = *(const u32x4*)((const uint16_t*)p.d_o + off);
      u32x4 r = {0u, 0u, 0u, 0u};
      if (p.o_lo != nullptr) r = *(const u32x4*)((const uint16_t*)p.o_lo + off);
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int hi = 0; hi < 2; ++hi)
          acc += (elem_to_f32<DT>(a[w], hi) + elem_to_f32<DT>(r[w], hi)) * elem_to_f32<DT>(b[w], hi);
    }
  }
#pragma unroll
  for (int s = kLpr / 2; s >= 1; s >>= 1) acc += __shfl_xor(acc, s, kLpr);
  if (row < rows && part == 0) p.out_delta[row] = acc;
}

typedef __attribute__((address_space(3))) void lds_void;

// Direct-to-LDS staging: buffer_load_dwordx4 ... lds writes lane i's 16 bytes to M0 + 16 i,
// so each lane picks the global chunk that belongs in its LDS slot.  Instruction j (0..7)
// fills LDS rows 8j..8j+7 of a row-major tile; this is the lane's byte offset inside the
// tile's global rows.
__device__ __forceinline__ int direct_voff(int j, int lane) {
  const int r = 8 * j + (lane >> 3);
  return r * 128 + (((lane & 7) ^ swz(r)) << 4);
}

// ------------------------------------------------------------------------------------
// dK, dV
// ------------------------------------------------------------------------------------
struct DkdvStage {
  char q_rm[8192];   // Q tile, row-major (rows = queries)
  char do_rm[8192];  // dO tile, row-major
  float lse[64];     // lse * log2(e) of the tile's 64 rows; 0 past the end
  float delta[256];  // delta of the tile's 64 rows (entries 64.. are load padding); 0 past the end
};

// classify() for wave-uniform bounds as one scalar value: bitwise terms, no branches.
__device__ __forceinline__ int classify_uniform(const MaskSpec& m, int q0, int q1, int k0, int k1) {
  const int c = m.causal != 0, w = m.window;
  const int empty = (k0 >= m.S) | (c & (k0 > q1)) | (c & (w > 0) & (k1 <= q0 - w) & (k0 >= m.sinks));
  const int full = ((c ^ 1) & (k1 < m.S)) |
                   (c & (k1 <= q0) & (k1 < m.S) & ((w <= 0) | (k0 > q1 - w) | (k1 < m.sinks)));
  return __builtin_amdgcn_readfirstlane(empty ? (int)kEmpty : full ? (int)kFull : (int)kPartial);
}

// The two staging buffers of the dK/dV pass, as distinct LDS objects so that the compiler
// can tell the buffer being read from the one the direct loads are filling.
__shared__ __attribute__((aligned(1024))) DkdvStage g_dkdv_stage0;
__shared__ __attribute__((aligned(1024))) DkdvStage g_dkdv_stage1;

// Per-wave state of the dK/dV pass: 32 keys (one column block) of one kv head.
template <int DT>
struct DkdvWave {
  int lane, l32, hl;
  int kw0, kw1;
  MaskSpec m;
  float c2;
  u32x4 kf[4], vf[4];  // K and -V rows as B operands [contraction step]
  f32x16 dk[2], dv[2];  // transposed accumulators [d block]
  int trb[2][2];        // this lane's byte offsets of the transposed reads [d block][row half]

  // The transposed reads of block (qb, t) address rows qb*32 + 16t + lr (+ 8) of a row-major
  // tile, lr = 4*(lane/32) + (lane%16)/4 < 8.  The swizzle depends on a row's low four bits
  // only, which the tile offset qb*32 + 16t leaves alone, and the d block flips chunk bit 2,
  // which the lane's own chunk bits (0..1) never touch: the lane part of every address is
  // one of four values and the rest is a constant.
  __device__ __forceinline__ void init_tr_offsets() {
    const int lr = 4 * hl + ((lane & 15) >> 2);
    const int lc = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int row = lr + 8 * hf;
        trb[db][hf] = row * 128 + (((lc ^ swz(row)) ^ (4 * db)) << 4) + 8 * (lane & 1);
      }
  }
  // lds_rm_transposed_operand(tile, db, qb, t, lane) from the offsets above
  __device__ __forceinline__ u32x4 tr_operand(const char* tile, int db, int qb, int t) const {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const char* base = tile + (qb * 32 + 16 * t) * 128;
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(__attribute__((address_space(3))) char*)(base + trb[db][0]));
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(__attribute__((address_space(3))) char*)(base + trb[db][1]));
    const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
    return u32x4{ua[0], ua[1], ub[0], ub[1]};
  }

  // one 32-query block qb of the staged tile (rows qr0 ..): both products for dK and dV
  template <bool PRECISE>
  __device__ __forceinline__ void block(const DkdvStage& sb, int qb, int qr0, bool partial) {
    f32x16 s, dp;
    f32x16 nd;  // delta of this lane's 16 rows: the initial accumulator of dO (-V)^T, which
                // therefore holds delta - dP, and dS = P (dP - delta) = -P (delta - dP)
    float L[16];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4 lv = *(const f32x4*)(sb.lse + qb * 32 + 8 * r4 + 4 * hl);
      const f32x4 dv4 = *(const f32x4*)(sb.delta + qb * 32 + 8 * r4 + 4 * hl);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        L[4 * r4 + x] = lv[x];
        nd[4 * r4 + x] = dv4[x];
      }
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const u32x4 aq = lds_rm_operand(sb.q_rm, qb, ks, l32, hl);
      const u32x4 ado = lds_rm_operand(sb.do_rm, qb, ks, l32, hl);
      s = mfma32<DT>(aq, kf[ks], ks == 0 ? f32x16{} : s);
      dp = mfma32<DT>(ado, vf[ks], ks == 0 ? nd : dp);
    }
    if (__builtin_expect(partial, 0)) {
      // lane = key column j, register r = query row qr0 + 4*hl + rr(r)
      const int j = kw0 + l32;
      const int base = qr0 + 4 * hl;
      const int lo = m.causal ? j - base : -(1 << 30);                 // rr >= lo: i >= j
      const bool sink = j < m.sinks;
      const int whi = m.window > 0 ? j + m.window - base : (1 << 30);  // rr < whi: in window
      const bool key_ok = j < m.S;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rr = 8 * (r >> 2) + (r & 3);
        const bool ok = key_ok && rr >= lo && (sink || rr < whi);
        s[r] = ok ? s[r] : -INFINITY;
      }
    }
    u32x4 pp[2], pds[2], pp_lo[2], pds_lo[2];  // [t]
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float pv[8], dsv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 8 * t + e;
        pv[e] = exp2_fast(__builtin_fmaf(s[r], c2, -L[r]));
        dsv[e] = -pv[e] * dp[r];
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        pp[t][w] = pack2<DT>(pv[2 * w], pv[2 * w + 1]);
        pds[t][w] = pack2<DT>(dsv[2 * w], dsv[2 * w + 1]);
        if (PRECISE) {
          pp_lo[t][w] = pack2_residual<DT>(pv[2 * w], pv[2 * w + 1], pp[t][w]);
          pds_lo[t][w] = pack2_residual<DT>(dsv[2 * w], dsv[2 * w + 1], pds[t][w]);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const u32x4 ado_t = tr_operand(sb.do_rm, db, qb, t);
        const u32x4 aq_t = tr_operand(sb.q_rm, db, qb, t);
        dv[db] = mfma32<DT>(ado_t, pp[t], dv[db]);
        dk[db] = mfma32<DT>(aq_t, pds[t], dk[db]);
        if (PRECISE) {
          dv[db] = mfma32<DT>(ado_t, pp_lo[t], dv[db]);
          dk[db] = mfma32<DT>(aq_t, pds_lo[t], dk[db]);
        }
      }
  }
};

// The whole dK/dV pass for one workgroup.  Every pass is inlined into its kernel: a call
// to an out-of-line pass makes the callee save the callee-saved vector registers it uses
// to scratch memory (up to 500 bytes per lane here), while the two variants of a branch
// share one allocation at the larger variant's pressure.
template <int DT, bool PRECISE, bool ROPE>
__device__ __forceinline__ void dkdv_block(const BwdArgs& a, int wg) {
  const BwdParams& p = a.p;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int S = p.S;
  const int hpg = p.H / p.G;

  // heaviest (earliest) key blocks first
  const int per_k = p.B * p.G;
  const int kblk = wg / per_k;
  const int rest = wg % per_k;
  const int b = rest / p.G;
  const int g = rest % p.G;
  const int K0 = kblk * kDkdvKeys;
  const int K1 = imin(K0 + kDkdvKeys, S) - 1;

  DkdvWave<DT> W;
  W.lane = lane;
  W.l32 = lane & 31;
  W.hl = lane >> 5;
  W.kw0 = K0 + wave * 32;
  W.kw1 = imin(W.kw0 + 31, S - 1);
  W.m = p.mask;
  W.c2 = p.scale_log2;
  W.init_tr_offsets();
  const bool active = W.kw0 < S;

  const __amdgpu_buffer_rsrc_t krs = slab_rsrc((const uint16_t*)p.k + (size_t)(b * p.G + g) * S * kHeadDim, S);
  const __amdgpu_buffer_rsrc_t vrs = slab_rsrc((const uint16_t*)p.v + (size_t)(b * p.G + g) * S * kHeadDim, S);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int off = (W.kw0 + W.l32) * 128 + ks * 32 + W.hl * 16;
    W.kf[ks] = buf_load16(krs, off);
    W.vf[ks] = buf_load16(vrs, off) ^ 0x80008000u;  // -V: flip both 16-bit signs
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the K/V operands are in registers before the loop
#pragma unroll
  for (int db = 0; db < 2; ++db) {
    W.dk[db] = f32x16{};
    W.dv[db] = f32x16{};
  }

  // Staging by direct loads into LDS (no registers): wave w loads LDS rows 16w..16w+15 of the
  // Q and dO tiles; wave 1 loads the delta row (a full 1 KiB load, of which the first 64
  // entries are the tile's).  Wave 0 loads the tile's 64 lse values into a register and,
  // once they have arrived, stores them scaled by log2(e), so that the exponent of every
  // score takes a single fma.  Rows past the end of the sequence read zero, which makes
  // their P V and dS contributions vanish (Q and dO rows are zero).
  const int voff0 = direct_voff(2 * wave, lane), voff1 = direct_voff(2 * wave + 1, lane);
  const TileRanges tr = query_tiles_for_keys(W.m, K0, K1);
  const int nq = tr.count();
  const int n_iter = nq * hpg;
  auto stage_dma = [&](DkdvStage* sb, int iter) __attribute__((always_inline)) -> float {
    const int hh = iter / nq;
    const int qt = tr.tile(iter % nq);
    const size_t slab = (size_t)(b * p.H + g * hpg + hh) * S;
    const __amdgpu_buffer_rsrc_t qr = slab_rsrc((const uint16_t*)p.q + slab * kHeadDim, S);
    const __amdgpu_buffer_rsrc_t dr = slab_rsrc((const uint16_t*)p.d_o + slab * kHeadDim, S);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(qr, (lds_void*)(sb->q_rm + 2048 * wave), 16, qt * kTile * 128 + voff0, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(qr, (lds_void*)(sb->q_rm + 2048 * wave + 1024), 16, qt * kTile * 128 + voff1, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(dr, (lds_void*)(sb->do_rm + 2048 * wave), 16, qt * kTile * 128 + voff0, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(dr, (lds_void*)(sb->do_rm + 2048 * wave + 1024), 16, qt * kTile * 128 + voff1, 0, 0, 0);
    float lv = 0.f;
    if (wave == 0) {
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p.lse + slab), 0, S * 4, 0x00020000);
      lv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (qt * kTile + lane) * 4, 0, 0));
    } else if (wave == 1) {
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p.delta + slab), 0, S * 4, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)sb->delta, 16, (qt * kTile + 4 * lane) * 4, 0, 0, 0);
    }
    return lv;
  };
  // after the wait for the loads: wave 0 stores the scaled lse
  auto stage_lse = [&](DkdvStage* sb, float lv) __attribute__((always_inline)) {
    if (wave == 0) {
      asm volatile("" : "+v"(lv));  // keeps the scaling (and so the wait for the load) here
      sb->lse[lane] = lv * kLog2e;
    }
  };
  auto compute = [&](const DkdvStage& sb, int iter) __attribute__((always_inline)) {
    if (!active) return;
    const int qt = tr.tile(iter % nq);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qr0 = qt * kTile + qb * 32;
      const int cls = classify_uniform(W.m, qr0, imin(qr0 + 31, S - 1), W.kw0, W.kw1);
      if (cls == kEmpty) continue;
      W.template block<PRECISE>(sb, qb, qr0, cls != kFull);
    }
  };

  float lv0 = 0.f;
  if (n_iter > 0) lv0 = stage_dma(&g_dkdv_stage0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  if (n_iter > 0) stage_lse(&g_dkdv_stage0, lv0);
  __syncthreads();
  // unrolled by two so that every LDS buffer is known at compile time (the loads into the
  // other buffer then need no wait before this buffer's reads)
  auto iter_body = [&](auto par, int it) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    DkdvStage* next = P ? &g_dkdv_stage0 : &g_dkdv_stage1;
    const bool more = it + 1 < n_iter;
    float lv = 0.f;
    if (more) lv = stage_dma(next, it + 1);
    compute(P ? g_dkdv_stage1 : g_dkdv_stage0, it);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): next stage landed, reads done
    if (more) stage_lse(next, lv);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the lse store is done
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  for (int it = 0; it < n_iter; it += 2) {
    iter_body(std::integral_constant<int, 0>{}, it);
    if (it + 1 >= n_iter) break;
    iter_body(std::integral_constant<int, 1>{}, it + 1);
  }

  if (!active) return;
  float* dkslab = p.dk + (size_t)(b * p.G + g) * S * kHeadDim;
  float* dvslab = p.dv + (size_t)(b * p.G + g) * S * kHeadDim;
  const int j = W.kw0 + W.l32;
  if (j >= S) return;
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d0 = db * 32 + 8 * r4 + 4 * W.hl;
      f32x4 kv = {W.dk[db][4 * r4] * p.scale, W.dk[db][4 * r4 + 1] * p.scale, W.dk[db][4 * r4 + 2] * p.scale,
                  W.dk[db][4 * r4 + 3] * p.scale};
      if constexpr (ROPE) kv = rope_back4(kv, j, a.rope, d0 / 2);  // gradient of the unrotated K
      const f32x4 vv = {W.dv[db][4 * r4], W.dv[db][4 * r4 + 1], W.dv[db][4 * r4 + 2], W.dv[db][4 * r4 + 3]};
      *(f32x4*)(dkslab + (size_t)j * kHeadDim + d0) = kv;
      *(f32x4*)(dvslab + (size_t)j * kHeadDim + d0) = vv;
    }
}

// Sink keys collect attention from every later query, so their dK and dV are sums of many
// large terms: in blocks holding sinks, P and dS enter the MFMAs as a rounded value plus
// its rounded residual (two products each), which keeps their rounding out of the sum.
// The same holds for every block when each query sees only a few keys (short sequences,
// short windows): then P is large and a key's dV sums few such terms per head, so the
// rounding of P would not average out (precise_all, set by the host).
template <int DT, bool ROPE>
__device__ __forceinline__ void dkdv_dispatch(const BwdArgs& a, int wg) {
  const int kblk = wg / (a.p.B * a.p.G);
  if (a.p.precise_all || (a.p.mask.window > 0 && kblk * kDkdvKeys < a.p.mask.sinks))
    dkdv_block<DT, true, ROPE>(a, wg);
  else
    dkdv_block<DT, false, ROPE>(a, wg);
}

template <int DT, bool ROPE>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_kernel(BwdArgs a) {
  dkdv_dispatch<DT, ROPE>(a, (int)blockIdx.x);
}

// ------------------------------------------------------------------------------------
// dQ
// ------------------------------------------------------------------------------------
// The staging buffers of the dQ pass (distinct LDS objects, see the dK/dV pass).
__shared__ __attribute__((aligned(1024))) char g_dq_k0[8192];
__shared__ __attribute__((aligned(1024))) char g_dq_k1[8192];
__shared__ __attribute__((aligned(1024))) char g_dq_v0[8192];
__shared__ __attribute__((aligned(1024))) char g_dq_v1[8192];

template <int DT, bool ROPE>
__device__ __forceinline__ void dq_body(const BwdArgs& a, int wg) {
  const BwdParams& p = a.p;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hl = lane >> 5;
  const int S = p.S;
  const MaskSpec m = p.mask;

  const int nhq = p.H / p.hpw;
  const int per_q = p.B * nhq;
  const int qblk = p.n_qblk - 1 - wg / per_q;
  const int rest = wg % per_q;
  const int b = rest / nhq;
  const int h = (rest % nhq) * p.hpw + (wave % p.hpw);
  const int g = h / (p.H / p.G);
  const int Q0 = qblk * kTile * p.qpw;
  const int Q1 = imin(Q0 + kTile * p.qpw, S) - 1;
  const int q0 = Q0 + (wave / p.hpw) * kTile;
  const int q1 = imin(q0 + kTile - 1, S - 1);
  const bool active = q0 < S;

  const size_t qslab_rows = (size_t)(b * p.H + h) * S;
  const __amdgpu_buffer_rsrc_t qrs = slab_rsrc((const uint16_t*)p.q + qslab_rows * kHeadDim, S);
  const __amdgpu_buffer_rsrc_t dors = slab_rsrc((const uint16_t*)p.d_o + qslab_rows * kHeadDim, S);
  const __amdgpu_buffer_rsrc_t krs = slab_rsrc((const uint16_t*)p.k + (size_t)(b * p.G + g) * S * kHeadDim, S);
  const __amdgpu_buffer_rsrc_t vrs = slab_rsrc((const uint16_t*)p.v + (size_t)(b * p.G + g) * S * kHeadDim, S);

  const TileRanges tr = key_tiles_for_rows(m, Q0, Q1);
  const int nt = tr.count();
  // rows of key tile n; past the last tile, row S (all loads out of range: zero, no traffic)
  auto tile_row = [&](int n) __attribute__((always_inline)) { return n < nt ? tr.tile(n) * kTile : S; };
  // direct loads: wave w fills LDS rows 16w..16w+15 of the K and V tiles
  const int dvo[2] = {direct_voff(2 * wave, lane), direct_voff(2 * wave + 1, lane)};
  auto stage = [&](char* kt, char* vt, int row0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(kt + 1024 * (2 * wave + u)), 16, row0 * 128 + dvo[u], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(vt + 1024 * (2 * wave + u)), 16, row0 * 128 + dvo[u], 0, 0, 0);
    }
  };
  stage(g_dq_k0, g_dq_v0, tile_row(0));

  u32x4 qf[2][4], df[2][4];
  float lse2[2], dlt[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int row = q0 + cb * 32 + l32;
    const bool ok = active && row < S;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int off = row * 128 + ks * 32 + hl * 16;
      qf[cb][ks] = buf_load16(qrs, off);
      df[cb][ks] = buf_load16(dors, off);
    }
    lse2[cb] = ok ? p.lse[qslab_rows + row] * kLog2e : INFINITY;
    dlt[cb] = ok ? p.delta[qslab_rows + row] : 0.f;
  }

  // -delta of the lane's query row, replicated over an accumulator: the initial value of
  // dP^T, which then holds dP - delta (loop-invariant, so set up once)
  f32x16 ndlt[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) ndlt[cb][r] = -dlt[cb];

  f32x16 dq[2][2];  // dQ^T [d block][column block]
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) dq[db][cb] = f32x16{};

  // lane offsets of the LDS operand reads (the swizzle depends on row bits 0..3 only, so the
  // key-half, step and buffer offsets are additive constants)
  int koff[4], toff[2][2];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) koff[ks] = rm_off(l32, ks * 2 + hl);
  {
    const int r0 = 4 * hl + ((lane & 15) >> 2);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int c0 = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      toff[db][0] = rm_off(r0, c0 >> 3) + (c0 & 7) * 2;
      toff[db][1] = rm_off(r0 + 8, c0 >> 3) + (c0 & 7) * 2;
    }
  }
  // a key half [k, k + 31] is fully visible to all 64 rows iff these hold
  const int lim_hi = m.causal ? imin(q0, S - 1) : S - 1;
  const int win_lo = m.window > 0 ? q1 - m.window + 1 : -(1 << 30);
  const float c2 = p.scale_log2;
  __builtin_amdgcn_s_waitcnt(0);  // Q, dO operands and the first K/V tiles have landed
  __syncthreads();

  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  auto half = [&](const char* kl, const char* vl, int kb, int kr0) __attribute__((always_inline)) {
    f32x16 s[2], dp[2];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const u32x4 ak = *(const u32x4*)(kl + kb * 4096 + koff[ks]);
      const u32x4 av = *(const u32x4*)(vl + kb * 4096 + koff[ks]);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        s[cb] = mfma32<DT>(ak, qf[cb][ks], ks == 0 ? f32x16{} : s[cb]);
        dp[cb] = mfma32<DT>(av, df[cb][ks], ks == 0 ? ndlt[cb] : dp[cb]);
      }
    }
    const bool full = __builtin_amdgcn_readfirstlane((int)(kr0 + 31 <= lim_hi) &
                                                     ((int)(kr0 >= win_lo) | (int)(kr0 + 31 < m.sinks))) != 0;
    if (__builtin_expect(!full, 0)) {
      // lane = query column i, register r = key kr0 + 4*hl + rr(r)
      const int base = kr0 + 4 * hl;
      const int kmax = m.S - 1 - base;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int i = q0 + cb * 32 + l32;
        const int causal_hi = m.causal ? i - base : kmax;
        const int hi = causal_hi < kmax ? causal_hi : kmax;
        const int wlo = m.window > 0 ? i - m.window + 1 - base : -(1 << 30);
        const int sink_hi = m.sinks - 1 - base;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rr = 8 * (r >> 2) + (r & 3);
          const bool ok = (rr <= hi) && (rr >= wlo || rr <= sink_hi);
          s[cb][r] = ok ? s[cb][r] : -INFINITY;
        }
      }
    }
    u32x4 pds[2][2];  // [cb][t]
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float dsv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * t + e;
          const float pv = exp2_fast(__builtin_fmaf(s[cb][r], c2, -lse2[cb]));
          dsv[e] = pv * dp[cb][r];
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) pds[cb][t][w] = pack2<DT>(dsv[2 * w], dsv[2 * w + 1]);
      }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const char* base = kl + (kb * 32 + 16 * t) * 128;
        const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(__attribute__((address_space(3))) char*)(base + toff[db][0]));
        const s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(__attribute__((address_space(3))) char*)(base + toff[db][1]));
        const u32x2 ux = __builtin_bit_cast(u32x2, x), uy = __builtin_bit_cast(u32x2, y);
        const u32x4 akt = u32x4{ux[0], ux[1], uy[0], uy[1]};
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) dq[db][cb] = mfma32<DT>(akt, pds[cb][t], dq[db][cb]);
      }
  };
  // one key tile; PAR = it % 2 fixes the LDS buffers at compile time
  auto tile = [&](auto par, int it) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    char* kc = P ? g_dq_k1 : g_dq_k0;
    char* vc = P ? g_dq_v1 : g_dq_v0;
    stage(P ? g_dq_k0 : g_dq_k1, P ? g_dq_v0 : g_dq_v1, tile_row(it + 1));
    const int k0 = tr.tile(it) * kTile;
    if (active) {
      half(kc, vc, 0, k0);
      if (k0 + 32 < S) half(kc, vc, 1, k0 + 32);
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): next tiles landed, reads done
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  for (int it = 0; it < nt; it += 2) {
    tile(std::integral_constant<int, 0>{}, it);
    if (it + 1 >= nt) break;
    tile(std::integral_constant<int, 1>{}, it + 1);
  }

  if (!active) return;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int i = q0 + cb * 32 + l32;
    if (i >= S) continue;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = db * 32 + 8 * r4 + 4 * hl;
        f32x4 w = {dq[db][cb][4 * r4] * p.scale, dq[db][cb][4 * r4 + 1] * p.scale,
                   dq[db][cb][4 * r4 + 2] * p.scale, dq[db][cb][4 * r4 + 3] * p.scale};
        if constexpr (ROPE) w = rope_back4(w, i, a.rope, d0 / 2);  // gradient of the unrotated Q
        *(f32x4*)(p.dq + (qslab_rows + i) * kHeadDim + d0) = w;
      }
  }
}

template <int DT, bool ROPE>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdArgs a) {
  dq_body<DT, ROPE>(a, (int)blockIdx.x);
}

// dK/dV and dQ in one launch: the dK/dV workgroups (heaviest key blocks first) come first,
// then the dQ workgroups (heaviest query blocks first), so dQ work fills the CUs that the
// light dK/dV blocks free while the heavy ones still run.  The two passes are independent
// (both only read Q, K, V, dO, lse, delta).
template <int DT, bool ROPE>
__global__ __launch_bounds__(256, 2) void bwd_fused_kernel(BwdArgs a) {
  const int n_dkdv = a.p.n_kblk * a.p.B * a.p.G;
  const int wg = (int)blockIdx.x;
  if (wg < n_dkdv)
    dkdv_dispatch<DT, ROPE>(a, wg);
  else
    dq_body<DT, ROPE>(a, wg - n_dkdv);
}

// Kernels by element type and by whether dQ / dK are rotated back at the store.
template <bool ROPE>
const void* bwd_kernel(int which, int dtype) {
  const bool bf = dtype == kDtBF16;
  if (which == 0) return bf ? (const void*)bwd_dkdv_kernel<kDtBF16, ROPE> : (const void*)bwd_dkdv_kernel<kDtF16, ROPE>;
  if (which == 1) return bf ? (const void*)bwd_dq_kernel<kDtBF16, ROPE> : (const void*)bwd_dq_kernel<kDtF16, ROPE>;
  return bf ? (const void*)bwd_fused_kernel<kDtBF16, ROPE> : (const void*)bwd_fused_kernel<kDtF16, ROPE>;
}

const void* pick_bwd(int which, const RopeSpec& rope, int dtype) {
  return rope.enabled ? bwd_kernel<true>(which, dtype) : bwd_kernel<false>(which, dtype);
}

}  // namespace

hipError_t launch_bwd_preprocess(const BwdParams& p, int dtype, hipStream_t s) {
  const long long rows = (long long)p.B * p.H * p.S;
  const int rows_per_block = (dtype == kDtF32) ? 16 : 32;
  dim3 grid((unsigned)((rows + rows_per_block - 1) / rows_per_block)), block(256);
  void* args[] = {(void*)&p};
  switch (dtype) {
    case kDtF32: return hipLaunchKernel((const void*)bwd_preprocess_kernel<kDtF32>, grid, block, args, 0, s);
    case kDtBF16: return hipLaunchKernel((const void*)bwd_preprocess_kernel<kDtBF16>, grid, block, args, 0, s);
    default: return hipLaunchKernel((const void*)bwd_preprocess_kernel<kDtF16>, grid, block, args, 0, s);
  }
}

hipError_t launch_bwd_dkdv_mfma(const BwdParams& p, const RopeSpec& rope, int dtype, hipStream_t s) {
  dim3 grid((unsigned)((long long)p.n_kblk * p.B * p.G)), block(256);
  BwdArgs a{p, rope};
  void* args[] = {(void*)&a};
  return hipLaunchKernel(pick_bwd(0, rope, dtype), grid, block, args, 0, s);
}

hipError_t launch_bwd_dq_mfma(const BwdParams& p, const RopeSpec& rope, int dtype, hipStream_t s) {
  dim3 grid((unsigned)((long long)p.n_qblk * p.B * (p.H / p.hpw))), block(256);
  BwdArgs a{p, rope};
  void* args[] = {(void*)&a};
  return hipLaunchKernel(pick_bwd(1, rope, dtype), grid, block, args, 0, s);
}

hipError_t launch_bwd_fused_mfma(const BwdParams& p, const RopeSpec& rope, int dtype, hipStream_t s) {
  const long long n = (long long)p.n_kblk * p.B * p.G + (long long)p.n_qblk * p.B * (p.H / p.hpw);
  dim3 grid((unsigned)n), block(256);
  BwdArgs a{p, rope};
  void* args[] = {(void*)&a};
  return hipLaunchKernel(pick_bwd(2, rope, dtype), grid, block, args, 0, s);
}

}  // namespace gqa
