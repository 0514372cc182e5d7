// Forward pass of causal grouped-query attention on gfx950 matrix cores (bf16 / f16).
//
// Work decomposition.  One workgroup = 4 wavefronts over one batch b and one kv head g,
// two workgroups per CU (two waves per SIMD).  Wave w owns a 64-row query tile of query
// head h (hpw heads x qpw row tiles per workgroup; all heads belong to kv group g, so every
// wave reads the same K/V tiles).  The workgroup walks the key tiles that hold at least
// one visible key: sink tiles, then the window/causal range; everything between is never
// loaded.  K and V tiles are staged row-major into LDS, double-buffered: the next tile's
// buffer loads (which read zero past the end of the sequence) are issued before this
// tile's math and written after it, one barrier per tile.
//
// Per wave, S^T = K Q^T runs on v_mfma_f32_32x32x16 with the wave's Q tile held in
// registers as the B operand, so each accumulator lane holds one query column: row
// statistics are in-lane plus one exchange between the two 32-lane halves.  All scores of
// a 64-key tile are issued first; one running-maximum decision covers the tile; then the
// probabilities of the first 32-key half feed O^T += V^T P^T on the matrix cores while the
// VALU exponentiates the second half.  V^T operands come from the row-major V tile through
// ds_read_b64_tr_b16 transposed reads, and P^T straight from the S^T accumulator registers
// (see gqa_device.h).  The online softmax runs in fp32: exp2 with scale*log2(e) folded into
// one FMA, row sums of the unrounded P in fp32 (so lse keeps fp32 accuracy), and a running
// maximum that is only raised when a tile's maximum exceeds it by more than 2^8, so the O
// rescale is skipped on almost every tile and P stays below 2^8.  Halves that are not fully
// visible are masked with one compare per element against per-lane bounds.
//
// The online softmax with running max and sum and the fused score/softmax/PV loop follow
// the "SnapKitty Transformer 8B" model card's FlashAttention Kernel section; the tiling,
// operand orientation and staging here are this library's own for CDNA4.
#include "gqa_device.h"

namespace gqa {

namespace {

constexpr float kRescaleThreshold = 8.0f;  // log2 units
constexpr float kLn2 = 0.69314718055994530942f;

// Per-wave state and the pieces of one key tile, processed as two 32-key halves.
template <int DT>
struct FwdWave {
  int lane, l32, hl;
  int q0, q1;
  MaskSpec m;
  float c2;
  u32x4 qf[2][4];   // Q tile as B operands [column block][contraction step]
  f32x16 o[2][2];   // O^T accumulators [d block][column block]
  float mrow[2];    // running maximum (log2 units) per column block
  float lrow[2];    // running sum (this lane's half of the keys)
  float alpha[2];   // rescale factor decided by the last softmax
  bool rescale;     // wave-uniform: the last softmax raised the maximum

  // S^T[cb] = K[kb] Q^T[cb] for key half kb of the tile in `kl` (row-major LDS tile)
  __device__ __forceinline__ void scores(const char* kl, int kb, f32x16 (&s)[2]) const {
    u32x4 a[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) a[ks] = lds_rm_operand(kl, kb, ks, l32, hl);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) s[cb] = mfma32<DT>(a[0], qf[cb][0], f32x16{});
#pragma unroll
    for (int ks = 1; ks < 4; ++ks)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) s[cb] = mfma32<DT>(a[ks], qf[cb][ks], s[cb]);
  }

  // O^T[db][cb] += V^T[db] P^T[cb] over key half kb of the tile in `vl` (row-major tile,
  // read transposed)
  __device__ __forceinline__ void accumulate(const char* vl, int kb, const u32x4 (&pf)[2][2]) {
    u32x4 a[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < 2; ++db) a[db][t] = lds_rm_transposed_operand(vl, db, kb, t, lane);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) o[db][cb] = mfma32<DT>(a[db][t], pf[cb][t], o[db][cb]);
  }

  // hide keys that are not visible (halves that are not fully visible only).  Register r of
  // this lane holds key k0 + 4*hl + rr(r) with rr(r) = 8*(r/4) + r%4 a compile-time constant,
  // so every test is one compare of rr against a per-lane bound.
  __device__ __forceinline__ void mask(f32x16 (&s)[2], int k0) const {
    const int base = k0 + 4 * hl;
    const int kmax = m.S - 1 - base;  // rr <= kmax: key inside the sequence
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int i = q0 + cb * 32 + l32;
      const int causal_hi = m.causal ? i - base : kmax;       // rr <= causal_hi: not in the future
      const int hi = causal_hi < kmax ? causal_hi : kmax;
      const int win_lo = m.window > 0 ? i - m.window + 1 - base : -(1 << 30);  // rr >= win_lo: in window
      const int sink_hi = m.sinks - 1 - base;                  // rr <= sink_hi: a sink
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rr = 8 * (r >> 2) + (r & 3);
        const bool ok = (rr <= hi) && (rr >= win_lo || rr <= sink_hi);
        s[cb][r] = ok ? s[cb][r] : -INFINITY;
      }
    }
  }

  // running-maximum update for one 64-key tile (both halves): sets rescale/alpha/mrow
  __device__ __forceinline__ void decide(const f32x16 (&s0)[2], const f32x16 (&s1)[2]) {
    float mx[2];
    bool need = false;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      float a = vmax(s0[cb][0], s0[cb][1]);
#pragma unroll
      for (int r = 2; r < 16; r += 2) a = vmax(vmax(a, s0[cb][r]), s0[cb][r + 1]);
#pragma unroll
      for (int r = 0; r < 16; r += 2) a = vmax(vmax(a, s1[cb][r]), s1[cb][r + 1]);
      mx[cb] = max_across_halves(a) * c2;
      need = need || (mx[cb] > mrow[cb] + kRescaleThreshold);
    }
    rescale = wave_any(need);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const float mnew = rescale ? vmax(mrow[cb], mx[cb]) : mrow[cb];
      alpha[cb] = (rescale && mnew != -INFINITY) ? exp2_fast(mrow[cb] - mnew) : 1.0f;
      mrow[cb] = mnew;
      lrow[cb] *= alpha[cb];
    }
  }

  // P^T of one half tile at the current maximum, packed into B operands [cb][t]
  __device__ __forceinline__ void probs(const f32x16 (&s)[2], u32x4 (&pf)[2][2]) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const float muse = (mrow[cb] == -INFINITY) ? 0.f : mrow[cb];
      float lsum = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = exp2_fast(__builtin_fmaf(s[cb][8 * t + e], c2, -muse));
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          pf[cb][t][w] = pack2<DT>(pv[2 * w], pv[2 * w + 1]);
          lsum += pv[2 * w] + pv[2 * w + 1];
        }
      }
      lrow[cb] += lsum;
    }
  }

  __device__ __forceinline__ void apply_rescale() {
    // keep this block a real branch: O *= 1 is an identity, and hoisting the 64 multiplies
    // out of the (rare) branch would put them on every step
    asm volatile("" ::: "memory");
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) o[db][cb] *= alpha[cb];
  }
};

template <int DT>
__global__ __launch_bounds__(256, 2) void fwd_mfma_kernel(FwdParams p) {
  __shared__ __attribute__((aligned(16))) char k_lds[2][8192];
  __shared__ __attribute__((aligned(16))) char v_lds[2][8192];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int nhq = p.H / p.hpw;
  const int per_q = p.B * nhq;
  const int qblk = p.n_qblk - 1 - (int)(blockIdx.x / per_q);
  const int rest = (int)(blockIdx.x % per_q);
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
  const bool active = W.q0 < S;
  const __amdgpu_buffer_rsrc_t qrs = slab_rsrc((const uint16_t*)p.q + (size_t)(b * p.H + h) * S * kHeadDim, S);
  const __amdgpu_buffer_rsrc_t krs = slab_rsrc((const uint16_t*)p.k + (size_t)(b * p.G + g) * S * kHeadDim, S);
  const __amdgpu_buffer_rsrc_t vrs = slab_rsrc((const uint16_t*)p.v + (size_t)(b * p.G + g) * S * kHeadDim, S);
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      W.qf[cb][ks] = buf_load16(qrs, (W.q0 + cb * 32 + W.l32) * 128 + ks * 32 + W.hl * 16);
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) W.o[db][cb] = f32x16{};
  W.mrow[0] = W.mrow[1] = -INFINITY;
  W.lrow[0] = W.lrow[1] = 0.f;
  W.alpha[0] = W.alpha[1] = 1.f;
  W.rescale = false;

  const TileRanges tr = key_tiles_for_rows(W.m, Q0, Q1);
  const int nt = tr.count();
  const int kind = wave >> 1;
  const int unit = tid & 127;
  const int ur0 = (unit >> 3) * 4;
  const int udc = unit & 7;
  Unit st;
  auto tile_row = [&](int n) __attribute__((always_inline)) { return n < nt ? tr.tile(n) * kTile : S; };

  const int flip = (unit >> 3) & 1;  // alternate row order by unit parity
  unit_load_buf_rm(st, kind == 0 ? krs : vrs, tile_row(0) + ur0, udc, flip);
  unit_store_rm_flip(kind == 0 ? k_lds[0] : v_lds[0], st, ur0, udc, flip);
  __syncthreads();
  for (int n = 0; n < nt; ++n) {
    unit_load_buf_rm(st, kind == 0 ? krs : vrs, tile_row(n + 1) + ur0, udc, flip);
    const int k0 = tr.tile(n) * kTile;
    f32x16 s0[2], s1[2];
    u32x4 p0[2][2], p1[2][2];
    W.scores(k_lds[n & 1], 0, s0);
    W.scores(k_lds[n & 1], 1, s1);
    if (__builtin_expect(classify(W.m, W.q0, W.q1, k0, k0 + 31) != kFull, 0)) W.mask(s0, k0);
    if (__builtin_expect(classify(W.m, W.q0, W.q1, k0 + 32, k0 + 63) != kFull, 0)) W.mask(s1, k0 + 32);
    W.decide(s0, s1);
    if (__builtin_expect(W.rescale, 0)) W.apply_rescale();
    W.probs(s0, p0);
    W.accumulate(v_lds[n & 1], 0, p0);
    W.probs(s1, p1);
    W.accumulate(v_lds[n & 1], 1, p1);
    unit_store_rm_flip(kind == 0 ? k_lds[(n + 1) & 1] : v_lds[(n + 1) & 1], st, ur0, udc, flip);
    __syncthreads();
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
  if (dtype == kDtBF16) return hipLaunchKernel((const void*)fwd_mfma_kernel<kDtBF16>, grid, block, args, 0, s);
  return hipLaunchKernel((const void*)fwd_mfma_kernel<kDtF16>, grid, block, args, 0, s);
}

}  // namespace gqa
