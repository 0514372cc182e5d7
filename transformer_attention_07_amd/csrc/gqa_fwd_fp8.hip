// Forward of causal grouped-query attention with FP8 (OCP e4m3) Q, K and V on gfx950's
// FP8 matrix cores: the FlashAttention-3 forward's "FP8 computation" of the "SnapKitty
// Transformer 8B" model card (Protected Inventions list), with per-tensor dequantisation
// factors.
//
// Both products run on v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales), twice the
// bf16 rate: S^T = K Q^T contracts the whole head dimension in one instruction per 32x32
// block, and O^T += V^T P^T contracts 64 keys at once with P rounded to e4m3.  The work
// decomposition, tile ranges, masks and the lazy online softmax are those of the bf16
// forward (gqa_fwd.hip), with one change: P must stay below e4m3's 448, so a half goes
// through the exact maximum path when a lane's partial row sum exceeds 256 (not 2^16);
// after that path every P is at most 2^8.  And the P V product takes the whole tile, so
// when the second half raises the maximum, the first half's P (still waiting in the
// operand, at the old maximum) is added to O before the rescale (see decide).
//
// Operand order.  A 32x32x64 operand gives each lane 32 bytes of one row (lane % 32) for
// one k-group (lane / 32); the instruction pairs element i of group g of both operands,
// so any assignment of (g, i) to the contraction index works if both operands use it.
//   * Q K^T: group g holds head dimensions 32 g .. 32 g + 31 in order, for both.
//   * V^T P^T: P^T comes from the S^T accumulators, where register r of a lane in group g
//     holds key 8 (r / 4) + 4 g + r % 4 of a 32-key block; so element i of group g is key
//     kappa(g, i) = 32 (i / 16) + 8 ((i % 16) / 4) + 4 g + i % 4 of the 64-key tile.  A
//     pre-pass writes V transposed, with each tile's keys stored in that order
//     (vt_permute_kernel), so a V^T operand is 32 contiguous bytes as well.
// LDS tiles are 64 rows x 64 bytes; the 16-byte chunk c of row r is stored at chunk
// c ^ ((r >> 2) & 3), which makes the operand reads (16 consecutive rows, one chunk each)
// conflict-free.  Tiles arrive by direct loads into LDS, triple-buffered, one barrier per
// tile, as in the bf16 forward.
#include "gqa_device.h"

namespace gqa {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void8;

constexpr float kRescaleThreshold8 = 8.0f;  // log2 units: P <= 2^8 after the exact path
constexpr float kSumGuard8 = 256.0f;        // a lane's partial row sum above this: exact path
constexpr float kLn2_8 = 0.69314718055994530942f;
// The running maximum of a row before its first visible key: finite and below every score
// (log2 units), so the first visible key exponentiates to +inf and the row-sum guard takes
// the exact path; masked keys (-inf) still give 0.
constexpr float kNoMax8 = -1.0e38f;

__device__ __forceinline__ f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c) {
  // cbsz = blgp = 0: both operands e4m3; block scales 2^(127 - 127) = 1
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

__device__ __forceinline__ int chunk_off8(int row, int c) { return row * 64 + ((c ^ ((row >> 2) & 3)) << 4); }

__device__ __forceinline__ i32x8 join(u32x4 a, u32x4 b) {
  return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

// Four fp32 values rounded to e4m3 (nearest even) in one dword, first value in byte 0.
__device__ __forceinline__ int pack4_e4m3(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

struct Fp8Wave {
  int lane, l32, hl;
  int q0, q1;
  MaskSpec m;
  float c2;
  i32x8 qf[2];      // Q^T operands [column block]
  f32x16 o[2][2];   // O^T accumulators [d block][column block]
  float mrow[2], lrow[2], alpha[2], nmuse[2];
  int lim_hi, win_lo;
  bool rescale;
  int off[2];       // this lane's two operand chunks in a tile (row l32, chunks 2 hl, 2 hl + 1)

  // operand of rows 32 blk + l32 of an LDS tile (K: key block; V^T: d block)
  __device__ __forceinline__ i32x8 operand(const char* tile, int blk) const {
    return join(*(const u32x4*)(tile + blk * 2048 + off[0]), *(const u32x4*)(tile + blk * 2048 + off[1]));
  }
  __device__ __forceinline__ void scores(i32x8 ka, f32x16 (&s)[2]) const {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) s[cb] = mfma8(ka, qf[cb], f32x16{});
  }
  __device__ __forceinline__ void accumulate(const i32x8 (&va)[2], const i32x8 (&pf)[2]) {
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) o[db][cb] = mfma8(va[db], pf[cb], o[db][cb]);
  }

  __device__ __forceinline__ bool half_full(int k) const {
    return __builtin_amdgcn_readfirstlane((int)(k + 31 <= lim_hi) & ((int)(k >= win_lo) | (int)(k + 31 < m.sinks))) != 0;
  }

  // keys of this half that are not visible: register r of this lane holds key
  // k0 + 4 hl + 8 (r / 4) + r % 4
  __device__ __forceinline__ void mask(f32x16 (&s)[2], int k0) const {
    const int base = k0 + 4 * hl;
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

  // H = 1: the first half's P already sits in bytes 0..15 of the P operands at the old
  // maximum, waiting for the tile's P V; when the maximum is raised, that half is added to
  // O first (a P V with the second half's bytes zero) so that the rescale covers it, and
  // its bytes are cleared, so the tile's P V adds the second half alone.
  template <int H>
  __device__ __forceinline__ void decide(const f32x16 (&s)[2], i32x8 (&pf)[2], const i32x8 (&va)[2]) {
    float mx[2];
    bool need = false;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      float a = vmax(s[cb][0], s[cb][1]);
#pragma unroll
      for (int r = 2; r < 16; r += 2) a = vmax(vmax(a, s[cb][r]), s[cb][r + 1]);
      uint32_t u = __builtin_bit_cast(uint32_t, a);
      auto pr = __builtin_amdgcn_permlane32_swap(u, u, false, false);
      mx[cb] = vmax(__builtin_bit_cast(float, (uint32_t)pr[0]), __builtin_bit_cast(float, (uint32_t)pr[1])) * c2;
      need = need | (mx[cb] > mrow[cb] + kRescaleThreshold8);
    }
    rescale = wave_any(need);
    if (__builtin_expect(rescale, 0)) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const float mnew = vmax(mrow[cb], mx[cb]);
        alpha[cb] = exp2_fast(mrow[cb] - mnew);  // finite: mrow starts at kNoMax8
        mrow[cb] = mnew;
        nmuse[cb] = -mnew;
        lrow[cb] *= alpha[cb];
      }
      if constexpr (H == 1) {
        i32x8 p0[2];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          p0[cb] = pf[cb];
#pragma unroll
          for (int w = 4; w < 8; ++w) p0[cb][w] = 0;
        }
        accumulate(va, p0);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
          for (int w = 0; w < 4; ++w) pf[cb][w] = 0;
      }
      apply_rescale();
    }
  }

  // P^T of one half at the current maximum, rounded to e4m3 into dwords 4 h .. 4 h + 3 of
  // the B operands (bytes 16 h + r: key kappa(hl, 16 h + r)); row sums of the unrounded P
  template <int H>
  __device__ __forceinline__ void probs(const f32x16 (&s)[2], i32x8 (&pf)[2], float (&ls)[2]) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      float pv[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) pv[e] = exp2_fast(__builtin_fmaf(s[cb][e], c2, nmuse[cb]));
      float lsum = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        pf[cb][4 * H + w] = pack4_e4m3(pv[4 * w], pv[4 * w + 1], pv[4 * w + 2], pv[4 * w + 3]);
        lsum += (pv[4 * w] + pv[4 * w + 1]) + (pv[4 * w + 2] + pv[4 * w + 3]);
      }
      ls[cb] = lsum;
    }
  }

  template <int H>
  __device__ __forceinline__ void softmax_half(const f32x16 (&s)[2], i32x8 (&pf)[2], const i32x8 (&va)[2]) {
    float ls[2];
    probs<H>(s, pf, ls);
    const bool need = !(ls[0] <= kSumGuard8) | !(ls[1] <= kSumGuard8);
    if (__builtin_expect(wave_any(need), 0)) {
      decide<H>(s, pf, va);
      probs<H>(s, pf, ls);
    }
    lrow[0] += ls[0];
    lrow[1] += ls[1];
  }

  __device__ __forceinline__ void apply_rescale() {
    asm volatile("" ::: "memory");
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) o[db][cb] *= alpha[cb];
  }
};

template <int VM>
__device__ __forceinline__ void lds_barrier8() {
  static_assert(VM >= 0 && VM < 16, "vmcnt field");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0070 | VM);  // vmcnt(VM) expcnt(7) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wave `wave` fills LDS bytes 1024 wave .. + 1023 (rows 16 wave .. 16 wave + 15) of a
// 64 x 64-byte tile: lane i writes LDS row 16 wave + i / 4, stored chunk i % 4, so it loads
// global chunk (i % 4) ^ (row >> 2 & 3) of that row.  `voff` is that byte offset within
// the tile's global rows (row pitch `pitch`); `base` moves it to the tile.
__device__ __forceinline__ int tile_voff(int wave, int lane, int pitch) {
  const int r = 16 * wave + (lane >> 2);
  return r * pitch + (((lane & 3) ^ ((r >> 2) & 3)) << 4);
}

__device__ __forceinline__ void stage8(__amdgpu_buffer_rsrc_t rs, char* tile, int base, int voff, int wave) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void8*)(tile + 1024 * wave), 16, base + voff, 0, 0, 0);
}

__global__ __launch_bounds__(256, 2) void fwd_fp8_kernel(Fp8FwdParams p) {
  __shared__ __attribute__((aligned(1024))) char k_lds0[4096];
  __shared__ __attribute__((aligned(1024))) char k_lds1[4096];
  __shared__ __attribute__((aligned(1024))) char k_lds2[4096];
  __shared__ __attribute__((aligned(1024))) char v_lds0[4096];
  __shared__ __attribute__((aligned(1024))) char v_lds1[4096];
  __shared__ __attribute__((aligned(1024))) char v_lds2[4096];

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

  Fp8Wave W;
  W.lane = lane;
  W.l32 = lane & 31;
  W.hl = lane >> 5;
  W.q0 = Q0 + (wave / p.hpw) * kTile;
  W.q1 = imin(W.q0 + kTile - 1, S - 1);
  W.m = p.mask;
  W.c2 = p.scale_log2;
  W.off[0] = chunk_off8(W.l32, 2 * W.hl);
  W.off[1] = chunk_off8(W.l32, 2 * W.hl + 1);
  const bool active = W.q0 < S;
  const size_t slab_q = (size_t)(b * p.H + h) * S * kHeadDim;  // bytes (1 per element)
  const size_t slab_k = (size_t)(b * p.G + g) * S * kHeadDim;
  const __amdgpu_buffer_rsrc_t qrs = byte_rsrc((const uint8_t*)p.q + slab_q, (uint32_t)S * kHeadDim);
  const __amdgpu_buffer_rsrc_t krs = byte_rsrc((const uint8_t*)p.k + slab_k, (uint32_t)S * kHeadDim);
  const __amdgpu_buffer_rsrc_t vrs = byte_rsrc((const uint8_t*)p.vt + (size_t)(b * p.G + g) * kHeadDim * p.s_pad,
                                               (uint32_t)kHeadDim * p.s_pad);

  const TileRanges tr = key_tiles_for_rows(W.m, Q0, Q1);
  const int nt = tr.count();
  const int kvoff = tile_voff(wave, lane, 64);
  const int vvoff = tile_voff(wave, lane, p.s_pad);
  // global byte offset of key tile n in K (rows) and in V^T (columns); past the last tile
  // both point past the end of their slab, so the loads return zeros
  auto k_base = [&](int n) __attribute__((always_inline)) { return (n < nt ? tr.tile(n) * kTile : S) * 64; };
  auto v_base = [&](int n) __attribute__((always_inline)) { return n < nt ? tr.tile(n) * kTile : kHeadDim * p.s_pad; };

  stage8(krs, k_lds0, k_base(0), kvoff, wave);
  stage8(vrs, v_lds0, v_base(0), vvoff, wave);
  stage8(krs, k_lds1, k_base(1), kvoff, wave);

#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int off = (W.q0 + cb * 32 + W.l32) * 64 + W.hl * 32;
    W.qf[cb] = join(buf_load16(qrs, off), buf_load16(qrs, off + 16));
  }
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) W.o[db][cb] = f32x16{};
  W.mrow[0] = W.mrow[1] = kNoMax8;
  W.lrow[0] = W.lrow[1] = 0.f;
  W.alpha[0] = W.alpha[1] = 1.f;
  W.nmuse[0] = W.nmuse[1] = -kNoMax8;
  W.lim_hi = __builtin_amdgcn_readfirstlane(W.m.causal ? imin(W.q0, S - 1) : S - 1);
  W.win_lo = __builtin_amdgcn_readfirstlane(W.m.window > 0 ? W.q1 - W.m.window + 1 : -(1 << 30));
  W.rescale = false;

  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // The bf16 forward's half-tile pipeline: a step softmaxes one 32-key half while the
  // matrix cores compute the scores of the next; the two halves' P fill one 64-key
  // operand, which feeds O^T += V^T P^T at the end of the tile.  K_{n+2} and V_{n+1} are
  // staged right after the barrier into the buffers of K_{n-1} and V_{n-2}.
  f32x16 sc[2], sn[2];
  i32x8 ka = W.operand(k_lds0, 0);
  W.scores(ka, sc);
  ka = W.operand(k_lds0, 1);

  auto tile = [&](auto par, int n) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    char* kn1 = P == 0 ? k_lds1 : P == 1 ? k_lds2 : k_lds0;
    char* kn2 = P == 0 ? k_lds2 : P == 1 ? k_lds0 : k_lds1;
    char* vn = P == 0 ? v_lds0 : P == 1 ? v_lds1 : v_lds2;
    char* vn1 = P == 0 ? v_lds1 : P == 1 ? v_lds2 : v_lds0;
    const int k0 = tr.tile(n) * kTile;
    i32x8 pf[2];
    stage8(krs, kn2, k_base(n + 2), kvoff, wave);
    stage8(vrs, vn1, v_base(n + 1), vvoff, wave);
    W.scores(ka, sn);                       // S(n, 1)
    const i32x8 va[2] = {W.operand(vn, 0), W.operand(vn, 1)};
    ka = W.operand(kn1, 0);
    if (__builtin_expect(!W.half_full(k0), 0)) W.mask(sc, k0);
    W.softmax_half<0>(sc, pf, va);
    W.scores(ka, sc);                       // S(n + 1, 0)
    ka = W.operand(kn1, 1);
    if (__builtin_expect(!W.half_full(k0 + 32), 0)) W.mask(sn, k0 + 32);
    W.softmax_half<1>(sn, pf, va);
    W.accumulate(va, pf);
    lds_barrier8<0>();
  };
  for (int n = 0; n < nt; n += 3) {
    tile(std::integral_constant<int, 0>{}, n);
    if (n + 1 >= nt) break;
    tile(std::integral_constant<int, 1>{}, n + 1);
    if (n + 2 >= nt) break;
    tile(std::integral_constant<int, 2>{}, n + 2);
  }

  if (!active) return;
  uint16_t* oslab = (uint16_t*)p.o + (size_t)(b * p.H + h) * S * kHeadDim;
  float* lse_row = p.lse + (size_t)(b * p.H + h) * S;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const float l = sum_across_halves(W.lrow[cb]);
    const int i = W.q0 + cb * 32 + W.l32;
    if (i >= S) continue;
    const float inv = p.o_scale / l;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = db * 32 + 8 * r4 + 4 * W.hl;
        const u32x2 w = {pack2<kDtBF16>(W.o[db][cb][4 * r4] * inv, W.o[db][cb][4 * r4 + 1] * inv),
                         pack2<kDtBF16>(W.o[db][cb][4 * r4 + 2] * inv, W.o[db][cb][4 * r4 + 3] * inv)};
        *(u32x2*)(oslab + (size_t)i * kHeadDim + d0) = w;
      }
    if (W.hl == 0) lse_row[i] = (W.mrow[cb] + log2f(l)) * kLn2_8;
  }
}

// V [n][S][64] e4m3 -> V^T [n][64][s_pad] with each 64-key tile's keys in the order of the
// P^T operand: byte 32 g + i of a tile row holds key kappa(g, i); keys at or past S are 0.
// One workgroup per (slab, tile): the tile is staged in LDS, then each thread writes 16
// bytes of one V^T row.
__global__ __launch_bounds__(256) void vt_permute_kernel(VtParams p) {
  __shared__ uint8_t t[kTile][kHeadDim + 4];
  const int ntile = p.s_pad / kTile;
  const long long n = blockIdx.x / ntile;
  const int tile = (int)(blockIdx.x % ntile);
  const int tid = threadIdx.x;
  {
    const int key = tid >> 2, c = tid & 3;
    const int j = tile * kTile + key;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (j < p.S) x = *(const u32x4*)((const uint8_t*)p.v + ((size_t)n * p.S + j) * kHeadDim + 16 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) *(uint32_t*)&t[key][16 * c + 4 * e] = x[e];
  }
  __syncthreads();
  const int d = tid >> 2, c = tid & 3;
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint32_t acc = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int pos = 16 * c + 4 * e + b;  // 32 g + i
      const int gg = pos >> 5, i = pos & 31;
      const int key = 32 * (i >> 4) + 8 * ((i & 15) >> 2) + 4 * gg + (i & 3);
      acc |= (uint32_t)t[key][d] << (8 * b);
    }
    w[e] = acc;
  }
  *(u32x4*)((uint8_t*)p.vt + ((size_t)n * kHeadDim + d) * p.s_pad + (size_t)tile * kTile + 16 * c) =
      u32x4{w[0], w[1], w[2], w[3]};
}

}  // namespace

hipError_t launch_vt_permute(const VtParams& p, hipStream_t s) {
  const long long blocks = p.n_slabs * (p.s_pad / kTile);
  void* args[] = {(void*)&p};
  return hipLaunchKernel((const void*)vt_permute_kernel, dim3((unsigned)blocks), dim3(256), args, 0, s);
}

hipError_t launch_fwd_fp8(const Fp8FwdParams& p, hipStream_t s) {
  const long long nblk = (long long)p.n_qblk * p.B * (p.H / p.hpw);
  void* args[] = {(void*)&p};
  return hipLaunchKernel((const void*)fwd_fp8_kernel, dim3((unsigned)nblk), dim3(256), args, 0, s);
}

}  // namespace gqa
