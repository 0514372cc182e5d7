// Forward pass of causal grouped-query attention on gfx950 matrix cores (bf16 / f16).
//
// One workgroup = 4 wavefronts over one batch b and one kv head g.  Wave w owns a
// 64-row query tile of query head h (hpw heads x qpw row tiles per workgroup; all heads
// belong to kv group g, so every wave reads the same K/V tiles).  The workgroup walks the
// key tiles that hold at least one visible key (sink tiles, then the window/causal
// range; everything between is never loaded).  Per key tile:
//   * K (row-major) and V (transposed) are staged into LDS, double-buffered: the next
//     tile's global loads are issued before this tile's math and written after it.
//   * S^T = K Q^T on MFMA: the Q tile of the wave lives in registers as the B operand,
//     so each lane of the accumulator holds one query column; row statistics are
//     in-lane plus one exchange between the two 32-lane halves.
//   * online softmax in fp32 (exp2 with scale*log2(e) folded into one FMA); the running
//     maximum is only raised when a tile's maximum exceeds it by more than 2^8, so the
//     rescale of O is skipped on almost every tile and P stays below 2^8.
//   * O^T += V^T P^T on MFMA with P^T taken from the S^T accumulator registers.
// Tiles that are fully visible skip the mask arithmetic; partial tiles (diagonal, window
// start, sink edge, ragged end) mask element by element.
// The online softmax with running max and sum and the fused score/softmax/PV loop follow
// the "SnapKitty Transformer 8B" model card's FlashAttention Kernel section; the tiling,
// operand orientation and staging here are this library's own for CDNA4.
#include "gqa_device.h"

namespace gqa {

namespace {

constexpr float kRescaleThreshold = 8.0f;  // log2 units
constexpr float kLn2 = 0.69314718055994530942f;

template <int DT>
__global__ __launch_bounds__(256, 2) void fwd_mfma_kernel(FwdParams p) {
  __shared__ __attribute__((aligned(16))) char smem[2][2][8192];  // [buffer][K | V^T]

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  // heaviest (latest) row blocks first
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
  const int q0 = Q0 + (wave / p.hpw) * kTile;
  const int q1 = imin(q0 + kTile - 1, S - 1);
  const bool active = q0 < S;
  const MaskSpec m = p.mask;

  const uint16_t* qslab = (const uint16_t*)p.q + (size_t)(b * p.H + h) * S * kHeadDim;
  const uint16_t* kslab = (const uint16_t*)p.k + (size_t)(b * p.G + g) * S * kHeadDim;
  const uint16_t* vslab = (const uint16_t*)p.v + (size_t)(b * p.G + g) * S * kHeadDim;

  // Q tile as B operands: column block cb (rows q0 + 32cb + l32), contraction step ks.
  u32x4 qf[2][4];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int row = q0 + cb * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (active && row < S)
        qf[cb][ks] = *(const u32x4*)(qslab + (size_t)row * kHeadDim + ks * 16 + hl * 8);
      else
        qf[cb][ks] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  // staging roles: threads 0..127 stage K (row-major), 128..255 stage V (transposed)
  const int kind = tid >> 7;
  const int unit = tid & 127;
  const int ur0 = (unit >> 3) * 4;
  const int udc = unit & 7;
  const uint16_t* stage_slab = kind == 0 ? kslab : vslab;
  Unit st;

  const TileRanges tr = key_tiles_for_rows(m, Q0, Q1);
  const int nt = tr.count();

  f32x16 o[2][2];  // O^T accumulators [d block][column block]
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) o[db][cb] = f32x16{};
  float mrow[2] = {-INFINITY, -INFINITY};
  float lrow[2] = {0.f, 0.f};
  const float c2 = p.scale_log2;

  if (nt > 0) {
    unit_load(st, stage_slab, tr.tile(0) * kTile + ur0, udc, S);
    if (kind == 0)
      unit_store_rm(smem[0][0], st, ur0, udc);
    else
      unit_store_tr(smem[0][1], st, ur0, udc);
  }
  __syncthreads();

  for (int it = 0; it < nt; ++it) {
    const int kt = tr.tile(it);
    const int k0 = kt * kTile;
    const bool more = it + 1 < nt;
    if (more) unit_load(st, stage_slab, tr.tile(it + 1) * kTile + ur0, udc, S);

    const int cls = active ? classify(m, q0, q1, k0, k0 + kTile - 1) : (int)kEmpty;
    if (cls != kEmpty) {
      const char* kl = smem[it & 1][0];
      const char* vl = smem[it & 1][1];

      // S^T[kb][cb] = K[kb] Q^T[cb]
      f32x16 s[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) s[kb][cb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const u32x4 a = lds_rm_operand(kl, kb, ks, l32, hl);
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) s[kb][cb] = mfma32<DT>(a, qf[cb][ks], s[kb][cb]);
        }
      }

      if (cls == kPartial) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
            const int i = q0 + cb * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int j = k0 + kb * 32 + acc_row(r, hl);
              if (!visible(m, i, j)) s[kb][cb][r] = -INFINITY;
            }
          }
      }

      // online softmax per query column; P^T packed into B operands [kb][cb][t]
      u32x4 pf[2][2][2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][cb][r]);
        mx = max_across_halves(mx) * c2;
        if (wave_any(mx > mrow[cb] + kRescaleThreshold)) {
          const float mnew = fmaxf(mrow[cb], mx);
          const float alpha = (mnew == -INFINITY) ? 1.f : exp2_fast(mrow[cb] - mnew);
          mrow[cb] = mnew;
          lrow[cb] *= alpha;
#pragma unroll
          for (int db = 0; db < 2; ++db) o[db][cb] *= alpha;
        }
        const float muse = (mrow[cb] == -INFINITY) ? 0.f : mrow[cb];
        float lsum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            float pv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              pv[e] = exp2_fast(__builtin_fmaf(s[kb][cb][8 * t + e], c2, -muse));
              lsum += pv[e];
            }
            pf[kb][cb][t] = u32x4{pack2<DT>(pv[0], pv[1]), pack2<DT>(pv[2], pv[3]),
                                  pack2<DT>(pv[4], pv[5]), pack2<DT>(pv[6], pv[7])};
          }
        lrow[cb] += lsum;
      }

      // O^T[db][cb] += V^T[db] P^T[cb]
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const u32x4 a = lds_tr_operand(vl, db, kb, t, l32, hl);
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) o[db][cb] = mfma32<DT>(a, pf[kb][cb][t], o[db][cb]);
          }
    }

    if (more) {
      if (kind == 0)
        unit_store_rm(smem[(it + 1) & 1][0], st, ur0, udc);
      else
        unit_store_tr(smem[(it + 1) & 1][1], st, ur0, udc);
    }
    __syncthreads();
  }

  if (!active) return;
  uint16_t* oslab = (uint16_t*)p.o + (size_t)(b * p.H + h) * S * kHeadDim;
  uint16_t* olo_slab = p.o_lo ? (uint16_t*)p.o_lo + (size_t)(b * p.H + h) * S * kHeadDim : nullptr;
  float* lse_row = p.lse + (size_t)(b * p.H + h) * S;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const float l = sum_across_halves(lrow[cb]);
    const int i = q0 + cb * 32 + l32;
    if (i >= S) continue;
    const float inv = 1.0f / l;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = db * 32 + 8 * r4 + 4 * hl;
        const float x0 = o[db][cb][4 * r4 + 0] * inv, x1 = o[db][cb][4 * r4 + 1] * inv;
        const float x2 = o[db][cb][4 * r4 + 2] * inv, x3 = o[db][cb][4 * r4 + 3] * inv;
        const u32x2 w = {pack2<DT>(x0, x1), pack2<DT>(x2, x3)};
        *(u32x2*)(oslab + (size_t)i * kHeadDim + d0) = w;
        if (olo_slab != nullptr) {
          const u32x2 r = {pack2_residual<DT>(x0, x1, w[0]), pack2_residual<DT>(x2, x3, w[1])};
          *(u32x2*)(olo_slab + (size_t)i * kHeadDim + d0) = r;
        }
      }
    if (hl == 0) lse_row[i] = (mrow[cb] + log2f(l)) * kLn2;
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
