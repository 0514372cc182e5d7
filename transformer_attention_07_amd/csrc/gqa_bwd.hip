// Backward pass of causal grouped-query attention on gfx950 matrix cores (bf16 / f16
// inputs, fp32 gradients).  Loss convention L = <O, dO>.
//
//   preprocess : delta_i = sum_c dO_ic O_ic                       (HBM-bound, fp32)
//   dK/dV      : per (b, g, 256-key block), 4 waves x 64 keys.  For every query head of
//                the group and every query tile that sees the block:
//                  S  = Q K^T        P = exp(scale*S - lse)   (recomputed from the saved lse)
//                  dP = dO V^T       dS = P * (dP - delta)
//                  dV^T += dO^T P    dK^T += Q^T dS           (scale applied at the end)
//                The sum over the H/G heads of the group stays in registers: no atomics.
//   dQ         : per (b, h, 64-row tile), the forward's decomposition.  For every key
//                tile it sees: S^T = K Q^T, dP^T = V dO^T, dS^T = P^T (dP^T - delta),
//                dQ^T += K^T dS^T.  Deterministic (each dQ element has one writer).
//
// The recompute of P from the saved log-sum-exp and dS = P * (dO V^T - D) follow the
// FlashAttention-3 backward entry of the "SnapKitty Transformer 8B" model card
// (Protected Inventions); that entry reduces dQ with atomics across query tiles, which
// this library replaces by the separate deterministic dQ pass.
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

// ------------------------------------------------------------------------------------
// dK, dV
// ------------------------------------------------------------------------------------
struct DkdvStage {
  char q_rm[8192];
  char q_tr[8192];
  char do_rm[8192];
  char do_tr[8192];
  float lse2[64];
  float delta[64];
};

template <int DT>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(16))) DkdvStage stage[2];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hl = lane >> 5;
  const int S = p.S;
  const MaskSpec m = p.mask;
  const int hpg = p.H / p.G;

  // heaviest (earliest) key blocks first
  const int per_k = p.B * p.G;
  const int kblk = (int)(blockIdx.x / per_k);
  const int rest = (int)(blockIdx.x % per_k);
  const int b = rest / p.G;
  const int g = rest % p.G;
  const int K0 = kblk * 4 * kTile;
  const int K1 = imin(K0 + 4 * kTile, S) - 1;
  const int kw0 = K0 + wave * kTile;
  const int kw1 = imin(kw0 + kTile - 1, S - 1);
  const bool active = kw0 < S;
  // Sink keys collect attention from every later query, so their dK and dV are sums of
  // many large terms: there P and dS enter the MFMAs as a rounded value plus its rounded
  // residual (two products each), which keeps the rounding of P and dS out of the sum.
  const bool precise = m.window > 0 && kw0 < m.sinks;

  const uint16_t* kslab = (const uint16_t*)p.k + (size_t)(b * p.G + g) * S * kHeadDim;
  const uint16_t* vslab = (const uint16_t*)p.v + (size_t)(b * p.G + g) * S * kHeadDim;

  // K and V rows of this wave as B operands: column block cb (keys kw0 + 32cb + l32)
  u32x4 kf[2][4], vf[2][4];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int row = kw0 + cb * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (active && row < S) {
        kf[cb][ks] = *(const u32x4*)(kslab + (size_t)row * kHeadDim + ks * 16 + hl * 8);
        vf[cb][ks] = *(const u32x4*)(vslab + (size_t)row * kHeadDim + ks * 16 + hl * 8);
      } else {
        kf[cb][ks] = u32x4{0u, 0u, 0u, 0u};
        vf[cb][ks] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }

  f32x16 dk[2][2], dv[2][2];  // transposed accumulators [d block][key column block]
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      dk[db][cb] = f32x16{};
      dv[db][cb] = f32x16{};
    }

  // staging roles: threads 0..127 stage Q units, 128..255 dO units (both RM and TR);
  // threads 0..63 also stage lse (in log2 units), 64..127 delta.
  const int kind = tid >> 7;
  const int unit = tid & 127;
  const int ur0 = (unit >> 3) * 4;
  const int udc = unit & 7;
  Unit st;
  float st_f = 0.f;

  const TileRanges tr = query_tiles_for_keys(m, K0, K1);
  const int nq = tr.count();
  const int n_iter = nq * hpg;
  const float c2 = p.scale_log2;

  auto load_stage = [&](int iter) {
    const int hh = iter / nq;
    const int qt = tr.tile(iter % nq);
    const int h = g * hpg + hh;
    const size_t slab = (size_t)(b * p.H + h) * S;
    const uint16_t* src = (const uint16_t*)(kind == 0 ? p.q : p.d_o) + slab * kHeadDim;
    unit_load(st, src, qt * kTile + ur0, udc, S);
    if (tid < 128) {
      const int i = qt * kTile + (tid & 63);
      if (tid < 64)
        st_f = (i < S) ? p.lse[slab + i] * kLog2e : INFINITY;
      else
        st_f = (i < S) ? p.delta[slab + i] : 0.f;
    }
  };
  auto store_stage = [&](int buf) {
    DkdvStage& sb = stage[buf];
    if (kind == 0) {
      unit_store_rm(sb.q_rm, st, ur0, udc);
      unit_store_tr(sb.q_tr, st, ur0, udc);
    } else {
      unit_store_rm(sb.do_rm, st, ur0, udc);
      unit_store_tr(sb.do_tr, st, ur0, udc);
    }
    if (tid < 64)
      sb.lse2[tid] = st_f;
    else if (tid < 128)
      sb.delta[tid - 64] = st_f;
  };

  if (n_iter > 0) {
    load_stage(0);
    store_stage(0);
  }
  __syncthreads();

  for (int it = 0; it < n_iter; ++it) {
    const int qt = tr.tile(it % nq);
    const bool more = it + 1 < n_iter;
    if (more) load_stage(it + 1);
    const DkdvStage& sb = stage[it & 1];

    if (active) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int qr0 = qt * kTile + qb * 32;
        if (qr0 >= S) continue;
        const int cls = classify(m, qr0, imin(qr0 + 31, S - 1), kw0, kw1);
        if (cls == kEmpty) continue;

        f32x16 s[2], dp[2];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          s[cb] = f32x16{};
          dp[cb] = f32x16{};
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const u32x4 aq = lds_rm_operand(sb.q_rm, qb, ks, l32, hl);
          const u32x4 ado = lds_rm_operand(sb.do_rm, qb, ks, l32, hl);
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
            s[cb] = mfma32<DT>(aq, kf[cb][ks], s[cb]);
            dp[cb] = mfma32<DT>(ado, vf[cb][ks], dp[cb]);
          }
        }

        // per-row statistics of the 16 rows this lane's registers hold
        float L[16], Dl[16];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 lv = *(const f32x4*)(sb.lse2 + qb * 32 + 8 * r4 + 4 * hl);
          const f32x4 dv4 = *(const f32x4*)(sb.delta + qb * 32 + 8 * r4 + 4 * hl);
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            L[4 * r4 + x] = lv[x];
            Dl[4 * r4 + x] = dv4[x];
          }
        }

        if (cls == kPartial) {
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
            const int j = kw0 + cb * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int i = qr0 + acc_row(r, hl);
              if (!visible(m, i, j)) s[cb][r] = -INFINITY;
            }
          }
        }

        u32x4 pp[2][2], pds[2][2], pp_lo[2][2], pds_lo[2][2];  // [cb][t]
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            float pv[8], dsv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int r = 8 * t + e;
              pv[e] = exp2_fast(__builtin_fmaf(s[cb][r], c2, -L[r]));
              dsv[e] = pv[e] * (dp[cb][r] - Dl[r]);
            }
            pp[cb][t] = u32x4{pack2<DT>(pv[0], pv[1]), pack2<DT>(pv[2], pv[3]), pack2<DT>(pv[4], pv[5]),
                              pack2<DT>(pv[6], pv[7])};
            pds[cb][t] = u32x4{pack2<DT>(dsv[0], dsv[1]), pack2<DT>(dsv[2], dsv[3]),
                               pack2<DT>(dsv[4], dsv[5]), pack2<DT>(dsv[6], dsv[7])};
            if (precise) {
#pragma unroll
              for (int w = 0; w < 4; ++w) {
                pp_lo[cb][t][w] = pack2_residual<DT>(pv[2 * w], pv[2 * w + 1], pp[cb][t][w]);
                pds_lo[cb][t][w] = pack2_residual<DT>(dsv[2 * w], dsv[2 * w + 1], pds[cb][t][w]);
              }
            }
          }

#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const u32x4 ado_t = lds_tr_operand(sb.do_tr, db, qb, t, l32, hl);
            const u32x4 aq_t = lds_tr_operand(sb.q_tr, db, qb, t, l32, hl);
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
              dv[db][cb] = mfma32<DT>(ado_t, pp[cb][t], dv[db][cb]);
              dk[db][cb] = mfma32<DT>(aq_t, pds[cb][t], dk[db][cb]);
            }
            if (precise) {
#pragma unroll
              for (int cb = 0; cb < 2; ++cb) {
                dv[db][cb] = mfma32<DT>(ado_t, pp_lo[cb][t], dv[db][cb]);
                dk[db][cb] = mfma32<DT>(aq_t, pds_lo[cb][t], dk[db][cb]);
              }
            }
          }
      }
    }

    if (more) store_stage((it + 1) & 1);
    __syncthreads();
  }

  if (!active) return;
  float* dkslab = p.dk + (size_t)(b * p.G + g) * S * kHeadDim;
  float* dvslab = p.dv + (size_t)(b * p.G + g) * S * kHeadDim;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int j = kw0 + cb * 32 + l32;
    if (j >= S) continue;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = db * 32 + 8 * r4 + 4 * hl;
        const f32x4 kv = {dk[db][cb][4 * r4] * p.scale, dk[db][cb][4 * r4 + 1] * p.scale,
                          dk[db][cb][4 * r4 + 2] * p.scale, dk[db][cb][4 * r4 + 3] * p.scale};
        const f32x4 vv = {dv[db][cb][4 * r4], dv[db][cb][4 * r4 + 1], dv[db][cb][4 * r4 + 2],
                          dv[db][cb][4 * r4 + 3]};
        *(f32x4*)(dkslab + (size_t)j * kHeadDim + d0) = kv;
        *(f32x4*)(dvslab + (size_t)j * kHeadDim + d0) = vv;
      }
  }
}

// ------------------------------------------------------------------------------------
// dQ
// ------------------------------------------------------------------------------------
struct DqStage {
  char k_rm[8192];
  char k_tr[8192];
  char v_rm[8192];
};

template <int DT>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(16))) DqStage stage[2];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hl = lane >> 5;
  const int S = p.S;
  const MaskSpec m = p.mask;

  const int nhq = p.H / p.hpw;
  const int per_q = p.B * nhq;
  const int qblk = p.n_qblk - 1 - (int)(blockIdx.x / per_q);
  const int rest = (int)(blockIdx.x % per_q);
  const int b = rest / nhq;
  const int h = (rest % nhq) * p.hpw + (wave % p.hpw);
  const int g = h / (p.H / p.G);
  const int Q0 = qblk * kTile * p.qpw;
  const int Q1 = imin(Q0 + kTile * p.qpw, S) - 1;
  const int q0 = Q0 + (wave / p.hpw) * kTile;
  const int q1 = imin(q0 + kTile - 1, S - 1);
  const bool active = q0 < S;

  const size_t qslab_rows = (size_t)(b * p.H + h) * S;
  const uint16_t* qslab = (const uint16_t*)p.q + qslab_rows * kHeadDim;
  const uint16_t* doslab = (const uint16_t*)p.d_o + qslab_rows * kHeadDim;
  const uint16_t* kslab = (const uint16_t*)p.k + (size_t)(b * p.G + g) * S * kHeadDim;
  const uint16_t* vslab = (const uint16_t*)p.v + (size_t)(b * p.G + g) * S * kHeadDim;

  u32x4 qf[2][4], df[2][4];
  float lse2[2], dlt[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int row = q0 + cb * 32 + l32;
    const bool ok = active && row < S;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ok) {
        qf[cb][ks] = *(const u32x4*)(qslab + (size_t)row * kHeadDim + ks * 16 + hl * 8);
        df[cb][ks] = *(const u32x4*)(doslab + (size_t)row * kHeadDim + ks * 16 + hl * 8);
      } else {
        qf[cb][ks] = u32x4{0u, 0u, 0u, 0u};
        df[cb][ks] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    lse2[cb] = ok ? p.lse[qslab_rows + row] * kLog2e : INFINITY;
    dlt[cb] = ok ? p.delta[qslab_rows + row] : 0.f;
  }

  f32x16 dq[2][2];  // dQ^T [d block][column block]
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) dq[db][cb] = f32x16{};

  // staging roles: threads 0..127 stage K (RM and TR), 128..255 stage V (RM)
  const int kind = tid >> 7;
  const int unit = tid & 127;
  const int ur0 = (unit >> 3) * 4;
  const int udc = unit & 7;
  const uint16_t* stage_slab = kind == 0 ? kslab : vslab;
  Unit st;

  const TileRanges tr = key_tiles_for_rows(m, Q0, Q1);
  const int nt = tr.count();
  const float c2 = p.scale_log2;

  auto store_stage = [&](int buf) {
    if (kind == 0) {
      unit_store_rm(stage[buf].k_rm, st, ur0, udc);
      unit_store_tr(stage[buf].k_tr, st, ur0, udc);
    } else {
      unit_store_rm(stage[buf].v_rm, st, ur0, udc);
    }
  };

  if (nt > 0) {
    unit_load(st, stage_slab, tr.tile(0) * kTile + ur0, udc, S);
    store_stage(0);
  }
  __syncthreads();

  for (int it = 0; it < nt; ++it) {
    const int kt = tr.tile(it);
    const int k0 = kt * kTile;
    const bool more = it + 1 < nt;
    if (more) unit_load(st, stage_slab, tr.tile(it + 1) * kTile + ur0, udc, S);
    const DqStage& sb = stage[it & 1];

    if (active) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int kr0 = k0 + kb * 32;
        if (kr0 >= S) continue;
        const int cls = classify(m, q0, q1, kr0, kr0 + 31);
        if (cls == kEmpty) continue;

        f32x16 s[2], dp[2];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          s[cb] = f32x16{};
          dp[cb] = f32x16{};
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const u32x4 ak = lds_rm_operand(sb.k_rm, kb, ks, l32, hl);
          const u32x4 av = lds_rm_operand(sb.v_rm, kb, ks, l32, hl);
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
            s[cb] = mfma32<DT>(ak, qf[cb][ks], s[cb]);
            dp[cb] = mfma32<DT>(av, df[cb][ks], dp[cb]);
          }
        }

        if (cls == kPartial) {
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
            const int i = q0 + cb * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int j = kr0 + acc_row(r, hl);
              if (!visible(m, i, j)) s[cb][r] = -INFINITY;
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
              dsv[e] = pv * (dp[cb][r] - dlt[cb]);
            }
            pds[cb][t] = u32x4{pack2<DT>(dsv[0], dsv[1]), pack2<DT>(dsv[2], dsv[3]),
                               pack2<DT>(dsv[4], dsv[5]), pack2<DT>(dsv[6], dsv[7])};
          }

#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const u32x4 akt = lds_tr_operand(sb.k_tr, db, kb, t, l32, hl);
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) dq[db][cb] = mfma32<DT>(akt, pds[cb][t], dq[db][cb]);
          }
      }
    }

    if (more) store_stage((it + 1) & 1);
    __syncthreads();
  }

  if (!active) return;
  float* dqslab = p.dq + qslab_rows * kHeadDim;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int i = q0 + cb * 32 + l32;
    if (i >= S) continue;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = db * 32 + 8 * r4 + 4 * hl;
        const f32x4 w = {dq[db][cb][4 * r4] * p.scale, dq[db][cb][4 * r4 + 1] * p.scale,
                         dq[db][cb][4 * r4 + 2] * p.scale, dq[db][cb][4 * r4 + 3] * p.scale};
        *(f32x4*)(dqslab + (size_t)i * kHeadDim + d0) = w;
      }
  }
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

hipError_t launch_bwd_dkdv_mfma(const BwdParams& p, int dtype, hipStream_t s) {
  dim3 grid((unsigned)((long long)p.n_kblk * p.B * p.G)), block(256);
  void* args[] = {(void*)&p};
  if (dtype == kDtBF16) return hipLaunchKernel((const void*)bwd_dkdv_kernel<kDtBF16>, grid, block, args, 0, s);
  return hipLaunchKernel((const void*)bwd_dkdv_kernel<kDtF16>, grid, block, args, 0, s);
}

hipError_t launch_bwd_dq_mfma(const BwdParams& p, int dtype, hipStream_t s) {
  dim3 grid((unsigned)((long long)p.n_qblk * p.B * (p.H / p.hpw))), block(256);
  void* args[] = {(void*)&p};
  if (dtype == kDtBF16) return hipLaunchKernel((const void*)bwd_dq_kernel<kDtBF16>, grid, block, args, 0, s);
  return hipLaunchKernel((const void*)bwd_dq_kernel<kDtF16>, grid, block, args, 0, s);
}

}  // namespace gqa
