// fp32 kernels of causal grouped-query attention (forward, dK/dV, dQ).
//
// These serve fp32 inputs, where the result must stay within 1e-4 of the exact value;
// they use plain fp32 vector arithmetic (one query or key row per lane, K/V or Q/dO
// rows staged through LDS 64 at a time, the same key-tile ranges as the bf16 kernels)
// and the precise device expf/logf.  Throughput is not their purpose: fp32 attention
// is far below the matrix-core rate either way, and the bf16/f16 kernels are the fast path.
#include "gqa_device.h"

namespace gqa {

namespace {

constexpr int kPad = kHeadDim + 1;  // LDS row pitch in floats (avoids bank conflicts)

// One wave per (b, h, 64-row tile); lane = query row.
template <bool ROPE>
__global__ __launch_bounds__(64) void fwd_f32_kernel(FwdParams p) {
  __shared__ float ks[kTile][kPad];
  __shared__ float vs[kTile][kPad];
  const int S = p.S;
  const int nqt = (S + kTile - 1) / kTile;
  const int qt = nqt - 1 - (int)(blockIdx.x % nqt);
  const int bh = (int)(blockIdx.x / nqt);
  const int b = bh / p.H, h = bh % p.H, g = h / (p.H / p.G);
  const int lane = threadIdx.x;
  const int i = qt * kTile + lane;
  const bool row_ok = i < S;
  const MaskSpec m = p.mask;

  const float* qrow = (const float*)p.q + ((size_t)bh * S + (row_ok ? i : 0)) * kHeadDim;
  const float* kslab = (const float*)p.k + (size_t)(b * p.G + g) * S * kHeadDim;
  const float* vslab = (const float*)p.v + (size_t)(b * p.G + g) * S * kHeadDim;
  float q[kHeadDim], acc[kHeadDim];
#pragma unroll
  for (int c = 0; c < kHeadDim; ++c) {
    q[c] = row_ok ? qrow[c] : 0.f;
    acc[c] = 0.f;
  }
  if constexpr (ROPE) {  // rotary embedding of the lane's query row, at position i
#pragma unroll
    for (int j = 0; j < kRopePairs; ++j) {
      float mc, ms;
      rope_cs(i, p.rope.rev[j], p.rope.mscale, false, mc, ms);
      rope_pair(q[2 * j], q[2 * j + 1], mc, ms);
    }
    if (p.q_rot != nullptr && row_ok) {
      float* rrow = (float*)p.q_rot + ((size_t)bh * S + i) * kHeadDim;
#pragma unroll
      for (int c = 0; c < kHeadDim; ++c) rrow[c] = q[c];
    }
  }
#pragma unroll
  for (int c = 0; c < kHeadDim; ++c) q[c] *= p.scale;
  float mx = -INFINITY, l = 0.f;

  const TileRanges tr = key_tiles_for_rows(m, qt * kTile, imin(qt * kTile + kTile - 1, S - 1));
  for (int it = 0; it < tr.count(); ++it) {
    const int k0 = tr.tile(it) * kTile;
    __syncthreads();
    const int j_ld = k0 + lane;
#pragma unroll 8
    for (int c = 0; c < kHeadDim; ++c) {
      ks[lane][c] = j_ld < S ? kslab[(size_t)j_ld * kHeadDim + c] : 0.f;
      vs[lane][c] = j_ld < S ? vslab[(size_t)j_ld * kHeadDim + c] : 0.f;
    }
    __syncthreads();
    if (!row_ok) continue;
    for (int jj = 0; jj < kTile; ++jj) {
      if (!visible(m, i, k0 + jj)) continue;
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < kHeadDim; ++c) s = __builtin_fmaf(q[c], ks[jj][c], s);
      const float mnew = fmaxf(mx, s);
      const float corr = expf(mx - mnew);  // mx = -inf on the first key: 0
      const float pj = expf(s - mnew);
      l = l * corr + pj;
#pragma unroll
      for (int c = 0; c < kHeadDim; ++c) acc[c] = acc[c] * corr + pj * vs[jj][c];
      mx = mnew;
    }
  }
  if (!row_ok) return;
  float* orow = (float*)p.o + ((size_t)bh * S + i) * kHeadDim;
  const float inv = 1.0f / l;
#pragma unroll
  for (int c = 0; c < kHeadDim; ++c) orow[c] = acc[c] * inv;
  p.lse[(size_t)bh * S + i] = mx + logf(l);
}

// One wave per (b, g, 64-key tile); lane = key row.  Loops over the heads of the group
// and the query tiles that see the key tile.
__global__ __launch_bounds__(64) void dkdv_f32_kernel(BwdParams p) {
  __shared__ float qs[kTile][kPad];
  __shared__ float ds_[kTile][kPad];
  __shared__ float own_k[kTile][kPad];
  __shared__ float own_v[kTile][kPad];
  __shared__ float lse_s[kTile];
  __shared__ float dl_s[kTile];
  const int S = p.S;
  const int nkt = (S + kTile - 1) / kTile;
  const int kt = (int)(blockIdx.x % nkt);
  const int bg = (int)(blockIdx.x / nkt);
  const int b = bg / p.G, g = bg % p.G;
  const int hpg = p.H / p.G;
  const int lane = threadIdx.x;
  const int j = kt * kTile + lane;
  const bool key_ok = j < S;
  const MaskSpec m = p.mask;

  const float* kslab = (const float*)p.k + (size_t)bg * S * kHeadDim;
  const float* vslab = (const float*)p.v + (size_t)bg * S * kHeadDim;
  for (int c = 0; c < kHeadDim; ++c) {
    own_k[lane][c] = key_ok ? kslab[(size_t)j * kHeadDim + c] : 0.f;
    own_v[lane][c] = key_ok ? vslab[(size_t)j * kHeadDim + c] : 0.f;
  }
  float dk[kHeadDim], dv[kHeadDim];
#pragma unroll
  for (int c = 0; c < kHeadDim; ++c) dk[c] = dv[c] = 0.f;

  const TileRanges tr = query_tiles_for_keys(m, kt * kTile, imin(kt * kTile + kTile - 1, S - 1));
  for (int hh = 0; hh < hpg; ++hh) {
    const int h = g * hpg + hh;
    const size_t slab = (size_t)(b * p.H + h) * S;
    const float* qslab = (const float*)p.q + slab * kHeadDim;
    const float* doslab = (const float*)p.d_o + slab * kHeadDim;
    for (int it = 0; it < tr.count(); ++it) {
      const int q0 = tr.tile(it) * kTile;
      __syncthreads();
      const int i_ld = q0 + lane;
      for (int c = 0; c < kHeadDim; ++c) {
        qs[lane][c] = i_ld < S ? qslab[(size_t)i_ld * kHeadDim + c] : 0.f;
        ds_[lane][c] = i_ld < S ? doslab[(size_t)i_ld * kHeadDim + c] : 0.f;
      }
      lse_s[lane] = i_ld < S ? p.lse[slab + i_ld] : 0.f;
      dl_s[lane] = i_ld < S ? p.delta[slab + i_ld] : 0.f;
      __syncthreads();
      if (!key_ok) continue;
      for (int ii = 0; ii < kTile; ++ii) {
        const int i = q0 + ii;
        if (i >= S || !visible(m, i, j)) continue;
        float s = 0.f, dpv = 0.f;
#pragma unroll
        for (int c = 0; c < kHeadDim; ++c) {
          s = __builtin_fmaf(qs[ii][c], own_k[lane][c], s);
          dpv = __builtin_fmaf(ds_[ii][c], own_v[lane][c], dpv);
        }
        const float pij = expf(s * p.scale - lse_s[ii]);
        const float dsij = pij * (dpv - dl_s[ii]);
#pragma unroll
        for (int c = 0; c < kHeadDim; ++c) {
          dv[c] = __builtin_fmaf(pij, ds_[ii][c], dv[c]);
          dk[c] = __builtin_fmaf(dsij, qs[ii][c], dk[c]);
        }
      }
    }
  }
  if (!key_ok) return;
  float* dkrow = p.dk + ((size_t)bg * S + j) * kHeadDim;
  float* dvrow = p.dv + ((size_t)bg * S + j) * kHeadDim;
#pragma unroll
  for (int c = 0; c < kHeadDim; ++c) {
    dkrow[c] = dk[c] * p.scale;
    dvrow[c] = dv[c];
  }
}

// One wave per (b, h, 64-row tile); lane = query row.
__global__ __launch_bounds__(64) void dq_f32_kernel(BwdParams p) {
  __shared__ float ks[kTile][kPad];
  __shared__ float vs[kTile][kPad];
  __shared__ float own_q[kTile][kPad];
  __shared__ float own_do[kTile][kPad];
  const int S = p.S;
  const int nqt = (S + kTile - 1) / kTile;
  const int qt = nqt - 1 - (int)(blockIdx.x % nqt);
  const int bh = (int)(blockIdx.x / nqt);
  const int b = bh / p.H, h = bh % p.H, g = h / (p.H / p.G);
  const int lane = threadIdx.x;
  const int i = qt * kTile + lane;
  const bool row_ok = i < S;
  const MaskSpec m = p.mask;

  const float* qrow = (const float*)p.q + ((size_t)bh * S + (row_ok ? i : 0)) * kHeadDim;
  const float* dorow = (const float*)p.d_o + ((size_t)bh * S + (row_ok ? i : 0)) * kHeadDim;
  for (int c = 0; c < kHeadDim; ++c) {
    own_q[lane][c] = row_ok ? qrow[c] : 0.f;
    own_do[lane][c] = row_ok ? dorow[c] : 0.f;
  }
  const float lse = row_ok ? p.lse[(size_t)bh * S + i] : 0.f;
  const float dl = row_ok ? p.delta[(size_t)bh * S + i] : 0.f;
  const float* kslab = (const float*)p.k + (size_t)(b * p.G + g) * S * kHeadDim;
  const float* vslab = (const float*)p.v + (size_t)(b * p.G + g) * S * kHeadDim;
  float dq[kHeadDim];
#pragma unroll
  for (int c = 0; c < kHeadDim; ++c) dq[c] = 0.f;

  const TileRanges tr = key_tiles_for_rows(m, qt * kTile, imin(qt * kTile + kTile - 1, S - 1));
  for (int it = 0; it < tr.count(); ++it) {
    const int k0 = tr.tile(it) * kTile;
    __syncthreads();
    const int j_ld = k0 + lane;
    for (int c = 0; c < kHeadDim; ++c) {
      ks[lane][c] = j_ld < S ? kslab[(size_t)j_ld * kHeadDim + c] : 0.f;
      vs[lane][c] = j_ld < S ? vslab[(size_t)j_ld * kHeadDim + c] : 0.f;
    }
    __syncthreads();
    if (!row_ok) continue;
    for (int jj = 0; jj < kTile; ++jj) {
      if (!visible(m, i, k0 + jj)) continue;
      float s = 0.f, dpv = 0.f;
#pragma unroll
      for (int c = 0; c < kHeadDim; ++c) {
        s = __builtin_fmaf(own_q[lane][c], ks[jj][c], s);
        dpv = __builtin_fmaf(own_do[lane][c], vs[jj][c], dpv);
      }
      const float pij = expf(s * p.scale - lse);
      const float dsij = pij * (dpv - dl);
#pragma unroll
      for (int c = 0; c < kHeadDim; ++c) dq[c] = __builtin_fmaf(dsij, ks[jj][c], dq[c]);
    }
  }
  if (!row_ok) return;
  float* dqrow = p.dq + ((size_t)bh * S + i) * kHeadDim;
#pragma unroll
  for (int c = 0; c < kHeadDim; ++c) dqrow[c] = dq[c] * p.scale;
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t s) {
  const long long n = (long long)p.B * p.H * ((p.S + kTile - 1) / kTile);
  void* args[] = {(void*)&p};
  const void* fn = p.rope.enabled ? (const void*)fwd_f32_kernel<true> : (const void*)fwd_f32_kernel<false>;
  return hipLaunchKernel(fn, dim3((unsigned)n), dim3(64), args, 0, s);
}

hipError_t launch_bwd_dkdv_f32(const BwdParams& p, hipStream_t s) {
  const long long n = (long long)p.B * p.G * ((p.S + kTile - 1) / kTile);
  void* args[] = {(void*)&p};
  return hipLaunchKernel((const void*)dkdv_f32_kernel, dim3((unsigned)n), dim3(64), args, 0, s);
}

hipError_t launch_bwd_dq_f32(const BwdParams& p, hipStream_t s) {
  const long long n = (long long)p.B * p.H * ((p.S + kTile - 1) / kTile);
  void* args[] = {(void*)&p};
  return hipLaunchKernel((const void*)dq_f32_kernel, dim3((unsigned)n), dim3(64), args, 0, s);
}

}  // namespace gqa
