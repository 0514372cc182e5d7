// Rotary position embedding with YaRN frequencies over [n_slabs][S][64] rows (bf16, f16
// or fp32): y = m R(pos0 + s) x, or m R^T for the backward.  The rotation is the RoFormer
// rotary embedding with the YaRN paper's "NTK-by-parts" frequencies and temperature, the
// YaRN RoPE with a 32x factor of the "SnapKitty Transformer 8B" model card (Model
// Specifications; Training Configuration rope_yarn, rope_yarn_factor; Protected
// Inventions: YaRN-scaled RoPE inside the attention kernels).
//
// HBM-bound streaming: a thread owns one 16-byte chunk (4 or 2 dimension pairs) of one
// position and walks a run of slabs (heads) at that position, so the angles' sine and
// cosine, the only non-trivial arithmetic, are computed once per position and chunk and
// reused for every slab of the run.  Consecutive threads cover consecutive chunks of
// consecutive rows: each load and store instruction of a wave moves 1 KiB of contiguous
// memory.  Four slabs' loads are in flight per thread.
#include "gqa_device.h"

namespace gqa {

namespace {

template <int DT>
struct RopeLayout {
  static constexpr int kEl = DT == kDtF32 ? 4 : 8;     // elements per 16-byte chunk
  static constexpr int kPairs = kEl / 2;
  static constexpr int kLanesPerRow = kHeadDim / kEl;  // 16 or 8
  static constexpr int kRows = 256 / kLanesPerRow;     // rows per block: 16 or 32
  static constexpr int kRowBytes = kHeadDim * (DT == kDtF32 ? 4 : 2);
};

template <int DT>
__device__ __forceinline__ u32x4 rotate_chunk(u32x4 w, int pos, const float (&mc)[4], const float (&ms)[4]) {
  if constexpr (DT == kDtF32) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      // elements go through scalars: clang's __builtin_bit_cast of a vector element
      // lvalue reads element 0
      const uint32_t a0 = w[2 * j], a1 = w[2 * j + 1];
      float x0 = __builtin_bit_cast(float, a0), x1 = __builtin_bit_cast(float, a1);
      rope_pair(x0, x1, mc[j], ms[j]);
      w[2 * j] = __builtin_bit_cast(uint32_t, x0);
      w[2 * j + 1] = __builtin_bit_cast(uint32_t, x1);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float x0 = elem_to_f32<DT>(w[j], 0), x1 = elem_to_f32<DT>(w[j], 1);
      rope_pair(x0, x1, mc[j], ms[j]);
      w[j] = pack2<DT>(x0, x1);
    }
  }
  return w;
}

template <int DT>
__global__ __launch_bounds__(256) void rope_kernel(RopeParams p) {
  using L = RopeLayout<DT>;
  const int t = threadIdx.x;
  const int rb = (int)(blockIdx.x % (unsigned)p.n_row_blocks);
  const long long chunk = blockIdx.x / (unsigned)p.n_row_blocks;
  const int row = rb * L::kRows + t / L::kLanesPerRow;
  if (row >= p.S) return;
  const int cpos = t % L::kLanesPerRow;  // chunk of the row
  const int pos = p.pos0 + row;
  float mc[4], ms[4];
#pragma unroll
  for (int j = 0; j < L::kPairs; ++j)
    rope_cs(pos, p.spec.rev[cpos * L::kPairs + j], p.spec.mscale, p.inverse != 0, mc[j], ms[j]);

  const long long n0 = chunk * p.slabs_per_block;
  const long long n1 = n0 + p.slabs_per_block < p.n_slabs ? n0 + p.slabs_per_block : p.n_slabs;
  const size_t stride = (size_t)p.S * L::kRowBytes;
  const size_t off0 = (size_t)n0 * stride + (size_t)row * L::kRowBytes + (size_t)cpos * 16;
  const char* xp = (const char*)p.x + off0;
  char* yp = (char*)p.y + off0;
  long long n = n0;
  for (; n + 4 <= n1; n += 4) {
    u32x4 w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) w[u] = *(const u32x4*)(xp + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) *(u32x4*)(yp + u * stride) = rotate_chunk<DT>(w[u], pos, mc, ms);
    xp += 4 * stride;
    yp += 4 * stride;
  }
  for (; n < n1; ++n) {
    *(u32x4*)yp = rotate_chunk<DT>(*(const u32x4*)xp, pos, mc, ms);
    xp += stride;
    yp += stride;
  }
}

}  // namespace

int rope_rows_per_block(int dtype) {
  return dtype == kDtF32 ? RopeLayout<kDtF32>::kRows : RopeLayout<kDtBF16>::kRows;
}

hipError_t launch_rope(const RopeParams& p, int dtype, hipStream_t s) {
  const long long chunks = (p.n_slabs + p.slabs_per_block - 1) / p.slabs_per_block;
  dim3 grid((unsigned)(chunks * p.n_row_blocks)), block(256);
  void* args[] = {(void*)&p};
  if (dtype == kDtBF16) return hipLaunchKernel((const void*)rope_kernel<kDtBF16>, grid, block, args, 0, s);
  if (dtype == kDtF16) return hipLaunchKernel((const void*)rope_kernel<kDtF16>, grid, block, args, 0, s);
  return hipLaunchKernel((const void*)rope_kernel<kDtF32>, grid, block, args, 0, s);
}

}  // namespace gqa
