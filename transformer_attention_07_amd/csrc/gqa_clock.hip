// Shader clock under matrix-core load, for reporting throughput against the peak at the
// clock the device actually runs (the published peaks assume 2.4 GHz).
//
// One 4-wave workgroup per compute unit keeps its four SIMDs busy with independent chains
// of v_mfma_f32_32x32x16_bf16 on non-trivial data.  Wave 0 of each workgroup reads the
// shader clock counter (s_memtime) and the constant 100 MHz counter (s_memrealtime) around
// the chains; their ratio is the clock.
#include "gqa_device.h"

namespace gqa {

namespace {

__global__ __launch_bounds__(256) void clock_probe_kernel(unsigned long long* out, int iters) {
  const int lane = threadIdx.x & 63;
  const uint32_t pa = 0x3F80BF80u ^ (uint32_t)(lane * 0x00010001u);  // +-1-ish bf16 pairs, varying by lane
  const uint32_t pb = 0xBF003F00u ^ (uint32_t)(lane * 0x00020002u);
  const u32x4 a = {pa, pb, pa ^ 0x80008000u, pb}, b = {pb, pa, pb ^ 0x80008000u, pa};
  f32x16 acc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = mfma32<kDtBF16>(a, b, acc[c]);
  }
  asm volatile("s_nop 0" ::"v"(acc[0][0]), "v"(acc[1][0]), "v"(acc[2][0]), "v"(acc[3][0]));
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    out[2 * blockIdx.x] = t1 - t0;
    out[2 * blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace

hipError_t launch_clock_probe(unsigned long long* out, int blocks, int iters, hipStream_t s) {
  void* args[] = {(void*)&out, (void*)&iters};
  return hipLaunchKernel((const void*)clock_probe_kernel, dim3((unsigned)blocks), dim3(256), args, 0, s);
}

}  // namespace gqa
