// The backward for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation): gqa_attn_bwd with its
// workspace, the fp32 delta vector [B][H][S], in a fixed array of device memory that the
// library owns.  Nothing here allocates; the kernels are gqa_attn_bwd's.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gqa.h"
#include "gqa_internal.h"

namespace {

constexpr size_t kScratchFloats = GQA_NOALLOC_MAX_ROWS;
constexpr size_t kScratchBytes = kScratchFloats * sizeof(float);  // 32 MiB

// The delta vector of gqa_attn_bwd_noalloc.  Each device holds its own copy, at its own
// address, from the library's load until the process ends.  In host code this name is a
// host-side stand-in, not a device address: host code uses the per-device address that
// device_scratch() looks up.
static __device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`, looked up on the first call
// on that device (with it current) and kept.
int device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GQA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return GQA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return GQA_OK;
}

}  // namespace

extern "C" int gqa_attn_bwd_noalloc(const gqa_problem* p, const void* q, const void* k, const void* v,
                                    const void* o, const void* o_lo, const float* lse, const void* d_o,
                                    float* dq, float* dk, float* dv, void* stream) {
  int rc = gqa::bwd_check_args(p, q, k, v, o, o_lo, lse, d_o, dq, dk, dv, true, nullptr, 0);
  if (rc != GQA_OK) return rc;
  const size_t need = gqa_attn_bwd_workspace_bytes(p);
  if (need == 0) return GQA_OK;  // empty problem
  if (need > kScratchBytes) return GQA_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((rc = device_scratch(&ws)) != GQA_OK) return rc;
  // delta is written in full by the preprocess pass before the gradient kernels read it, so
  // nothing in the array needs clearing
  return gqa_attn_bwd(p, q, k, v, o, o_lo, lse, d_o, dq, dk, dv, ws, kScratchBytes, stream);
}
