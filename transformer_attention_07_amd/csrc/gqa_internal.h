// Internal declarations shared by the libgqa kernels and the C-ABI layer.
//
// Visibility rule (see include/gqa.h): key j is visible to query i iff
//   j <= i  and  (window == 0  or  j > i - window  or  j < num_sinks)      (causal)
//   always                                                               (non-causal)
// restricted to 0 <= j < S.  The kernels work on square tiles of 64 keys; for a block
// of query rows [q0, q1] the helpers below give the key tiles that contain at least one
// visible key (all others are never loaded) and classify each tile as FULL (no mask
// arithmetic needed) or PARTIAL (mask element by element).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gqa.h"

namespace gqa {

constexpr int kTile = 64;   // keys per key tile and query rows per wave tile
constexpr int kDkdvKeys = 128;  // keys per dK/dV workgroup (4 waves x 32 keys)
constexpr int kHeadDim = 64;

enum TileClass : int { kEmpty = 0, kPartial = 1, kFull = 2 };

struct MaskSpec {
  int S;
  int causal;
  int window;
  int sinks;
};

__host__ __device__ inline int imin(int a, int b) { return a < b ? a : b; }
__host__ __device__ inline int imax(int a, int b) { return a > b ? a : b; }

// Is key j visible to query i (both inside [0, S))?
__host__ __device__ inline bool visible(const MaskSpec& m, int i, int j) {
  if (j >= m.S) return false;
  if (!m.causal) return true;
  if (j > i) return false;
  if (m.window > 0 && j <= i - m.window && j >= m.sinks) return false;
  return true;
}

// Class of the block rows [q0, q1] x keys [k0, k1] (inclusive bounds, q1 < S assumed).
// FULL is only returned when every pair is visible; PARTIAL is always a safe answer.
__host__ __device__ inline int classify(const MaskSpec& m, int q0, int q1, int k0, int k1) {
  if (k0 >= m.S) return kEmpty;
  if (!m.causal) return (k1 < m.S) ? kFull : kPartial;
  if (k0 > q1) return kEmpty;
  if (m.window > 0) {
    // union over the rows of the in-window keys is (q0 - W, q1]; sinks are [0, NS)
    bool hits_window = k1 > q0 - m.window;
    bool hits_sinks = k0 < m.sinks;
    if (!hits_window && !hits_sinks) return kEmpty;
  }
  bool full = (k1 <= q0) && (k1 < m.S);
  if (full && m.window > 0) full = (k0 > q1 - m.window) || (k1 < m.sinks);
  return full ? kFull : kPartial;
}

// Key tiles a block of query rows [q0, q1] must visit, as at most two disjoint tile
// ranges [a0, a1) and [b0, b1) (sink tiles, then window/causal tiles).
struct TileRanges {
  int a0, a1, b0, b1;
  __host__ __device__ int count() const { return (a1 - a0) + (b1 - b0); }
  __host__ __device__ int tile(int n) const { return n < (a1 - a0) ? a0 + n : b0 + (n - (a1 - a0)); }
};

__host__ __device__ inline TileRanges key_tiles_for_rows(const MaskSpec& m, int q0, int q1) {
  TileRanges r{0, 0, 0, 0};
  const int nt = (m.S + kTile - 1) / kTile;
  if (!m.causal) {
    r.b0 = 0;
    r.b1 = nt;
    return r;
  }
  const int last = q1 / kTile + 1;  // exclusive
  if (m.window <= 0 || q0 - m.window + 1 <= 0) {
    r.b0 = 0;
    r.b1 = last;
    return r;
  }
  const int wfirst = (q0 - m.window + 1) / kTile;
  const int sink_end = (imin(m.sinks, q1 + 1) + kTile - 1) / kTile;  // exclusive
  if (sink_end >= wfirst) {
    r.b0 = 0;
    r.b1 = last;
  } else {
    r.a0 = 0;
    r.a1 = sink_end;
    r.b0 = wfirst;
    r.b1 = last;
  }
  return r;
}

// Query tiles that see at least one key of the key rows [k0, k1]: as two disjoint tile
// ranges of query tiles (used by the dK/dV pass, which walks queries for fixed keys).
__host__ __device__ inline TileRanges query_tiles_for_keys(const MaskSpec& m, int k0, int k1) {
  TileRanges r{0, 0, 0, 0};
  const int nt = (m.S + kTile - 1) / kTile;
  if (!m.causal) {
    r.b0 = 0;
    r.b1 = nt;
    return r;
  }
  const int first = k0 / kTile;  // queries i >= k0
  if (m.window <= 0 || k0 < m.sinks) {
    // sinks are seen by every later query; without a window every later query sees them
    r.b0 = first;
    r.b1 = nt;
    return r;
  }
  // non-sink keys [k0, k1] are seen by queries i with j <= i < j + W, i.e. [k0, k1 + W - 1]
  const int last_row = imin(m.S - 1, k1 + m.window - 1);
  r.b0 = first;
  r.b1 = last_row / kTile + 1;
  return r;
}

// ---------------------------------------------------------------------------------
// Kernel parameter blocks (passed by value).
// ---------------------------------------------------------------------------------

// Rotary position embedding with YaRN frequencies, as the kernels take it: the per-pair
// frequencies are worked out on the host from the configuration (like the softmax scale);
// the angles of each position and the rotations run on the device.
constexpr int kRopePairs = kHeadDim / 2;
struct RopeSpec {
  double rev[kRopePairs];  // pair i turns rev[i] revolutions per position (theta'_i / 2 pi)
  float mscale;            // factor on each rotated vector (YaRN's attention temperature)
  int enabled;             // forward: rotate Q in registers before the scores
};

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  void* o_lo;        // optional: O minus its rounded value, in the element type
  float* lse;
  int B, H, G, S;
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e)
  MaskSpec mask;
  int hpw;           // heads per workgroup (a divisor of H/G): waves 0..hpw-1 share rows
  int qpw;           // 64-row query tiles per workgroup (4 / hpw)
  int n_qblk;        // workgroup row blocks per head = ceil(S / (64 * qpw))
  int xcd_hg;        // > 0: head groups per XCD (workgroup order that keeps kv heads on one
                     // XCD, see fwd_block_order); 0: plain q-block-major order
  int xcd_kv;        // with xcd_hg: > 0 = head groups per kv head, an XCD finishing one kv
                     // head before the next; 0 = its kv heads' row blocks interleaved
  void* q_rot;       // with rope.enabled: optional output of the rotated Q (element type)
  RopeSpec rope;     // query i sits at position i
};

// y = mscale R(pos0 + s) x (R^T with inverse) for the rows s of x, y [n_slabs][S][64].
struct RopeParams {
  const void* x;
  void* y;           // == x (in place) or disjoint
  long long n_slabs;
  int S;
  int pos0;          // pos0 + S - 1 fits in int
  int slabs_per_block;
  int n_row_blocks;  // ceil(S / rows per block)
  int inverse;
  RopeSpec spec;
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* o_lo;  // optional rounding residual of O (preprocess only)
  const void* d_o;
  const float* lse;
  const float* delta;
  float* out_delta;
  float* dq;
  float* dk;
  float* dv;
  int B, H, G, S;
  float scale;
  float scale_log2;
  MaskSpec mask;
  int hpw, qpw, n_qblk;  // dQ pass: same row decomposition as the forward
  int n_kblk;            // dK/dV pass: kDkdvKeys-key blocks per kv head
  int precise_all;       // dK/dV pass: every block takes P and dS as rounded value plus
                         // rounded residual (short sequences and short windows, where P is large)
};

// The only argument of the dK/dV, dQ and one-launch backward kernels: the parameters and
// the rotation table (with rope.enabled they rotate dQ and dK back, m R^T at their
// positions, as they store them).  One block, so no argument offset is computed by hand.
struct BwdArgs {
  BwdParams p;
  RopeSpec rope;
};

// Launchers (return hipSuccess or the launch error).  Element type by dtype code.
// Decode (few query rows against a key/value cache), split over the visible key tiles.
// Rows of a (batch, kv head) pair: r = hh * Sq + t for query head g * hpg + hh and query
// row t (position Skv - Sq + t), in chunks of kDecodeRows; every wave of the split kernel
// is one partial over its own key tiles and writes its unnormalised O, running maximum
// (log2 units of the scaled score) and row sum, which the merge kernel combines.
constexpr int kDecodeRows = 128;  // rows per chunk (four 32-row MFMA column blocks)
constexpr int kDecodeWaves = 4;   // waves (= partials) per workgroup

struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* part_o;     // [n_sets][n_part][kDecodeRows][64]
  float* part_ml;    // [n_sets][n_part][2][kDecodeRows]: maximum, row sum
  int B, H, G, Sq, Skv;
  int hpg;           // H / G
  int rows;          // hpg * Sq
  int nrc;           // row chunks per (b, g) = ceil(rows / kDecodeRows)
  int nsplit;        // workgroups per (b, g, chunk)
  int shared_tiles;  // 0: each of a workgroup's 4 waves is a partial (chunks of <= 32 rows);
                     // 1: one wave per 32-row block sharing the tiles, the workgroup a partial
  int n_part;        // partials per set: 4 * nsplit, or nsplit when shared_tiles
  float scale_log2;  // scale * log2(e)
  MaskSpec mask;     // S = Skv, causal
  TileRanges tiles;  // key tiles visible to at least one row (sinks, then window)
};

hipError_t launch_decode(const DecodeParams& p, int dtype, hipStream_t s);

// FP8 forward: Q, K (e4m3, [B][H|G][S][64]) and V^T permuted by vt_permute ([B][G][64][s_pad]).
struct Fp8FwdParams {
  const void* q;
  const void* k;
  const void* vt;
  void* o;           // bf16 [B][H][S][64]
  float* lse;
  int B, H, G, S;
  int s_pad;         // S rounded up to a multiple of 64
  float scale_log2;  // softmax scale * q and k dequantisation factors * log2(e)
  float o_scale;     // V's dequantisation factor
  MaskSpec mask;
  int hpw, qpw, n_qblk;
  int xcd_hg, xcd_kv;  // workgroup order, as FwdParams
};

struct VtParams {
  const void* v;     // e4m3 [n_slabs][S][64]
  void* vt;          // e4m3 [n_slabs][64][s_pad]
  long long n_slabs;
  int S;
  int s_pad;
};

hipError_t launch_clock_probe(unsigned long long* out, int blocks, int iters, hipStream_t s);
hipError_t launch_vt_permute(const VtParams& p, hipStream_t s);
hipError_t launch_fwd_fp8(const Fp8FwdParams& p, hipStream_t s);

hipError_t launch_rope(const RopeParams& p, int dtype, hipStream_t s);
int rope_rows_per_block(int dtype);

hipError_t launch_fwd_mfma(const FwdParams& p, int dtype, hipStream_t s);

// Host side: gqa_attn_bwd's argument checks (GQA_OK for a valid or empty problem); with
// own_workspace the workspace is the library's and is not checked.
int bwd_check_args(const gqa_problem* p, const void* q, const void* k, const void* v, const void* o,
                   const void* o_lo, const float* lse, const void* d_o, const float* dq, const float* dk,
                   const float* dv, bool own_workspace, const void* workspace, size_t workspace_bytes);
hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t s);
hipError_t launch_bwd_preprocess(const BwdParams& p, int dtype, hipStream_t s);
hipError_t launch_bwd_dkdv_mfma(const BwdParams& p, const RopeSpec& rope, int dtype, hipStream_t s);
hipError_t launch_bwd_dq_mfma(const BwdParams& p, const RopeSpec& rope, int dtype, hipStream_t s);
hipError_t launch_bwd_fused_mfma(const BwdParams& p, const RopeSpec& rope, int dtype, hipStream_t s);
hipError_t launch_bwd_dkdv_f32(const BwdParams& p, hipStream_t s);
hipError_t launch_bwd_dq_f32(const BwdParams& p, hipStream_t s);

}  // namespace gqa
