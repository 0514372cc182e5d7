// C-ABI of libgqa: argument validation, problem normalisation and kernel dispatch.
// Everything is checked on the host before the first HIP call; see include/gqa.h.
#include "gqa.h"

#include <math.h>

#include <atomic>
#include <climits>
#include <initializer_list>

#include "gqa_internal.h"

namespace {

using gqa::BwdParams;
using gqa::FwdParams;
using gqa::MaskSpec;

constexpr float kLog2e = 1.44269504088896340736f;
// The dK/dV pass takes P and dS with their rounding residuals in every block for sequences
// up to this length or windows up to this width (see BwdParams::precise_all).
constexpr int kPreciseMaxSeq = 256;
constexpr int kPreciseMaxWindow = 64;

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// Shape and flag checks shared by every entry point.
int check_problem(const gqa_problem* p) {
  if (p == nullptr) return GQA_ERR_INVALID_ARG;
  if (p->B < 0 || p->S < 0 || p->H < 1 || p->G < 1 || p->D < 1) return GQA_ERR_INVALID_ARG;
  if (p->H % p->G != 0) return GQA_ERR_INVALID_ARG;
  if (!(isfinite(p->scale) && p->scale > 0.f)) return GQA_ERR_INVALID_ARG;
  if (p->causal != 0 && p->causal != 1) return GQA_ERR_INVALID_ARG;
  if (p->window < 0 || p->num_sinks < 0) return GQA_ERR_INVALID_ARG;
  if (p->causal == 0 && (p->window != 0 || p->num_sinks != 0)) return GQA_ERR_INVALID_ARG;
  if (p->dtype != GQA_F32 && p->dtype != GQA_BF16 && p->dtype != GQA_F16) return GQA_ERR_INVALID_ARG;
  if ((long long)p->B * p->H > INT_MAX / 2) return GQA_ERR_UNSUPPORTED;
  if (p->D != gqa::kHeadDim || p->S > GQA_MAX_SEQ) return GQA_ERR_UNSUPPORTED;
  return GQA_OK;
}

bool empty_problem(const gqa_problem* p) { return p->B == 0 || p->S == 0; }

// The window and sink rule with the no-op cases folded away: a window of S or more
// keys hides nothing, sinks only matter under a window, and more sinks than keys make
// every key a sink.
MaskSpec normalised_mask(const gqa_problem* p) {
  MaskSpec m{p->S, p->causal, p->window, p->num_sinks};
  if (m.window >= m.S) m.window = 0;
  if (m.window == 0) m.sinks = 0;
  if (m.sinks >= m.S) {
    m.window = 0;
    m.sinks = 0;
  }
  return m;
}

// Heads per workgroup for the kernels that give each of the 4 waves one 64-row tile of
// one query head: as many heads of one kv group as divide H/G (up to 4), the remaining
// waves taking further row tiles of the same heads.
void row_decomposition(const gqa_problem* p, int* hpw, int* qpw, int* n_qblk) {
  const int hpg = p->H / p->G;
  *hpw = (hpg % 4 == 0) ? 4 : (hpg % 2 == 0) ? 2 : 1;
  *qpw = 4 / *hpw;
  *n_qblk = (p->S + gqa::kTile * *qpw - 1) / (gqa::kTile * *qpw);
}

int grid_ok(long long blocks) { return blocks > 0 && blocks <= INT_MAX; }

int current_cu_count();

// Workgroup order of the 16-bit forward (the kernels' fwd_block_order).  Workgroup j runs
// on XCD j mod 8, each XCD with its own L2.  When the head groups (B * H / hpw) split into
// eight equal shares of whole kv heads, each XCD serves one share, so a kv head's K/V tiles
// stay in one L2; and when one kv head's workgroups fill at least four rounds of an XCD's
// workgroup slots (two per CU), the XCD finishes each kv head before starting the next,
// which holds a single kv head's tiles per L2 at a time (on smaller grids that order
// would leave light row blocks of one kv head ahead of heavy ones of the next).
void xcd_block_order(const gqa_problem* p, int hpw, int n_qblk, int* xcd_hg, int* xcd_kv) {
  *xcd_hg = 0;
  *xcd_kv = 0;
  const long long nhg = (long long)p->B * (p->H / hpw);
  const int per_kv = (p->H / p->G) / hpw;  // head groups of one kv head
  if (nhg % 8 != 0 || (nhg / 8) % per_kv != 0) return;
  *xcd_hg = (int)(nhg / 8);
  const int cus = current_cu_count();
  const long long slots_per_xcd = cus > 0 ? 2LL * cus / 8 : 64;
  if ((long long)n_qblk * per_kv >= 4 * slots_per_xcd) *xcd_kv = per_kv;
}

// Compute units of the current device (cached per device; 0 if the query fails).
int current_cu_count() {
  static std::atomic<int> cached[64] = {};  // calls may come from several host threads
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

int fill_bwd(const gqa_problem* p, BwdParams* bp) {
  *bp = BwdParams{};
  bp->B = p->B;
  bp->H = p->H;
  bp->G = p->G;
  bp->S = p->S;
  bp->scale = p->scale;
  bp->scale_log2 = p->scale * kLog2e;
  bp->mask = normalised_mask(p);
  row_decomposition(p, &bp->hpw, &bp->qpw, &bp->n_qblk);
  bp->n_kblk = (p->S + gqa::kDkdvKeys - 1) / gqa::kDkdvKeys;
  // few keys per query: large P, whose rounding a key's dV and dK would not average out
  bp->precise_all = (p->S <= kPreciseMaxSeq || (bp->mask.window > 0 && bp->mask.window <= kPreciseMaxWindow)) ? 1 : 0;
  if (!grid_ok((long long)bp->n_qblk * p->B * (p->H / bp->hpw))) return GQA_ERR_UNSUPPORTED;
  if (!grid_ok((long long)bp->n_kblk * p->B * p->G)) return GQA_ERR_UNSUPPORTED;
  if (!grid_ok((long long)p->B * p->H * ((p->S + 63) / 64))) return GQA_ERR_UNSUPPORTED;
  return GQA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? GQA_OK : GQA_ERR_HIP; }

// ---- rotary position embedding ----
constexpr double kTwoPi = 6.28318530717958647693;

bool overlaps(const void* a, size_t abytes, const void* b, size_t bbytes) {
  if (a == nullptr || b == nullptr) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + bbytes && y < x + abytes;
}

size_t elem_bytes(int dtype) { return dtype == GQA_F32 ? 4 : 2; }

// A buffer the call reads or writes: address and bytes (nullptr: absent).
struct Span {
  const void* ptr;
  size_t bytes;
};

// True if an output overlaps an input or another output.  Every kernel reads its inputs
// while other workgroups write outputs, so no aliasing is allowed except where an entry
// point says so (the rotation's in-place form).
bool aliased(std::initializer_list<Span> outs, std::initializer_list<Span> ins) {
  for (auto o = outs.begin(); o != outs.end(); ++o) {
    for (const Span& i : ins)
      if (overlaps(o->ptr, o->bytes, i.ptr, i.bytes)) return true;
    for (auto o2 = o + 1; o2 != outs.end(); ++o2)
      if (overlaps(o->ptr, o->bytes, o2->ptr, o2->bytes)) return true;
  }
  return false;
}

// Byte sizes of a problem's tensors (see the layout in gqa.h).
struct Sizes {
  size_t q, kv, row, q32, kv32;  // Q/O/dO, K/V (element type); lse/delta; dQ; dK/dV
};
Sizes sizes_of(const gqa_problem* p) {
  const size_t rows_q = (size_t)p->B * p->H * p->S, rows_kv = (size_t)p->B * p->G * p->S;
  const size_t e = elem_bytes(p->dtype), D = (size_t)p->D;
  return Sizes{rows_q * D * e, rows_kv * D * e, rows_q * sizeof(float), rows_q * D * 4, rows_kv * D * 4};
}

// The configuration as the kernels take it: YaRN's per-pair frequencies (RoFormer's
// base^(-2i/D), kept for pairs that turn more than beta times over the original context,
// divided by the factor for those turning fewer than alpha times, linearly blended in
// between), in revolutions per position, and the factor m on each rotated vector.
int make_rope_spec(const gqa_rope* r, gqa::RopeSpec* spec) {
  if (r == nullptr) return GQA_ERR_INVALID_ARG;
  if (!(isfinite(r->base) && r->base > 1.0)) return GQA_ERR_INVALID_ARG;
  if (!(isfinite(r->factor) && r->factor >= 1.0)) return GQA_ERR_INVALID_ARG;
  if (!(isfinite(r->mscale) && r->mscale >= 0.0)) return GQA_ERR_INVALID_ARG;
  if (r->factor > 1.0) {
    if (!(isfinite(r->orig_ctx) && r->orig_ctx > 0.0)) return GQA_ERR_INVALID_ARG;
    if (!(isfinite(r->alpha) && isfinite(r->beta) && r->beta > r->alpha)) return GQA_ERR_INVALID_ARG;
  }
  *spec = gqa::RopeSpec{};
  const int D = gqa::kHeadDim;
  for (int i = 0; i < D / 2; ++i) {
    double theta = pow(r->base, -2.0 * i / D);
    if (r->factor > 1.0) {
      const double turns = r->orig_ctx * theta / kTwoPi;
      double ramp = (turns - r->alpha) / (r->beta - r->alpha);
      ramp = ramp < 0.0 ? 0.0 : ramp > 1.0 ? 1.0 : ramp;
      theta = (1.0 - ramp) * theta / r->factor + ramp * theta;
    }
    spec->rev[i] = theta / kTwoPi;
  }
  const double m = r->mscale > 0.0 ? r->mscale : r->factor > 1.0 ? 0.1 * log(r->factor) + 1.0 : 1.0;
  spec->mscale = (float)m;
  spec->enabled = 1;
  return GQA_OK;
}

// Launch plan of the rotation kernel: blocks of rows x runs of up to 16 slabs (the sines and
// cosines of a run's rows are computed once), shorter runs while that leaves fewer than 8
// blocks per compute unit.
int plan_rope(const gqa::RopeSpec& spec, const void* x, void* y, long long n_slabs, int S, long long pos0,
              int inverse, int dtype, gqa::RopeParams* rp) {
  *rp = gqa::RopeParams{};
  rp->x = x;
  rp->y = y;
  rp->n_slabs = n_slabs;
  rp->S = S;
  rp->pos0 = (int)pos0;
  rp->inverse = inverse;
  rp->spec = spec;
  const int rows = gqa::rope_rows_per_block(dtype);
  rp->n_row_blocks = (S + rows - 1) / rows;
  const int cus = current_cu_count();
  const long long want = 8LL * (cus > 0 ? cus : 256);
  long long spb = 16;
  while (spb > 1 && rp->n_row_blocks * ((n_slabs + spb - 1) / spb) < want) spb /= 2;
  rp->slabs_per_block = (int)spb;
  return grid_ok(rp->n_row_blocks * ((n_slabs + spb - 1) / spb)) ? GQA_OK : GQA_ERR_UNSUPPORTED;
}


// ---- decode ----
int check_decode(const gqa_decode_problem* p) {
  if (p == nullptr) return GQA_ERR_INVALID_ARG;
  if (p->B < 0 || p->Sq < 0 || p->Skv < 0 || p->H < 1 || p->G < 1 || p->D < 1) return GQA_ERR_INVALID_ARG;
  if (p->H % p->G != 0) return GQA_ERR_INVALID_ARG;
  if (!(isfinite(p->scale) && p->scale > 0.f)) return GQA_ERR_INVALID_ARG;
  if (p->window < 0 || p->num_sinks < 0) return GQA_ERR_INVALID_ARG;
  if (p->dtype != GQA_F32 && p->dtype != GQA_BF16 && p->dtype != GQA_F16) return GQA_ERR_INVALID_ARG;
  if (p->Sq > p->Skv) return GQA_ERR_INVALID_ARG;  // the rows are the newest Sq positions of the cache
  if (p->D != gqa::kHeadDim || p->dtype == GQA_F32) return GQA_ERR_UNSUPPORTED;
  if (p->Skv > GQA_MAX_SEQ || (long long)p->B * p->H * p->Sq > INT_MAX / 2) return GQA_ERR_UNSUPPORTED;
  return GQA_OK;
}

bool empty_decode(const gqa_decode_problem* p) { return p->B == 0 || p->Sq == 0; }

// Split plan shared by the workspace query and the launch: rows per (b, g) in chunks of
// 128, the visible key tiles of the newest Sq positions, and enough splits per chunk to
// fill every compute unit (see below).  Workspace: per chunk and partial, O (128 x 64 fp32)
// plus maximum and sum (2 x 128 fp32).
int plan_decode(const gqa_decode_problem* p, gqa::DecodeParams* dp, size_t* ws_bytes) {
  using gqa::kDecodeRows;
  using gqa::kDecodeWaves;
  *dp = gqa::DecodeParams{};
  dp->B = p->B;
  dp->H = p->H;
  dp->G = p->G;
  dp->Sq = p->Sq;
  dp->Skv = p->Skv;
  dp->hpg = p->H / p->G;
  const long long rows = (long long)dp->hpg * p->Sq;
  if (rows > INT_MAX / 2) return GQA_ERR_UNSUPPORTED;
  dp->rows = (int)rows;
  dp->nrc = (int)((rows + kDecodeRows - 1) / kDecodeRows);
  dp->scale_log2 = p->scale * kLog2e;
  gqa_problem q{p->B, p->H, p->G, p->Skv, p->D, p->scale, 1, p->window, p->num_sinks, p->dtype};
  dp->mask = normalised_mask(&q);
  dp->tiles = gqa::key_tiles_for_rows(dp->mask, p->Skv - p->Sq, p->Skv - 1);
  const int nt = dp->tiles.count();
  const long long sets = (long long)p->B * p->G * dp->nrc;
  // Chunks of at most 32 rows: every wave of a 4-wave workgroup is a partial over its own
  // tiles (one workgroup per CU, 128 KiB of LDS), at least 2 tiles per wave.  Larger chunks:
  // one wave per 32-row block sharing the tiles, the workgroup a partial (64 KiB of LDS, two
  // per CU), at least 4 tiles per workgroup.
  dp->shared_tiles = rows > 32 ? 1 : 0;
  const int cus = current_cu_count();
  const long long target = cus > 0 ? (long long)cus * (dp->shared_tiles ? 2 : 1) : 1;
  long long nsplit = (target + sets - 1) / sets;
  const long long min_tiles = dp->shared_tiles ? 4 : 8;
  const long long cap = nt / min_tiles > 1 ? nt / min_tiles : 1;
  if (nsplit > cap) nsplit = cap;
  if (nsplit < 1) nsplit = 1;
  dp->nsplit = (int)nsplit;
  dp->n_part = (int)(nsplit * (dp->shared_tiles ? 1 : kDecodeWaves));
  if (!grid_ok(sets * nsplit) || !grid_ok(((long long)p->B * p->H * p->Sq + 3) / 4)) return GQA_ERR_UNSUPPORTED;
  const size_t parts = (size_t)sets * dp->n_part;
  const size_t bytes = parts * ((size_t)kDecodeRows * gqa::kHeadDim + 2 * kDecodeRows) * sizeof(float);
  *ws_bytes = (bytes + 255) & ~(size_t)255;
  return GQA_OK;
}


// Forward launch with validated, non-empty arguments; rope == nullptr for plain attention.
int run_fwd(const gqa_problem* p, const void* q, const void* k, const void* v, void* o, void* o_lo, float* lse,
            const gqa::RopeSpec* rope, void* q_rot, hipStream_t s) {
  FwdParams fp{};
  fp.q = q;
  fp.k = k;
  fp.v = v;
  fp.o = o;
  fp.o_lo = o_lo;
  fp.lse = lse;
  fp.B = p->B;
  fp.H = p->H;
  fp.G = p->G;
  fp.S = p->S;
  fp.scale = p->scale;
  fp.scale_log2 = p->scale * kLog2e;
  fp.mask = normalised_mask(p);
  row_decomposition(p, &fp.hpw, &fp.qpw, &fp.n_qblk);
  xcd_block_order(p, fp.hpw, fp.n_qblk, &fp.xcd_hg, &fp.xcd_kv);
  if (rope != nullptr) {
    fp.rope = *rope;
    fp.q_rot = q_rot;
  }
  if (p->dtype == GQA_F32) return hip_status(gqa::launch_fwd_f32(fp, s));
  return hip_status(gqa::launch_fwd_mfma(fp, p->dtype, s));
}

int fwd_grid_ok(const gqa_problem* p) {
  if (p->dtype == GQA_F32) return grid_ok((long long)p->B * p->H * ((p->S + 63) / 64));
  int hpw, qpw, n_qblk;
  row_decomposition(p, &hpw, &qpw, &n_qblk);
  return grid_ok((long long)n_qblk * p->B * (p->H / hpw));
}


int run_dkdv(const gqa_problem* p, const void* q, const void* k, const void* v, const float* lse, const void* d_o,
             const float* delta, float* dk, float* dv, const gqa::RopeSpec* rope, void* stream) {
  int rc = check_problem(p);
  if (rc != GQA_OK) return rc;
  if (empty_problem(p)) return GQA_OK;
  if (!q || !k || !v || !lse || !d_o || !delta || !dk || !dv) return GQA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(lse) || !aligned16(d_o) ||
      !aligned16(delta) || !aligned16(dk) || !aligned16(dv))
    return GQA_ERR_INVALID_ARG;
  const Sizes z = sizes_of(p);
  if (aliased({{dk, z.kv32}, {dv, z.kv32}}, {{q, z.q}, {k, z.kv}, {v, z.kv}, {lse, z.row}, {d_o, z.q}, {delta, z.row}})) return GQA_ERR_INVALID_ARG;
  BwdParams bp;
  if ((rc = fill_bwd(p, &bp)) != GQA_OK) return rc;
  bp.q = q;
  bp.k = k;
  bp.v = v;
  bp.lse = lse;
  bp.d_o = d_o;
  bp.delta = delta;
  bp.dk = dk;
  bp.dv = dv;
  hipStream_t s = (hipStream_t)stream;
  if (p->dtype == GQA_F32) return hip_status(gqa::launch_bwd_dkdv_f32(bp, s));
  return hip_status(gqa::launch_bwd_dkdv_mfma(bp, rope ? *rope : gqa::RopeSpec{}, p->dtype, s));
}

int run_dq(const gqa_problem* p, const void* q, const void* k, const void* v, const float* lse, const void* d_o,
           const float* delta, float* dq, const gqa::RopeSpec* rope, void* stream) {
  int rc = check_problem(p);
  if (rc != GQA_OK) return rc;
  if (empty_problem(p)) return GQA_OK;
  if (!q || !k || !v || !lse || !d_o || !delta || !dq) return GQA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(lse) || !aligned16(d_o) ||
      !aligned16(delta) || !aligned16(dq))
    return GQA_ERR_INVALID_ARG;
  const Sizes z = sizes_of(p);
  if (aliased({{dq, z.q32}}, {{q, z.q}, {k, z.kv}, {v, z.kv}, {lse, z.row}, {d_o, z.q}, {delta, z.row}})) return GQA_ERR_INVALID_ARG;
  BwdParams bp;
  if ((rc = fill_bwd(p, &bp)) != GQA_OK) return rc;
  bp.q = q;
  bp.k = k;
  bp.v = v;
  bp.lse = lse;
  bp.d_o = d_o;
  bp.delta = delta;
  bp.dq = dq;
  hipStream_t s = (hipStream_t)stream;
  if (p->dtype == GQA_F32) return hip_status(gqa::launch_bwd_dq_f32(bp, s));
  return hip_status(gqa::launch_bwd_dq_mfma(bp, rope ? *rope : gqa::RopeSpec{}, p->dtype, s));
}

int run_grads(const gqa_problem* p, const void* q, const void* k, const void* v, const float* lse, const void* d_o,
              const float* delta, float* dq, float* dk, float* dv, const gqa::RopeSpec* rope, void* stream) {
  int rc = check_problem(p);
  if (rc != GQA_OK) return rc;
  if (empty_problem(p)) return GQA_OK;
  if (!q || !k || !v || !lse || !d_o || !delta || !dq || !dk || !dv) return GQA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(lse) || !aligned16(d_o) ||
      !aligned16(delta) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return GQA_ERR_INVALID_ARG;
  const Sizes z = sizes_of(p);
  if (aliased({{dq, z.q32}, {dk, z.kv32}, {dv, z.kv32}}, {{q, z.q}, {k, z.kv}, {v, z.kv}, {lse, z.row}, {d_o, z.q}, {delta, z.row}})) return GQA_ERR_INVALID_ARG;
  BwdParams bp;
  if ((rc = fill_bwd(p, &bp)) != GQA_OK) return rc;
  // When the dK/dV workgroups fill at most two rounds of workgroup slots (two per CU), the
  // causal spread of their work sets the pass's length; then dK/dV and dQ go in one launch
  // and dQ workgroups fill the CUs that the short key blocks free (3 % faster at B=4 H=32
  // S=4096).  With more rounds the difference is within 1 % either way: two launches.
  const long long n_dkdv = (long long)bp.n_kblk * p->B * p->G;
  const int cus = current_cu_count();
  if (p->dtype == GQA_F32 || cus <= 0 || n_dkdv > 4LL * cus) {
    if ((rc = run_dkdv(p, q, k, v, lse, d_o, delta, dk, dv, rope, stream)) != GQA_OK) return rc;
    return run_dq(p, q, k, v, lse, d_o, delta, dq, rope, stream);
  }
  if (!grid_ok(n_dkdv + (long long)bp.n_qblk * p->B * (p->H / bp.hpw))) return GQA_ERR_UNSUPPORTED;
  bp.q = q;
  bp.k = k;
  bp.v = v;
  bp.lse = lse;
  bp.d_o = d_o;
  bp.delta = delta;
  bp.dq = dq;
  bp.dk = dk;
  bp.dv = dv;
  return hip_status(gqa::launch_bwd_fused_mfma(bp, rope ? *rope : gqa::RopeSpec{}, p->dtype, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int gqa_abi_version(void) { return GQA_ABI_VERSION; }

const char* gqa_status_str(int status) {
  switch (status) {
    case GQA_OK: return "GQA_OK";
    case GQA_ERR_INVALID_ARG: return "GQA_ERR_INVALID_ARG: invalid argument";
    case GQA_ERR_UNSUPPORTED: return "GQA_ERR_UNSUPPORTED: valid problem without a kernel in this build";
    case GQA_ERR_WORKSPACE: return "GQA_ERR_WORKSPACE: workspace missing or too small";
    case GQA_ERR_HIP: return "GQA_ERR_HIP: kernel launch failed";
    default: return "unknown gqa_status";
  }
}

int64_t gqa_visible_pairs(const gqa_problem* p) {
  const int rc = check_problem(p);
  if (rc == GQA_ERR_INVALID_ARG || p == nullptr) return -1;
  const int64_t S = p->S;
  if (S == 0) return 0;
  const MaskSpec m = normalised_mask(p);
  if (!m.causal) return S * S;
  if (m.window == 0) return S * (S + 1) / 2;
  const int64_t W = m.window, NS = m.sinks;  // 0 < W < S, NS < S
  // sum_i min(i + 1, W): ramp to W, then W per row
  int64_t pairs = W * (W + 1) / 2 + (S - W) * W;
  // sinks older than the window: row i >= W adds min(NS, i - W + 1)
  const int64_t n = S - W;
  pairs += (n <= NS) ? n * (n + 1) / 2 : NS * (NS + 1) / 2 + (n - NS) * NS;
  return pairs;
}


int gqa_clock_probe(unsigned long long* out, int32_t blocks, int32_t iters, void* stream) {
  if (out == nullptr || !aligned16(out) || blocks < 1 || blocks > 65536 || iters < 1 || iters > 10000000)
    return GQA_ERR_INVALID_ARG;
  return hip_status(gqa::launch_clock_probe(out, blocks, iters, (hipStream_t)stream));
}

int gqa_attn_fwd(const gqa_problem* p, const void* q, const void* k, const void* v, void* o, void* o_lo,
                 float* lse, void* stream) {
  int rc = check_problem(p);
  if (rc != GQA_OK) return rc;
  if (empty_problem(p)) return GQA_OK;
  if (!q || !k || !v || !o || !lse) return GQA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) || !aligned16(o_lo))
    return GQA_ERR_INVALID_ARG;
  if (o_lo != nullptr && p->dtype == GQA_F32) return GQA_ERR_INVALID_ARG;
  const Sizes z = sizes_of(p);
  if (aliased({{o, z.q}, {o_lo, z.q}, {lse, z.row}}, {{q, z.q}, {k, z.kv}, {v, z.kv}})) return GQA_ERR_INVALID_ARG;
  if (!fwd_grid_ok(p)) return GQA_ERR_UNSUPPORTED;
  return run_fwd(p, q, k, v, o, o_lo, lse, nullptr, nullptr, (hipStream_t)stream);
}

int gqa_rope_apply(const gqa_rope* r, const void* x, void* y, int64_t n_slabs, int32_t S, int32_t D, int64_t pos0,
                   int32_t inverse, int32_t dtype, void* stream) {
  gqa::RopeSpec spec;
  int rc = make_rope_spec(r, &spec);
  if (rc != GQA_OK) return rc;
  if (dtype != GQA_F32 && dtype != GQA_BF16 && dtype != GQA_F16) return GQA_ERR_INVALID_ARG;
  if (n_slabs < 0 || S < 0 || D < 1 || pos0 < 0 || (inverse != 0 && inverse != 1)) return GQA_ERR_INVALID_ARG;
  if (pos0 + (int64_t)S > (int64_t)INT_MAX) return GQA_ERR_INVALID_ARG;
  if (D != gqa::kHeadDim) return GQA_ERR_UNSUPPORTED;
  if (n_slabs == 0 || S == 0) return GQA_OK;
  if (!x || !y || !aligned16(x) || !aligned16(y)) return GQA_ERR_INVALID_ARG;
  const size_t bytes = (size_t)n_slabs * S * D * elem_bytes(dtype);
  if (x != y && overlaps(x, bytes, y, bytes)) return GQA_ERR_INVALID_ARG;
  gqa::RopeParams rp;
  if ((rc = plan_rope(spec, x, y, n_slabs, S, pos0, inverse, dtype, &rp)) != GQA_OK) return rc;
  return hip_status(gqa::launch_rope(rp, dtype, (hipStream_t)stream));
}

int gqa_attn_fwd_rope(const gqa_problem* p, const gqa_rope* r, const void* q, const void* k, const void* v,
                      void* o, void* o_lo, float* lse, void* q_rot, void* k_rot, void* stream) {
  int rc = check_problem(p);
  if (rc != GQA_OK) return rc;
  gqa::RopeSpec spec;
  if ((rc = make_rope_spec(r, &spec)) != GQA_OK) return rc;
  if (empty_problem(p)) return GQA_OK;
  if (!q || !k || !v || !o || !lse || !k_rot) return GQA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) || !aligned16(o_lo) ||
      !aligned16(q_rot) || !aligned16(k_rot))
    return GQA_ERR_INVALID_ARG;
  if (o_lo != nullptr && p->dtype == GQA_F32) return GQA_ERR_INVALID_ARG;
  const Sizes z = sizes_of(p);
  if (aliased({{o, z.q}, {o_lo, z.q}, {lse, z.row}, {q_rot, z.q}, {k_rot, z.kv}}, {{q, z.q}, {k, z.kv}, {v, z.kv}}))
    return GQA_ERR_INVALID_ARG;
  if (!fwd_grid_ok(p)) return GQA_ERR_UNSUPPORTED;
  gqa::RopeParams rp;
  if ((rc = plan_rope(spec, k, k_rot, (long long)p->B * p->G, p->S, 0, 0, p->dtype, &rp)) != GQA_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  if ((rc = hip_status(gqa::launch_rope(rp, p->dtype, s))) != GQA_OK) return rc;
  return run_fwd(p, q, k_rot, v, o, o_lo, lse, &spec, q_rot, s);
}

size_t gqa_attn_bwd_workspace_bytes(const gqa_problem* p) {
  if (check_problem(p) != GQA_OK || empty_problem(p)) return 0;
  const size_t bytes = (size_t)p->B * p->H * p->S * sizeof(float);
  return (bytes + 255) & ~(size_t)255;
}

int gqa_attn_bwd_preprocess(const gqa_problem* p, const void* o, const void* o_lo, const void* d_o, float* delta,
                            void* stream) {
  int rc = check_problem(p);
  if (rc != GQA_OK) return rc;
  if (empty_problem(p)) return GQA_OK;
  if (!o || !d_o || !delta) return GQA_ERR_INVALID_ARG;
  if (!aligned16(o) || !aligned16(o_lo) || !aligned16(d_o) || !aligned16(delta)) return GQA_ERR_INVALID_ARG;
  if (o_lo != nullptr && p->dtype == GQA_F32) return GQA_ERR_INVALID_ARG;
  const Sizes z = sizes_of(p);
  if (aliased({{delta, z.row}}, {{o, z.q}, {o_lo, z.q}, {d_o, z.q}})) return GQA_ERR_INVALID_ARG;
  BwdParams bp;
  if ((rc = fill_bwd(p, &bp)) != GQA_OK) return rc;
  bp.o = o;
  bp.o_lo = o_lo;
  bp.d_o = d_o;
  bp.out_delta = delta;
  const long long rows = (long long)p->B * p->H * p->S;
  if (!grid_ok(rows / 16 + 1)) return GQA_ERR_UNSUPPORTED;
  return hip_status(gqa::launch_bwd_preprocess(bp, p->dtype, (hipStream_t)stream));
}


int gqa_attn_bwd_dkdv(const gqa_problem* p, const void* q, const void* k, const void* v, const float* lse,
                      const void* d_o, const float* delta, float* dk, float* dv, void* stream) {
  return run_dkdv(p, q, k, v, lse, d_o, delta, dk, dv, nullptr, stream);
}

int gqa_attn_bwd_dq(const gqa_problem* p, const void* q, const void* k, const void* v, const float* lse,
                    const void* d_o, const float* delta, float* dq, void* stream) {
  return run_dq(p, q, k, v, lse, d_o, delta, dq, nullptr, stream);
}

int gqa_attn_bwd_grads(const gqa_problem* p, const void* q, const void* k, const void* v, const float* lse,
                       const void* d_o, const float* delta, float* dq, float* dk, float* dv, void* stream) {
  return run_grads(p, q, k, v, lse, d_o, delta, dq, dk, dv, nullptr, stream);
}

}  // extern "C"

namespace gqa {

// gqa_attn_bwd's argument checks, in its order: the problem, the pointers, the workspace
// (unless own_workspace: the caller brings none), then overlaps.
int bwd_check_args(const gqa_problem* p, const void* q, const void* k, const void* v, const void* o,
                   const void* o_lo, const float* lse, const void* d_o, const float* dq, const float* dk,
                   const float* dv, bool own_workspace, const void* workspace, size_t workspace_bytes) {
  const int rc = check_problem(p);
  if (rc != GQA_OK) return rc;
  if (empty_problem(p)) return GQA_OK;
  if (!q || !k || !v || !o || !lse || !d_o || !dq || !dk || !dv) return GQA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) || !aligned16(d_o) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return GQA_ERR_INVALID_ARG;
  if (!own_workspace) {
    if (workspace == nullptr || workspace_bytes < gqa_attn_bwd_workspace_bytes(p)) return GQA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return GQA_ERR_INVALID_ARG;
  }
  const Sizes z = sizes_of(p);
  if (aliased({{dq, z.q32}, {dk, z.kv32}, {dv, z.kv32}, {own_workspace ? nullptr : workspace, z.row}},
              {{q, z.q}, {k, z.kv}, {v, z.kv}, {o, z.q}, {o_lo, z.q}, {lse, z.row}, {d_o, z.q}}))
    return GQA_ERR_INVALID_ARG;
  if (o_lo != nullptr && (p->dtype == GQA_F32 || !aligned16(o_lo))) return GQA_ERR_INVALID_ARG;
  return GQA_OK;
}

}  // namespace gqa

extern "C" {

int gqa_attn_bwd(const gqa_problem* p, const void* q, const void* k, const void* v, const void* o,
                 const void* o_lo, const float* lse, const void* d_o, float* dq, float* dk, float* dv,
                 void* workspace, size_t workspace_bytes, void* stream) {
  int rc = gqa::bwd_check_args(p, q, k, v, o, o_lo, lse, d_o, dq, dk, dv, false, workspace, workspace_bytes);
  if (rc != GQA_OK || empty_problem(p)) return rc;
  BwdParams bp;
  if ((rc = fill_bwd(p, &bp)) != GQA_OK) return rc;
  float* delta = (float*)workspace;
  if ((rc = gqa_attn_bwd_preprocess(p, o, o_lo, d_o, delta, stream)) != GQA_OK) return rc;
  return run_grads(p, q, k, v, lse, d_o, delta, dq, dk, dv, nullptr, stream);
}

int gqa_attn_bwd_rope(const gqa_problem* p, const gqa_rope* r, const void* q_rot, const void* k_rot, const void* v,
                      const void* o, const void* o_lo, const float* lse, const void* d_o, float* dq, float* dk,
                      float* dv, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_problem(p);
  if (rc != GQA_OK) return rc;
  gqa::RopeSpec spec;
  if ((rc = make_rope_spec(r, &spec)) != GQA_OK) return rc;
  if (empty_problem(p)) return GQA_OK;
  if (p->dtype != GQA_F32) {
    // 16-bit: the dK/dV and dQ kernels rotate their results back as they store them
    if (!q_rot || !k_rot || !v || !o || !lse || !d_o || !dq || !dk || !dv) return GQA_ERR_INVALID_ARG;
    if (!aligned16(q_rot) || !aligned16(k_rot) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
        !aligned16(d_o) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
      return GQA_ERR_INVALID_ARG;
    if (workspace == nullptr || workspace_bytes < gqa_attn_bwd_workspace_bytes(p)) return GQA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return GQA_ERR_INVALID_ARG;
    const Sizes z = sizes_of(p);
    if (aliased({{dq, z.q32}, {dk, z.kv32}, {dv, z.kv32}, {workspace, z.row}},
                {{q_rot, z.q}, {k_rot, z.kv}, {v, z.kv}, {o, z.q}, {o_lo, z.q}, {lse, z.row}, {d_o, z.q}}))
      return GQA_ERR_INVALID_ARG;
    BwdParams bp;
    if ((rc = fill_bwd(p, &bp)) != GQA_OK) return rc;
    float* delta = (float*)workspace;
    if ((rc = gqa_attn_bwd_preprocess(p, o, o_lo, d_o, delta, stream)) != GQA_OK) return rc;
    return run_grads(p, q_rot, k_rot, v, lse, d_o, delta, dq, dk, dv, &spec, stream);
  }
  // fp32: the backward, then the two back-rotations in place (plans checked before anything
  // is enqueued)
  gqa::RopeParams rq, rk;
  if ((rc = plan_rope(spec, dq, dq, (long long)p->B * p->H, p->S, 0, 1, GQA_F32, &rq)) != GQA_OK) return rc;
  if ((rc = plan_rope(spec, dk, dk, (long long)p->B * p->G, p->S, 0, 1, GQA_F32, &rk)) != GQA_OK) return rc;
  rc = gqa_attn_bwd(p, q_rot, k_rot, v, o, o_lo, lse, d_o, dq, dk, dv, workspace, workspace_bytes, stream);
  if (rc != GQA_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  if ((rc = hip_status(gqa::launch_rope(rq, GQA_F32, s))) != GQA_OK) return rc;
  return hip_status(gqa::launch_rope(rk, GQA_F32, s));
}

size_t gqa_attn_fwd_fp8_workspace_bytes(const gqa_problem* p) {
  if (check_problem(p) != GQA_OK || empty_problem(p)) return 0;
  const size_t s_pad = ((size_t)p->S + gqa::kTile - 1) / gqa::kTile * gqa::kTile;
  const size_t bytes = (size_t)p->B * p->G * gqa::kHeadDim * s_pad;
  return (bytes + 255) & ~(size_t)255;
}

int gqa_attn_fwd_fp8(const gqa_problem* p, const gqa_fp8_scales* sc, const void* q8, const void* k8, const void* v8,
                     void* o, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_problem(p);
  if (rc != GQA_OK) return rc;
  if (sc == nullptr || !(isfinite(sc->q) && sc->q > 0.f) || !(isfinite(sc->k) && sc->k > 0.f) ||
      !(isfinite(sc->v) && sc->v > 0.f))
    return GQA_ERR_INVALID_ARG;
  if (p->dtype != GQA_BF16) return GQA_ERR_UNSUPPORTED;
  if (empty_problem(p)) return GQA_OK;
  if (!q8 || !k8 || !v8 || !o || !lse) return GQA_ERR_INVALID_ARG;
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8) || !aligned16(o) || !aligned16(lse) || !aligned16(workspace))
    return GQA_ERR_INVALID_ARG;
  if (workspace == nullptr || workspace_bytes < gqa_attn_fwd_fp8_workspace_bytes(p)) return GQA_ERR_WORKSPACE;
  const Sizes z = sizes_of(p);  // element type bf16: the e4m3 inputs are half of those sizes
  if (aliased({{o, z.q}, {lse, z.row}, {workspace, gqa_attn_fwd_fp8_workspace_bytes(p)}},
              {{q8, z.q / 2}, {k8, z.kv / 2}, {v8, z.kv / 2}}))
    return GQA_ERR_INVALID_ARG;
  gqa::Fp8FwdParams fp{};
  fp.q = q8;
  fp.k = k8;
  fp.vt = workspace;
  fp.o = o;
  fp.lse = lse;
  fp.B = p->B;
  fp.H = p->H;
  fp.G = p->G;
  fp.S = p->S;
  fp.s_pad = (p->S + gqa::kTile - 1) / gqa::kTile * gqa::kTile;
  fp.scale_log2 = p->scale * sc->q * sc->k * kLog2e;
  fp.o_scale = sc->v;
  fp.mask = normalised_mask(p);
  row_decomposition(p, &fp.hpw, &fp.qpw, &fp.n_qblk);
  // plain longest-first order (xcd_hg = xcd_kv = 0): the XCD-aware order cuts this kernel's
  // HBM reads threefold but, the kernel being far from bandwidth-bound, costs it ~1 %
  gqa::VtParams vp{};
  vp.v = v8;
  vp.vt = workspace;
  vp.n_slabs = (long long)p->B * p->G;
  vp.S = p->S;
  vp.s_pad = fp.s_pad;
  if (!grid_ok((long long)fp.n_qblk * p->B * (p->H / fp.hpw)) || !grid_ok(vp.n_slabs * (fp.s_pad / gqa::kTile)))
    return GQA_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  if ((rc = hip_status(gqa::launch_vt_permute(vp, s))) != GQA_OK) return rc;
  return hip_status(gqa::launch_fwd_fp8(fp, s));
}

size_t gqa_attn_decode_workspace_bytes(const gqa_decode_problem* p) {
  if (check_decode(p) != GQA_OK || empty_decode(p)) return 0;
  gqa::DecodeParams dp;
  size_t bytes = 0;
  if (plan_decode(p, &dp, &bytes) != GQA_OK) return 0;
  return bytes;
}

int gqa_attn_decode(const gqa_decode_problem* p, const void* q, const void* k, const void* v, void* o, float* lse,
                    void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_decode(p);
  if (rc != GQA_OK) return rc;
  if (empty_decode(p)) return GQA_OK;
  if (!q || !k || !v || !o || !lse) return GQA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) || !aligned16(workspace))
    return GQA_ERR_INVALID_ARG;
  gqa::DecodeParams dp;
  size_t need = 0;
  if ((rc = plan_decode(p, &dp, &need)) != GQA_OK) return rc;
  if (workspace == nullptr || workspace_bytes < need) return GQA_ERR_WORKSPACE;
  const size_t e = elem_bytes(p->dtype), qrows = (size_t)p->B * p->H * p->Sq;
  const size_t kvb = (size_t)p->B * p->G * p->Skv * p->D * e;
  if (aliased({{o, qrows * p->D * e}, {lse, qrows * sizeof(float)}, {workspace, need}},
              {{q, qrows * p->D * e}, {k, kvb}, {v, kvb}}))
    return GQA_ERR_INVALID_ARG;
  dp.q = q;
  dp.k = k;
  dp.v = v;
  dp.o = o;
  dp.lse = lse;
  const size_t parts = (size_t)p->B * p->G * dp.nrc * dp.n_part;
  dp.part_o = (float*)workspace;
  dp.part_ml = dp.part_o + parts * gqa::kDecodeRows * gqa::kHeadDim;
  return hip_status(gqa::launch_decode(dp, p->dtype, (hipStream_t)stream));
}

}  // extern "C"
