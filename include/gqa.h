/*
 * libgqa -- fused causal grouped-query attention for AMD Instinct MI355X (gfx950).
 *
 * The operation (forward), for batch b, query head h and query position i:
 *
 *     g      = h / (H / G)                              query heads share kv heads in
 *                                                       contiguous groups
 *     s_ij   = scale * sum_c Q[b,h,i,c] * K[b,g,j,c]    scaled dot product, scale = 1/sqrt(D)
 *     vis_ij = j <= i  and  (window == 0  or  j > i - window  or  j < num_sinks)
 *     P_ij   = exp(s_ij - lse_i) over visible j, 0 elsewhere
 *     lse_i  = log sum_{visible j} exp(s_ij)             natural log of the scaled scores
 *     O[b,h,i,:] = sum_j P_ij V[b,g,j,:]
 *
 * Sources.  The scaled-dot-product causal softmax, the P.V product and the grouped head
 * map are those of "nx_f32_gqa_gate.nx source" (nishifamily.com): its header comment
 * states the causal scaled softmax attention, and its test T2 gives the map
 * kv = qh / (H/G).  Window and sinks are the "SnapKitty Transformer 8B" model card's
 * attention parameters (Model Specifications: Sliding Window, Attention Sinks; the
 * FlashAttention Inference call flash_attention_fwd(Q, K, V, causal=True,
 * sliding_window=..., num_sinks=...)).  The card gives only sizes; this library reads a
 * window of W as "the W most recent keys, self included" and sinks as the first
 * num_sinks key positions, exempt from the window but still causal.  The backward
 * (recompute P from the saved log-sum-exp, dS = P * (dO V^T - D)) is the card's
 * FlashAttention-3 backward entry in its Protected Inventions list, with
 * D_i = sum_c dO[i,c] O[i,c] and loss L = <O, dO>.
 *
 * Layout.  All tensors are dense and row-major (contiguous, innermost index last):
 *     Q, O, dO     [B][H][S][D]      element type from gqa_problem.dtype
 *     K, V         [B][G][S][D]      same element type
 *     lse, delta   [B][H][S]         fp32
 *     dQ           [B][H][S][D]      fp32
 *     dK, dV       [B][G][S][D]      fp32
 * Query and key sequences have the same length S and the causal diagonal is j = i.
 *
 * Ownership.  The caller allocates and frees every buffer; device pointers must be
 * device memory of the current HIP device, 16-byte aligned.  The library allocates
 * nothing, never synchronises, and enqueues its kernels on `stream` (a hipStream_t
 * passed as void*; NULL = the null stream) and returns.  Results are ready when the
 * stream reaches that point.  The library keeps no state between calls, so calls on
 * different streams may run concurrently if their output buffers do not overlap.
 * Within a call, an output (workspaces included) may overlap neither an input nor another
 * output, except in gqa_rope_apply's in-place form; such a call returns
 * GQA_ERR_INVALID_ARG before anything is enqueued.
 *
 * Errors.  Every argument is validated on the host before any HIP call; a non-OK
 * status means nothing was enqueued, except GQA_ERR_HIP (a launch failed: earlier
 * kernels of the same call may have been enqueued).  No exception crosses this ABI.
 * S == 0 or B == 0 is a valid empty problem and returns GQA_OK without a launch.
 *
 * Supported: D == 64; dtype GQA_BF16 and GQA_F16 (MFMA kernels) and GQA_F32 (fp32
 * kernels for reference-precision runs).  causal == 0 means full (non-causal)
 * attention and then requires window == 0 and num_sinks == 0.  Sequences (S, and a
 * decode cache's Skv) hold at most GQA_MAX_SEQ = 2^23 positions: the kernels address a
 * head's rows with 32-bit byte offsets, tile padding included; longer ones return
 * GQA_ERR_UNSUPPORTED.
 */
#ifndef GQA_H_
#define GQA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GQA_ABI_VERSION 1
#define GQA_MAX_SEQ (1 << 23) /* longest S / Skv the attention entry points accept */
#define GQA_NOALLOC_MAX_ROWS (1 << 23) /* largest B * H * S of gqa_attn_bwd_noalloc */

typedef enum gqa_status {
  GQA_OK = 0,
  GQA_ERR_INVALID_ARG = 1, /* null pointer, bad sizes or flags, misaligned pointer      */
  GQA_ERR_UNSUPPORTED = 2, /* valid problem this build has no kernel for (e.g. D != 64)   */
  GQA_ERR_WORKSPACE = 3,   /* backward workspace missing or smaller than required        */
  GQA_ERR_HIP = 4          /* a HIP launch reported an error                             */
} gqa_status;

typedef enum gqa_dtype { GQA_F32 = 0, GQA_BF16 = 1, GQA_F16 = 2 } gqa_dtype;

typedef struct gqa_problem {
  int32_t B;         /* batch                                                          */
  int32_t H;         /* query heads; H % G == 0                                        */
  int32_t G;         /* key/value heads                                                */
  int32_t S;         /* sequence length of queries and keys                            */
  int32_t D;         /* head dimension (64)                                            */
  float scale;       /* softmax scale applied to q.k; finite and > 0 (1/sqrt(D))       */
  int32_t causal;    /* 1: key j visible to query i only if j <= i; 0: full attention  */
  int32_t window;    /* 0: no window; W > 0: also require j > i - W (unless a sink)     */
  int32_t num_sinks; /* keys j < num_sinks ignore the window (still causal); >= 0      */
  int32_t dtype;     /* gqa_dtype of Q, K, V, O and dO                                 */
} gqa_problem;

/* ABI version of the loaded library (GQA_ABI_VERSION it was built with). */
int gqa_abi_version(void);

/* Static, human-readable name of a gqa_status value; never NULL. */
const char* gqa_status_str(int status);

/* Number of visible (query, key) pairs of one (batch, head), computed on the host from
 * the visibility rule above; -1 if the problem is invalid.  The algorithmic work of the
 * forward is 4 * D * pairs * B * H flop (Q K^T and P V), of the backward
 * 10 * D * pairs * B * H flop (S, dP, dV, dK, dQ). */
int64_t gqa_visible_pairs(const gqa_problem* p);

/* Shader clock under matrix-core load (a measurement helper, not part of the attention):
 * `blocks` workgroups of 4 waves run `iters` iterations of four independent bf16 MFMA
 * chains each; out[2 b] receives workgroup b's shader-clock cycles and out[2 b + 1] the
 * 100 MHz reference ticks over the same interval (clock in MHz = 100 * out[2b] / out[2b+1]).
 * out: device memory, 2 * blocks uint64, 16-byte aligned.  1 <= blocks <= 65536,
 * 1 <= iters <= 10^7; GQA_ERR_INVALID_ARG otherwise. */
int gqa_clock_probe(unsigned long long* out, int32_t blocks, int32_t iters, void* stream);

/* Forward.  Reads Q, K, V; writes O (dtype) and lse (fp32, natural log, of the scaled
 * scores).  lse is what the backward needs to recompute P.
 * o_lo (optional, NULL to skip; must be NULL for GQA_F32): same shape and dtype as O,
 * receives O's rounding residual (exact O minus the stored O, rounded to dtype).  Passed
 * back to the backward it makes delta = rowsum(dO * O) carry about twice dtype's
 * mantissa, which matters where many queries put large weight on the same keys (sinks):
 * there each row's delta error is multiplied by a large P in dK. */
int gqa_attn_fwd(const gqa_problem* p, const void* q, const void* k, const void* v, void* o,
                 void* o_lo, float* lse, void* stream);

/* Bytes of device workspace gqa_attn_bwd needs (the fp32 delta vector [B][H][S]),
 * rounded up to 256; 0 for an invalid or empty problem. */
size_t gqa_attn_bwd_workspace_bytes(const gqa_problem* p);

/* Backward of L = <O, dO>: dQ, dK, dV (fp32, overwritten, not accumulated into) from the
 * forward's inputs, its output O (and optionally o_lo, see gqa_attn_fwd; NULL if not
 * kept) and its lse.  Runs gqa_attn_bwd_preprocess into the workspace, then
 * gqa_attn_bwd_grads, on one stream.  Deterministic: no floating-point atomics, so
 * repeated calls give bit-identical results. */
int gqa_attn_bwd(const gqa_problem* p, const void* q, const void* k, const void* v,
                 const void* o, const void* o_lo, const float* lse, const void* d_o, float* dq,
                 float* dk, float* dv, void* workspace, size_t workspace_bytes, void* stream);

/* gqa_attn_bwd for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  The workspace (the fp32
 * delta vector) is a fixed array inside the library, GQA_NOALLOC_MAX_ROWS floats (32 MiB),
 * which each device the library runs on holds until the process ends; the call allocates
 * nothing.  Arguments, results (bit-identical to gqa_attn_bwd's) and errors as
 * gqa_attn_bwd, except: a problem with B * H * S > GQA_NOALLOC_MAX_ROWS returns
 * GQA_ERR_WORKSPACE before anything is enqueued; the first call on a device looks up the
 * array's address there (GQA_ERR_HIP if that fails).  Every call on one device shares that
 * device's array: calls that may overlap on one device (several streams, several host
 * threads) race on it and must be ordered by the caller. */
int gqa_attn_bwd_noalloc(const gqa_problem* p, const void* q, const void* k, const void* v,
                         const void* o, const void* o_lo, const float* lse, const void* d_o, float* dq,
                         float* dk, float* dv, void* stream);

/* Backward step 1: delta[b,h,i] = sum_c dO[b,h,i,c] * (O + o_lo)[b,h,i,c], accumulated in
 * fp32 (o_lo may be NULL). */
int gqa_attn_bwd_preprocess(const gqa_problem* p, const void* o, const void* o_lo,
                            const void* d_o, float* delta, void* stream);

/* Backward step 2: dK and dV.  Each kv head's gradient sums over the H/G query heads that
 * read it; the sum stays in registers (no atomics). */
int gqa_attn_bwd_dkdv(const gqa_problem* p, const void* q, const void* k, const void* v,
                      const float* lse, const void* d_o, const float* delta, float* dk,
                      float* dv, void* stream);

/* Backward step 3: dQ, one pass per query tile over its visible key tiles. */
int gqa_attn_bwd_dq(const gqa_problem* p, const void* q, const void* k, const void* v,
                    const float* lse, const void* d_o, const float* delta, float* dq,
                    void* stream);

/* Backward steps 2 and 3 together: dK, dV and dQ from delta, with results bit-identical to
 * gqa_attn_bwd_dkdv followed by gqa_attn_bwd_dq.  For 16-bit inputs, when the dK/dV pass
 * has no more workgroups than the device holds at once (two per compute unit), its work
 * per workgroup is very uneven under a causal mask (the first key block sees every query,
 * the last one almost none); then both passes go in one launch, so that dQ work fills the
 * compute units the short key blocks leave idle.  Otherwise, and for GQA_F32, the two
 * passes are launched one after the other.  Arguments and errors as for those two. */
int gqa_attn_bwd_grads(const gqa_problem* p, const void* q, const void* k, const void* v,
                       const float* lse, const void* d_o, const float* delta, float* dq,
                       float* dk, float* dv, void* stream);

/* ---------------------------------------------------------------------------------------
 * Decode: a few new query rows per head against a long key/value cache.
 *
 * The same operation as the forward, for the last Sq positions of a sequence of Skv keys:
 * query row t of head h sits at position i = Skv - Sq + t and sees key j iff
 *     j <= i  and  (window == 0  or  j > i - window  or  j < num_sinks)
 * (always causal).  This is generation with a key/value cache: the model card's inference
 * call flash_attention_fwd(Q, K, V, causal=True, sliding_window=..., num_sinks=...) with the
 * cache as K and V and only the newest tokens as Q ("SnapKitty Transformer 8B" model card:
 * FlashAttention Inference and Text Generation examples, and the KV Cache column of its
 * Memory Usage table).
 *
 * Layout (dense, row-major):
 *     Q, O   [B][H][Sq][D]    element type from dtype (GQA_BF16 or GQA_F16)
 *     K, V   [B][G][Skv][D]   the cache, same element type
 *     lse    [B][H][Sq]       fp32, natural log of the scaled scores
 * The key range is split across workgroups (split-KV): each writes a partial softmax state
 * (unnormalised O, running maximum, row sum) to the workspace, and a second kernel merges
 * the partials of every row with the log-sum-exp rule.  The split depends only on the
 * problem and the device's compute-unit count, so results are deterministic on a device. */
typedef struct gqa_decode_problem {
  int32_t B;         /* batch                                                          */
  int32_t H;         /* query heads; H % G == 0                                        */
  int32_t G;         /* key/value heads                                                */
  int32_t Sq;        /* query rows per head, 1 <= Sq <= Skv (0 with B == 0: empty)     */
  int32_t Skv;       /* keys in the cache                                              */
  int32_t D;         /* head dimension (64)                                            */
  float scale;       /* softmax scale applied to q.k; finite and > 0                   */
  int32_t window;    /* 0: no window; W > 0: also require j > i - W (unless a sink)     */
  int32_t num_sinks; /* keys j < num_sinks ignore the window (still causal); >= 0      */
  int32_t dtype;     /* gqa_dtype of Q, K, V and O: GQA_BF16 or GQA_F16                */
} gqa_decode_problem;

/* Bytes of device workspace gqa_attn_decode needs on the current device (the partial
 * softmax states of every split), rounded up to 256; 0 for an invalid or empty problem. */
size_t gqa_attn_decode_workspace_bytes(const gqa_decode_problem* p);

/* Decode attention.  Reads Q, K, V; writes O (dtype) and lse (fp32).  The workspace (device
 * memory, at least gqa_attn_decode_workspace_bytes, 16-byte aligned) is scratch owned by the
 * caller; its contents need no initialisation and are meaningless afterwards.  Errors:
 * GQA_ERR_INVALID_ARG for bad sizes, pointers or alignment (Sq > Skv included),
 * GQA_ERR_UNSUPPORTED for D != 64, GQA_F32 or Skv > GQA_MAX_SEQ, GQA_ERR_WORKSPACE for a
 * missing or short workspace, GQA_ERR_HIP if a launch fails.  B == 0 returns GQA_OK without a launch. */
int gqa_attn_decode(const gqa_decode_problem* p, const void* q, const void* k, const void* v,
                    void* o, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * Rotary position embedding with YaRN frequencies ("SnapKitty Transformer 8B" model card:
 * YaRN RoPE, 32x factor, in the Model Specifications table; rope_yarn and
 * rope_yarn_factor 32.0 with max_seq_len 204800 in its Training Configuration; YaRN-scaled
 * RoPE inside the attention kernels in its Protected Inventions list).  The card gives no
 * formula; this library follows the published methods it names:
 *
 *   RoFormer rotary embedding: the dimension pair (2i, 2i+1), i < D/2, of the vector at
 *   position p is rotated by the angle p * theta'_i:
 *       y_{2i}   = m (x_{2i} cos - x_{2i+1} sin),   y_{2i+1} = m (x_{2i} sin + x_{2i+1} cos)
 *   YaRN frequencies ("NTK-by-parts"): theta_i = base^(-2i/D), r_i = orig_ctx theta_i / (2 pi),
 *       gamma_i = clamp((r_i - alpha) / (beta - alpha), 0, 1),
 *       theta'_i = (1 - gamma_i) theta_i / factor + gamma_i theta_i      (factor > 1)
 *       theta'_i = theta_i                                               (factor == 1)
 *   and m = YaRN's attention temperature 0.1 ln(factor) + 1 on each of q and k (or mscale).
 *
 * The model card's setting: base 10000, factor 32, orig_ctx 204800 / 32 = 6400, alpha 1,
 * beta 32, mscale 0 (the YaRN value, 1.3466).  Base, the original context and the ramp
 * bounds are the YaRN and RoFormer papers' values, not the card's.  The D/2 frequencies
 * are worked out on the host in fp64 from this struct; each position's angles and the
 * rotation run in the kernels, the angle reduced to one revolution in fp64 so that any
 * position below 2^31 keeps fp32 accuracy. */
typedef struct gqa_rope {
  double base;     /* frequency base, > 1 (10000)                                        */
  double factor;   /* YaRN context scale, >= 1; 1 = plain rotary embedding (32)          */
  double orig_ctx; /* original context length of the ramp, > 0 when factor > 1 (6400)   */
  double alpha;    /* pairs turning fewer than alpha times over orig_ctx: theta / factor  */
  double beta;     /* pairs turning more than beta times keep theta; beta > alpha (1, 32) */
  double mscale;   /* factor m on each rotated vector, >= 0; 0 = YaRN's 0.1 ln(factor) + 1 */
} gqa_rope;

/* y = m R(pos0 + s) x for every row s of x, or m R(pos0 + s)^T x with inverse = 1 (the
 * backward of the rotation).  x, y: [n_slabs][S][D] rows of dtype (GQA_BF16, GQA_F16 or
 * GQA_F32), device memory, 16-byte aligned, either the same buffer (in place) or not
 * overlapping.  D == 64.  0 <= pos0 and pos0 + S <= 2^31 - 1.  Errors: GQA_ERR_INVALID_ARG
 * for a bad configuration, size, pointer or flag; GQA_ERR_UNSUPPORTED for D != 64;
 * GQA_ERR_HIP if the launch fails.  n_slabs == 0 or S == 0 returns GQA_OK, no launch. */
int gqa_rope_apply(const gqa_rope* r, const void* x, void* y, int64_t n_slabs, int32_t S, int32_t D,
                   int64_t pos0, int32_t inverse, int32_t dtype, void* stream);

/* Forward with the rotation in front: O = attention(R Q, R K, V), query and key i at
 * position i.  K is rotated into k_rot ([B][G][S][D], dtype; required), which is what the
 * backward reads and what a key/value cache holds.  Q is rotated in the forward kernel's
 * registers (never stored) unless q_rot is given ([B][H][S][D], dtype; NULL to skip), which
 * then receives the rotated Q for the backward.  Everything else as gqa_attn_fwd; q_rot and
 * k_rot must not overlap the inputs.  The rotated operands are rounded to dtype. */
int gqa_attn_fwd_rope(const gqa_problem* p, const gqa_rope* r, const void* q, const void* k, const void* v,
                      void* o, void* o_lo, float* lse, void* q_rot, void* k_rot, void* stream);

/* Backward of gqa_attn_fwd_rope: dQ, dK, dV of L = <O, dO> with respect to the unrotated
 * Q, K and V.  Takes the rotated q_rot and k_rot of the forward; computes what gqa_attn_bwd
 * gives for them (the gradients with respect to R Q and R K) and rotates dQ and dK back
 * with m R^T: for 16-bit inputs inside the dK/dV and dQ kernels as they store their results
 * (bit-identical to a separate rotation), for GQA_F32 by the rotation kernel in place
 * afterwards.  Workspace and errors as gqa_attn_bwd (gqa_attn_bwd_workspace_bytes). */
int gqa_attn_bwd_rope(const gqa_problem* p, const gqa_rope* r, const void* q_rot, const void* k_rot,
                      const void* v, const void* o, const void* o_lo, const float* lse, const void* d_o,
                      float* dq, float* dk, float* dv, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * FP8 forward: the forward above with Q, K and V in FP8 (OCP e4m3, one byte per element)
 * and per-tensor dequantisation factors -- the "FP8 computation" of the model card's
 * FlashAttention-3 forward (Protected Inventions list).  Both products run on the FP8
 * matrix cores: S = scale * (q_scale Q8)(k_scale K8)^T, P = softmax, and O = P (v_scale V8)
 * with P rounded to e4m3 for the second product; row sums, lse and accumulation in fp32.
 *
 * Layout: Q8 [B][H][S][D], K8 and V8 [B][G][S][D] (e4m3 bytes); O [B][H][S][D] in
 * p->dtype, which must be GQA_BF16; lse [B][H][S] fp32 (natural log of the scaled scores).
 * The workspace (gqa_attn_fwd_fp8_workspace_bytes) receives V transposed per kv head, in
 * the key order the kernel's operands need; its contents need no initialisation.
 * Errors as gqa_attn_fwd, plus GQA_ERR_INVALID_ARG for a missing or non-positive scale,
 * GQA_ERR_WORKSPACE for a missing or short workspace, GQA_ERR_UNSUPPORTED for an output
 * dtype other than GQA_BF16. */
typedef struct gqa_fp8_scales {
  float q, k, v; /* element value = scale * e4m3 code value; finite and > 0 */
} gqa_fp8_scales;

size_t gqa_attn_fwd_fp8_workspace_bytes(const gqa_problem* p);

int gqa_attn_fwd_fp8(const gqa_problem* p, const gqa_fp8_scales* scales, const void* q8, const void* k8,
                     const void* v8, void* o, float* lse, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_H_ */
