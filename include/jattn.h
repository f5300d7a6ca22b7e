/*
 * jattn.h -- C ABI of libjattn.so: jagged (unpadded, variable-length)
 * dot-product attention, forward and backward, for AMD MI355X (gfx950).
 *
 * What is computed.  "Training GEM at LLM scale" (Meta engineering post):
 *   - section "Jagged Sequence Flash Attention": attention over jagged
 *     tensors without padding, custom additive attention bias, query and
 *     key/value lengths that differ per sample, and a backward pass;
 *   - section "Generalized Dot-Product Attention (GDPA)": the same two
 *     matrix products with GELU or SiLU applied element-wise in place of
 *     softmax (no normalisation);
 *   - section "BlockAttention": a fixed 64-token block-diagonal mask, and
 *     the sliding-window attention that preceded it (each token attends to
 *     nearby tokens of its own sequence; tiles outside the window are never
 *     visited).
 * For sample b and head h, with Q_b [lq,D], K_b, V_b [lk,D]:
 *   S = scale * Q_b K_b^T + bias_b[h]
 *   softmax:  P = softmax_row(S), O = P V, LSE_i = ln sum_j exp(S_ij)
 *   GDPA:     P = act(S),        O = P V   (act = erf-GELU, SiLU, or the
 *             ALU-only polynomial GELU of the GDPA section, which is accurate
 *             on the bounded scores that QK-norm gives)
 *   block-diagonal: only pairs with floor(i/64) == floor(j/64) take part.
 *   sliding window (left, right): only pairs with i - left <= j <= i + right
 *     take part (self-attention: lq_b == lk_b).  The pages fix no window
 *     size or direction; (left, right) = (>= max length, 0) is causal.
 * There is no causal mask.  Zero-length samples: rows with lk = 0 get O = 0,
 * LSE = -inf and dQ = 0; rows with lq = 0 get dK = dV = 0.  The library
 * writes these zeros itself and never assumes zeroed output buffers.
 *
 * Layouts (device memory, row-major, caller-owned):
 *   q, o, dout, dq     [Tq, H, D]   Tq = q_offsets[B]
 *   k, v, dk, dv       [Tk, H, D]   Tk = kv_offsets[B]
 *   lse                [Tq, H] float32 (softmax only)
 *   bias, dbias        samples concatenated: sample b is [H, lq_b, lk_b]
 *                      row-major at element offset sum_{j<b} H lq_j lk_j
 *   offsets            host int64 [B+1], offsets[0] = 0, non-decreasing.
 * Value pointers must be 16-byte aligned; bias/dbias element-aligned.
 *
 * Ownership and threading.  The caller owns every device buffer, including
 * the workspace (size from jattn_plan_info).  The library never allocates
 * device memory.  A plan is host memory owned by the library, immutable
 * after creation and safe to share between threads.  jattn_fwd, jattn_bwd
 * and jattn_bwd_stages enqueue their kernels on the given stream (a
 * hipStream_t; NULL = the null stream) and return without waiting; device
 * faults surface at the caller's next synchronisation.  jattn_plan_upload is
 * the exception: it waits for its copy (see there).
 *
 * Sharing one workspace.  The workspace holds the uploaded plan, which every
 * call only reads, and a scratch region (row statistics Di and LSE * log2 e)
 * that the backward writes and reads (see the stages below).  Forwards may
 * therefore run concurrently on one workspace; a softmax backward (mask NONE
 * or WINDOW) must not overlap another backward on the same workspace.
 *
 * Errors.  Every call returns JATTN_OK (0) or a negative JATTN_E_* code.
 * Arguments are validated on the host before anything is enqueued; on
 * error nothing is launched.  jattn_last_error() gives a text for the most
 * recent failure on the calling thread.  Nothing is thrown across the ABI.
 */
#ifndef JATTN_H
#define JATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define JATTN_OK 0
#define JATTN_E_NULL (-1)        /* a required pointer is NULL */
#define JATTN_E_OFFSETS (-2)     /* offsets[0] != 0, decreasing, or a total >= 2^31 rows */
#define JATTN_E_SHAPE (-3)       /* bad B, H, D, block-diagonal with lq != lk, or a sample whose rows span
                                    >= 2^31 bytes in the widest of in/out/grad dtype */
#define JATTN_E_UNSUPPORTED (-4) /* unsupported dtype / activation / mask combination */
#define JATTN_E_ALIGN (-5)       /* misaligned device pointer */
#define JATTN_E_WORKSPACE (-6)   /* workspace missing or too small */
#define JATTN_E_STATE (-7)       /* e.g. LSE missing for a softmax backward */
#define JATTN_E_HIP (-8)         /* a HIP runtime call or launch failed */
#define JATTN_E_ARG (-9)         /* other invalid argument */

/* activation (desc.act) */
#define JATTN_SOFTMAX 0
#define JATTN_GELU_ERF 1 /* GDPA with x * Phi(x) */
#define JATTN_SILU 2     /* GDPA with x * sigmoid(x) */
#define JATTN_GELU_POLY 3 /* GDPA with the ALU-only GELU: 0.5 x (1 + t(u)),
                             u = sqrt(2/pi) (x + 0.044715 x^3),
                             t(u) = u - u^3/3 + 2 u^5/15 (tanh's Taylor
                             polynomial through order 6); for the bounded
                             scores of QK-norm inputs; bf16 inputs only */

/* mask (desc.mask) */
#define JATTN_MASK_NONE 0
#define JATTN_MASK_BLOCKDIAG64 1 /* BlockAttention, requires lq_b == lk_b */
#define JATTN_MASK_WINDOW 2      /* sliding window (window_left, window_right),
                                    requires lq_b == lk_b and bf16 inputs */

/* element types */
#define JATTN_BF16 0
#define JATTN_F32 1
#define JATTN_MXFP8 2 /* desc.in_dtype only: inputs are MXFP8 tensors made by
                         jattn_mx_quantize (see the MXFP8 section below) */

/* unit order across workers (desc.order) */
#define JATTN_HEAVY_FIRST 0 /* cost-sorted units dealt round-robin */
#define JATTN_ZIGZAG 1      /* cost-sorted units dealt boustrophedon */
#define JATTN_LPT 2         /* cost-sorted units to the least-loaded worker */

/* plan parts (jattn_plan_export "which") */
#define JATTN_PLAN_FWD 0  /* forward units (b, h, q-tile) */
#define JATTN_PLAN_DKDV 1 /* dK/dV units (b, h, kv-tile) */
#define JATTN_PLAN_DQ 2   /* dQ units (b, h, q-tile) */
#define JATTN_PLAN_BLOCK 3 /* block-diagonal units (b, h, 64-block) */

typedef struct jattn_plan jattn_plan; /* opaque */

typedef struct {
  int32_t B, H, D;      /* D in {32, 64, 128}; H >= 1; B >= 0 */
  float scale;          /* softmax/GDPA scale; <= 0 selects 1/sqrt(D) */
  int32_t act;          /* JATTN_SOFTMAX | JATTN_GELU_ERF | JATTN_SILU | JATTN_GELU_POLY */
  int32_t mask;         /* JATTN_MASK_NONE | JATTN_MASK_BLOCKDIAG64 | JATTN_MASK_WINDOW */
  int32_t has_bias;     /* 0/1: additive bias input */
  int32_t want_dbias;   /* 0/1: backward writes dBias (needs has_bias) */
  int32_t in_dtype;     /* q, k, v, bias, dout: JATTN_BF16 | JATTN_F32 */
  int32_t out_dtype;    /* o */
  int32_t grad_dtype;   /* dq, dk, dv */
  int32_t split_operands; /* 0/1: P and dS enter the PV-type products as
                             bf16 hi + lo pairs (two MFMAs) for accuracy.
                             Accuracy contract: GDPA (GELU / SiLU) rows are
                             not normalised, so with plain bf16 P the error of
                             O = P V grows as 2^-8 sum_j |P_ij| |V_j| (about
                             0.15 at 4000 keys of N(0,1) data); a 2e-2
                             max-abs bound on long key sets needs split = 1
                             and fp32 outputs.  Softmax normalises by the sum
                             of the rounded P and does not need it; for dV /
                             dK sums over thousands of queries it does. */
  int32_t order;        /* JATTN_HEAVY_FIRST | JATTN_ZIGZAG | JATTN_LPT */
  int32_t num_workers;  /* persistent workers per kernel; 0 = default.  The
                           bf16 dK/dV pass at D <= 64 without bias or window
                           on 64- or 128-key tiles (not erf-GELU) runs two
                           workgroups per CU and is planned over twice this
                           number; the bf16 forward without bias or window
                           on 128-row query tiles runs three at D <= 64 and
                           (softmax) two at D = 128, planned over three or
                           two times it; the bf16 softmax dQ pass without
                           bias or window (at D = 128 also without split
                           operands) runs two, over twice it
                           (jattn_plan_summary reports each pass's) */
  int32_t dbias_dtype;  /* dbias: JATTN_BF16 | JATTN_F32 */
  int32_t window_left;  /* JATTN_MASK_WINDOW: keys before the query it sees (>= 0) */
  int32_t window_right; /* JATTN_MASK_WINDOW: keys after the query it sees (>= 0);
                           both are ignored for other masks */
  int32_t rope;         /* 0/1, JATTN_MASK_BLOCKDIAG64 only: rotary position
                           embedding of Q and K fused into the block kernels
                           (section "BlockAttention": RoPE backward fused into
                           the attention epilogue).  Rotate-half pairs
                           (j, j + D/2) at position m (token index inside the
                           sample) turn by m * rope_base^(-2j/D); q, k stay
                           un-rotated in memory and dq, dk are the gradients
                           with respect to them. */
  float rope_base;      /* <= 0 selects 10000 */
} jattn_desc;

/* Per-kernel plan figures.  tile_rows: rows of the unit's own tile (q rows
 * for fwd/dq, kv rows for dkdv, 64 for block); step_rows: rows consumed per
 * inner-loop step (kv for fwd/dq, q for dkdv). */
typedef struct {
  int32_t tile_rows, step_rows, num_workers, n_units;
} jattn_kernel_plan;

typedef struct {
  int64_t workspace_bytes; /* device workspace needed by fwd and bwd */
  int64_t Tq, Tk;          /* total query / key rows */
  int64_t bias_elems;      /* sum_b H lq_b lk_b */
  double flops_fwd;        /* algorithmic: 4 H D sum(lq lk) (allowed pairs) */
  double flops_bwd;        /* 2.5 x flops_fwd */
  jattn_kernel_plan fwd, dkdv, dq, block;
} jattn_plan_summary;

/* Build a plan on the host from host offset arrays (int64 [B+1] each).
 * Validates offsets and the descriptor, enumerates the valid tiles of every
 * kernel and orders them across workers ("Training GEM at LLM scale",
 * section "Generalized Dot-Product Attention (GDPA)": valid tiles are
 * precomputed on the CPU, empty ones skipped, and assigned in zigzag order).
 * On success *out owns the plan (free with jattn_plan_destroy).  Touches no
 * GPU. */
int jattn_plan_create(const jattn_desc* desc, const int64_t* q_offsets,
                      const int64_t* kv_offsets, jattn_plan** out);

/* Fill *summary.  Host only. */
int jattn_plan_info(const jattn_plan* plan, jattn_plan_summary* summary);

/* Copy a plan part to host memory as int32.  which = JATTN_PLAN_* * 2 + part,
 * part 0 = units as (b, h, tile, cost) quadruples in worker order (with a
 * sliding window, cost counts the steps that meet the tile's window; the
 * first of them follows from the tile index and the window),
 * part 1 = worker offsets [num_workers + 1].  *n receives the number of
 * int32 written (or needed, when dst is NULL).  Host only. */
int jattn_plan_export(const jattn_plan* plan, int32_t which, int32_t* dst, int64_t cap,
                      int64_t* n);

/* Copy the plan into the caller's device workspace, on `stream`, and wait
 * for the copy to finish (hipStreamSynchronize(stream)): the call blocks the
 * host until everything enqueued on that stream before it has run, and the
 * plan's host memory may then be freed.  Must be done once per (plan,
 * workspace) pair before jattn_fwd / jattn_bwd use that workspace; the plan
 * region is never modified by fwd/bwd. */
int jattn_plan_upload(const jattn_plan* plan, void* workspace, int64_t workspace_bytes,
                      void* stream);

/* Forward.  Writes o (out_dtype) and, for softmax with mask NONE or WINDOW, lse.
 * Tail handling ("Jagged Sequence Flash Attention" section): keys past a
 * sample's end are read as zeros and score 0; their exp terms are removed
 * from the row sum by subtraction instead of a -inf mask.  A row whose best
 * valid score is below 0 (where the subtraction would cancel or, once the
 * valid terms underflow, give NaN) instead drops those keys in the one key
 * step that holds them, so any finite bias is handled exactly.
 * bias: required iff desc.has_bias.  lse may be NULL (not written) for
 * softmax; it must be NULL-or-ignored for GDPA and block mode, which keep
 * no row statistics ("BlockAttention" section: no logsumexp traffic). */
int jattn_fwd(const jattn_plan* plan, const void* q, const void* k, const void* v,
              const void* bias, void* o, float* lse, void* workspace, void* stream);

/* Backward.  Given dout, writes dq, dk, dv (grad_dtype) and, if
 * desc.want_dbias, dbias (dbias_dtype).  Softmax with mask NONE or WINDOW needs o and
 * the forward's lse (JATTN_E_STATE otherwise); GDPA needs neither; block
 * mode recomputes its row statistics in-tile and needs neither.  Uses the
 * workspace's scratch region for row statistics.  No atomics: every output
 * element has exactly one writer, so results are run-to-run identical
 * ("Jagged Sequence Flash Attention" section: separate dQ pass, no atomic
 * adds). */
int jattn_bwd(const jattn_plan* plan, const void* q, const void* k, const void* v,
              const void* bias, const void* o, const float* lse, const void* dout, void* dq,
              void* dk, void* dv, void* dbias, void* workspace, void* stream);

/* Backward stages (bit mask for jattn_bwd_stages). */
#define JATTN_BWD_PREP 1 /* Di = rowsum(dO * O) and LSE * log2(e) into the workspace
                            (softmax, mask NONE or WINDOW) */
#define JATTN_BWD_DKDV 2 /* dK, dV (and dBias) */
#define JATTN_BWD_DQ 4   /* dQ */
#define JATTN_BWD_ALL 7

/* Same as jattn_bwd but runs only the stages in `stages`, on one stream.
 * Softmax plans (mask NONE or WINDOW) keep row statistics in the workspace:
 * DKDV reads Di and LSE * log2 e, which PREP writes.  With bf16 inputs (except
 * D = 128 with fp32 O) the DQ stage forms them itself from O, dO and LSE and
 * writes them too: a call with DQ then skips PREP and runs DQ before DKDV,
 * and DQ alone needs no earlier PREP.  Otherwise (fp32 inputs, or D = 128
 * with fp32 O) DQ and DKDV both read them, and PREP must have completed (in
 * this call or an earlier one on an ordered stream) before either.  DKDV
 * run alone needs an earlier PREP or DQ of the same inputs.  Block mode has
 * a single fused stage, run when DKDV or DQ is requested. */
int jattn_bwd_stages(const jattn_plan* plan, int32_t stages, const void* q, const void* k,
                     const void* v, const void* bias, const void* o, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv, void* dbias, void* workspace,
                     void* stream);

/* Backward with a fixed scratch: the same computation, kernels and results
 * as jattn_bwd (all stages), for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  The row statistics that jattn_bwd keeps in the workspace's
 * scratch region (Di and LSE * log2 e, 2 * align256(4 Tq H) bytes) live
 * instead in a fixed device array of the library, 32 MiB per GPU, held from
 * the first call on that GPU until the process ends; the call itself
 * allocates nothing.  `workspace` must still hold the uploaded plan
 * (jattn_plan_upload), which is only read; its scratch region is not
 * touched.  The array is found on the current device: `stream` must belong
 * to it (JATTN_E_ARG otherwise).  Plans whose row statistics exceed 32 MiB
 * (softmax without the block mask and Tq * H above about 4.19 million rows)
 * are refused with JATTN_E_WORKSPACE before anything is enqueued; GDPA and
 * block-mode plans use no row statistics and have no such limit.  Every call
 * on one GPU shares that GPU's array: two calls whose kernels overlap on
 * the same GPU (on unordered streams) race on it.  Each call overwrites the
 * rows it reads before reading them, so nothing needs clearing between
 * calls. */
int jattn_bwd_fixed_scratch(const jattn_plan* plan, const void* q, const void* k, const void* v,
                            const void* bias, const void* o, const float* lse, const void* dout, void* dq,
                            void* dk, void* dv, void* dbias, void* workspace, void* stream);

void jattn_plan_destroy(jattn_plan* plan);

/* QK-norm ("Training GEM at LLM scale", section "Generalized Dot-Product
 * Attention (GDPA)", item on the ALU-only activation: the polynomial GELU is
 * accurate on the bounded input range that query/key normalisation
 * enforces), read as row-wise L2 normalisation: each of `rows` rows of D
 * contiguous elements (a [T, H, D] tensor has rows = T * H) becomes
 *   y = x * r,   r = 1 / max(||x||_2, 1e-12),
 * so that |q . k| <= 1 for normalised rows.  Forward writes y (y_dtype) and,
 * if rnorm is not NULL, r per row (float32).  Backward, given dy = dL/dy,
 * writes dx = r (dy - y (y . dy)) (the projection term only where
 * ||x|| > 1e-12), recomputing y and r from x.  x, y, dy, dx: device memory,
 * 16-byte aligned; D in {32, 64, 128}; dtypes JATTN_BF16 | JATTN_F32.  y may
 * be x and dx may be dy when the element types match.  Enqueued on `stream`;
 * errors as for the other calls (validated on the host, nothing launched on
 * error; rows = 0 is a no-op). */
int jattn_l2norm_fwd(const void* x, void* y, float* rnorm, int64_t rows, int32_t D, int32_t x_dtype,
                     int32_t y_dtype, void* stream);
int jattn_l2norm_bwd(const void* x, const void* dy, void* dx, int64_t rows, int32_t D, int32_t x_dtype,
                     int32_t dy_dtype, int32_t dx_dtype, void* stream);

/* ---- MXFP8 attention --------------------------------------------------
 * "Training GEM at LLM scale", section "Mixed Ultra-Low-Precision Training",
 * part "Low Precision Flash Attention": the attention products run as MXFP8
 * block-scaled matrix products; every input tensor is quantised once, with
 * one shared power-of-two scale per square 32 x 32 block (so a block and its
 * transpose share it), and the kernel converts P to MXFP8 itself, taking
 * its shared exponent from the row maximum softmax already keeps.
 *
 * A plan with desc.in_dtype = JATTN_MXFP8 (D = 64 or 128, mask NONE, no
 * bias, softmax / erf-GELU / SiLU) runs through the calls below; jattn_fwd
 * and jattn_bwd refuse it.  An MXFP8 tensor of a jagged [T, H, D] bf16
 * tensor (T = Tq for Q, Tk for K and V) is three device arrays:
 *   codes    uint8 [T, H, D]        FP8 E4M3 codes (OCP format), row-major
 *   codes_t  uint8 [RB, H, D, 32]   the same codes per 32-token block,
 *                                   feature-major; tokens past a sample's
 *                                   end are zero
 *   scales   uint8 [RB, H, D / 32]  E8M0 byte X + 127 of each block: the
 *                                   block's values are codes * 2^X
 * RB = sum_b ceil(len_b / 32); blocks never straddle two samples.  X is the
 * smallest integer with amax * 2^-X <= 448 (amax = the block's largest
 * magnitude), so nothing saturates; elements are rounded to nearest, ties to
 * even.  Sizes: jattn_mx_sizes.  The arrays are caller-owned; codes and
 * codes_t 16-byte aligned, scales 4-byte aligned. */
#define JATTN_MX_Q 0  /* rows of the query offsets (Q, dO) */
#define JATTN_MX_KV 1 /* rows of the key/value offsets (K, V) */

typedef struct {
  void* codes;   /* uint8 [T, H, D] */
  void* codes_t; /* uint8 [RB, H, D, 32]; may be NULL where not read */
  void* scales;  /* uint8 [RB, H, D / 32] */
} jattn_mx_tensor;

/* Bytes of the three arrays of an MXFP8 tensor with the query (JATTN_MX_Q)
 * or key/value (JATTN_MX_KV) rows of the plan (the scales size rounded up to
 * a multiple of 4: the kernels read scale bytes as aligned dwords).  Host
 * only. */
int jattn_mx_sizes(const jattn_plan* plan, int32_t rows, int64_t* codes_bytes, int64_t* codes_t_bytes,
                   int64_t* scales_bytes);

/* Quantise a bf16 [T, H, D] tensor (16-byte aligned) into out->codes,
 * out->scales and, when out->codes_t is not NULL, out->codes_t; `workspace`
 * holds the uploaded plan (its block tables).  Enqueued on `stream`. */
int jattn_mx_quantize(const jattn_plan* plan, int32_t rows, const void* x, const jattn_mx_tensor* out,
                      void* workspace, void* stream);

/* MXFP8 forward: reads q->codes, k->codes, v->codes_t and the three scale
 * arrays; writes o (out_dtype, [Tq, H, D]) and, for softmax, lse [Tq, H]
 * (may be NULL).  S = scale Q K^T and O = P V are MXFP8 products with fp32
 * accumulation; P is rounded to E4M3 with one shared exponent per row and
 * 64-key step (from the step's row maximum), or per row and 32-key block of
 * the largest |P| for GDPA; the row sum uses the unrounded P.  Zero-length
 * samples and the tail handling are as for jattn_fwd. */
int jattn_mx_fwd(const jattn_plan* plan, const jattn_mx_tensor* q, const jattn_mx_tensor* k,
                 const jattn_mx_tensor* v, void* o, float* lse, void* workspace, void* stream);

/* MXFP8 backward, the stages in `stages` (JATTN_BWD_* mask, as for
 * jattn_bwd_stages; JATTN_BWD_ALL for the whole backward): given dout as an
 * MXFP8 tensor (JATTN_MX_Q rows) and, for softmax, o and the forward's lse,
 * writes dq, dk, dv (grad_dtype).  Reads
 * q and dout (codes, codes_t, scales), k (codes, codes_t, scales) and v
 * (codes, scales).  Di = rowsum(dout * o) uses the dequantised dout.  The
 * products S, dP, dV = P^T dO, dK = dS^T Q, dQ = dS K are MXFP8 with fp32
 * accumulation; P is rounded to E4M3 with the fixed exponent -8 (P <= 1
 * given the row's LSE; GDPA: one exponent per 32 x 32 block) and dS with one
 * exponent per 32 x 32 block (query block x key block), so the dK and dQ
 * products share its scales.  No atomics: dK/dV and dQ are separate passes.
 * Uses the workspace's scratch region for Di and LSE * log2 e. */
int jattn_mx_bwd(const jattn_plan* plan, int32_t stages, const jattn_mx_tensor* q, const jattn_mx_tensor* k,
                 const jattn_mx_tensor* v, const void* o, const float* lse, const jattn_mx_tensor* dout,
                 void* dq, void* dk, void* dv, void* workspace, void* stream);

/* Static text for a status code. */
const char* jattn_strerror(int status);

/* Detail of the calling thread's most recent failure ("" if none). */
const char* jattn_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* JATTN_H */
