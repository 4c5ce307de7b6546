/*
 * qkvnr — packed-QKV split + per-head RMSNorm + RoPE for MI355X (gfx950).
 *
 * C ABI of the library libqkvnr.so.  Plain pointers and sizes only.
 *
 * What the entry points compute (sources are the three public pages this
 * library is built from):
 *   - torchtitan "[muse_spark][perf] Split the packed qkv inside the q/k
 *     region": Problem items 1-4 and Solution items 1-3 with the before/after
 *     diagram.  The fused projection's packed output is split into q, k and v;
 *     q and k get a per-head RMSNorm with a learned weight and then RoPE (no
 *     rotation on NoPE layers); v is copied; the backward writes one packed
 *     grad directly, with no concatenation of three grads.
 *   - DeepSpeed "[muon] Per-head Newton-Schulz for fused QKV projections",
 *     "What this PR does": the two fused layouts (sectioned and interleaved per
 *     KV group), each a partition of the row into n_q + 2*n_kv head blocks of
 *     head_dim values, and the exact-total guard that declines any other width.
 *   - TensorRT-LLM "MLA DSpark: run each drafter layer's kv path beside its q
 *     path", Description: the latent kv row's RMSNorm/RoPE kernel stores its
 *     result straight into the paged context pool at the block table's
 *     page/offset, bitwise what a staged buffer plus a scatter would write.
 *
 * Definitions (per token t at position p = positions[t]):
 *   RMSNorm of a head x[0..D):  y_d = x_d * w_d / sqrt(mean_d(x_d^2) + eps)
 *   RoPE, rotate-half, R = rotated width, i < R/2, phi_i = p * theta^(-2i/R):
 *     y_i       = x_i cos(phi_i) - x_{i+R/2} sin(phi_i)
 *     y_{i+R/2} = x_{i+R/2} cos(phi_i) + x_i sin(phi_i)
 *   The angle is taken as the real number p * theta^(-2i/R): the kernels form it
 *   in fp64 and reduce it in turns, so large positions (>= 1e5) keep full
 *   accuracy.  Arithmetic is fp32; each output is rounded once (nearest-even).
 *
 * Conventions common to every entry point:
 *   - All pointers are device pointers (HIP device memory), owned by the
 *     caller.  The library never allocates, frees or keeps a pointer after it
 *     returns.  Outputs must not overlap inputs.
 *   - Work is enqueued on `stream` (0 = the default stream); a return value of
 *     QKVNR_OK means "enqueued", not "finished".  Faults inside a kernel
 *     surface at the caller's next synchronisation, as for any HIP launch.
 *   - Every argument is validated on the host before any HIP call is made; a
 *     negative return code means nothing was enqueued.
 *   - Tensors of activations use the layout's dtype (bf16 or fp32), the norm
 *     weights too.  Norm-weight gradients are fp32.  positions are int32.
 *   - Every tensor pointer (except positions, block tables and fp32 weight
 *     gradients, which need 4-byte alignment) must be 16-byte aligned, and the
 *     packed input's row stride in bytes must be a multiple of 16.
 *   - T == 0 is valid: nothing is read or written and every tensor pointer may
 *     be NULL, except that the backward still zeroes the norm-weight
 *     gradients, whose pointers must then be valid.
 *   - Calls on one stream are ordered; calls that overlap on different streams
 *     and write the same memory race, as for any kernel.
 *   - A large batch may be enqueued as several launches of the same kernel
 *     (a dispatch holds fewer than 2^32 work-items); the results do not
 *     depend on it.
 */
#ifndef QKVNR_H
#define QKVNR_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QKVNR_VERSION 10500 /* major * 10000 + minor * 100 + patch */

/* Return codes. */
#define QKVNR_OK 0
#define QKVNR_EINVAL (-1)      /* a null pointer, a bad size, or a width that is not the exact total */
#define QKVNR_EALIGN (-2)      /* a pointer or the input row stride is not aligned as required */
#define QKVNR_EUNSUPPORTED (-3)/* a shape the library has no kernel for, or no gfx950 device current */
#define QKVNR_EHIP (-4)        /* a HIP runtime call or launch failed; qkvnr_strerror has its text */

/* Packed layouts. */
#define QKVNR_INTERLEAVED 0 /* [T, n_kv, q_per_kv + 2, head_dim]: per kv group q..., k, v */
#define QKVNR_SECTIONED 1   /* [T, (n_q + 2 n_kv) * head_dim]: n_q q heads, n_kv k, n_kv v */
#define QKVNR_LATENT 2      /* [T, norm_dim + rope_dim]: one MLA latent row per token */

/* Storage dtypes. */
#define QKVNR_BF16 0
#define QKVNR_FP32 1

/*
 * Layout descriptor of the packed input.
 *
 *   kind          QKVNR_INTERLEAVED, QKVNR_SECTIONED or QKVNR_LATENT.
 *   dtype         QKVNR_BF16 or QKVNR_FP32 (LATENT: BF16 only).
 *   T             tokens (rows); 0 <= T < 2^31.
 *   n_kv          kv heads = kv groups (GQA kinds), >= 1.  Ignored for LATENT.
 *   q_per_kv      q heads per kv group (GQA kinds), >= 1; n_q = n_kv * q_per_kv.
 *                 Ignored for LATENT.
 *   head_dim      D, 64 or 128 (GQA kinds).  Ignored for LATENT.
 *   rope_dim      GQA kinds: 0 (NoPE layer: no rotation, positions unused) or
 *                 head_dim (rotate the whole head).  LATENT: 64, the rotated
 *                 tail of the row.
 *   norm_dim      LATENT only: 512, the normalised head of the row.
 *   width         elements of the packed row.  Must equal exactly
 *                 (n_q + 2 n_kv) * head_dim for the GQA kinds and
 *                 norm_dim + rope_dim for LATENT (the exact-total guard);
 *                 any other width is QKVNR_EINVAL.
 *   in_row_stride elements from one token's packed row to the next, >= width.
 *                 The backward writes dqkv with the same row stride (elements
 *                 of a row beyond `width` are not touched).
 */
typedef struct qkvnr_layout {
  int32_t kind;
  int32_t dtype;
  int64_t T;
  int32_t n_kv;
  int32_t q_per_kv;
  int32_t head_dim;
  int32_t rope_dim;
  int32_t norm_dim;
  int32_t reserved;
  int64_t width;
  int64_t in_row_stride;
} qkvnr_layout;

/*
 * Forward: split, per-head RMSNorm of q and k, RoPE of q and k (unless
 * rope_dim == 0), copy of v, contiguous outputs.
 * (torchtitan page: Problem items 1-3, Solution items 1 and 3, diagram "after".
 *  TensorRT-LLM page: Description, the latent RMSNorm/RoPE before its store.)
 *
 * GQA kinds:
 *   qkv        packed input, `layout` describes it.
 *   positions  [T] int32, 0 <= p < 2^31; may be NULL when rope_dim == 0.
 *   q_norm_w   [head_dim] weight shared by every q head.
 *   k_norm_w   [head_dim] weight shared by every k head.
 *   eps        added to the mean square inside the square root; >= 0, finite.
 *   theta      RoPE base, > 0 and finite when rope_dim > 0.
 *   q          out [T, n_q, head_dim]; q head h = g * q_per_kv + s for slot s of group g.
 *   k, v       out [T, n_kv, head_dim]; v is a bit-exact copy of the v slots.
 * LATENT kind:
 *   q_norm_w, q and v must be NULL; k_norm_w is the [norm_dim] weight;
 *   k is out [T, norm_dim + rope_dim]: [RMSNorm(row[0:norm_dim]) || RoPE(row[norm_dim:])].
 */
int qkvnr_forward(const qkvnr_layout* layout, const void* qkv, const int32_t* positions,
                  const void* q_norm_w, const void* k_norm_w, float eps, double theta,
                  void* q, void* k, void* v, hipStream_t stream);

/*
 * Backward of qkvnr_forward for the GQA kinds: inverse RoPE of the incoming
 * grads, then the RMSNorm backward, written as one packed grad in the input's
 * layout (no concatenation), plus the norm-weight grads.
 * (torchtitan page: Problem item 4, Solution item 3, diagram "after".)
 *
 *   qkv, positions, q_norm_w, k_norm_w, eps, theta: as given to the forward
 *              (the backward recomputes the norm statistics from qkv).
 *   dq         [T, n_q, head_dim], dk and dv [T, n_kv, head_dim]: grads of the outputs.
 *   dqkv       out, packed like qkv (row stride in_row_stride); its v slots are
 *              a bit-exact copy of dv.
 *   dq_norm_w  out [head_dim] fp32, dk_norm_w out [head_dim] fp32: overwritten
 *              with the sums over all tokens and heads.  Block partial sums are
 *              combined with fp32 atomics into 16 workspace slots, so the last
 *              bits may differ from run to run; a second, one-block launch on
 *              `stream` folds the slots into the outputs.
 *   workspace  device scratch of at least qkvnr_backward_workspace_bytes(layout)
 *              bytes, 16-byte aligned, owned by the caller.  It must be all
 *              zero before its first use; every call that completes leaves it
 *              all zero again, so one zero-filled buffer serves any number of
 *              calls in sequence.  Calls that may run at the same time (on
 *              different streams) need different workspaces.  After a call
 *              that returned QKVNR_EHIP (a launch failed once kernels were
 *              enqueued; the library still enqueues the fold that zeroes the
 *              slots, but that launch may have failed too) or did not complete
 *              (a device fault), zero it again.  It may be NULL when T == 0.
 * LATENT is QKVNR_EUNSUPPORTED.
 */
int qkvnr_backward(const qkvnr_layout* layout, const void* qkv, const int32_t* positions,
                   const void* q_norm_w, const void* k_norm_w, float eps, double theta,
                   const void* dq, const void* dk, const void* dv, void* dqkv,
                   float* dq_norm_w, float* dk_norm_w, void* workspace, int64_t workspace_bytes,
                   hipStream_t stream);

/* Bytes of workspace qkvnr_backward needs for `layout` (at most
 * QKVNR_BACKWARD_WORKSPACE_MAX for any supported layout). */
int64_t qkvnr_backward_workspace_bytes(const qkvnr_layout* layout);
#define QKVNR_BACKWARD_WORKSPACE_MAX 16384

/*
 * qkvnr_backward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops that may
 * not call hipMalloc, harnesses that forbid allocation.  Same arguments (less
 * workspace and workspace_bytes), arithmetic, results and errors as
 * qkvnr_backward.  The weight-grad partial-sum slots live in a static device
 * array inside the library, QKVNR_NOALLOC_SCRATCH_BYTES bytes, one copy per GPU,
 * held until the process ends.  No hipMalloc, hipFree or allocating call is
 * made.
 *   - The first call on a device looks the array up (hipGetSymbolAddress) and
 *     enqueues, on `stream`, a small kernel that zeroes it.  Every completed
 *     call leaves it zero; a call whose fold failed to launch (QKVNR_EHIP)
 *     makes the next call on that device zero it again first.
 *   - Every call on one GPU shares that GPU's array: calls that may overlap in
 *     time on one GPU (different streams, no ordering between them) race, and
 *     their weight grads are wrong.  Order such calls, or give each stream
 *     its own workspace through qkvnr_backward.
 *   - A layout whose slots (qkvnr_backward_workspace_bytes) exceed the array
 *     is QKVNR_EINVAL; every supported head_dim fits.
 */
int qkvnr_backward_noalloc(const qkvnr_layout* layout, const void* qkv, const int32_t* positions,
                           const void* q_norm_w, const void* k_norm_w, float eps, double theta,
                           const void* dq, const void* dk, const void* dv, void* dqkv,
                           float* dq_norm_w, float* dk_norm_w, hipStream_t stream);
#define QKVNR_NOALLOC_SCRATCH_BYTES 16384

/*
 * Forward that stores k and v (GQA kinds) or the latent row (LATENT) straight
 * into a paged pool at the block table's page/offset, instead of a contiguous
 * buffer that is scattered afterwards.  Same arithmetic as qkvnr_forward, only
 * the store index differs, so the pool rows are bitwise what qkvnr_forward
 * followed by a scatter would write.
 * (TensorRT-LLM page: Description, the direct pool write; Test Coverage, the
 *  bitwise comparison with the staged write.)
 *
 *   block_table    [ceil(T / tokens_per_req), bt_stride] int32 page ids.
 *   tokens_per_req tokens per request: token t belongs to request t / tokens_per_req.
 *   page_size      rows per page, P >= 1.
 *   num_pages      pages in the pool.
 *   Token t at position p goes to page block_table[b][p / P], row p % P of it.
 *   A token whose p / P >= bt_stride, or whose page id is outside
 *   [0, num_pages), is not stored (its pool rows are left as they were); the
 *   caller should treat that as an error in its own table.
 * GQA kinds:
 *   q       out [T, n_q, head_dim], contiguous as in qkvnr_forward.
 *   k_pool  [num_pages, page_size, n_kv, head_dim]; v_pool likewise.
 * LATENT kind:
 *   q_norm_w, q and v_pool must be NULL; k_norm_w is the [norm_dim] weight;
 *   k_pool is [num_pages, page_size, norm_dim + rope_dim].
 */
int qkvnr_forward_paged(const qkvnr_layout* layout, const void* qkv, const int32_t* positions,
                        const void* q_norm_w, const void* k_norm_w, float eps, double theta,
                        const int32_t* block_table, int32_t bt_stride, int32_t tokens_per_req,
                        int32_t page_size, int32_t num_pages, void* q, void* k_pool,
                        void* v_pool, hipStream_t stream);

/*
 * Rotate-half RoPE, in place, of the rope part of every head of x: the q
 * path's rotation of its heads' rope parts in the MLA drafter layer, which
 * runs beside the latent kv path (TensorRT-LLM page: Description, the q path
 * "q_a_proj -> q_a_layernorm -> q_b_proj -> rope_into -> k absorption").  No
 * norm.  Same rotation and angle handling as qkvnr_forward: pairs
 * (i, i + R/2) of the R = rope_dim values at rope_offset turn by
 * pos * theta^(-2i/R), formed in fp64 and reduced in turns; one rounding.
 *
 *   dtype        QKVNR_BF16 (QKVNR_FP32 is QKVNR_EUNSUPPORTED).
 *   T            tokens, >= 0 (T == 0 is a no-op; x and positions may be NULL).
 *   heads        heads per token, >= 1.
 *   token_stride elements from one token to the next (>= heads * head_stride).
 *   head_stride  elements from one head to the next within a token.
 *   rope_offset  first rotated element within a head; rope_offset + rope_dim
 *                <= head_stride.  rope_offset, head_stride and token_stride
 *                must be multiples of 8 elements (QKVNR_EALIGN otherwise).
 *   rope_dim     64 or 128 (others QKVNR_EUNSUPPORTED).
 *   positions    [T] int32, 4-byte aligned.
 *   x            in/out, 16-byte aligned; only the rope parts are read and
 *                written.  Must not overlap positions.
 */
int qkvnr_rope_inplace(int32_t dtype, int64_t T, int32_t heads, int64_t token_stride,
                       int32_t head_stride, int32_t rope_offset, int32_t rope_dim,
                       const int32_t* positions, double theta, void* x, hipStream_t stream);

/*
 * Per-head Newton-Schulz on fused QKV weights (DeepSpeed page "[muon]
 * Per-head Newton-Schulz for fused QKV projections", "What this PR does" and
 * "Not in this PR").
 *
 * qkvnr_fused_head_blocks: the exact-total guard.  A fused q|k|v weight is
 * split into head blocks of head_dim rows only when its row count is exactly
 * (n_q + 2 n_kv) * head_dim; then *blocks = n_q + 2 n_kv (12 for 8 query heads
 * over 2 kv heads) and QKVNR_OK.  Any other row count (a transposed Conv1D
 * weight, a config whose fused total does not describe the weight) is
 * QKVNR_EINVAL with *blocks = 0: such a weight stays on the full-matrix path.
 * The guard is the same for the sectioned and the interleaved order, whose
 * blocks differ only in order.  Host only: no HIP call.
 */
int qkvnr_fused_head_blocks(int32_t n_q, int32_t n_kv, int32_t head_dim, int64_t weight_rows,
                            int64_t* blocks);

/*
 * Gram matrices X X^T of bf16 blocks, as partial sums over column slices:
 * the first product of each Newton-Schulz step (and G G^T for the first).
 * Both factors are rows of X, read along the long side; v_mfma_f32_32x32x16_bf16.
 *
 *   blocks  number of blocks, 0 .. 2^22 (0 is a no-op).
 *   d       block side (rows of each block): 32, 64, 96 or 128 (others
 *           QKVNR_EUNSUPPORTED).
 *   cols    block width, a positive multiple of 8 (QKVNR_EALIGN otherwise), at
 *           most 2^30 (QKVNR_EINVAL otherwise).
 *   x       [blocks, d, cols] bf16, row-major, 16-byte aligned.
 *   parts   column slices, 1..65535: slice p covers columns
 *           [p * S, min(cols, (p + 1) * S)), S = ceil(ceil(cols / parts) / 16) * 16.
 *   out     [blocks, parts, d, d] fp32, 4-byte aligned, must not overlap x;
 *           out[b][p] is block b's Gram matrix over slice p (zero for an empty slice).
 */
int qkvnr_gram_partials(int64_t blocks, int32_t d, int64_t cols, const void* x, int32_t parts,
                        float* out, hipStream_t stream);

/*
 * One Newton-Schulz step's polynomial for every block: from A (the Gram matrix
 * X X^T of the block's wide orientation, d x d, given as `parts` partial sums
 * that are added), P = a I + b A + c A A with Muon's quintic coefficients
 * (a, b, c) = (3.4445, -4.7750, 2.0315); the step itself is X <- P X.  With
 * first != 0, A is G G^T of the unnormalised block: it is divided by
 * (||G||_F + eps)^2 (the norm is the square root of its trace) and P by
 * (||G||_F + eps), so that P G is the first step from G / (||G||_F + eps).  P is
 * multiplied by `scale` (pass the block scale max(1, rows/cols)**0.5 on the
 * last step, 1 otherwise).  The update P X is qkvnr_ns_update (or any batched
 * GEMM).
 *
 *   dtype   QKVNR_BF16 or QKVNR_FP32: the type of p.
 *   blocks  number of blocks, 0 .. 2^22 (0 is a no-op).
 *   d       block side, 1..128 (others QKVNR_EUNSUPPORTED).
 *   gram    [blocks, parts, d, d] fp32, row-major, 16-byte aligned; read
 *           only (the partials are added in order as they are loaded).
 *   parts   >= 1.
 *   p       out [blocks, d, d] in dtype, row-major; must not overlap gram.
 */
int qkvnr_ns_poly(int32_t dtype, int64_t blocks, int32_t d, float* gram, int32_t parts,
                  int32_t first, float scale, float eps, void* p, hipStream_t stream);

/*
 * One Newton-Schulz update of bf16 blocks, Y = P X per block (fp32 products,
 * rounded once to bf16), and optionally the partial Gram matrices Y Y^T that
 * the next step's qkvnr_ns_poly needs, taken from the same pass: Y is written
 * once and not read back.  (DeepSpeed page, "What this PR does": each head
 * block is orthogonalised on its own; every step is X <- P X.)
 *
 *   blocks  number of blocks, 0 .. 2^22 (0 is a no-op).
 *   d       block side: 64 or 128 (others QKVNR_EUNSUPPORTED).
 *   cols    block width, a positive multiple of 8 (QKVNR_EALIGN otherwise), at
 *           most 2^30 (QKVNR_EINVAL otherwise).
 *   p       [blocks, d, d] bf16, row-major, 16-byte aligned (qkvnr_ns_poly's
 *           bf16 output).
 *   x       [blocks, d, cols] bf16, row-major, 16-byte aligned.
 *   y       out [blocks, d, cols] bf16, 16-byte aligned; must not overlap x or p.
 *   parts   column slices, 1..65535, as for qkvnr_gram_partials.
 *   gram    NULL, or out [blocks, parts, d, d] fp32, 4-byte aligned, must not
 *           overlap p, x or y: what qkvnr_gram_partials(blocks, d, cols, y,
 *           parts, gram) would write, up to the order of the fp32 sums.
 */
int qkvnr_ns_update(int64_t blocks, int32_t d, int64_t cols, const void* p, const void* x, void* y,
                    int32_t parts, float* gram, hipStream_t stream);

/*
 * The whole Newton-Schulz iteration of every block as one d x d matrix M, so
 * that the result is M G (qkvnr_ns_apply): two passes over the blocks instead
 * of two a step.  (DeepSpeed page, "What this PR does": each head block is
 * orthogonalised on its own by Muon's quintic Newton-Schulz steps.)  Each step
 * multiplies X by P = a I + b X X^T + c (X X^T)^2 with (a, b, c) = (3.4445,
 * -4.7750, 2.0315), a polynomial in G G^T, so from A'_0 = G G^T / (||G||_F +
 * eps)^2:  P_k = a I + b A'_k + c A'_k A'_k,  A'_{k+1} = P_k A'_k P_k,
 * M_{k+1} = P_k M_k,  and M = M_steps * scale / (||G||_F + eps): in exact
 * arithmetic the same M G as `steps` calls of qkvnr_ns_poly and an update.
 * Every product is taken from operands split into two bf16 terms (hi + lo,
 * within 2^-16 of the value) with fp32 accumulation, and M is written as the
 * same two terms: M's entries grow with the block's condition while M G stays
 * near orthogonal, so M needs more than bf16's 8 bits.
 *
 *   blocks  number of blocks, 0 .. 2^22 (0 is a no-op).
 *   d       block side: 64 or 128 (others QKVNR_EUNSUPPORTED).
 *   gram    [blocks, parts, d, d] fp32, 16-byte aligned: G G^T as partial sums
 *           (qkvnr_gram_partials), added in order; read only.
 *   parts   1..65535.
 *   steps   Newton-Schulz steps, 1..64.
 *   scale   > 0 and finite: the block scale max(1, rows/cols)**0.5.
 *   eps     >= 0 and finite.
 *   m       out [blocks, 2, d, d] bf16, 16-byte aligned: hi terms, then lo
 *           terms, of each block's M; must not overlap gram.
 */
int qkvnr_ns_collapse(int64_t blocks, int32_t d, const float* gram, int32_t parts, int32_t steps, float scale,
                      float eps, void* m, hipStream_t stream);

/*
 * Y = M X for bf16 blocks with M given as two bf16 terms (qkvnr_ns_collapse's
 * output): both products are added in fp32 before Y's one rounding to bf16.
 *
 *   blocks, d, cols, parts: as for qkvnr_ns_update (d 64 or 128).
 *   m       [blocks, 2, d, d] bf16, 16-byte aligned.
 *   x       [blocks, d, cols] bf16, 16-byte aligned.
 *   y       out [blocks, d, cols] bf16, 16-byte aligned; must not overlap x or m
 *           (QKVNR_EINVAL).
 */
int qkvnr_ns_apply(int64_t blocks, int32_t d, int64_t cols, const void* m, const void* x, void* y, int32_t parts,
                   hipStream_t stream);

/*
 * The QKV projection with the forward region fused into its epilogue.
 * (torchtitan page: Problem item 1, the region's input is the packed output of
 *  the attention's QKV projection; Results, the region is timed with the GEMMs
 *  left out.)
 * packed = x w_qkv^T is formed in fp32 and never stored or rounded; each of its
 * head blocks is split out as qkvnr_forward splits the packed input, q and k
 * get qkvnr_forward's per-head RMSNorm and RoPE, v is rounded once, and q, k, v
 * are written as qkvnr_forward writes them.
 *
 *   layout     kind QKVNR_INTERLEAVED or QKVNR_SECTIONED (others
 *              QKVNR_EUNSUPPORTED), dtype QKVNR_BF16 (QKVNR_FP32 is
 *              QKVNR_EUNSUPPORTED), T, n_kv, q_per_kv, head_dim, rope_dim and
 *              width as for qkvnr_forward; in_row_stride is not used (there is
 *              no packed tensor) but must pass the same check (>= width).
 *   hidden     columns of x and w_qkv: a positive multiple of 64, at most 2^30
 *              (QKVNR_EINVAL otherwise).
 *   x          [T, hidden] bf16, row-major, 16-byte aligned.
 *   w_qkv      [width, hidden] bf16, row-major, 16-byte aligned: row j is packed
 *              column j, so its head blocks follow the layout's order.
 *   positions, q_norm_w, k_norm_w, eps, theta, q, k, v: as for qkvnr_forward
 *              (v is x w_v^T rounded once, not a copy).
 * Outputs must not overlap any input (QKVNR_EINVAL).  T == 0 enqueues nothing.
 */
int qkvnr_proj_forward(const qkvnr_layout* layout, int64_t hidden, const void* x, const void* w_qkv,
                       const int32_t* positions, const void* q_norm_w, const void* k_norm_w, float eps,
                       double theta, void* q, void* k, void* v, hipStream_t stream);

/* Static text for a return code.  For QKVNR_EHIP and the validation errors it
 * returns the last detailed message recorded on the calling thread. */
const char* qkvnr_strerror(int code);

/* QKVNR_VERSION of the built library. */
int qkvnr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QKVNR_H */
