/*
 * salad.h - C interface of the hybrid block-sparse + ReLU-linear attention
 * operator for AMD Instinct MI355X (gfx950).
 *
 * The operator (SALAD, "High-Sparsity Attention paralleling with Linear
 * Attention for Diffusion Transformer"): a sparse softmax-attention branch over
 * the key blocks a block mask keeps, and beside it a ReLU linear-attention
 * branch over all tokens that shares Q, K and V; the linear output passes a
 * projection and a scalar gate in (0,1) and is added to the sparse output.
 * Sources: the "SALAD" explainer on gist.science, technical summary sections
 * 2.1 (two parallel branches, shared Q/K/V, ReLU linear attention), 2.2
 * (zero-initialised projection, sigmoid-bounded scale s), 2.3 (dropping
 * low-scale branches at inference) and 5 (sliding-window and Top-K masks); the
 * sciencestack "SALAD" page, TL;DR and abstract (90% sparsity, input-dependent
 * scalar gate) and Figure 1 (spatio-temporal sliding window, ST-SWA).
 *
 * Conventions shared by every entry point:
 *  - Tensors q, k, v, out are [batch, heads, n_pad, head_dim], contiguous,
 *    head_dim innermost, in the shape's dtype (fp32 or bf16), with the tokens
 *    in the shape's storage order (see salad_shape): frame-major by default,
 *    slot n holding the token t = n / (H*W), y = (n / W) % H, x = n % W.
 *    Slots N = T*H*W .. n_pad-1 are padding: their contents are never read
 *    into a result (any bit pattern is allowed) and output rows there are
 *    written as 0.
 *  - A block mask is CSR over rows r = (b*heads + h)*nb + qb, nb = n_pad/block:
 *    row_ptr int32 [batch*heads*nb + 1], col_idx int32, key blocks ascending
 *    within a row.
 *  - Every pointer argument except the shape and spec structs is DEVICE memory
 *    owned by the caller; the library allocates nothing, keeps no pointer after
 *    it returns, and holds no global mutable state (thread-safe).
 *  - `stream` is a hipStream_t (NULL = the null stream).  All device work is
 *    enqueued on it; no call synchronises.  Calls sharing one workspace must be
 *    ordered on one stream.
 *  - Arguments are validated before any launch; on error nothing is enqueued
 *    and a negative salad_status is returned.  A failed launch returns
 *    SALAD_EHIP.  The library never prints or aborts.
 *  - Device pointers must be 16-byte aligned.
 */
#ifndef SALAD_H
#define SALAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SALAD_VERSION 100 /* 1.0.0 */

#if defined(__GNUC__)
#define SALAD_API __attribute__((visibility("default")))
#else
#define SALAD_API
#endif
#define SALAD_MAX_HEADS 128

typedef enum {
  SALAD_OK = 0,
  SALAD_EINVAL = -1,        /* bad argument (null pointer, inconsistent shape) */
  SALAD_EUNSUPPORTED = -2,  /* valid but not built: head_dim not 64/128, block not 64/128, heads > 128 */
  SALAD_ENOSPACE = -3,      /* workspace or col_idx capacity too small */
  SALAD_EINFEASIBLE = -4,   /* a window head asks for more block pairs than it has candidates */
  SALAD_EHIP = -5           /* a HIP launch failed */
} salad_status;

typedef enum { SALAD_F32 = 0, SALAD_BF16 = 1 } salad_dtype;

typedef enum { SALAD_MASK_WINDOW = 0, SALAD_MASK_TOPK = 1, SALAD_MASK_SICS = 2 } salad_mask_kind;

/* Layer shape.  Requirements: batch, heads >= 1; heads <= SALAD_MAX_HEADS;
 * head_dim in {64, 128}; T, H, W >= 1; block in {64, 128};
 * n_pad == ceil(T*H*W / block) * block (so every block holds a valid token).
 *
 * Storage order of the tokens.  cuboid_t = cuboid_h = cuboid_w = 0: frame-major,
 * block j = the frame-major run [j*block, (j+1)*block).  Otherwise 3-D cuboid
 * blocks (SPADE explainer, blueprint part "Der Bauplan (vDiT-SSR)": the video's
 * block grid cut into flat, tall or mixed shapes), with cuboid_t * cuboid_h *
 * cuboid_w == block, all >= 1.  The cuboid grid has ceil(T/cuboid_t) x
 * ceil(H/cuboid_h) x ceil(W/cuboid_w) cells; a cell is full when it lies inside
 * the grid, partial when it meets a far edge that its extent does not divide.
 * Slots hold every full cell in lexicographic (t, y, x) cell order, one block
 * each, then every partial cell in lexicographic order packed into the last
 * blocks; tokens inside a cell frame-major.  salad_token_order lists the order
 * and salad_permute_tokens moves tensors into and out of it.  The window mask
 * measures distances on the stored blocks' token sets; top-k, SICS, the gate
 * and both attention branches take the blocks as stored. */
typedef struct {
  int32_t batch, heads, head_dim;
  int32_t T, H, W;
  int32_t n_pad, block;
  int32_t dtype; /* salad_dtype */
  int32_t cuboid_t, cuboid_h, cuboid_w; /* 0, 0, 0 = frame-major */
} salad_shape;

/* Mask request for one head (host struct, one per head).
 *
 * SALAD_MASK_WINDOW - static spatio-temporal sliding window ("SALAD" explainer,
 *   section 5; sciencestack Figure 1, ST-SWA).  r*(qb, kb) is the least
 *   Chebyshev spatial distance max(|dy|, |dx|) over token pairs of the two
 *   blocks at most t_window frames apart (infinite if none).  Candidates have
 *   finite r* and, when r_max >= 0, r* <= r_max.  density <= 0 keeps every
 *   candidate; otherwise candidates are ranked by (qb != kb, r*, |qb - kb|, qb,
 *   kb) and the first K = floor(density * nb * nb + 0.5) are kept (the diagonal
 *   ranks first).  Identical for every batch index.
 * SALAD_MASK_TOPK - dynamic Top-K over pooled block scores ("SALAD" explainer,
 *   section 5).  pq, pk = float32 block means of Q and K over valid tokens
 *   (sequential float32 sum in token order, then one division); score(qb, kb) =
 *   sequential float32 sum over channels of separately rounded products
 *   pq[c]*pk[c]; each query block keeps the k = max(1, floor(density*nb + 0.5))
 *   highest (capped at nb), ties to the lower kb.  t_window, r_max unused.
 * SALAD_MASK_SICS - key blocks scored by the sum of intra-block cosine
 *   similarities ("SPADE" explainer, scheme generation, "Der sofortige
 *   Entscheidungsträger"): SICS(kb) = sum over valid token pairs i, j of kb of
 *   cos(k_i, k_j) = || sum_i k_i / |k_i| ||^2 in a fixed float32 order (|k|^2
 *   sequential over channels; zero vectors contribute nothing; correctly
 *   rounded sqrt and division; block sum sequential over tokens; squared norm
 *   sequential over channels; no fused multiply-add).  Per (b, h) the m =
 *   max(1, floor(density*nb + 0.5)) highest blocks (ties to the lower kb) are
 *   kept for every query block, plus each query block's own block: m or m + 1
 *   per row.  t_window, r_max unused. */
typedef struct {
  int32_t kind;     /* salad_mask_kind */
  int32_t t_window; /* window: +- frames */
  int32_t r_max;    /* window: spatial cap, -1 = none */
  float density;    /* fraction of block pairs kept */
} salad_mask_spec;

/* Version number (SALAD_VERSION of the built library). */
SALAD_API int salad_version(void);

/* Static description of a status code; never NULL. */
SALAD_API const char* salad_status_str(int status);

/* Number of col_idx entries salad_build_mask writes for this shape and these
 * specs (pure host function, no device work).  Exact for window heads (K when
 * density > 0, else the number of candidate pairs) and top-k heads (k * nb per
 * (b, h)); for SICS heads it is the upper bound (m + 1) * nb per (b, h), since
 * whether the diagonal block is among a head's m chosen blocks depends on K.
 * Negative salad_status on invalid arguments, and SALAD_EINFEASIBLE when a
 * window head with density > 0 asks for K block pairs but has fewer candidate
 * pairs (the "SALAD" explainer, section 5, names static sliding-window masks;
 * the window rule is given with salad_mask_spec).  The candidate count depends
 * on the shape and the spec only; it takes O(nb log nb) host time without a
 * spatial cap (r_max < 0) in frame-major order, otherwise time proportional to
 * nb times the blocks of the frames a block's window spans. */
SALAD_API int64_t salad_mask_nnz(const salad_shape* shape, const salad_mask_spec* specs);

/* Device workspace, in bytes, that salad_build_mask, salad_gate_from_q,
 * salad_linear_state, salad_attn_fwd and salad_attn_fwd_branches need for this
 * shape (one buffer serves all of them).  Pure host function; 0 on invalid
 * shape. */
SALAD_API size_t salad_workspace_bytes(const salad_shape* shape);

/* Build the CSR block mask for every (b, h) from the per-head specs.
 * Validation (before any launch) includes the window feasibility of
 * salad_mask_nnz: SALAD_EINFEASIBLE when a window head asks for more pairs
 * than it has candidates, SALAD_EUNSUPPORTED when the mask would hold more
 * than INT32_MAX entries (row_ptr is int32).
 *   specs    host array [heads]
 *   q, k     device tensors; q is read when some head is SALAD_MASK_TOPK or a
 *            gate is requested, k when some head is SALAD_MASK_TOPK or
 *            SALAD_MASK_SICS (either may be NULL when not read)
 *   row_ptr  device int32 [batch*heads*nb + 1], written
 *   col_idx  device int32 [col_cap], written in [0, row_ptr[last])
 *   col_cap  must be >= salad_mask_nnz(shape, specs), else SALAD_ENOSPACE
 *   w_g, gate  optional (both NULL, or both device pointers): also compute
 *            the gate of salad_gate_from_q from the same pass over Q that pools
 *            the query blocks, saving a second read of Q
 *   ws       device workspace of ws_bytes >= salad_workspace_bytes(shape)
 * The static window part depends only on the shape and specs and may be cached
 * by the caller. */
SALAD_API int salad_build_mask(const salad_shape* shape, const salad_mask_spec* specs,
                     const void* q, const void* k,
                     int32_t* row_ptr, int32_t* col_idx, int64_t col_cap,
                     const float* w_g, float* gate,
                     void* ws, size_t ws_bytes, void* stream);

/* Bits of the result of salad_check_mask. */
#define SALAD_MASK_BAD_START 1   /* row_ptr[0] != 0 */
#define SALAD_MASK_BAD_ROW_PTR 2 /* row_ptr decreases, is negative, or passes col_cap */
#define SALAD_MASK_BAD_COL 4     /* a col_idx entry outside [0, nb) */
#define SALAD_MASK_BAD_ORDER 8   /* a row's key blocks not strictly ascending */

/* Check a CSR block mask against what salad_attn_fwd, salad_attn_apply,
 * salad_attn_fwd_branches and salad_attn_bwd assume of it (they index the key
 * and value tensors with col_idx unchecked and walk each row in order):
 * row_ptr[0] == 0, row_ptr non-decreasing with row_ptr[rows] <= col_cap,
 * every entry in [0, nb), each row strictly ascending.  Masks made by
 * salad_build_mask always pass; a caller that builds its own (a hand-made or
 * learned block mask in place of the window or Top-K rules of the "SALAD"
 * explainer, section 5) can check it first.
 *   row_ptr  device int32 [batch*heads*nb + 1]
 *   col_idx  device int32 [col_cap]: col_cap is the number of elements the
 *            allocation holds; the check reads no entry at or beyond it, nor
 *            the entries of a row whose row_ptr bounds are bad
 *   result   device int32 [1], written: 0 for a valid mask, else the OR of
 *            the SALAD_MASK_BAD_* bits found
 * One small kernel on `stream`; no workspace. */
SALAD_API int salad_check_mask(const salad_shape* shape, const int32_t* row_ptr, const int32_t* col_idx,
                               int64_t col_cap, int32_t* result, void* stream);

/* Storage order of the shape's tokens: order[p] = frame-major index
 * t*H*W + y*W + x of the token stored at slot p, for p < N, and order[p] = p
 * for the padding slots p in [N, n_pad).  order: HOST int32 [n_pad].  Pure
 * host function (the identity for frame-major shapes). */
SALAD_API int salad_token_order(const salad_shape* shape, int32_t* order);

/* Move the token axis of a [batch, heads, n_pad, head_dim] tensor of the
 * shape's dtype between frame-major order and the shape's storage order
 * (order as listed by salad_token_order):
 *   inverse = 0: dst[b, h, p, :] = src[b, h, order[p], :]  (into storage order)
 *   inverse = 1: dst[b, h, order[p], :] = src[b, h, p, :]  (back to frame-major)
 * Padding slots are copied unchanged.  src, dst: device, 16-byte aligned, not
 * overlapping (SALAD_EINVAL otherwise).  A plain copy for frame-major shapes.
 * Needs no workspace. */
SALAD_API int salad_permute_tokens(const salad_shape* shape, int inverse, const void* src,
                                   void* dst, void* stream);

/* Gate from Q: gate[b*heads + h] = sigmoid(mean over the N valid tokens of
 * q[b, h, n, :] . w_g), the stand-in used here for the input-aware scale s of
 * the "SALAD" explainer, section 2.2.  w_g: device float [head_dim];
 * gate: device float [batch*heads]. */
SALAD_API int salad_gate_from_q(const salad_shape* shape, const void* q, const float* w_g,
                      float* gate, void* ws, size_t ws_bytes, void* stream);

/* Linear-attention state ("SALAD" explainer, section 2.1: ReLU linear
 * attention, O(N)): S[b,h] = sum over valid tokens n of ReLU(k_n) v_n^T
 * (head_dim x head_dim, row index over k's channel) and z[b,h] = sum over
 * valid n of ReLU(k_n), accumulated in fp32 in a fixed order (bitwise
 * reproducible run to run).  S: device float [batch*heads*head_dim*head_dim];
 * z: device float [batch*heads*head_dim]. */
SALAD_API int salad_linear_state(const salad_shape* shape, const void* k, const void* v,
                       float* S, float* z, void* ws, size_t ws_bytes, void* stream);

/* The fused layer forward:
 *   out[i] = o_s[i] + gate[b,h] * (o_l[i] . w_lin)        for tokens i < N
 *   out[i] = 0                                             for N <= i < n_pad
 * o_s: softmax attention of query i over the keys (< N) of the key blocks its
 *   query block keeps in (row_ptr, col_idx), logits scale*<q_i,k_j>; a row
 *   keeping no block gives 0.
 * Precondition on the mask (here and in salad_attn_apply,
 *   salad_attn_fwd_branches and salad_attn_bwd): it is a valid CSR as
 *   salad_check_mask defines it.  Entries are used as key-block indices
 *   without a check, so an entry >= nb reads outside k and v; masks from
 *   salad_build_mask always hold, others can be checked with salad_check_mask.
 * o_l: ReLU(q_i)^T S / (ReLU(q_i)^T z + eps) with S, z as salad_linear_state.
 * Equal inputs give bitwise equal outputs.  For bf16 shapes with 64-token
 *   blocks the kernel walks each head's kept lists in one of two orders,
 *   chosen on the device from how much neighbouring query blocks' lists
 *   overlap (a function of the mask alone); the choice changes only the
 *   order of floating-point sums.
 *   gate   device float [batch*heads], values in (0,1) by the method's design
 *          (any finite value is accepted)
 *   w_lin  device [head_dim*head_dim] in the shape's dtype, row-major, applied
 *          on the right (o_l . w_lin), shared by all heads
 *   eps    > 0 keeps the ReLU normaliser finite
 *   scale  softmax scale; <= 0 selects 1/sqrt(head_dim)
 *   drop_tau  branch dropping ("SALAD" explainer, section 2.3): heads whose
 *          gate < drop_tau skip the linear branch entirely: no linear state
 *          is computed for them and out = o_s; pass 0 to keep every branch
 *   out    device, shape of q
 *   lse    NULL, or device float [batch*heads*n_pad] (bf16 shapes only, else
 *          SALAD_EUNSUPPORTED): receives each row's log2-sum-exp of its scaled
 *          scores, m + log2(sum_j 2^(x_j - m)) with x_j = scale*<q_i,k_j>*log2(e)
 *          over the kept keys (+inf for padding rows and rows that keep no
 *          key), for salad_attn_bwd */
SALAD_API int salad_attn_fwd(const salad_shape* shape, const void* q, const void* k, const void* v,
                   const int32_t* row_ptr, const int32_t* col_idx,
                   const float* gate, const void* w_lin, float eps, float scale,
                   float drop_tau, void* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/* salad_attn_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same launches and the same results, with the workspace taken from a
 * static device array inside the library (32 MiB on each GPU that loads the
 * library, held until the process ends) instead of a caller buffer.  The
 * call itself allocates nothing.  Only the linear-state part of the
 * workspace layout is used; SALAD_ENOSPACE when it exceeds 32 MiB (at
 * head_dim 128 about batch*heads > 240).  Every call on one GPU shares that
 * GPU's array: calls that overlap in time on one GPU (two streams, two host
 * threads without ordering) race and give wrong results; calls ordered on one
 * stream are safe.  Nothing in the array needs to start at zero.  The first
 * call on each device looks up the array's address (hipGetSymbolAddress) with
 * that device current; `stream` must belong to the current device. */
SALAD_API int salad_attn_fwd_noalloc(const salad_shape* shape, const void* q, const void* k, const void* v,
                                     const int32_t* row_ptr, const int32_t* col_idx, const float* gate,
                                     const void* w_lin, float eps, float scale, float drop_tau, void* out,
                                     float* lse, void* stream);

/* salad_attn_fwd in two calls, for callers that reuse the linear state or
 * time the steps apart.  salad_linear_prepare computes S and z (as
 * salad_linear_state) and keeps, in the workspace, the state with gate and
 * projection folded in: S'' = gate[b,h] * S . w_lin.  salad_attn_apply then
 * runs the sparse branch and the linear epilogue in one kernel, reading that
 * folded state: its gate argument serves branch dropping only and must be the
 * gate given to salad_linear_prepare.  Branch dropping ("SALAD" explainer,
 * section 2.3) starts here: salad_linear_prepare computes no state for heads
 * with gate < drop_tau (their workspace slots are left as they were), so
 * salad_attn_apply must get a drop_tau at least as large.  Between the two
 * calls the workspace must not be used by another call.  salad_attn_fwd ==
 * prepare + apply with the same drop_tau. */
SALAD_API int salad_linear_prepare(const salad_shape* shape, const void* k, const void* v,
                                   const float* gate, const void* w_lin, float drop_tau, void* ws,
                                   size_t ws_bytes, void* stream);
SALAD_API int salad_attn_apply(const salad_shape* shape, const void* q, const void* k,
                               const void* v, const int32_t* row_ptr, const int32_t* col_idx,
                               const float* gate, float eps, float scale, float drop_tau,
                               void* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/* The two branches separately, for parity checks: out_sparse = o_s and
 * out_lin = o_l (before projection and gate), both shaped like q, rows >= N
 * zero.  Either output pointer may be NULL to skip that branch. */
SALAD_API int salad_attn_fwd_branches(const salad_shape* shape, const void* q, const void* k,
                            const void* v, const int32_t* row_ptr, const int32_t* col_idx,
                            float eps, float scale, void* out_sparse, void* out_lin,
                            void* ws, size_t ws_bytes, void* stream);

/* ---- backward (for fine-tuning) ------------------------------------------
 * The layer is trained, not only run: the "SALAD" explainer's technical
 * summary, section 2.2, makes the projection on the linear branch a learnable
 * layer initialised at zero and the scale s the output of a small learned
 * module, and section 3 reports the fine-tuning budget.  salad_attn_bwd gives
 * the gradients of a loss L through out = o_s + g * (o_l W_lin) from dout =
 * dL/dout. */

/* Device workspace, in bytes, that salad_attn_bwd needs for this shape (it
 * includes salad_workspace_bytes).  Pure host function; 0 on invalid shape. */
SALAD_API size_t salad_bwd_workspace_bytes(const salad_shape* shape);

/* Gradients of the fused forward (salad_attn_fwd without branch dropping) for
 * bf16 shapes:
 *   q, k, v, out, dout  device bf16 [batch, heads, n_pad, head_dim]: the
 *                       forward's inputs, its output, and dL/dout (rows from N
 *                       on are not read)
 *   lse                 the forward's lse output (16-byte aligned), or NULL:
 *                       then the kernel recomputes it (one more pass of Q K^T
 *                       over the kept blocks)
 *   row_ptr, col_idx    the CSR mask the forward used
 *   gate                device float [batch*heads]; w_lin device bf16
 *                       [head_dim, head_dim]; eps, scale as in salad_attn_fwd
 *   dq, dk, dv          device bf16, same shape as q (written; padding rows 0)
 *   dw_lin              device float [head_dim, head_dim] (written: summed over
 *                       every batch index and head)
 *   dgate               device float [batch*heads] (written)
 *   ws                  device workspace of salad_bwd_workspace_bytes(shape)
 * Accumulation is fp32 (bf16 MFMA products), every sum in a fixed order:
 * bitwise reproducible run to run.  Given the forward's lse, dQ runs in one
 * pass over the kept tiles; without it a first pass recomputes the statistic.
 * fp32 shapes return SALAD_EUNSUPPORTED. */
SALAD_API int salad_attn_bwd(const salad_shape* shape, const void* q, const void* k,
                             const void* v, const int32_t* row_ptr, const int32_t* col_idx,
                             const float* gate, const void* w_lin, float eps, float scale,
                             const void* out, const float* lse, const void* dout, void* dq,
                             void* dk, void* dv,
                             float* dw_lin, float* dgate, void* ws, size_t ws_bytes,
                             void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SALAD_H */
