"""CPU oracle for hybrid block-sparse + ReLU-linear attention (SALAD-style).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import or call anything in this package.  The
product path (the HIP library and its Python binding) never uses it, and this
package never imports the product path.  It shares no code with it: only the
seeded input generator (``synth``), which draws numbers and holds none of the
operator's arithmetic, serves both sides.

What it computes, and where the pages say so:

* Sparse branch: softmax attention in which each query block attends only to
  the key blocks its mask keeps ("SALAD" explainer, technical summary section
  2.1, sparse branch carries most of the modelling at high sparsity; sciencestack
  "SALAD" TL;DR and abstract, 90% sparsity).  Written as dense masked softmax:
  logits of dropped blocks are -inf.
* Linear branch: ReLU linear attention, O(N), global over all tokens, sharing
  Q/K/V with the sparse branch (explainer section 2.1).  Written in its
  quadratic form (ReLU(Q) ReLU(K)^T) V, row-normalised.
* Mix: out = sparse + s * (linear . W_lin), with s in (0,1) a per-head gate
  (explainer section 2.2, LWSS projection and ITADS sigmoid gate; sciencestack
  TL;DR, input-dependent scalar gate).
* Masks: a static spatio-temporal sliding window or a dynamic top-k over pooled
  block scores (explainer section 5, applies to sliding-window and Top-K sparse
  attention; sciencestack Figure 1, ST-SWA), or key blocks ranked by the sum of
  intra-block cosine similarities (SPADE explainer, scheme generation).  The
  pages fix none of the rules; the readings used here are stated in ``masks.py``.
* Gradients (for fine-tuning, explainer sections 2.2 and 3): dq, dk, dv, dW_lin
  and dgate of the same forward by reverse-mode differentiation, in
  ``backward.py``.
* Token order: frame-major runs or 3-D cuboid blocks (SPADE explainer, the
  vDiT-SSR blueprint part); the storage rule is stated in ``layout.py``.

All floating-point work is fp64 on the exact values of the (bf16 or fp32)
inputs, except the pooled-score ranking of the top-k mask, whose fp32 order of
operations is part of its definition (see ``masks.py``).

Parity status per function: every function here is pinned by the CPU tests
(closed forms, library special cases, invariants, brute force); none is
"parity unpinned".  The readings of the mask rules themselves cannot be pinned
by the pages, which print no mask rule.
"""

from .attention import (
    layer_forward,
    linear_attention,
    linear_attention_from_state,
    linear_state,
    mix,
    sparse_attention,
    sparse_lse2,
)
from .backward import layer_backward, layer_backward_sampled
from .layout import cuboid_order, permute_tokens, slot_coords
from .masks import (
    InfeasibleMask,
    build_masks,
    csr_from_keep,
    gate_from_q,
    keep_from_csr,
    pooled_means_f32,
    pooled_scores_f32,
    sics_block_scores_f32,
    sics_select,
    topk_count,
    topk_select,
    window_count,
    window_rstar_bruteforce,
    window_rstar_segments,
    window_select,
)

__all__ = [
    "InfeasibleMask",
    "build_masks",
    "csr_from_keep",
    "cuboid_order",
    "gate_from_q",
    "keep_from_csr",
    "layer_backward",
    "layer_backward_sampled",
    "layer_forward",
    "linear_attention",
    "linear_attention_from_state",
    "linear_state",
    "mix",
    "permute_tokens",
    "pooled_means_f32",
    "pooled_scores_f32",
    "slot_coords",
    "sparse_attention",
    "sparse_lse2",
    "topk_count",
    "topk_select",
    "window_count",
    "window_rstar_bruteforce",
    "window_rstar_segments",
    "window_select",
]
