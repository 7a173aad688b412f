// Internal declarations shared by the HIP translation units of libsalad.
// Nothing here is part of the public interface (include/salad.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "salad.h"

#define SALAD_HIDDEN __attribute__((visibility("hidden")))

namespace salad {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kRstarInf = 1 << 30;
// int32 words after the 9 per-XCD cuts of the forward item split: one layout
// mode per head (sched.hip)
constexpr int kPairModeSlots = SALAD_MAX_HEADS;

// Geometry of the latent grid and its blocking, as kernels see it.
struct Geom {
  int B, Hh, D;     // batch, heads, head_dim
  int T, H, W;      // latent grid
  int N, n_pad, blk, nb;
};

// Token storage order of a shape: frame-major runs (ct == 0) or cuboid blocks.
// Tokens are stored cuboid by cuboid: every full ct x ch x cw cuboid in
// lexicographic cuboid order (one block each), then the partial cuboids at the
// grid's far edges in lexicographic order; frame-major inside a cuboid.
struct Cuboid {
  int ct, ch, cw;      // cuboid extents, 0 = frame-major order
  int nt, ny, nx;      // cuboids per axis (rounded up)
  int Ft, Fy, Fx;      // full cuboids per axis (rounded down)
  int rt, ry, rx;      // extent of the last cuboid on each axis
  int F;               // full cuboids: blocks [0, F) are exactly one cuboid each
  int box_cap;         // boxes a block's token set can need (upper bound)
};

// Axis-aligned box of tokens, bounds inclusive: (t0, t1, y0, y1), (x0, x1, -, -).
struct Box {
  int4 ty;
  int4 x;
};

// Per-head mask parameters, passed by value in kernel arguments.
struct HeadTable {
  int n_heads;
  int kind[SALAD_MAX_HEADS];       // salad_mask_kind
  int t_window[SALAD_MAX_HEADS];
  int r_max[SALAD_MAX_HEADS];
  int count[SALAD_MAX_HEADS];      // window: K pairs (-1 = keep all); top-k: k per row
  int pool[SALAD_MAX_HEADS];       // pool Q (bit 0) / K (bit 1) for this head
  int group[SALAD_MAX_HEADS];      // window heads: index of their (t_window, r_max) group
  // Direct row pointers (no SICS head, nb <= kDirectRowsMaxNb): every head's
  // entry count per batch is known before the launch, so row (b, h, qb)
  // starts at b * batch_nnz + base[h] + (the head's entries in rows < qb).
  int direct_rows;
  int batch_nnz;
  int base[SALAD_MAX_HEADS];
};
// Largest block count for direct row pointers: each window row sums the
// counts of the rows before it in its head (nb^2 / 2 reads per head).
constexpr int kDirectRowsMaxNb = 4096;

// Workspace layout for one shape, computed on the host.
struct Workspace {
  size_t bytes;
  // mask build
  size_t off_rt;                   // uint16 [nb][nb]: r* of one window group (0xffff = no candidate)
  size_t off_hist, hist_bins;      // int32 [hist_bins]: that group's candidates per rank bin
  size_t off_thr;                  // int64 [heads] threshold keys
  size_t off_rowcnt;               // int32 [B*H*nb]
  size_t off_psum_q, off_psum_k;   // float [B*H*nb*D]
  size_t off_scores;               // float [heads per batch][nb][nb] (top-k scores)
  size_t off_sics, off_sics_pack;  // float / int32 [B*H*nb] (SICS scores, selection)
  size_t off_nbox, off_boxes;      // cuboid order: int32 [nb] box counts, Box [nb][box_cap]
  // linear state
  int lin_splits, lin_chunk;
  size_t off_spart, off_zpart;     // float [splits][B*H][D*D], [splits][B*H][D]
  size_t off_z;                    // float [B*H][D]
  size_t off_sft;                  // folded state, transposed: bf16 or f32 [B*H][D*D]
  size_t off_split;                // int32 [9 + kPairModeSlots]: attention items per XCD, layout modes
  size_t mask_end, lin_end;
};

// Backward workspace: the forward layout (its linear-state partials are reused
// to rebuild S, z) followed by the regions of the backward pass.
struct BwdWorkspace {
  Workspace fwd;
  size_t bytes;
  int red_splits, red_chunk;          // token split of the dS / dW reduction
  size_t off_s32, off_z;              // float [BH][D][D], [BH][D]: S, z
  size_t off_s_hi, off_s_lo;          // bf16 [BH][D][D]: S (rows c)
  size_t off_st_hi, off_st_lo;        // bf16 [BH][D][D]: S^T (rows e)
  size_t off_dq, off_dden, off_lse;   // float [BH][n_pad]: D_i, dden_i, (spare)
  size_t off_du, off_ol;              // bf16 [BH][n_pad][D]: dU, o_l
  size_t off_gpart;                   // float [BH][n_pad/32]: dgate partials
  size_t off_dspart, off_dzpart, off_dwpart;  // float [splits][BH][D*D | D | D*D]
  size_t off_ds_hi, off_ds_lo;        // bf16 [BH][D][D]: dS_lin (rows c)
  size_t off_dst_hi, off_dst_lo;      // bf16 [BH][D][D]: dS_lin^T (rows e)
  size_t off_dz;                      // float [BH][D]: dz_lin
  size_t off_dwh;                     // float [BH][D][D]: g * per-head dW_lin
  size_t off_colcnt, off_colptr;      // int32 [BH*nb], [BH*nb + 1]
  size_t off_rowidx;                  // int32 [BH*nb*nb]
  size_t off_bits;                    // uint32 [BH*nb][ceil(nb/32)]: transposed mask bitmap
  size_t off_split_q, off_split_k;    // int32 [9 + kPairModeSlots], [9]: dQ items per XCD and layout modes,
                                      // dK/dV items per XCD
};

// ---- XCD assignment of attention items (sched.hip) ----------------------------
// Item i of a job covers `per` consecutive rows of one of n_seq sequences of
// nrows rows (the last item of a sequence may be short); ptr is the CSR or CSC
// pointer array over the n_seq*nrows rows.  split[x] .. split[x+1]-1 are the
// items XCD x runs, cut by estimated work (kept blocks * tpb + ovh per item),
// each run at most xcd_items_cap(n_items) long: the consumer launches 8 times
// that many workgroups.
//
// With mode_heads > 0 (forward kernels whose workgroups own two neighbouring
// query blocks, per = 2), the same launch also chooses, per head, how those
// workgroups walk the kept lists: mode 0, the union of both blocks' lists with
// all four waves (tiles kept by both blocks are loaded once); mode 1, each wave
// pair its own block's list (no wave sits out a tile its block does not keep).
// Mode 1 is chosen when sampled neighbouring lists of the head (batch 0)
// overlap little: their union is more than 5/4 of the longer list.  Word
// split[9 + x] receives the mode of sequence x (head x % mode_heads) for every
// x < min(n_seq, kPairModeSlots).  Both modes compute the same attention, up
// to the order of floating-point sums.
__host__ __device__ inline int xcd_items_cap(int n_items) { return (n_items + 7) / 8 + (n_items + 31) / 32; }
struct ItemSplit {
  const int32_t* ptr;  // pointer array over n_seq * nrows rows
  int32_t* split;      // [9] output, then [mode_heads] modes when mode_heads > 0
  int n_seq, nrows, per, tpb, ovh;
  const int32_t* col = nullptr;  // the rows' entries (needed for the modes)
  int mode_heads = 0;            // 0: no modes; else heads <= kPairModeSlots
};
// One workgroup per job (one or two jobs per launch).
SALAD_HIDDEN hipError_t launch_item_splits(const ItemSplit* jobs, int n_jobs, hipStream_t st);

SALAD_HIDDEN bool make_geom(const salad_shape* s, Geom* g);
SALAD_HIDDEN void make_cuboid(const salad_shape* s, Cuboid* c);
SALAD_HIDDEN Workspace plan_workspace(const Geom& g, const Cuboid& cu, int dtype);

// ---- token order (layout.hip) -----------------------------------------------
SALAD_HIDDEN hipError_t launch_permute_tokens(const Geom& g, const Cuboid& cu, int dtype,
                                              int inverse, const void* src, void* dst,
                                              hipStream_t st);
// Box lists of every block's token set (cuboid order only) into the workspace.
SALAD_HIDDEN hipError_t launch_block_boxes(const Geom& g, const Cuboid& cu, char* ws,
                                           const Workspace& L, hipStream_t st);

// ---- mask builder (mask.hip) ------------------------------------------------
SALAD_HIDDEN hipError_t launch_build_mask(const Geom& g, const Cuboid& cu, int dtype,
                                          const HeadTable& ht,
                                          const void* q, const void* k, int32_t* row_ptr,
                                          int32_t* col_idx, int64_t col_cap,
                                          const float* w_g, float* gate, char* ws,
                                          const Workspace& L, hipStream_t st);
// Number of candidate (qb, kb) pairs of a window head with this t_window and
// r_max (window_count.hip, host only).
SALAD_HIDDEN int64_t window_candidates(const Geom& g, const Cuboid& cu, int t_window, int r_max);
// CSR structure check (check.hip): writes the SALAD_MASK_BAD_* bits to out[0].
SALAD_HIDDEN hipError_t launch_check_mask(const Geom& g, const int32_t* row_ptr, const int32_t* col_idx,
                                          int64_t col_cap, int32_t* out, hipStream_t st);
SALAD_HIDDEN hipError_t launch_gate_from_q(const Geom& g, int dtype, const void* q,
                                           const float* w_g, float* gate, char* ws,
                                           const Workspace& L, hipStream_t st);

// Heads whose top-k scores (nb x nb floats each) the workspace holds at once:
// all of them up to 64 MiB of scores, at least one.
inline int topk_heads_per_batch(const Geom& g) {
  const int64_t per_head = (int64_t)g.nb * g.nb * 4;
  const int64_t cap = ((int64_t)64 << 20) / per_head;
  return (int)std::max<int64_t>(1, std::min<int64_t>((int64_t)g.B * g.Hh, cap));
}

// ---- linear state (linear.hip) ----------------------------------------------
// Split partials of S and z.  With a gate, heads whose gate < drop_tau are
// skipped (nothing written for them).  For bf16, a non-null w_lin makes the
// partials S_c W_lin (the fused forward: pass it exactly when the fold runs in
// mode 0); the fp32 kernel ignores it.
SALAD_HIDDEN hipError_t launch_linear_state(const Geom& g, int dtype, const void* k,
                                            const void* v, const float* gate, float drop_tau,
                                            const void* w_lin, char* ws, const Workspace& L,
                                            hipStream_t st);
// Reduce the split partials and fold.  mode 0: folded state g*S*W_lin (fused
// forward; heads with g < drop_tau skipped; for bf16 the product with W_lin
// was taken by the partial kernel); 1: S itself (linear branch alone); 2:
// reduce only.  S_out / z_out (may be null) receive the fp32 state in modes 1
// and 2; z always lands in the workspace.
SALAD_HIDDEN hipError_t launch_linear_fold(const Geom& g, int dtype, const float* gate,
                                           const void* w_lin, int mode, float drop_tau,
                                           float* S_out, float* z_out, char* ws,
                                           const Workspace& L, hipStream_t st);

// ---- backward (linear_bwd.hip, attn_bwd.hip) ---------------------------------
SALAD_HIDDEN BwdWorkspace plan_bwd_workspace(const Geom& g, const Cuboid& cu, int dtype);
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const float* gate;
  const void* w_lin;
  const void* out;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* dw_lin;
  float* dgate;
  const float* lse;     // forward's log2-sum-exp [BH][n_pad], or null (recomputed)
  float eps;
  float scale;
};
// Linear-branch backward up to dS_lin, dz_lin, dW_lin, dgate and the per-token
// D_i, dU, dden (needs S, z in the workspace).
SALAD_HIDDEN hipError_t launch_linear_bwd(const Geom& g, const BwdArgs& a, char* ws,
                                          const BwdWorkspace& L, hipStream_t st);
// Transposed mask (CSC) of the CSR rows.
SALAD_HIDDEN hipError_t launch_mask_transpose(const Geom& g, const int32_t* row_ptr,
                                              const int32_t* col_idx, char* ws,
                                              const BwdWorkspace& L, hipStream_t st);
// Sparse-branch backward plus the linear parts of dq, dk, dv.
SALAD_HIDDEN hipError_t launch_attn_bwd(const Geom& g, const BwdArgs& a, char* ws,
                                        const BwdWorkspace& L, hipStream_t st);

// ---- attention (attn_bf16.hip, attn_f32.hip) --------------------------------
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const void* sft;      // folded linear state, transposed [BH][D][D] (bf16 or f32)
  const float* z;       // [BH][D]
  const float* gate;    // [BH] (branch dropping), may be null
  float* lse;           // [BH][n_pad] log2-sum-exp of the scaled scores (bf16 path), may be null
  int32_t* split;       // [9] cuts of the item sequence per XCD (bf16 path; written before the launch)
  float drop_tau;
  float eps;
  float scale;
  int has_sparse;
  int has_lin;
};
SALAD_HIDDEN hipError_t launch_attn_bf16(const Geom& g, const AttnArgs& a, hipStream_t st);
SALAD_HIDDEN hipError_t launch_attn_f32(const Geom& g, const AttnArgs& a, hipStream_t st);

}  // namespace salad
