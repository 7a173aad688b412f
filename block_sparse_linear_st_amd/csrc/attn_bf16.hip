// attn_bf16.hip - fused hybrid attention forward for gfx950, bf16 in/out.
//
// One workgroup (4 waves) owns 128 query rows: two 64-token query blocks, or
// one 128-token block.  Each wave owns 32 rows.  The workgroup walks the
// ascending union of its query blocks' kept key-block lists (a two-way merge of
// the CSR rows, read through the scalar cache) in 64-key tiles (32-key tiles
// for 128-token blocks, see tile_keys below); a wave computes
// a tile only when its own query block keeps that key block, so dropped blocks
// cost nothing and key blocks kept by both query blocks are loaded once.
//
// Per tile, with MFMA 32x32x16 bf16 (fp32 accumulate):
//   S^T = K Q^T      A = K tile (LDS), B = Q fragments held in registers
//   online softmax   a row's scores of a tile sit in lanes l and l^32, so the row max
//                    and row sum need one v_permlane32_swap each
//   O^T += V^T P^T   A = V^T fragments read from the row-major V tile with the
//                    gfx950 LDS transpose read (ds_read_b64_tr_b16), B = P taken
//                    straight from the S^T accumulators, converted to bf16
// The transposed orientation keeps every per-query quantity (max, sum, scale)
// in the lane that owns the query.  With 64-key tiles the loop is software
// pipelined inside each wave (pipe_step): the QK^T of tile u runs beside the
// exponentials of tile u-1 and the PV of tile u-1 beside the row max of tile u,
// K tiles travelling one step ahead of V tiles.  The softmax rescale is lazy: the running
// max used for the exponentials only moves when a row's max grows by more than
// 2^8, so most tiles skip rescaling O; the final O/l is exact either way.
//
// K/V tiles travel HBM -> LDS with global_load_lds_dwordx4 (no registers, no
// VALU), double buffered: the next tile's loads are issued before the current
// tile's MFMAs.  Rows are 16-byte-chunk XOR-swizzled so that the K fragment
// reads (16 consecutive rows, one chunk) and the V transpose reads (4 rows x 4
// chunks per half-wave) spread over all banks.
//
// Epilogue: o_s = O / l (and, when asked, each row's log2-sum-exp m + log2 l
// for the backward pass); the linear branch ("SALAD" explainer, section 2.1)
// and its gated projection (section 2.2) arrive pre-folded as S''^T =
// (g S W_lin)^T in bf16 (rounded once, as P is before the PV product), so
// g*(o_l W_lin) = (S''^T ReLU(Q)^T) / (ReLU(Q) z + eps) is (D/32)*(D/16) more
// MFMAs on the Q fragments already in registers.  Heads whose gate is below drop_tau skip it (section 2.3).  The
// 128 x D bf16 result is staged through LDS for 16-byte coalesced stores.
//
// The per-lane LDS read offsets inside a tile are computed once; the tile loop
// is unrolled over the two buffers, so every fragment read is that offset plus
// an immediate.
//
// Work items map to workgroups so that each XCD (blockIdx % 8) gets a
// contiguous range of (head, query group) items: neighbouring query blocks,
// whose window lists overlap, share that XCD's L2.  The ranges are cut by
// estimated work (sched.hip) rather than by count, so that heads of different
// density do not leave some XCDs idle at the end.
#include <type_traits>

#include "attn_common.h"

namespace salad {
namespace {

using namespace fwd;

// S^T, softmax and O^T update of one wave on one 32-key tile held in buffer
// CUR (a tile's steps in order, one QK^T chain); kbase, vbase are the per-lane
// read bases (chunk c of a K row is kbase ^ (c << 5), output tile t of a V
// transpose read is vbase ^ (t << 6)).
template <int D, int CUR>
__device__ __attribute__((always_inline)) inline void compute_tile32(const unsigned char* smem, uint32_t kbase,
                                    uint32_t vbase, const bf16x8 (&qf)[D / 16],
                                    f32x16 (&o)[D / 32], float& m_used, float& l_run, int key0,
                                    int N, float c_log2, int lane) {
  using LY = Lay<D, 32>;
  constexpr int NC = D / 16, NT = D / 32;
  const int g32 = lane >> 5;
  const unsigned char* Kt = smem + CUR * LY::BUF_B;
  const unsigned char* Vt = Kt + LY::TILE_B;
  // S^T = K Q^T over the tile's 32 keys: one chain, K fragments one step ahead
  f32x16 s;
#pragma unroll
  for (int i = 0; i < 16; ++i) s[i] = 0.0f;
  {
    auto kfrag = [&](int c) __attribute__((always_inline)) {
      return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(Kt + (kbase ^ (c << 5))));
    };
    bf16x8 a0 = kfrag(0);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      bf16x8 a1 = a0;
      if (c + 1 < NC) a1 = kfrag(c + 1);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[c], s, 0, 0, 0);
      a0 = a1;
    }
  }
  if (key0 + 32 > N) {
    // keys past N get -inf added (bit patterns, no per-key compare masks)
    const int rem = N - key0 - g32 * 4;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] += past_n_bias(rem, (i >> 2) * 8 + (i & 3));
  }
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
  mx = pair_max(mx) * c_log2;
  if (__ballot(mx > m_used + 8.0f)) {
    const float m_new = fmaxf(m_used, mx);
    const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_used - m_new);
    l_run *= alpha;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[t][i] *= alpha;
    m_used = m_new;
  }
  const float neg_m = m_used == -INFINITY ? 0.0f : -m_used;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float rs = 0.0f;
  bf16x8 pf[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = __builtin_amdgcn_exp2f(fmaf(s[h * 8 + j], c_log2, neg_m));
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w[j] = pack_bf16x2(p[2 * j], p[2 * j + 1]);
      rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[j]), ones, rs, false);
    }
    pf[h] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
  }
  l_run += pair_sum(rs);
  // O^T += V^T P^T, V^T fragments by transpose reads laid out as in the 64-key tile
  auto vfrag = [&](int t, int ks) __attribute__((always_inline)) {
    uint2 tr[2];
    const uint32_t v0 = vbase ^ (t << 6);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const unsigned char* ad = Vt + v0 + (ks * 16 + 8 * h) * LY::ROW_B;
      tr[h] = __builtin_bit_cast(
          uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(ad)));
    }
    return __builtin_bit_cast(bf16x8, make_uint4(tr[0].x, tr[0].y, tr[1].x, tr[1].y));
  };
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int t = 0; t < NT; ++t)
      o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfrag(t, ks), pf[ks], o[t], 0, 0, 0);
}

// ---- software-pipelined 64-key tiles ------------------------------------------
// Within one wave the steps of a tile are serial (QK^T -> softmax -> PV).  The
// pipelined loop overlaps two tiles instead: in step u a wave runs
//   phase A: S_u = K_u Q^T (MFMA) beside the exponentials of S_{u-1} (VALU),
//   phase B: O^T += V_{u-1}^T P_{u-1}^T (MFMA) beside the row max of S_u (VALU),
// then decides whether tile u moves the reference max.  K tiles are loaded one
// step ahead of V tiles (tile u's K and V share LDS slot u % 2), so step u reads
// K_u and V_{u-1}.  Scheduling groups pin the MFMA/VALU interleave.

// Exponentials of chunk c (of NC) of the 32 scores a lane holds for one tile:
// score v = 16 kt + 8 h + j sits in s[kt][8 h + j]; p = 2^(s * c_log2 - m),
// packed to bf16 pairs (word v / 2) and summed (the sum adds the rounded values).
template <int NC>
__device__ __attribute__((always_inline)) inline void exp_chunk(int c, const f32x16 (&s)[2], float c_log2,
                                                                float neg_m, uint32_t (&w)[16], float& rs) {
  constexpr int PER = 32 / NC;  // scores per chunk (4 or 8)
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int q = 0; q < PER / 2; ++q) {
    const int v = c * PER + 2 * q;
    const float p0 = __builtin_amdgcn_exp2f(fmaf(s[v / 16][v % 16], c_log2, neg_m));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(s[(v + 1) / 16][(v + 1) % 16], c_log2, neg_m));
    w[v / 2] = pack_bf16x2(p0, p1);
    rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[v / 2]), ones, rs, false);
  }
}

__device__ __attribute__((always_inline)) inline void words_to_frags(const uint32_t (&w)[16], bf16x8 (&pf)[4]) {
#pragma unroll
  for (int g4 = 0; g4 < 4; ++g4)
    pf[g4] = __builtin_bit_cast(bf16x8, make_uint4(w[4 * g4], w[4 * g4 + 1], w[4 * g4 + 2], w[4 * g4 + 3]));
}

// One pipelined step of a wave.  QK: the wave keeps tile u (sn receives its
// scores); PV: it kept tile u-1 (sp holds those scores).  Returns nothing; o,
// m_used, l_run are updated.  CUR = u % 2.
template <int D, int CUR, bool QK, bool PV>
__device__ __attribute__((always_inline)) inline void pipe_step(
    const unsigned char* smem, const uint32_t (&ka)[D / 16], const uint32_t (&va)[D / 32],
    const bf16x8 (&qf)[D / 16], f32x16 (&o)[D / 32], const f32x16 (&sp)[2], f32x16 (&sn)[2], float& m_used,
    float& l_run, int key0, int N, float c_log2, int lane) {
  using LY = Lay<D, 64>;
  constexpr int NC = D / 16, NT = D / 32;
  constexpr int VPC = 3 * (32 / NC);  // VALU instructions per exponential chunk
  const int g32 = lane >> 5;
  const unsigned char* Kt = smem + CUR * LY::BUF_B;                      // K of tile u
  const unsigned char* Vt = smem + (CUR ^ 1) * LY::BUF_B + LY::TILE_B;   // V of tile u-1
  auto kfrag = [&](int half, int c) __attribute__((always_inline)) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(Kt + ka[c] + half * 32 * LY::ROW_B));
  };
  auto vfrag = [&](int t, int ks) __attribute__((always_inline)) {
    uint2 tr[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const unsigned char* ad = Vt + va[t] + (ks * 16 + 8 * h) * LY::ROW_B;
      tr[h] = __builtin_bit_cast(
          uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(ad)));
    }
    return __builtin_bit_cast(bf16x8, make_uint4(tr[0].x, tr[0].y, tr[1].x, tr[1].y));
  };

  // ---- phase A
  uint32_t w[16];
  float rs = 0.0f;
  const float neg_m = m_used == -INFINITY ? 0.0f : -m_used;
  if constexpr (QK) {
    bf16x8 a0 = kfrag(0, 0), b0 = kfrag(1, 0);
    bf16x8 a1 = kfrag(0, 1), b1 = kfrag(1, 1);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      bf16x8 a2 = a1, b2 = b1;
      if (c + 2 < NC) { a2 = kfrag(0, c + 2); b2 = kfrag(1, c + 2); }
      sn[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[c], c == 0 ? f32x16{} : sn[0], 0, 0, 0);
      sn[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b0, qf[c], c == 0 ? f32x16{} : sn[1], 0, 0, 0);
      if constexpr (PV) exp_chunk<NC>(c, sp, c_log2, neg_m, w, rs);
      a0 = a1; b0 = b1; a1 = a2; b1 = b2;
      if (c + 2 < NC) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (PV) __builtin_amdgcn_sched_group_barrier(0x002, VPC / 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (PV) __builtin_amdgcn_sched_group_barrier(0x002, VPC - VPC / 2, 0);
    }
  } else if constexpr (PV) {
#pragma unroll
    for (int c = 0; c < NC; ++c) exp_chunk<NC>(c, sp, c_log2, neg_m, w, rs);
  }
  if constexpr (PV) l_run += pair_sum(rs);

  // scores of keys past N (only the tile holding token N-1 and beyond)
  if constexpr (QK) {
    if (key0 + 64 > N) {
      const int rem = N - key0 - g32 * 4;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) sn[kt][i] += past_n_bias(rem, kt * 32 + (i >> 2) * 8 + (i & 3));
    }
  }

  // ---- phase B
  float mx = -INFINITY;
  if constexpr (PV) {
    bf16x8 pf[4];
    words_to_frags(w, pf);
    constexpr int NOPS = 4 * NT;  // (ks, t) in order
    constexpr int MPO = 32 / NOPS;  // max3 inputs pairs per op: 16 pairs over NOPS ops
    bf16x8 vf0 = vfrag(0, 0), vf1 = vfrag(1 % NT, (1 / NT) % 4);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < NOPS; ++i) {
      const int ks = i / NT, t = i % NT;
      bf16x8 vf2 = vf1;
      if (i + 2 < NOPS) vf2 = vfrag((i + 2) % NT, (i + 2) / NT);
      o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf0, pf[ks], o[t], 0, 0, 0);
      if constexpr (QK) {
#pragma unroll
        for (int q = 0; q < MPO; ++q) {
          const int v = i * MPO + q;
          mx = fmaxf(mx, sn[v / 16][v % 16]);
        }
      }
      vf0 = vf1; vf1 = vf2;
      if (i + 2 < NOPS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (QK) __builtin_amdgcn_sched_group_barrier(0x002, MPO / 2, 0);
    }
  } else if constexpr (QK) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sn[kt][i]);
  }
  if constexpr (QK) {
    // tile u moves the reference max only when some row grew by more than 2^8
    mx = pair_max(mx) * c_log2;
    if (__ballot(mx > m_used + 8.0f)) {
      const float m_new = fmaxf(m_used, mx);
      const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_used - m_new);
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[t][i] *= alpha;
      m_used = m_new;
    }
  }
}

// 64-key tiles for 64-token blocks (64 KiB of LDS at head_dim 128, two
// workgroups per CU, software-pipelined); 32-key tiles for 128-token blocks,
// whose workgroups walk one block's list with every wave active: 35 KiB of LDS
// and at most 168 registers give three workgroups (three waves per SIMD) per CU.
template <int BLK>
constexpr int tile_keys() { return BLK == 64 ? 64 : 32; }

template <int D, int BLK>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(BLK == 128 ? 3 : 2, BLK == 128 ? 3 : 2)))
k_attn_bf16(Geom g, AttnArgs a, int n_items, float c_log2) {
  constexpr int NW = 4;             // waves per workgroup
  constexpr int KT = tile_keys<BLK>();
  using LY = Lay<D, KT, NW>;
  constexpr int ROWS = NW * 32;     // query rows per workgroup
  constexpr int QPW = ROWS / BLK;   // query blocks per workgroup
  constexpr int NC = D / 16;
  constexpr int NT = D / 32;
  constexpr int TPB = BLK / KT;   // tiles per key block
  constexpr int SMEM_B = ROWS * LY::OST * 2 > 2 * LY::BUF_B ? ROWS * LY::OST * 2 : 2 * LY::BUF_B;
  static_assert(D * D * 2 <= SMEM_B, "the folded linear state must fit in the tile buffers");
  constexpr int THREADS = NW * 64;
  __shared__ __align__(1024) unsigned char smem[SMEM_B];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g32 = lane >> 5, l32 = lane & 31;

  // XCD-aware item order: workgroup w runs on XCD w % 8, which takes its own
  // contiguous run of items, cut by estimated work before the launch.
  const const_i32_ptr cuts = (const_i32_ptr)a.split;
  const int xcd = (int)(blockIdx.x & 7);
  const int item = cuts[xcd] + (int)(blockIdx.x >> 3);
  if (item >= cuts[xcd + 1] || item >= n_items) return;
  const int qgroups = (g.nb + QPW - 1) / QPW;
  const int bh = item / qgroups, qg = item - bh * qgroups;
  const int qb_base = qg * QPW;
  const int qsub = QPW == 2 ? (wave >> 1) : 0;
  const bool wave_rows = qb_base + qsub < g.nb;
  const int row0 = qb_base * BLK + wave * 32;
  const int my_row = row0 + l32;

  const __bf16* Qb = static_cast<const __bf16*>(a.q) + (int64_t)bh * g.n_pad * D;
  const __bf16* Kb = static_cast<const __bf16*>(a.k) + (int64_t)bh * g.n_pad * D;
  const __bf16* Vb = static_cast<const __bf16*>(a.v) + (int64_t)bh * g.n_pad * D;

  bf16x8 qf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (wave_rows && my_row < g.N) qf[c] = load_bf16x8(Qb + (int64_t)my_row * D + c * 16 + g32 * 8);
    else qf[c] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
  }
  wait_vmem();  // Q is in registers before the loop's own loads start

  f32x16 o[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] = 0.0f;
  float m_used = -INFINITY, l_run = 0.0f;

  if (a.has_sparse) {
    // kept lists of the workgroup's query blocks, read through the scalar cache
    const const_i32_ptr col = (const_i32_ptr)a.col_idx;
    const const_i32_ptr rptr = (const_i32_ptr)a.row_ptr;
    const int64_t rbase = (int64_t)bh * g.nb + qb_base;
    int i0 = 0, e0 = 0, i1 = 0, e1 = 0;
    if (qb_base < g.nb) { i0 = rptr[rbase]; e0 = rptr[rbase + 1]; }
    if (QPW == 2 && qb_base + 1 < g.nb) { i1 = e0; e1 = rptr[rbase + 2]; }
    // this head's layout (64-key tiles only): 0 walks the union of the two
    // lists, 1 gives each wave pair its own block's list
    const bool own_lists = KT == 64 && cuts[9 + (bh < kPairModeSlots ? bh : bh % g.Hh)] != 0;
    const int i0s = i0, e0s = e0, i1s = i1, e1s = e1;
    int c0 = i0 < e0 ? col[i0] : INT32_MAX;
    int c1 = i1 < e1 ? col[i1] : INT32_MAX;
    // current tile
    int kb = 0, sub = 0, flags = 0;
    bool valid = false;
    auto advance = [&](int& nkb, int& nsub, int& nflags, bool& nvalid) __attribute__((always_inline)) {
      if (valid && sub + 1 < TPB && kb * BLK + (sub + 1) * KT < g.N) {
        nkb = kb; nsub = sub + 1; nflags = flags; nvalid = true;
        return;
      }
      nkb = min(c0, c1);
      nvalid = nkb != INT32_MAX;
      nflags = (c0 == nkb ? 1 : 0) | (c1 == nkb ? 2 : 0);
      nsub = 0;
      if (c0 == nkb) { ++i0; c0 = i0 < e0 ? col[i0] : INT32_MAX; }
      if (c1 == nkb) { ++i1; c1 = i1 < e1 ? col[i1] : INT32_MAX; }
    };
    advance(kb, sub, flags, valid);
    // LDS byte address of the buffers (uniform); the wave index is uniform too
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    DmaOffsets<D, KT, NW> doff;
    doff.init(wave_u, lane);
    constexpr bool PIPE = KT == 64;  // 64-key tiles: the software-pipelined loop
    if (valid && !own_lists) {
      if constexpr (PIPE) issue_half<D, KT, NW, true>(lds0, Kb, kb * BLK + sub * KT, g.N, wave_u, lane, doff);
      else issue_tile<D, KT, NW>(lds0, Kb, Vb, kb * BLK + sub * KT, g.N, wave_u, lane, doff);
    }
    wait_vmem();
    __syncthreads();
    // per-lane LDS read offsets inside a tile, fixed for the whole loop (kept opaque so that
    // they stay in registers rather than being recomputed at every read): all of them for
    // 64-key tiles, one base per read kind for 32-key tiles (fewer registers)
    uint32_t ka[NC], va[NT], kbase = 0, vbase = 0;
    {
      const int sw = LY::kswz(l32);
      const int sl = lane & 15, dh = (lane >> 4) & 1;
      const int row = 4 * g32 + (sl >> 2);  // + 16 ks + 8 h, which leave the swizzle unchanged
      if constexpr (KT == 64) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          ka[c] = (uint32_t)(l32 * LY::ROW_B + (((2 * c + g32) ^ sw) << 4));
          asm volatile("" : "+v"(ka[c]));
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int chunk = 4 * t + 2 * dh + ((sl & 3) >> 1);
          va[t] = (uint32_t)(row * LY::ROW_B + ((chunk ^ LY::vswz(row)) << 4) + (sl & 1) * 8);
          asm volatile("" : "+v"(va[t]));
        }
      } else {
        kbase = (uint32_t)(l32 * LY::ROW_B + ((g32 ^ sw) << 4));
        vbase = (uint32_t)(row * LY::ROW_B + (((2 * dh + ((sl & 3) >> 1)) ^ LY::vswz(row)) << 4) + (sl & 1) * 8);
        asm volatile("" : "+v"(kbase), "+v"(vbase));
      }
    }
    // two copies of the step, one per buffer, so that every LDS offset is an immediate
    auto step = [&](auto cur_c) __attribute__((always_inline)) {
      constexpr int CUR = decltype(cur_c)::value;
      int nkb, nsub, nflags;
      bool nvalid;
      advance(nkb, nsub, nflags, nvalid);
      if (nvalid)
        issue_tile<D, KT, NW>(lds0 + (CUR ^ 1) * LY::BUF_B, Kb, Vb, nkb * BLK + nsub * KT, g.N, wave_u, lane,
                          doff);
      if (wave_rows && ((flags >> qsub) & 1))
        compute_tile32<D, CUR>(smem, kbase, vbase, qf, o, m_used, l_run, kb * BLK + sub * KT, g.N, c_log2, lane);
      wait_vmem();  // the next tile has landed in LDS ...
      __syncthreads();  // ... for every wave, and nobody still reads the current one
      kb = nkb; sub = nsub; flags = nflags; valid = nvalid;
    };
    if (PIPE && own_lists) {
      // Each wave pair walks its own block's list in 32-key tiles through its
      // own half of the LDS (two buffers), the pairs in step: max(L0, L1) * 2
      // steps, a pair whose list is done idles at the barriers.
      using LP = Lay<D, 32, 2>;
      const int wp = wave_u & 1, qs = wave_u >> 1;
      const uint32_t pbase = lds0 + qs * 2 * LP::BUF_B;
      const unsigned char* psmem = smem + qs * 2 * LP::BUF_B;
      DmaOffsets<D, 32, 2> poff;
      poff.init(wp, lane);
      uint32_t kb32, vb32;
      {
        const int sw = LP::kswz(l32), sl = lane & 15, dh = (lane >> 4) & 1;
        const int row = 4 * g32 + (sl >> 2);
        kb32 = (uint32_t)(l32 * LP::ROW_B + ((g32 ^ sw) << 4));
        vb32 = (uint32_t)(row * LP::ROW_B + (((2 * dh + ((sl & 3) >> 1)) ^ LP::vswz(row)) << 4) + (sl & 1) * 8);
        asm volatile("" : "+v"(kb32), "+v"(vb32));
      }
      constexpr int TP = BLK / 32;  // 32-key tiles per key block
      const int ib = qs == 0 ? i0s : i1s;
      const int len = qs == 0 ? e0s - i0s : e1s - i1s;
      const int nsteps = max(e0s - i0s, e1s - i1s) * TP;
      // tile of step s: sub-tile s % TP of list entry s / TP, if it holds a key below N
      auto tile_at = [&](int s_, int& kb_) __attribute__((always_inline)) -> bool {
        const int e = s_ / TP;
        if (e >= len) return false;
        kb_ = col[ib + e];
        return kb_ * BLK + (s_ % TP) * 32 < g.N;
      };
      int s = 0, kb_c = 0;
      bool v_c = nsteps > 0 && tile_at(0, kb_c);
      if (v_c) issue_tile<D, 32, 2>(pbase, Kb, Vb, kb_c * BLK, g.N, wp, lane, poff);
      wait_vmem();
      __syncthreads();
      auto ostep = [&](auto cur_c) __attribute__((always_inline)) {
        constexpr int CUR = decltype(cur_c)::value;
        int kb_n = 0;
        const bool v_n = s + 1 < nsteps && tile_at(s + 1, kb_n);
        if (v_n)
          issue_tile<D, 32, 2>(pbase + (CUR ^ 1) * LP::BUF_B, Kb, Vb, kb_n * BLK + ((s + 1) % TP) * 32, g.N, wp,
                               lane, poff);
        if (wave_rows && v_c)
          compute_tile32<D, CUR>(psmem, kb32, vb32, qf, o, m_used, l_run, kb_c * BLK + (s % TP) * 32, g.N, c_log2,
                                 lane);
        wait_vmem();      // the next tile has landed in LDS ...
        __syncthreads();  // ... for both waves of the pair, and nobody still reads the current one
        kb_c = kb_n; v_c = v_n; ++s;
      };
      while (s < nsteps) {
        ostep(std::integral_constant<int, 0>{});
        if (s >= nsteps) break;
        ostep(std::integral_constant<int, 1>{});
      }
    } else if constexpr (PIPE) {
      // step u: tile u is (kb, sub, flags, valid), tile u-1 (pflags, pvalid); scores of
      // alternate tiles in sA / sB; one more step after the last tile finishes it
      f32x16 sA[2], sB[2];
      int pflags = 0;
      bool pvalid = false;
      auto pstep = [&](auto cur_c) __attribute__((always_inline)) {
        constexpr int CUR = decltype(cur_c)::value;
        int nkb, nsub, nflags;
        bool nvalid;
        advance(nkb, nsub, nflags, nvalid);
        if (nvalid)
          issue_half<D, KT, NW, true>(lds0 + (CUR ^ 1) * LY::BUF_B, Kb, nkb * BLK + nsub * KT, g.N, wave_u, lane,
                                      doff);
        if (valid)
          issue_half<D, KT, NW, false>(lds0 + CUR * LY::BUF_B + LY::TILE_B, Vb, kb * BLK + sub * KT, g.N, wave_u,
                                       lane, doff);
        const bool kc = valid && wave_rows && ((flags >> qsub) & 1);
        const bool kp = pvalid && wave_rows && ((pflags >> qsub) & 1);
        f32x16(&sp)[2] = CUR ? sA : sB;
        f32x16(&sn)[2] = CUR ? sB : sA;
        const int key0 = kb * BLK + sub * KT;
        if (kc && kp)
          pipe_step<D, CUR, true, true>(smem, ka, va, qf, o, sp, sn, m_used, l_run, key0, g.N, c_log2, lane);
        else if (kc)
          pipe_step<D, CUR, true, false>(smem, ka, va, qf, o, sp, sn, m_used, l_run, key0, g.N, c_log2, lane);
        else if (kp)
          pipe_step<D, CUR, false, true>(smem, ka, va, qf, o, sp, sn, m_used, l_run, key0, g.N, c_log2, lane);
        wait_vmem();      // K of tile u+1 and V of tile u have landed ...
        __syncthreads();  // ... for every wave, and nobody still reads K_u or V_{u-1}
        pflags = flags; pvalid = valid;
        kb = nkb; sub = nsub; flags = nflags; valid = nvalid;
      };
      while (valid || pvalid) {
        pstep(std::integral_constant<int, 0>{});
        if (!(valid || pvalid)) break;
        pstep(std::integral_constant<int, 1>{});
      }
    } else {
      while (valid) {
        step(std::integral_constant<int, 0>{});
        if (!valid) break;
        step(std::integral_constant<int, 1>{});
      }
    }
  }

  // ---- epilogue -------------------------------------------------------------
  const float inv_l = l_run > 0.0f ? 1.0f / l_run : 0.0f;
  // log2-sum-exp of each row's scaled scores, kept for the backward pass
  if (a.lse != nullptr && a.has_sparse && wave_rows && g32 == 0)
    a.lse[(int64_t)bh * g.n_pad + my_row] =
        (my_row < g.N && l_run > 0.0f) ? m_used + __log2f(l_run) : INFINITY;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] *= inv_l;

  bool lin = a.has_lin != 0;
  if (lin && a.gate != nullptr && a.gate[bh] < a.drop_tau) lin = false;  // uniform
  if (lin) {
    // S''^T of this head into LDS, rows swizzled like K tiles: every wave reads
    // all of it, so one copy per workgroup instead of one per wave
    const __bf16* st = static_cast<const __bf16*>(a.sft) + (int64_t)bh * D * D;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    constexpr int PER = D * LY::CPR / THREADS;  // 1 KiB loads per wave
    __syncthreads();  // the tile buffers are free
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int blk1k = wave_u * PER + i;
      const int P = blk1k * 64 + lane;
      const int r = P / LY::CPR, p = P % LY::CPR;
      lds_dma16(st + r * D + (p ^ LY::kswz(r)) * 8, lds0 + blk1k * 1024);
    }
    const float* z = a.z + (int64_t)bh * D;
    bf16x8 rq[NC];
    float den = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      rq[c] = relu8(qf[c]);
#pragma unroll
      for (int j = 0; j < 8; ++j) den += (float)rq[c][j] * z[c * 16 + g32 * 8 + j];
    }
    den = pair_sum(den) + a.eps;
    const float inv_den = 1.0f / den;
    wait_vmem();
    __syncthreads();
    if (wave_rows) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int row = t * 32 + l32;
        const unsigned char* rh = smem + row * LY::ROW_B;
        const int sw = LY::kswz(row);
        if constexpr (BLK == 64) {
          f32x16 la;
#pragma unroll
          for (int i = 0; i < 16; ++i) la[i] = 0.0f;
#pragma unroll
          for (int c = 0; c < NC; ++c)
            la = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(rh + (((2 * c + g32) ^ sw) << 4))),
                rq[c], la, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 16; ++i) o[t][i] += la[i] * inv_den;
        } else {
          // no spare registers for a separate sum at 168 per lane: the term goes
          // straight into O, o = (o_s den + S''^T relu(q)) / den
#pragma unroll
          for (int i = 0; i < 16; ++i) o[t][i] *= den;
#pragma unroll
          for (int c = 0; c < NC; ++c)
            o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(rh + (((2 * c + g32) ^ sw) << 4))),
                rq[c], o[t], 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 16; ++i) o[t][i] *= inv_den;
        }
      }
    }
  }

  // stage [ROWS][D] bf16 through LDS, then 16-byte coalesced stores
  __syncthreads();
  __bf16* ost = reinterpret_cast<__bf16*>(smem);
  const bool row_ok = wave_rows && my_row < g.N;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = t * 32 + i4 * 8 + g32 * 4;
      uint2 w = make_uint2(0, 0);
      if (row_ok) w = make_uint2(pack_bf16x2(o[t][i4 * 4 + 0], o[t][i4 * 4 + 1]),
                                 pack_bf16x2(o[t][i4 * 4 + 2], o[t][i4 * 4 + 3]));
      *reinterpret_cast<uint2*>(ost + (wave * 32 + l32) * LY::OST + d0) = w;
    }
  __syncthreads();
  __bf16* Ob = static_cast<__bf16*>(a.out) + (int64_t)bh * g.n_pad * D;
  constexpr int CPR = D / 8;
  for (int ch = tid; ch < ROWS * CPR; ch += THREADS) {
    const int r = ch / CPR, dc = ch % CPR;
    const int row = qb_base * BLK + r;
    if (row < g.n_pad)
      *reinterpret_cast<uint4*>(Ob + (int64_t)row * D + dc * 8) =
          *reinterpret_cast<const uint4*>(ost + r * LY::OST + dc * 8);
  }
}

template <int D, int BLK>
hipError_t launch(const Geom& g, const AttnArgs& a, hipStream_t st) {
  constexpr int QPW = 128 / BLK;
  const int qgroups = (g.nb + QPW - 1) / QPW;
  const int n_items = g.B * g.Hh * qgroups;
  // work per item in tile steps: kept blocks times tiles per block, plus
  // about three 64-key steps for the item's own loads and epilogue
  constexpr int KT = tile_keys<BLK>();
  constexpr int TPB = BLK / KT;
  ItemSplit job{a.row_ptr, a.split, g.B * g.Hh, g.nb, QPW, TPB, 3 * 64 / KT};
  if (KT == 64 && QPW == 2) {
    job.col = a.col_idx;
    job.mode_heads = g.Hh;
  }
  hipError_t e = launch_item_splits(&job, 1, st);
  if (e != hipSuccess) return e;
  const int grid = 8 * xcd_items_cap(n_items);
  const float c_log2 = a.scale * 1.4426950408889634f;
  hipLaunchKernelGGL((k_attn_bf16<D, BLK>), dim3(grid), dim3(256), 0, st, g, a, n_items, c_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const Geom& g, const AttnArgs& a, hipStream_t st) {
  if (g.D == 128) return g.blk == 64 ? launch<128, 64>(g, a, st) : launch<128, 128>(g, a, st);
  return g.blk == 64 ? launch<64, 64>(g, a, st) : launch<64, 128>(g, a, st);
}

}  // namespace salad
