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
// in the lane that owns the query.  The softmax rescale is lazy: the running
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
// (g S W_lin)^T in hi + lo bf16, so g*(o_l W_lin) = (S''^T ReLU(Q)^T) /
// (ReLU(Q) z + eps) is 2*(D/32)*(D/16) more MFMAs on the Q fragments already
// in registers.  Heads whose gate is below drop_tau skip it (section 2.3).  The
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

#include "internal.h"

namespace salad {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
typedef __attribute__((address_space(3))) void* lds_ptr;

// KT keys per LDS tile: 64, or 32 for 128-token blocks (a smaller tile leaves
// room for three workgroups per CU).
template <int D, int KT>
struct Lay {
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int ROW_B = D * 2;           // bytes per row
  static constexpr int TILE_B = KT * ROW_B;     // one K or V tile
  static constexpr int BUF_B = 2 * TILE_B;      // K then V
  static constexpr int RPB = 16 / CPR;          // rows per 256-byte bank period
  static constexpr int LOADS = KT * CPR / 256;  // 1 KiB loads per thread per tile (K or V)
  static constexpr int OST = D + 8;             // output staging stride (bf16)
  static constexpr int SMEM_B = 128 * OST * 2 > 2 * BUF_B ? 128 * OST * 2 : 2 * BUF_B;
  // the folded linear state (hi, lo) goes through LDS in one pass when both fit, else one part at a time
  static constexpr int LIN_PASSES = 2 * D * D * 2 <= SMEM_B ? 1 : 2;
  static_assert(D * D * 2 <= SMEM_B, "one part of the folded linear state must fit");
  // 16 consecutive rows reading one logical chunk hit 16 different physical chunks
  __device__ static int kswz(int r) { return (r / RPB) % CPR; }
  // 4 consecutive rows x 4 consecutive chunks (a half-wave transpose read) are disjoint
  __device__ static int vswz(int r) { return 4 * ((r / RPB) % (CPR / 4)); }
};

__device__ inline bf16x8 load_bf16x8(const __bf16* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__device__ inline bf16x8 relu8(bf16x8 x) {
  uint4 u = __builtin_bit_cast(uint4, x);
  auto r = [](uint32_t w) {
    return ((w & 0x8000u) ? 0u : (w & 0xffffu)) | ((w & 0x80000000u) ? 0u : (w & 0xffff0000u));
  };
  u.x = r(u.x); u.y = r(u.y); u.z = r(u.z); u.w = r(u.w);
  return __builtin_bit_cast(bf16x8, u);
}

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// the own value combined with the one of lane l ^ 32 (max or sum), bit-identical in both lanes
__device__ inline float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// s_waitcnt vmcnt(0) as a compiler-visible instruction (gfx9 encoding: vmcnt 0,
// expcnt 7, lgkmcnt 15), so the compiler knows every vector load has landed.
__device__ __attribute__((always_inline)) inline void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// One direct HBM -> LDS load: every lane's 16 bytes at gptr land at LDS byte
// address m0_base + 16 * lane.  Written as inline asm so that the compiler,
// which cannot tell the two LDS buffers apart, does not stall every LDS read
// until this load lands; the kernel waits for it explicitly (vmcnt) before the
// barrier that publishes the buffer.  The instruction has no register result.
// M0 is set inside the asm; the compiler uses M0 nowhere in these kernels.
__device__ __attribute__((always_inline)) inline void lds_dma16(const void* gptr, uint32_t m0_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(m0_base)
               : "memory", "m0");
}
// The same with a wave-uniform 64-bit base in SGPRs and a 32-bit lane offset.
__device__ __attribute__((always_inline)) inline void lds_dma16_s(uint32_t voff, const void* sbase,
                                                                  uint32_t m0_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m0_base)
               : "memory", "m0");
}

__device__ __attribute__((always_inline)) inline const __bf16* uniform_ptr(const __bf16* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<const __bf16*>(((uint64_t)hi << 32) | lo);
}

// Per-lane byte offsets, inside a tile, of the 16-byte chunks this lane loads
// (row r, logical chunk p ^ swizzle(r)); they do not depend on the tile.
template <int D, int KT>
struct DmaOffsets {
  uint32_t k[Lay<D, KT>::LOADS], v[Lay<D, KT>::LOADS];
  __device__ void init(int wave, int lane) {
    using LY = Lay<D, KT>;
#pragma unroll
    for (int i = 0; i < LY::LOADS; ++i) {
      const int P = (wave * LY::LOADS + i) * 64 + lane;
      const int r = P / LY::CPR, p = P % LY::CPR;
      k[i] = (uint32_t)(r * LY::ROW_B + ((p ^ LY::kswz(r)) << 4));
      v[i] = (uint32_t)(r * LY::ROW_B + ((p ^ LY::vswz(r)) << 4));
    }
  }
};

// Issue the loads of one K and V tile into the LDS buffer at byte address
// `buf`.  Whole tiles use a uniform base plus the fixed lane offsets;
// the tile that runs past the last valid token loads row N-1 in place of the
// missing rows (always in bounds, always finite); their scores are masked to
// -inf, so they contribute exact zeros.
template <int D, int KT>
__device__ __attribute__((always_inline)) inline void issue_tile(uint32_t buf, const __bf16* Kb,
                                                                 const __bf16* Vb, int key0, int N,
                                                                 int wave, int lane,
                                                                 const DmaOffsets<D, KT>& off) {
  using LY = Lay<D, KT>;
  if (key0 + KT <= N) {
    const __bf16* kbase = uniform_ptr(Kb + (int64_t)key0 * D);
    const __bf16* vbase = uniform_ptr(Vb + (int64_t)key0 * D);
#pragma unroll
    for (int i = 0; i < LY::LOADS; ++i) {
      const uint32_t m0 = buf + (wave * LY::LOADS + i) * 1024;
      lds_dma16_s(off.k[i], kbase, m0);
      lds_dma16_s(off.v[i], vbase, m0 + LY::TILE_B);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < LY::LOADS; ++i) {
    const int blk1k = wave * LY::LOADS + i;  // which 1 KiB of the tile this instruction fills
    const int P = blk1k * 64 + lane;         // physical 16-byte chunk in the tile
    const int r = P / LY::CPR, p = P % LY::CPR;
    const int n = min(max(key0 + r, 0), N - 1);
    lds_dma16(Kb + (int64_t)n * D + (p ^ LY::kswz(r)) * 8, buf + blk1k * 1024);
    lds_dma16(Vb + (int64_t)n * D + (p ^ LY::vswz(r)) * 8, buf + LY::TILE_B + blk1k * 1024);
  }
}

// S^T, softmax and O^T update of one wave on one 64-key tile held in buffer
// CUR; ka, va are the per-lane read offsets.
template <int D, int CUR>
__device__ __attribute__((always_inline)) inline void compute_tile64(const unsigned char* smem, const uint32_t (&ka)[D / 16],
                                    const uint32_t (&va)[D / 32], const bf16x8 (&qf)[D / 16],
                                    f32x16 (&o)[D / 32], float& m_used, float& l_run, int key0,
                                    int N, float c_log2, int lane) {
  using LY = Lay<D, 64>;
  constexpr int NC = D / 16, NT = D / 32;
  const int g32 = lane >> 5, l32 = lane & 31;
  const unsigned char* Kt = smem + CUR * LY::BUF_B;
  const unsigned char* Vt = Kt + LY::TILE_B;

  // S^T = K Q^T: two accumulator chains (key rows 0-31 and 32-63) interleaved,
  // K fragments read two contraction steps ahead of their MFMA
  f32x16 s[2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[kt][i] = 0.0f;
  {
    // ka[c]: byte offset of row l32's chunk (2c + g32) inside a K tile (row 32 + l32 has the same swizzle)
    auto kfrag = [&](int half, int c) __attribute__((always_inline)) {
      return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(Kt + ka[c] + half * 32 * LY::ROW_B));
    };
    bf16x8 a0 = kfrag(0, 0), b0 = kfrag(1, 0);
    bf16x8 a1 = kfrag(0, 1), b1 = kfrag(1, 1);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      bf16x8 a2 = a1, b2 = b1;
      if (c + 2 < NC) { a2 = kfrag(0, c + 2); b2 = kfrag(1, c + 2); }
      s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[c], s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b0, qf[c], s[1], 0, 0, 0);
      a0 = a1; b0 = b1; a1 = a2; b1 = b2;
    }
  }
  // mask padded keys (only the tile that holds token N-1 and beyond)
  if (key0 + 64 > N) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = key0 + kt * 32 + (i >> 2) * 8 + g32 * 4 + (i & 3);
        if (key >= N) s[kt][i] = -INFINITY;
      }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][i]);
  mx = pair_max(mx) * c_log2;
  // lazy rescale: move the reference max only when some row grew by more than 2^8
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
  // P in bf16; the row sum adds the same rounded values the PV product uses
  // (v_dot2 with (1, 1) sums a packed pair in fp32)
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float rs = 0.0f;
  bf16x8 pf[4];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float p[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) p[j] = __builtin_amdgcn_exp2f(fmaf(s[kt][h * 8 + j], c_log2, neg_m));
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        w[j] = pack_bf16x2(p[2 * j], p[2 * j + 1]);
        rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[j]), ones, rs, false);
      }
      pf[kt * 2 + h] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
    }
  l_run += pair_sum(rs);

  // O^T += V^T P^T.  For 16-key step ks and half h, lane (group a = lane/16,
  // s = lane%16) points the transpose read at key ks*16 + 8h + 4*g32 + s/4 and
  // channels t*32 + 16*(a%2) + 4*(s%4) .. +3; lane i of the group then holds
  // channel t*32 + 16*(a%2) + i of those 4 keys, which are the keys its P
  // fragment carries in slots 4h .. 4h+3.
  // The NT output tiles are independent chains; the V fragments of the next
  // 16-key step are read while the current step's MFMAs run.
  // va[t]: byte offset, inside a V tile, of this lane's transpose-read address for
  // output tile t at 16-key step 0, half 0; steps and halves add whole rows
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
  bf16x8 vf[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) vf[t] = vfrag(t, 0);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    bf16x8 vn[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) vn[t] = ks + 1 < 4 ? vfrag(t, ks + 1) : vf[t];
#pragma unroll
    for (int t = 0; t < NT; ++t)
      o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[t], pf[ks], o[t], 0, 0, 0);
#pragma unroll
    for (int t = 0; t < NT; ++t) vf[t] = vn[t];
  }
}

// The same on one 32-key tile: one QK^T chain; kbase, vbase are the per-lane
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
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = key0 + (i >> 2) * 8 + g32 * 4 + (i & 3);
      if (key >= N) s[i] = -INFINITY;
    }
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

// 64-key tiles for 64-token blocks (64 KiB of LDS at head_dim 128, two
// workgroups per CU); 32-key tiles for 128-token blocks, whose workgroups walk
// one block's list with every wave active: 35 KiB of LDS and at most 168
// registers give three workgroups (three waves per SIMD) per CU.
template <int BLK>
constexpr int tile_keys() { return BLK == 128 ? 32 : 64; }

template <int D, int BLK>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(tile_keys<BLK>() == 32 ? 3 : 2, tile_keys<BLK>() == 32 ? 3 : 2)))
k_attn_bf16(Geom g, AttnArgs a, int n_items, float c_log2) {
  constexpr int KT = tile_keys<BLK>();
  using LY = Lay<D, KT>;
  constexpr int QPW = 128 / BLK;  // query blocks per workgroup
  constexpr int NC = D / 16;
  constexpr int NT = D / 32;
  constexpr int TPB = BLK / KT;   // tiles per key block
  __shared__ __align__(1024) unsigned char smem[LY::SMEM_B];

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
    DmaOffsets<D, KT> doff;
    doff.init(wave_u, lane);
    if (valid) issue_tile<D, KT>(lds0, Kb, Vb, kb * BLK + sub * KT, g.N, wave_u, lane, doff);
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
        issue_tile<D, KT>(lds0 + (CUR ^ 1) * LY::BUF_B, Kb, Vb, nkb * BLK + nsub * KT, g.N, wave_u, lane,
                          doff);
      if (wave_rows && ((flags >> qsub) & 1)) {
        if constexpr (KT == 64)
          compute_tile64<D, CUR>(smem, ka, va, qf, o, m_used, l_run, kb * BLK + sub * KT, g.N, c_log2, lane);
        else
          compute_tile32<D, CUR>(smem, kbase, vbase, qf, o, m_used, l_run, kb * BLK + sub * KT, g.N, c_log2,
                                 lane);
      }
      wait_vmem();  // the next tile has landed in LDS ...
      __syncthreads();  // ... for every wave, and nobody still reads the current one
      kb = nkb; sub = nsub; flags = nflags; valid = nvalid;
    };
    while (valid) {
      step(std::integral_constant<int, 0>{});
      if (!valid) break;
      step(std::integral_constant<int, 1>{});
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
    if constexpr (LY::LIN_PASSES == 1) {
      // S''^T (hi, lo) of this head into LDS, rows swizzled like K tiles: every
      // wave reads all of it, so one copy per workgroup instead of one per wave
      const __bf16* hi = static_cast<const __bf16*>(a.sft_hi) + (int64_t)bh * D * D;
      const __bf16* lo = static_cast<const __bf16*>(a.sft_lo) + (int64_t)bh * D * D;
      const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;
      const int wave_u = __builtin_amdgcn_readfirstlane(wave);
      constexpr int PER = D * LY::CPR / 256;  // 1 KiB loads per wave per matrix
      __syncthreads();  // the tile buffers are free
  #pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int blk1k = wave_u * PER + i;
        const int P = blk1k * 64 + lane;
        const int r = P / LY::CPR, p = P % LY::CPR;
        lds_dma16(hi + r * D + (p ^ LY::kswz(r)) * 8, lds0 + blk1k * 1024);
        lds_dma16(lo + r * D + (p ^ LY::kswz(r)) * 8, lds0 + D * D * 2 + blk1k * 1024);
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
      den = pair_sum(den);
      const float inv_den = 1.0f / (den + a.eps);
      wait_vmem();
      __syncthreads();
      if (wave_rows) {
  #pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int row = t * 32 + l32;
          const unsigned char* rh = smem + row * LY::ROW_B;
          const unsigned char* rl = rh + D * D * 2;
          const int sw = LY::kswz(row);
          f32x16 la;
  #pragma unroll
          for (int i = 0; i < 16; ++i) la[i] = 0.0f;
  #pragma unroll
          for (int c = 0; c < NC; ++c) {
            const int off = ((2 * c + g32) ^ sw) << 4;
            la = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(rh + off)), rq[c], la, 0, 0, 0);
            la = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(rl + off)), rq[c], la, 0, 0, 0);
          }
  #pragma unroll
          for (int i = 0; i < 16; ++i) o[t][i] += la[i] * inv_den;
        }
      }
  
    } else {
      // S''^T hi, then lo, through LDS one part at a time; the linear term goes
      // straight into O: o = (o_s den + S''^T relu(q)) / den
      const __bf16* part[2] = {static_cast<const __bf16*>(a.sft_hi) + (int64_t)bh * D * D,
                               static_cast<const __bf16*>(a.sft_lo) + (int64_t)bh * D * D};
      const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;
      const int wave_u = __builtin_amdgcn_readfirstlane(wave);
      constexpr int PER = D * LY::CPR / 256;  // 1 KiB loads per wave per matrix
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
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[t][i] *= den;
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        __syncthreads();  // the buffers are free
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          const int blk1k = wave_u * PER + i;
          const int P = blk1k * 64 + lane;
          const int r = P / LY::CPR, p = P % LY::CPR;
          lds_dma16(part[pp] + r * D + (p ^ LY::kswz(r)) * 8, lds0 + blk1k * 1024);
        }
        wait_vmem();
        __syncthreads();
        if (wave_rows) {
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const unsigned char* rh = smem + (t * 32 + l32) * LY::ROW_B;
            const int sw = LY::kswz(t * 32 + l32);
#pragma unroll
            for (int c = 0; c < NC; ++c)
              o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(rh + (((2 * c + g32) ^ sw) << 4))),
                  rq[c], o[t], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[t][i] *= inv_den;
    }
  }

  // stage [128 rows][D] bf16 through LDS, then 16-byte coalesced stores
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
  for (int ch = tid; ch < 128 * CPR; ch += 256) {
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
  // work per item in tile steps: kept key blocks times tiles per block, plus
  // about three 64-key steps for the item's own loads and epilogue
  constexpr int TPB = BLK / tile_keys<BLK>();
  const ItemSplit job{a.row_ptr, a.split, g.B * g.Hh, g.nb, QPW, TPB, 3 * 64 / tile_keys<BLK>()};
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
