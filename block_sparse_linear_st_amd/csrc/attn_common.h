// attn_common.h - LDS tile layout, direct HBM -> LDS loads and small lane
// helpers of the bf16 forward attention kernel (attn_bf16.hip).
//
// MFMA 32x32x16 bf16 operand layouts, lane l = 32*g + m (g = l/32):
//   A (32 x 16): lane l holds A[m][8g .. 8g+7];  B (16 x 32): B[8g .. 8g+7][m];
//   C (32 x 32): register i of lane l holds C[8*(i/4) + 4g + i%4][m].
#pragma once

#include "internal.h"

namespace salad {
namespace fwd {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
typedef __attribute__((address_space(3))) void* lds_ptr;

// KT keys per LDS tile: 64, or 32 for 128-token blocks (a smaller tile leaves
// room for three workgroups per CU).
template <int D, int KT, int NW = 4>
struct Lay {
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int ROW_B = D * 2;           // bytes per row
  static constexpr int TILE_B = KT * ROW_B;     // one K or V tile
  static constexpr int BUF_B = 2 * TILE_B;      // K then V
  static constexpr int RPB = 16 / CPR;          // rows per 256-byte bank period
  static constexpr int LOADS = KT * CPR / (64 * NW);  // 1 KiB loads per wave per tile (K or V), NW waves
  static constexpr int OST = D + 8;             // output staging stride (bf16)
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

// 0 for a key at offset kofs < rem inside its tile, -inf past it (rem = keys of
// the tile below N, for this lane): an arithmetic select, so that masking a
// tile's 16 or 32 scores keeps no compare masks alive in scalar registers.
__device__ __attribute__((always_inline)) inline float past_n_bias(int rem, int kofs) {
  return __int_as_float((int)(((uint32_t)((rem - 1 - kofs) >> 31)) & 0xff800000u));
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
template <int D, int KT, int NW = 4>
struct DmaOffsets {
  uint32_t k[Lay<D, KT, NW>::LOADS], v[Lay<D, KT, NW>::LOADS];
  __device__ void init(int wave, int lane) {
    using LY = Lay<D, KT, NW>;
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
// `buf` (NW waves share them).  Whole tiles use a uniform base plus the fixed lane offsets;
// the tile that runs past the last valid token loads row N-1 in place of the
// missing rows (always in bounds, always finite); their scores are masked to
// -inf, so they contribute exact zeros.
template <int D, int KT, int NW = 4>
__device__ __attribute__((always_inline)) inline void issue_tile(uint32_t buf, const __bf16* Kb,
                                                                 const __bf16* Vb, int key0, int N,
                                                                 int wave, int lane,
                                                                 const DmaOffsets<D, KT, NW>& off) {
  using LY = Lay<D, KT, NW>;
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

// The loads of one K tile or one V tile alone (IS_K: the K swizzle, else the
// V swizzle) into the LDS tile at byte address `tile`, shared by NW waves.
template <int D, int KT, int NW, bool IS_K>
__device__ __attribute__((always_inline)) inline void issue_half(uint32_t tile, const __bf16* Xb, int key0, int N,
                                                                 int wave, int lane,
                                                                 const DmaOffsets<D, KT, NW>& off) {
  using LY = Lay<D, KT, NW>;
  if (key0 + KT <= N) {
    const __bf16* base = uniform_ptr(Xb + (int64_t)key0 * D);
#pragma unroll
    for (int i = 0; i < LY::LOADS; ++i)
      lds_dma16_s(IS_K ? off.k[i] : off.v[i], base, tile + (wave * LY::LOADS + i) * 1024);
    return;
  }
#pragma unroll
  for (int i = 0; i < LY::LOADS; ++i) {
    const int blk1k = wave * LY::LOADS + i;
    const int P = blk1k * 64 + lane;
    const int r = P / LY::CPR, p = P % LY::CPR;
    const int n = min(max(key0 + r, 0), N - 1);
    const int sw = IS_K ? LY::kswz(r) : LY::vswz(r);
    lds_dma16(Xb + (int64_t)n * D + (p ^ sw) * 8, tile + blk1k * 1024);
  }
}

}  // namespace fwd
}  // namespace salad
