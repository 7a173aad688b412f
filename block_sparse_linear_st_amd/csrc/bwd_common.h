// bwd_common.h - LDS tile layout and MFMA fragment helpers of the backward
// kernels (v_mfma_f32_32x32x16_bf16, fp32 accumulate).
//
// Operand layouts of the 32x32x16 bf16 MFMA, lane l = 32*g + m (g = l/32):
//   A (32 x 16): lane l holds A[m][8g .. 8g+7];  B (16 x 32): B[8g .. 8g+7][m];
//   C (32 x 32): register i of lane l holds C[8*(i/4) + 4g + i%4][m].
// A tile of C whose column index is the lane (a query or a key) therefore
// serves directly as the B operand of the next product when its 32 rows are
// the contraction: for 16-row step h2 the lane's slot j carries row
// 16*h2 + 8*(j/4) + 4g + j%4 ("slot order"); the matching A operand is read
// from a row-major LDS tile with the transpose read ds_read_b64_tr_b16, which
// hands lane l the column 32t + m of 4 consecutive rows.
//
// LDS tiles hold rows of D bf16 in 16-byte chunks, chunk p of row r stored at
// chunk p ^ swz(r).  swz gives 16 consecutive rows 16 different chunks (direct
// 16-byte fragment reads of one logical chunk: conflict free) and puts 4
// consecutive rows in 4 disjoint groups of 4 chunks (transpose reads: conflict
// free).
#pragma once

#include "internal.h"

namespace salad {
namespace bwd {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int D>
struct TileLay {
  static constexpr int CPR = D / 8;        // 16-byte chunks per row
  static constexpr int ROW_B = D * 2;      // bytes per row
  static constexpr int RPB = 16 / CPR;     // rows per 256-byte bank period
  __host__ __device__ static constexpr int swz(int r) { return 4 * ((r / RPB) % (4 / RPB)) + ((r >> 2) & 3); }
  __host__ __device__ static constexpr int off(int r, int chunk) { return r * ROW_B + ((chunk ^ swz(r)) << 4); }
  // The offset rebuild used by the dQ kernel: for every row r < 16 and chunk,
  // rows r + 16 k (k < 4) have the same swizzle, chunk 2c + x is the chunk-x
  // offset XOR (c << 5), chunk 4t + x is the chunk-x offset XOR (t << 6), and
  // for r < 8 row r + 8 is row r's chunk-(x ^ 2) offset plus 8 rows.
  static constexpr bool xor_rebuild_holds() {
    for (int r = 0; r < 16; ++r)
      for (int x = 0; x < CPR; ++x) {
        for (int k = 1; k < 4; ++k)
          if (off(r + 16 * k, x) != off(r, x) + 16 * k * ROW_B) return false;
        for (int c = 0; 2 * c + (x & 1) < CPR; ++c)
          if ((x & 1) == x && off(r, 2 * c + x) != (off(r, x) ^ (c << 5))) return false;
        for (int t = 0; 4 * t + (x & 3) < CPR; ++t)
          if (x < 4 && off(r, 4 * t + x) != (off(r, x) ^ (t << 6))) return false;
        if (r < 8 && x < 4 && off(r + 8, x) != off(r, x ^ 2) + 8 * ROW_B) return false;
      }
    return true;
  }
  static_assert(CPR == 8 || CPR == 16, "head_dim 64 or 128");
};
static_assert(TileLay<64>::xor_rebuild_holds() && TileLay<128>::xor_rebuild_holds(),
              "LDS offset rebuild by XOR does not match the swizzle");

__device__ inline f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline void zero(f32x16& c) {
#pragma unroll
  for (int i = 0; i < 16; ++i) c[i] = 0.0f;
}

__device__ inline uint32_t pack2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// Row m of a C tile, as the B operand of a product whose contraction runs over
// the tile's rows: step h2 (rows 16*h2 .. 16*h2+15 in slot order).
__device__ inline bf16x8 c_to_b(const f32x16& c, int h2) {
  return __builtin_bit_cast(bf16x8, make_uint4(pack2(c[8 * h2 + 0], c[8 * h2 + 1]), pack2(c[8 * h2 + 2], c[8 * h2 + 3]),
                                               pack2(c[8 * h2 + 4], c[8 * h2 + 5]), pack2(c[8 * h2 + 6], c[8 * h2 + 7])));
}

// Direct fragment: lane l gets tile[r0 + l%32][16*c + 8*(l/32) .. +7]
// (A operand with rows = tile rows, or B operand with columns = tile rows;
// contraction over the tile's columns).
template <int D>
__device__ inline bf16x8 frag_direct(const unsigned char* tile, int r0, int c, int lane) {
  using TL = TileLay<D>;
  const int r = r0 + (lane & 31);
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(tile + TL::off(r, 2 * c + (lane >> 5))));
}

// Transposed fragment: lane l gets tile[rows 16*ks + slot order][32*t + l%32]
// (A operand whose rows are tile columns 32t .. 32t+31, contraction over the
// tile rows 16ks .. 16ks+15 in slot order).
template <int D>
__device__ inline bf16x8 frag_tr(const unsigned char* tile, int ks, int t, int lane) {
  using TL = TileLay<D>;
  const int sl = lane & 15, dh = (lane >> 4) & 1, g = lane >> 5;
  const int chunk = 4 * t + 2 * dh + ((sl & 3) >> 1);
  uint2 tr[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = ks * 16 + 8 * h + 4 * g + (sl >> 2);
    const unsigned char* ad = tile + TL::off(row, chunk) + (sl & 1) * 8;
    tr[h] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                          (__attribute__((address_space(3))) s16x4*)(ad)));
  }
  return __builtin_bit_cast(bf16x8, make_uint4(tr[0].x, tr[0].y, tr[1].x, tr[1].y));
}

// s_waitcnt vmcnt(0) as a compiler-visible instruction (gfx9 encoding: vmcnt 0,
// expcnt 7, lgkmcnt 15).
__device__ __attribute__((always_inline)) inline void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// One direct HBM -> LDS load: lane l's 16 bytes at gptr land at LDS byte
// address m0_base + 16 l.  Inline asm with no register result, so that the
// compiler does not hold LDS reads of the other buffer behind it; callers wait
// with wait_vmem() before the barrier that publishes the buffer.
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

// DMA of a ROWS-row tile (64, or 32) of a row-major [*, D] bf16 array into a
// swizzled LDS tile.  NW waves share it; wave w fills its 1 KiB blocks
// w*LOADS .. w*LOADS+LOADS-1.  The per-lane byte offsets inside a tile do not
// depend on the tile: they are computed once.
template <int D, int NW, int ROWS = 64>
struct TileDma {
  using TL = TileLay<D>;
  static constexpr int LOADS = ROWS * TL::ROW_B / 1024 / NW;
  static_assert(LOADS >= 1, "tile too small for the waves");
  uint32_t off[LOADS];
  int wave_u, lane;
  __device__ void init(int w, int l) {
    wave_u = w;
    lane = l;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int P = (w * LOADS + i) * 64 + l;
      const int r = P / TL::CPR, p = P % TL::CPR;
      off[i] = (uint32_t)(r * TL::ROW_B + ((p ^ TL::swz(r)) << 4));
    }
  }
  // rows [row0, row0 + ROWS) into the tile at LDS byte address lds; rows past
  // `last` repeat row `last` (only in the tile that holds it)
  __device__ __attribute__((always_inline)) void issue(uint32_t lds, const __bf16* src, int row0, int last) const {
    if (row0 + ROWS <= last + 1) {
      const __bf16* base = uniform_ptr(src + (int64_t)row0 * D);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) lds_dma16_s(off[i], base, lds + (wave_u * LOADS + i) * 1024);
      return;
    }
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int P = (wave_u * LOADS + i) * 64 + lane;
      const int r = P / TL::CPR, p = P % TL::CPR;
      const int gr = min(row0 + r, last);
      lds_dma16(src + (int64_t)gr * D + ((p ^ TL::swz(r)) << 3), lds + (wave_u * LOADS + i) * 1024);
    }
  }
};

__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)p;
}

// fp32 value rounded to bf16 (hi) and the bf16 of the remainder (lo).
__device__ inline void split_hi_lo(float x, __bf16& hi, __bf16& lo) {
  hi = (__bf16)x;
  lo = (__bf16)(x - (float)hi);
}

__device__ inline bf16x8 relu8(bf16x8 x) {
  uint4 u = __builtin_bit_cast(uint4, x);
  auto r = [](uint32_t w) {
    return ((w & 0x8000u) ? 0u : (w & 0xffffu)) | ((w & 0x80000000u) ? 0u : (w & 0xffff0000u));
  };
  u.x = r(u.x); u.y = r(u.y); u.z = r(u.z); u.w = r(u.w);
  return __builtin_bit_cast(bf16x8, u);
}

__device__ inline float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// C-layout row index of register i for lane group g
__device__ inline int crow(int i, int g) { return 8 * (i >> 2) + 4 * g + (i & 3); }

// The fp32 values of `row` (global, 16-byte aligned) at the C-layout rows of this
// lane group: out[t][i] = row[32*t + crow(i, g)] (D/8 loads of 16 bytes, all
// issued before any is used).
template <int D>
__device__ inline void rows_f32(const float* row, int g, float (&out)[D / 32][16]) {
  float4 w[D / 32][4];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int q = 0; q < 4; ++q) w[t][q] = *reinterpret_cast<const float4*>(row + 32 * t + 8 * q + 4 * g);
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      out[t][4 * q + 0] = w[t][q].x;
      out[t][4 * q + 1] = w[t][q].y;
      out[t][4 * q + 2] = w[t][q].z;
      out[t][4 * q + 3] = w[t][q].w;
    }
}

// Scheduling groups (same mask bits as the scheduling barrier): the next
// `n` instructions of a kind, in program order, form a group.
#define SG_MFMA(n) __builtin_amdgcn_sched_group_barrier(0x008, (n), 0)
#define SG_DSREAD(n) __builtin_amdgcn_sched_group_barrier(0x100, (n), 0)
#define SG_VMREAD(n) __builtin_amdgcn_sched_group_barrier(0x020, (n), 0)

// Which of the D bf16 values of `row` (global, 16-byte aligned) at the C-layout
// rows of this lane group are > 0: bit 16*t + i stands for row[32*t + crow(i, g)].
// Those are D/8 runs of 4 consecutive values; all loads are issued first.
template <int D>
__device__ inline uint64_t positive_rows(const __bf16* row, int g) {
  uint2 w[D / 32][4];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int q = 0; q < 4; ++q) w[t][q] = *reinterpret_cast<const uint2*>(row + 32 * t + 8 * q + 4 * g);
  uint64_t m = 0;
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t v = ((r < 2 ? w[t][q].x : w[t][q].y) >> (16 * (r & 1))) & 0xffffu;
        const uint32_t mag = v & 0x7fffu;
        const bool pos = !(v & 0x8000u) && mag != 0u && mag <= 0x7f80u;  // > 0, not NaN
        m |= (uint64_t)pos << (16 * t + 4 * q + r);
      }
  return m;
}

}  // namespace bwd
}  // namespace salad
