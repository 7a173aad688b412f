// linear.hip - the ReLU linear-attention state on gfx950.
//
// S[b,h] = sum_n ReLU(k_n) v_n^T and z[b,h] = sum_n ReLU(k_n) over the valid
// tokens ("SALAD" explainer, technical summary section 2.1: ReLU linear
// attention, O(N)).  Two passes:
//
//  1. k_lin_partial_*: grid (splits, B*H).  Each workgroup reduces one token
//     chunk of one head into a D x D fp32 partial.  The bf16 kernel streams
//     64-token tiles of K and V straight into LDS through a ring of four
//     buffers (three tiles in flight while one is reduced: one workgroup per
//     CU keeps 96 KiB of loads outstanding against HBM latency) and runs
//     32x32x16 bf16 MFMAs with the token index as the contraction; both
//     operands are read with the LDS transpose read, ReLU is applied to the K
//     fragment in registers.  Products of bf16 values are exact and the sums
//     are fp32.  The fp32 kernel does the same with VALU FMAs.
//     For the fused bf16 forward the workgroup multiplies its partial by W_lin
//     before storing it (the partial S_c W_lin of chunk c, by linearity), with
//     W_lin staged in LDS beside the ring and the fp32 partial split into
//     hi + lo bf16 MFMA operands, so that the fold needs no W_lin.
//  2. k_lin_fold: grid (B*H, D/2).  Sums the partials over the splits in a fixed
//     order (bitwise reproducible; loads batched 8 splits deep), then, for the
//     fused forward, folds gate and
//     projection into the state:  S'' = g * S * W_lin, so that the attention
//     epilogue computes g*(o_l W_lin) = ReLU(q)^T S'' / (ReLU(q)^T z + eps) with
//     one product.  S'' is stored transposed ([dv][dk]) because that is the
//     operand layout the attention epilogue reads; for the bf16 kernels it is
//     rounded to bf16 once, the MFMA operand type, as the attention kernel
//     rounds the probabilities P before the PV product.
#include <algorithm>

#include "internal.h"

namespace salad {
namespace {

constexpr int kTok = 64;  // tokens staged per LDS tile

__device__ inline uint32_t relu_bf16x2(uint32_t w) {
  // zero each 16-bit half whose sign bit is set (negative values and -0)
  uint32_t lo = (w & 0x8000u) ? 0u : (w & 0xffffu);
  uint32_t hi = (w & 0x80000000u) ? 0u : (w & 0xffff0000u);
  return lo | hi;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr;

// s_waitcnt vmcnt(0) as a compiler-visible instruction (gfx9 encoding)
__device__ __attribute__((always_inline)) inline void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// one direct HBM -> LDS load (lane l's 16 bytes land at m0_base + 16 l); inline
// asm so that the compiler does not stall LDS reads of the other buffer on it
__device__ __attribute__((always_inline)) inline void lds_dma16(const void* gptr, uint32_t m0_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(m0_base)
               : "memory", "m0");
}

__device__ __attribute__((always_inline)) inline uint4 relu_u4(uint4 u) {
  u.x = relu_bf16x2(u.x); u.y = relu_bf16x2(u.y); u.z = relu_bf16x2(u.z); u.w = relu_bf16x2(u.w);
  return u;
}

// Token-major tiles of K and V (64 tokens x D bf16) go HBM -> LDS directly.
// Both MFMA operands need 8 tokens of one channel per lane: they come from the
// gfx950 LDS transpose read.  For 16-token step ks and half h, lane (group
// a = lane/16, s = lane%16) points at token ks*16 + 8h + 4*(lane/32) + s/4 and
// channels c0 + 16*(a%2) + 4*(s%4) .. +3; lane i of the group receives channel
// c0 + 16*(a%2) + i of those 4 tokens, i.e. operand slots 4h .. 4h+3.  A and B
// use the same token for the same slot, so the contraction is over tokens.
template <int D>
struct LinLay {
  static constexpr int CPR = D / 8;
  static constexpr int ROW_B = D * 2;
  static constexpr int TILE_B = kTok * ROW_B;
  static constexpr int BUF_B = 2 * TILE_B;
  static constexpr int RPB = 16 / CPR;
  static constexpr int LOADS = kTok * CPR / 256;
  __device__ static int swz(int r) { return 4 * ((r / RPB) % (CPR / 4)); }
};

template <int D>
__device__ __attribute__((always_inline)) inline bf16x8 tr_frag(const unsigned char* tile, int ks, int c0,
                                                               int lane) {
  using LY = LinLay<D>;
  const int sl = lane & 15, a = lane >> 4;
  const int chunk = (c0 >> 3) + 2 * (a & 1) + ((sl & 3) >> 1);
  uint2 tr[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = ks * 16 + 8 * h + 4 * (lane >> 5) + (sl >> 2);
    const unsigned char* ad = tile + row * LY::ROW_B + ((chunk ^ LY::swz(row)) << 4) + (sl & 1) * 8;
    tr[h] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                          (__attribute__((address_space(3))) s16x4*)(ad)));
  }
  return __builtin_bit_cast(bf16x8, make_uint4(tr[0].x, tr[0].y, tr[1].x, tr[1].y));
}

// vmcnt(n) as an s_waitcnt immediate (gfx9: low 4 bits at [3:0], high 2 at [15:14];
// expcnt and lgkmcnt left at their maxima)
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// PREMUL: the workgroup's partial is stored as S_c W_lin instead of S_c.  The
// MFMA operands are then swapped so that the accumulators hold S_c^T (a lane
// owns one K channel, its registers run over V channels): split into hi + lo
// bf16 they are the A operand of S_c W_lin directly, contracted over the V
// channel, with W_lin read from LDS by the same transpose read as a V tile.
template <int D, bool PREMUL>
__global__ void __launch_bounds__(256, 1)
k_lin_partial_bf16(Geom g, const __bf16* __restrict__ K, const __bf16* __restrict__ V, int chunk,
                   float* __restrict__ spart, float* __restrict__ zpart, const float* __restrict__ gate,
                   float drop_tau, const __bf16* __restrict__ W) {
  using LY = LinLay<D>;
  constexpr int TD = D / 32;           // 32-wide output tiles per dimension
  constexpr int TPW = TD * TD / 4;     // output tiles per wave
  constexpr int RING = 4;              // tile buffers: three tiles in flight while one is reduced
  constexpr int PER = 2 * LY::LOADS;   // DMA instructions per thread per tile
  constexpr int W_B = PREMUL ? D * LY::ROW_B : 0;  // W_lin, rows laid out like a V tile's
  // 160 KiB at D = 128: the whole of a gfx950 CU's LDS
  __shared__ __align__(1024) unsigned char smem[RING * LY::BUF_B + W_B];

  const int split = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n0 = split * chunk, n1 = min(g.N, n0 + chunk);
  const int T = (n1 - n0 + kTok - 1) / kTok;
  const __bf16* Kb = K + (int64_t)bh * g.n_pad * D;
  const __bf16* Vb = V + (int64_t)bh * g.n_pad * D;
  const int ti = TD == 4 ? wave : wave >> 1;
  const int tj0 = TD == 4 ? 0 : (wave & 1);

  f32x16 acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[t][i] = 0.0f;
  float zacc = 0.0f;

  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  auto issue = [&](int tt) __attribute__((always_inline)) {
    const int t0 = n0 + tt * kTok, buf = tt % RING;
#pragma unroll
    for (int i = 0; i < LY::LOADS; ++i) {
      const int blk1k = wave_u * LY::LOADS + i;
      const int P = blk1k * 64 + lane;
      const int r = P / LY::CPR, p = P % LY::CPR;
      const int n = min(t0 + r, g.N - 1);
      const int c = (p ^ LY::swz(r)) * 8;
      lds_dma16(Kb + (int64_t)n * D + c, lds0 + buf * LY::BUF_B + blk1k * 1024);
      lds_dma16(Vb + (int64_t)n * D + c, lds0 + buf * LY::BUF_B + LY::TILE_B + blk1k * 1024);
    }
  };
  if constexpr (PREMUL) {
    // W_lin (L2-resident after the first workgroups) goes in first: loads
    // complete in order, so the wait for tile 0 covers it too
    constexpr int WL = D * LY::CPR / 256;  // 16-byte pieces per thread
#pragma unroll
    for (int i = 0; i < WL; ++i) {
      const int blk1k = wave_u * WL + i;
      const int P = blk1k * 64 + lane;
      const int r = P / LY::CPR, p = P % LY::CPR;
      lds_dma16(W + r * D + (p ^ LY::swz(r)) * 8, lds0 + RING * LY::BUF_B + blk1k * 1024);
    }
  }
  for (int tt = 0; tt < RING - 1 && tt < T; ++tt) issue(tt);
  // the gate is read once the first tiles are on their way, so that its latency
  // does not delay them
  if (gate != nullptr && gate[bh] < drop_tau) {  // dropped head: no linear state
    wait_vmem();
    return;
  }
  for (int tt = 0; tt < T; ++tt) {
    // tile tt has landed once at most min(T - 1 - tt, RING - 2) later tiles are outstanding
    const int ahead = min(T - 1 - tt, RING - 2);
    if (ahead >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * PER));
    else if (ahead == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER));
    else wait_vmem();
    __syncthreads();  // every wave's part of tile tt is in; tile tt - 1's buffer is free
    if (tt + RING - 1 < T) issue(tt + RING - 1);
    const int t0 = n0 + tt * kTok;
    const unsigned char* Kt = smem + (tt % RING) * LY::BUF_B;
    const unsigned char* Vt = Kt + LY::TILE_B;
    const int valid = n1 - t0;  // tokens of this tile inside the chunk
#pragma unroll
    for (int ks = 0; ks < kTok / 16; ++ks) {
      uint4 au = relu_u4(__builtin_bit_cast(uint4, tr_frag<D>(Kt, ks, ti * 32, lane)));
      if (valid < kTok) {  // zero the slots of tokens past the chunk end
        const int tb = ks * 16 + 4 * (lane >> 5);
        if (tb + 0 >= valid) { au.x &= 0xffff0000u; }
        if (tb + 1 >= valid) { au.x &= 0x0000ffffu; }
        if (tb + 2 >= valid) { au.y &= 0xffff0000u; }
        if (tb + 3 >= valid) { au.y &= 0x0000ffffu; }
        if (tb + 8 >= valid) { au.z &= 0xffff0000u; }
        if (tb + 9 >= valid) { au.z &= 0x0000ffffu; }
        if (tb + 10 >= valid) { au.w &= 0xffff0000u; }
        if (tb + 11 >= valid) { au.w &= 0x0000ffffu; }
      }
      const bf16x8 af = __builtin_bit_cast(bf16x8, au);
#pragma unroll
      for (int j = 0; j < 8; ++j) zacc += (float)af[j];
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int tj = TD == 4 ? t : tj0;
        const bf16x8 vf = tr_frag<D>(Vt, ks, tj * 32, lane);
        if constexpr (PREMUL)
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, af, acc[t], 0, 0, 0);  // S^T tile (tj, ti)
        else
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, vf, acc[t], 0, 0, 0);  // S tile (ti, tj)
      }
    }
  }

  // partial S (or S W_lin): lane holds rows (i/4)*8 + (lane/32)*4 + i%4 of row
  // tile ti, column lane%32 of column tile tj
  const int g32 = lane >> 5, l32 = lane & 31;
  float* sp = spart + ((int64_t)split * g.B * g.Hh + bh) * D * D;
  if constexpr (PREMUL) {
    if (T == 0) {  // no tile step waited for W_lin
      wait_vmem();
      __syncthreads();
    }
    // C[dk][j] = sum_dv S[dk][dv] W[dv][j] for this wave's dk tile ti.  acc[t][8 s + e]
    // is S^T[dv][dk] at dv = 32 t + 16 s + 8 (e / 4) + 4 g32 + e % 4, which is the
    // V-channel slot order the transpose read gives W's rows for step 2 t + s.
    constexpr int JT = TD;  // output column tiles
    const unsigned char* Ws = smem + RING * LY::BUF_B;
    f32x16 out[JT];
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
#pragma unroll
      for (int i = 0; i < 16; ++i) out[jt][i] = 0.0f;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int tj = TD == 4 ? t : tj0;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8 ah, al;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = acc[t][8 * s + e];
          ah[e] = (__bf16)x;
          al[e] = (__bf16)(x - (float)ah[e]);
        }
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
          const bf16x8 wf = tr_frag<D>(Ws, 2 * tj + s, jt * 32, lane);
          out[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, wf, out[jt], 0, 0, 0);
          out[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, wf, out[jt], 0, 0, 0);
        }
      }
    }
    if constexpr (TD == 2) {
      // D = 64: waves 2 ti and 2 ti + 1 hold the two V-channel halves of row
      // tile ti; the second passes its sums through ring slot T % RING (free:
      // every wave is past the step that last read it) and the first adds them
      float* xb = reinterpret_cast<float*>(smem + (T % RING) * LY::BUF_B) + ti * (JT * 16 * 64);
      if (tj0 == 1) {
#pragma unroll
        for (int jt = 0; jt < JT; ++jt)
#pragma unroll
          for (int i = 0; i < 16; ++i) xb[(jt * 16 + i) * 64 + lane] = out[jt][i];
      }
      __syncthreads();
      if (tj0 == 1) return;
#pragma unroll
      for (int jt = 0; jt < JT; ++jt)
#pragma unroll
        for (int i = 0; i < 16; ++i) out[jt][i] += xb[(jt * 16 + i) * 64 + lane];
    }
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = ti * 32 + (i >> 2) * 8 + g32 * 4 + (i & 3);
        sp[r * D + jt * 32 + l32] = out[jt][i];
      }
  } else {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int tj = TD == 4 ? t : tj0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = ti * 32 + (i >> 2) * 8 + g32 * 4 + (i & 3);
        sp[r * D + tj * 32 + l32] = acc[t][i];
      }
    }
  }
  // z: the lane pair (l, l^32) covers all tokens of channel ti*32 + l%32
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(zacc), __float_as_uint(zacc), false, false);
  const float zs = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  if (tj0 == 0 && lane < 32) zpart[((int64_t)split * g.B * g.Hh + bh) * D + ti * 32 + l32] = zs;
}

template <int D>
__global__ void __launch_bounds__(256)
k_lin_partial_f32(Geom g, const float* __restrict__ K, const float* __restrict__ V, int chunk,
                  float* __restrict__ spart, float* __restrict__ zpart, const float* __restrict__ gate,
                  float drop_tau) {
  if (gate != nullptr && gate[blockIdx.y] < drop_tau) return;  // dropped head: no linear state
  constexpr int TT = 32;                 // tokens per LDS tile
  constexpr int COLS = D * D / 256;      // outputs per thread (one row segment)
  constexpr int SEGS = D / COLS;         // row segments
  __shared__ float Ks[TT][D], Vs[TT][D];
  const int split = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int n0 = split * chunk, n1 = min(g.N, n0 + chunk);
  const float* Kb = K + (int64_t)bh * g.n_pad * D;
  const float* Vb = V + (int64_t)bh * g.n_pad * D;
  const int r = tid / SEGS, c0 = (tid % SEGS) * COLS;
  float acc[COLS];
#pragma unroll
  for (int j = 0; j < COLS; ++j) acc[j] = 0.0f;
  float zacc = 0.0f;
  for (int nt = n0; nt < n1; nt += TT) {
    __syncthreads();
    for (int i = tid; i < TT * D; i += 256) {
      const int tok = i / D, c = i % D, n = nt + tok;
      Ks[tok][c] = n < n1 ? fmaxf(Kb[(int64_t)n * D + c], 0.0f) : 0.0f;
      Vs[tok][c] = n < n1 ? Vb[(int64_t)n * D + c] : 0.0f;
    }
    __syncthreads();
    for (int tok = 0; tok < TT; ++tok) {
      const float kv = Ks[tok][r];
      zacc += kv;
#pragma unroll
      for (int j = 0; j < COLS; ++j) acc[j] = fmaf(kv, Vs[tok][c0 + j], acc[j]);
    }
  }
  float* sp = spart + ((int64_t)split * g.B * g.Hh + bh) * D * D;
#pragma unroll
  for (int j = 0; j < COLS; ++j) sp[r * D + c0 + j] = acc[j];
  if (c0 == 0) zpart[((int64_t)split * g.B * g.Hh + bh) * D + r] = zacc;
}

// dst[256 u + tid] = src[256 u + tid] for u < N: every load issued before the
// first store
template <int N>
__device__ __attribute__((always_inline)) inline void stage16(const uint4* __restrict__ src,
                                                             uint4* __restrict__ dst, int tid) {
  uint4 x[N];
#pragma unroll
  for (int u = 0; u < N; ++u) x[u] = src[256 * u + tid];
#pragma unroll
  for (int u = 0; u < N; ++u) dst[256 * u + tid] = x[u];
}

// grid (B*H, D/2), 256 threads: reduce 2 rows of S and the same 2 channels of z
// over the splits (in ordered parts), then fold.  mode 0: S'' = g*S*W (WITH_W);
// 1: S'' = S; 2: state only; 3: S'' = g*S, the partials already carrying W_lin.
// In modes 0 and 3 heads with g < drop_tau are skipped (their partials were
// never written).
template <typename WT, bool BF16OUT, bool WITH_W>
__global__ void __launch_bounds__(256)
k_lin_fold(Geom g, int splits, const float* __restrict__ spart, const float* __restrict__ zpart,
           const float* __restrict__ gate, const WT* __restrict__ w, int mode, float drop_tau,
           float* __restrict__ S_out, float* __restrict__ z_out, float* __restrict__ z_ws,
           void* __restrict__ sft) {
  constexpr int FR = 2;  // rows of S per workgroup
  __shared__ float Srows[FR][128];
  __shared__ float4 parts[256];
  __shared__ float zsp[FR][256];  // z of channels r0, r0 + 1: one entry per split (splits <= 256)
  __shared__ WT Ws[WITH_W ? 128 * 128 : 1];  // W_lin, staged once per workgroup (mode 0)
  const int D = g.D, bh = blockIdx.x, r0 = blockIdx.y * FR, tid = threadIdx.x;
  const int64_t BH = (int64_t)g.B * g.Hh;
  if ((mode == 0 || mode == 3) && gate[bh] < drop_tau) return;
  // this workgroup's z entries (channel r0 + i / splits, split i % splits), loaded
  // beside the partial rows so that both take one round trip
  // (indices past the last entry reload it: straight-line loads, none waited on here)
  float zv[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int i = min(tid + 256 * u, FR * splits - 1);
    const int rr = i / splits, sp = i - rr * splits;
    zv[u] = zpart[(int64_t)sp * BH * D + (int64_t)bh * D + r0 + rr];
  }
  const int nvec = FR * D / 4;  // float4s in this row block (64 or 32)
  const int np = 256 / nvec;    // threads per float4 (4 or 8)
  // np threads per float4: part p sums splits [p * len, (p + 1) * len) in
  // split order with loads batched 8 deep; the parts then add in part order
  // (a fixed order, so S is reproducible)
  const int v = tid % nvec, part = tid / nvec;
  const int len = (splits + np - 1) / np;
  const int s0 = min(splits, part * len), s1 = min(splits, s0 + len);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  {
    const int e = v * 4;  // element offset inside the row block
    const float* src = spart + (int64_t)bh * D * D + (int64_t)r0 * D + e;
    const int64_t stride = BH * D * D;
    // up to 8 loads in flight, added in split order
    for (int sp = s0; sp < s1; sp += 8) {
      float4 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (sp + u < s1) x[u] = *reinterpret_cast<const float4*>(src + (sp + u) * stride);
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (sp + u < s1) {
          acc.x += x[u].x; acc.y += x[u].y; acc.z += x[u].z; acc.w += x[u].w;
        }
    }
    parts[tid] = acc;
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int i = tid + 256 * u;
    if (i < FR * splits) {
      const int rr = i / splits;
      zsp[rr][i - rr * splits] = zv[u];
    }
  }
  __syncthreads();
  if (part == 0) {
    for (int p = 1; p < np; ++p) {
      const float4 b = parts[p * nvec + v];
      acc.x += b.x; acc.y += b.y; acc.z += b.z; acc.w += b.w;
    }
    const int e = v * 4, rr = e / D, c = e % D;
    Srows[rr][c] = acc.x; Srows[rr][c + 1] = acc.y; Srows[rr][c + 2] = acc.z; Srows[rr][c + 3] = acc.w;
    if (S_out) *reinterpret_cast<float4*>(S_out + (int64_t)bh * D * D + (int64_t)r0 * D + e) = acc;
  }
  if (tid < FR) {
    // z summed over the splits in split order
    float z = 0.0f;
    for (int sp = 0; sp < splits; ++sp) z += zsp[tid][sp];
    z_ws[(int64_t)bh * D + r0 + tid] = z;
    if (z_out) z_out[(int64_t)bh * D + r0 + tid] = z;
  }
  if (mode == 2) return;
  if constexpr (WITH_W) {
    // 16-byte copies (w_lin is 16-byte aligned), all of a thread's loads in flight at once
    constexpr int PER16 = 16 / (int)sizeof(WT);
    const uint4* src = reinterpret_cast<const uint4*>(w);
    uint4* dst = reinterpret_cast<uint4*>(Ws);
    if (D == 128) stage16<128 * 128 / PER16 / 256>(src, dst, tid);
    else stage16<64 * 64 / PER16 / 256>(src, dst, tid);
  }
  __syncthreads();
  const float gv = mode == 0 || mode == 3 ? gate[bh] : 1.0f;
  // S''[r0+rr][j] for column j, stored transposed at [j][r0+rr]
  for (int i = tid; i < FR * D; i += 256) {
    const int j = i / FR, rr = i % FR;
    float v;
    if (WITH_W) {
      float s = 0.0f;
      for (int kk = 0; kk < D; ++kk) s = fmaf(Srows[rr][kk], (float)Ws[kk * D + j], s);
      v = gv * s;
    } else {
      v = gv * Srows[rr][j];
    }
    const int64_t o = (int64_t)bh * D * D + (int64_t)j * D + r0 + rr;
    if (BF16OUT) static_cast<__bf16*>(sft)[o] = (__bf16)v;
    else static_cast<float*>(sft)[o] = v;
  }
}

}  // namespace

hipError_t launch_linear_state(const Geom& g, int dtype, const void* k, const void* v,
                               const float* gate, float drop_tau, const void* w_lin, char* ws,
                               const Workspace& L, hipStream_t st) {
  float* spart = reinterpret_cast<float*>(ws + L.off_spart);
  float* zpart = reinterpret_cast<float*>(ws + L.off_zpart);
  dim3 grid(L.lin_splits, g.B * g.Hh);
  if (dtype == SALAD_BF16) {
    const __bf16* kb = static_cast<const __bf16*>(k);
    const __bf16* vb = static_cast<const __bf16*>(v);
    const __bf16* wb = static_cast<const __bf16*>(w_lin);
    if (g.D == 128) {
      if (wb)
        hipLaunchKernelGGL((k_lin_partial_bf16<128, true>), grid, dim3(256), 0, st, g, kb, vb, L.lin_chunk,
                           spart, zpart, gate, drop_tau, wb);
      else
        hipLaunchKernelGGL((k_lin_partial_bf16<128, false>), grid, dim3(256), 0, st, g, kb, vb, L.lin_chunk,
                           spart, zpart, gate, drop_tau, wb);
    } else {
      if (wb)
        hipLaunchKernelGGL((k_lin_partial_bf16<64, true>), grid, dim3(256), 0, st, g, kb, vb, L.lin_chunk,
                           spart, zpart, gate, drop_tau, wb);
      else
        hipLaunchKernelGGL((k_lin_partial_bf16<64, false>), grid, dim3(256), 0, st, g, kb, vb, L.lin_chunk,
                           spart, zpart, gate, drop_tau, wb);
    }
  } else {
    if (g.D == 128)
      hipLaunchKernelGGL(k_lin_partial_f32<128>, grid, dim3(256), 0, st, g,
                         static_cast<const float*>(k), static_cast<const float*>(v), L.lin_chunk,
                         spart, zpart, gate, drop_tau);
    else
      hipLaunchKernelGGL(k_lin_partial_f32<64>, grid, dim3(256), 0, st, g,
                         static_cast<const float*>(k), static_cast<const float*>(v), L.lin_chunk,
                         spart, zpart, gate, drop_tau);
  }
  return hipGetLastError();
}

hipError_t launch_linear_fold(const Geom& g, int dtype, const float* gate, const void* w_lin,
                              int mode, float drop_tau, float* S_out, float* z_out, char* ws,
                              const Workspace& L, hipStream_t st) {
  const float* spart = reinterpret_cast<const float*>(ws + L.off_spart);
  const float* zpart = reinterpret_cast<const float*>(ws + L.off_zpart);
  float* z_ws = reinterpret_cast<float*>(ws + L.off_z);
  void* sft = ws + L.off_sft;
  dim3 grid(g.B * g.Hh, g.D / 2);
  if (dtype == SALAD_BF16)  // mode 0: the bf16 partials already carry W_lin
    hipLaunchKernelGGL((k_lin_fold<__bf16, true, false>), grid, dim3(256), 0, st, g, L.lin_splits, spart,
                       zpart, gate, static_cast<const __bf16*>(nullptr), mode == 0 ? 3 : mode, drop_tau, S_out,
                       z_out, z_ws, sft);
  else if (mode == 0)
    hipLaunchKernelGGL((k_lin_fold<float, false, true>), grid, dim3(256), 0, st, g, L.lin_splits, spart,
                       zpart, gate, static_cast<const float*>(w_lin), mode, drop_tau, S_out, z_out, z_ws, sft);
  else
    hipLaunchKernelGGL((k_lin_fold<float, false, false>), grid, dim3(256), 0, st, g, L.lin_splits, spart,
                       zpart, gate, static_cast<const float*>(nullptr), mode, drop_tau, S_out, z_out, z_ws,
                       sft);
  return hipGetLastError();
}

}  // namespace salad
