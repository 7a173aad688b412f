// linear.hip - the ReLU linear-attention state on gfx950.
//
// S[b,h] = sum_n ReLU(k_n) v_n^T and z[b,h] = sum_n ReLU(k_n) over the valid
// tokens ("SALAD" explainer, technical summary section 2.1: ReLU linear
// attention, O(N)).  Two passes:
//
//  1. k_lin_partial_*: grid (splits, B*H).  Each workgroup reduces one token
//     chunk of one head into a D x D fp32 partial.  The bf16 kernel stages 64
//     tokens of ReLU(K) and V in LDS, token-major, and runs 32x32x16 bf16 MFMAs
//     with the token index as the contraction (each operand lane gathers 8
//     tokens of one channel); products of bf16 values are exact and the sums are
//     fp32.  The fp32 kernel does the same with VALU FMAs.
//  2. k_lin_fold: grid (B*H, D/8).  Sums the partials over the splits in a fixed
//     order (bitwise reproducible), then, for the fused forward, folds gate and
//     projection into the state:  S'' = g * S * W_lin, so that the attention
//     epilogue computes g*(o_l W_lin) = ReLU(q)^T S'' / (ReLU(q)^T z + eps) with
//     one product.  S'' is stored transposed ([dv][dk]) because that is the
//     operand layout the attention epilogue reads; for the bf16 kernels it is
//     split into hi + lo bf16 parts (hi = bf16(S''), lo = bf16(S'' - hi)), which
//     keeps about 16 significant bits through the bf16 MFMA.
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

template <int D>
__global__ void __launch_bounds__(256)
k_lin_partial_bf16(Geom g, const __bf16* __restrict__ K, const __bf16* __restrict__ V, int chunk,
                   float* __restrict__ spart, float* __restrict__ zpart) {
  constexpr int ST = D + 8;            // LDS row stride (bf16)
  constexpr int CPR = D / 8;           // 16-byte chunks per token row
  constexpr int NCH = kTok * CPR / 256;  // chunks per thread per tensor
  constexpr int TD = D / 32;           // 32-wide output tiles per dimension
  constexpr int TPW = TD * TD / 4;     // output tiles per wave
  __shared__ __align__(16) __bf16 Ks[kTok * ST];
  __shared__ __align__(16) __bf16 Vs[kTok * ST];
  __shared__ float zred[256 / CPR][D];

  const int split = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n0 = split * chunk, n1 = min(g.N, n0 + chunk);
  const __bf16* Kb = K + (int64_t)bh * g.n_pad * D;
  const __bf16* Vb = V + (int64_t)bh * g.n_pad * D;

  f32x16 acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[t][i] = 0.0f;
  float zacc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) zacc[j] = 0.0f;

  // output tiles of this wave: D=128 -> row tile = wave, col tiles 0..3;
  // D=64 -> row tile wave/2, col tile wave%2
  const int ti = TD == 4 ? wave : wave >> 1;
  const int tj0 = TD == 4 ? 0 : (wave & 1);
  const int gsel = lane >> 5, l32 = lane & 31;

  for (int nt = n0; nt < n1; nt += kTok) {
    uint4 kr[NCH], vr[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = tid + 256 * i, tok = ch / CPR, dc = ch % CPR;
      const int n = nt + tok;
      if (n < n1) {
        kr[i] = *reinterpret_cast<const uint4*>(Kb + (int64_t)n * D + dc * 8);
        vr[i] = *reinterpret_cast<const uint4*>(Vb + (int64_t)n * D + dc * 8);
      } else {
        kr[i] = make_uint4(0, 0, 0, 0);
        vr[i] = make_uint4(0, 0, 0, 0);
      }
      kr[i].x = relu_bf16x2(kr[i].x);
      kr[i].y = relu_bf16x2(kr[i].y);
      kr[i].z = relu_bf16x2(kr[i].z);
      kr[i].w = relu_bf16x2(kr[i].w);
    }
    __syncthreads();  // previous tile fully consumed
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = tid + 256 * i, tok = ch / CPR, dc = ch % CPR;
      *reinterpret_cast<uint4*>(Ks + tok * ST + dc * 8) = kr[i];
      *reinterpret_cast<uint4*>(Vs + tok * ST + dc * 8) = vr[i];
      const uint32_t w[4] = {kr[i].x, kr[i].y, kr[i].z, kr[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        zacc[2 * j] += __uint_as_float(w[j] << 16);
        zacc[2 * j + 1] += __uint_as_float(w[j] & 0xffff0000u);
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kTok / 16; ++ks) {
      const int tok0 = ks * 16 + gsel * 8;
      bf16x8 a;
#pragma unroll
      for (int j = 0; j < 8; ++j) a[j] = Ks[(tok0 + j) * ST + ti * 32 + l32];
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int tj = TD == 4 ? t : tj0;
        bf16x8 b;
#pragma unroll
        for (int j = 0; j < 8; ++j) b[j] = Vs[(tok0 + j) * ST + tj * 32 + l32];
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[t], 0, 0, 0);
      }
    }
  }

  // partial S: lane holds rows (i/4)*8 + gsel*4 + i%4 of tile ti, column l32 of tile tj
  float* sp = spart + ((int64_t)split * g.B * g.Hh + bh) * D * D;
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int tj = TD == 4 ? t : tj0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = ti * 32 + (i >> 2) * 8 + gsel * 4 + (i & 3);
      sp[r * D + tj * 32 + l32] = acc[t][i];
    }
  }
  // z: threads sharing tid % CPR hold the same 8 channels
  const int dc = tid % CPR, grp = tid / CPR;
#pragma unroll
  for (int j = 0; j < 8; ++j) zred[grp][dc * 8 + j] = zacc[j];
  __syncthreads();
  if (tid < D) {
    float s = 0.0f;
    for (int r = 0; r < 256 / CPR; ++r) s += zred[r][tid];
    zpart[((int64_t)split * g.B * g.Hh + bh) * D + tid] = s;
  }
}

template <int D>
__global__ void __launch_bounds__(256)
k_lin_partial_f32(Geom g, const float* __restrict__ K, const float* __restrict__ V, int chunk,
                  float* __restrict__ spart, float* __restrict__ zpart) {
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

// grid (B*H, D/8), 256 threads.  mode 0: S'' = g*S*W; 1: S'' = S; 2: state only.
template <typename WT, bool BF16OUT>
__global__ void __launch_bounds__(256)
k_lin_fold(Geom g, int splits, const float* __restrict__ spart, const float* __restrict__ zpart,
           const float* __restrict__ gate, const WT* __restrict__ w, int mode,
           float* __restrict__ S_out, float* __restrict__ z_out, float* __restrict__ z_ws,
           void* __restrict__ sft_hi, void* __restrict__ sft_lo) {
  constexpr int FR = 8;
  __shared__ float Srows[FR][128];
  const int D = g.D, bh = blockIdx.x, r0 = blockIdx.y * FR, tid = threadIdx.x;
  const int64_t BH = (int64_t)g.B * g.Hh;
  for (int i = tid; i < FR * D; i += 256) {
    const int rr = i / D, c = i % D;
    float s = 0.0f;
    for (int sp = 0; sp < splits; ++sp) s += spart[((int64_t)sp * BH + bh) * D * D + (r0 + rr) * D + c];
    Srows[rr][c] = s;
    if (S_out) S_out[(int64_t)bh * D * D + (r0 + rr) * D + c] = s;
  }
  if (blockIdx.y == 0) {
    for (int c = tid; c < D; c += 256) {
      float s = 0.0f;
      for (int sp = 0; sp < splits; ++sp) s += zpart[((int64_t)sp * BH + bh) * D + c];
      z_ws[(int64_t)bh * D + c] = s;
      if (z_out) z_out[(int64_t)bh * D + c] = s;
    }
  }
  if (mode == 2) return;
  __syncthreads();
  const float gv = mode == 0 ? gate[bh] : 1.0f;
  // S''[r0+rr][j] for j = column; stored transposed at [j][r0+rr]
  for (int i = tid; i < FR * D; i += 256) {
    const int j = i / FR, rr = i % FR;
    float v;
    if (mode == 0) {
      float s = 0.0f;
      for (int kk = 0; kk < D; ++kk) s = fmaf(Srows[rr][kk], (float)w[kk * D + j], s);
      v = gv * s;
    } else {
      v = Srows[rr][j];
    }
    const int64_t o = (int64_t)bh * D * D + (int64_t)j * D + r0 + rr;
    if (BF16OUT) {
      const __bf16 hi = (__bf16)v;
      const __bf16 lo = (__bf16)(v - (float)hi);
      static_cast<__bf16*>(sft_hi)[o] = hi;
      static_cast<__bf16*>(sft_lo)[o] = lo;
    } else {
      static_cast<float*>(sft_hi)[o] = v;
    }
  }
}

}  // namespace

hipError_t launch_linear_state(const Geom& g, int dtype, const void* k, const void* v, char* ws,
                               const Workspace& L, hipStream_t st) {
  float* spart = reinterpret_cast<float*>(ws + L.off_spart);
  float* zpart = reinterpret_cast<float*>(ws + L.off_zpart);
  dim3 grid(L.lin_splits, g.B * g.Hh);
  if (dtype == SALAD_BF16) {
    if (g.D == 128)
      hipLaunchKernelGGL(k_lin_partial_bf16<128>, grid, dim3(256), 0, st, g,
                         static_cast<const __bf16*>(k), static_cast<const __bf16*>(v), L.lin_chunk,
                         spart, zpart);
    else
      hipLaunchKernelGGL(k_lin_partial_bf16<64>, grid, dim3(256), 0, st, g,
                         static_cast<const __bf16*>(k), static_cast<const __bf16*>(v), L.lin_chunk,
                         spart, zpart);
  } else {
    if (g.D == 128)
      hipLaunchKernelGGL(k_lin_partial_f32<128>, grid, dim3(256), 0, st, g,
                         static_cast<const float*>(k), static_cast<const float*>(v), L.lin_chunk,
                         spart, zpart);
    else
      hipLaunchKernelGGL(k_lin_partial_f32<64>, grid, dim3(256), 0, st, g,
                         static_cast<const float*>(k), static_cast<const float*>(v), L.lin_chunk,
                         spart, zpart);
  }
  return hipGetLastError();
}

hipError_t launch_linear_fold(const Geom& g, int dtype, const float* gate, const void* w_lin,
                              int mode, float* S_out, float* z_out, char* ws, const Workspace& L,
                              hipStream_t st) {
  const float* spart = reinterpret_cast<const float*>(ws + L.off_spart);
  const float* zpart = reinterpret_cast<const float*>(ws + L.off_zpart);
  float* z_ws = reinterpret_cast<float*>(ws + L.off_z);
  void* hi = ws + L.off_sft_hi;
  void* lo = ws + L.off_sft_lo;
  dim3 grid(g.B * g.Hh, g.D / 8);
  if (dtype == SALAD_BF16)
    hipLaunchKernelGGL((k_lin_fold<__bf16, true>), grid, dim3(256), 0, st, g, L.lin_splits, spart,
                       zpart, gate, static_cast<const __bf16*>(w_lin), mode, S_out, z_out, z_ws,
                       hi, lo);
  else
    hipLaunchKernelGGL((k_lin_fold<float, false>), grid, dim3(256), 0, st, g, L.lin_splits, spart,
                       zpart, gate, static_cast<const float*>(w_lin), mode, S_out, z_out, z_ws, hi,
                       lo);
  return hipGetLastError();
}

}  // namespace salad
