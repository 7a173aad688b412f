// linear_bwd.hip - backward of the ReLU linear-attention branch and of the
// gated projection, plus the transposed (CSC) block mask the key-side sparse
// kernel walks.
//
// The layer is fine-tuned ("SALAD" explainer, technical summary section 2.2:
// the projection on the linear branch is a learnable, zero-initialised layer
// and the scale s comes from a small learned module; section 3: the fine-tuning
// budget), so the gradients of out = o_s + g (o_l W_lin) are needed with
// respect to Q, K, V, W_lin and g.  With phi = ReLU, u = phi(q) S,
// den = phi(q).z + eps, o_l = u / den, t = dout W_lin^T and r = <t, o_l>:
//
//   dgate  = sum_n r_n                      dW_lin = sum_heads g o_l^T dout
//   D_n    = <dout_n, out_n> - g r_n        (= <dout_n, o_s,n>, for the softmax backward)
//   dU_n   = g t_n / den_n                  dden_n = -g r_n / den_n
//   dq_lin = (S dU_n + z dden_n) * [q_n > 0]
//   dS     = sum_n phi(q_n) dU_n^T          dz = sum_n phi(q_n) dden_n
//   dk_lin = (dS v_j + dz) * [k_j > 0]      dv_lin = dS^T phi(k_j)
//
// Kernels: k_lin_bwd_rows (chunks of a head's rows per workgroup, tokens in
// lanes: u^T = S^T phi(q)^T and t^T = W dout^T on MFMAs with S^T (hi + lo bf16)
// and W in LDS) writes D, dden, dU, o_l and per-32-row dgate sums; k_lin_bwd_red reduces
// dS, dz and the per-head dW over token chunks with the token index as the MFMA
// contraction (both operands by LDS transpose reads); the folds sum the chunks
// in a fixed order (bitwise reproducible) and lay dS out as hi + lo bf16 in
// both orientations.  dq_lin, dk_lin and dv_lin are formed in the sparse
// kernels (attn_bwd.hip), which hold the needed operands in registers.
#include <algorithm>

#include "bwd_common.h"

namespace salad {

using namespace bwd;

namespace {

constexpr int kTT = 64;  // tokens per tile of the reduction kernel

__device__ inline bf16x8 ld8(const __bf16* p) { return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p)); }

// Per-token quantities of the linear branch's backward, tokens in lanes:
// u^T = S^T phi(q)^T (S^T as hi + lo bf16) and t^T = W_lin dO^T on MFMAs, then
// den, o_l = u / den, r = <t, o_l>, D = <dO, out> - g r, dden = -g r / den and
// dU = g t / den, with per-32-row dgate sums.  The head's S^T (hi, lo) and
// W_lin sit in LDS: one workgroup per CU walks a contiguous chunk of a head's
// rows, 128 rows (four waves of 32) per iteration, and reads the three D x D
// operands from LDS.  The next iteration's Q, dO and out rows are loaded into
// registers while the current ones are reduced.  Rows from N to n_pad get
// zeros (D, dden, dU, o_l).
template <int D>
__global__ void __launch_bounds__(256, 1)
k_lin_bwd_rows(Geom g, int chunk, const __bf16* __restrict__ Q, const __bf16* __restrict__ dO,
               const __bf16* __restrict__ Out, const __bf16* __restrict__ st_hi, const __bf16* __restrict__ st_lo,
               const float* __restrict__ z, const __bf16* __restrict__ W, const float* __restrict__ gate, float eps,
               float* __restrict__ Dq, float* __restrict__ dden, __bf16* __restrict__ dU, __bf16* __restrict__ OL,
               float* __restrict__ gpart) {
  using TL = TileLay<D>;
  constexpr int NC = D / 16, NT = D / 32, SST = D + 8;
  constexpr int MB = D * TL::ROW_B;          // one D x D operand
  constexpr int ROWS = 128;                  // rows per iteration
  __shared__ __align__(1024) unsigned char smem[3 * MB + ROWS * SST * 2];
  __bf16* stage = reinterpret_cast<__bf16*>(smem + 3 * MB);
  const int split = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, gg = lane >> 5, m = lane & 31;
  const int n0 = split * chunk, n1 = min(g.n_pad, n0 + chunk);
  const int64_t hb = (int64_t)bh * g.n_pad;
  const float gv = gate[bh];

  // S^T hi, S^T lo and W into LDS, 64 rows per DMA tile, swizzled like the K tiles
  {
    TileDma<D, 4> dma;
    dma.init(__builtin_amdgcn_readfirstlane(wave), lane);
    const uint32_t lds0 = lds_addr(smem);
    const __bf16* src[3] = {st_hi + (int64_t)bh * D * D, st_lo + (int64_t)bh * D * D, W};
#pragma unroll
    for (int mtx = 0; mtx < 3; ++mtx)
#pragma unroll
      for (int r0 = 0; r0 < D; r0 += 64) dma.issue(lds0 + mtx * MB + r0 * TL::ROW_B, src[mtx], r0, D - 1);
  }
  float4 zf[NC][2];
  {
    const float* zb = z + (int64_t)bh * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      zf[c][0] = *reinterpret_cast<const float4*>(zb + 16 * c + 8 * gg);
      zf[c][1] = *reinterpret_cast<const float4*>(zb + 16 * c + 8 * gg + 4);
    }
  }
  // this lane's row of an iteration starting at row i0 (clamped into the padded range)
  bf16x8 qf[NC], dof[NC], of[NC];
  auto load_rows = [&](int i0, bf16x8 (&q)[NC], bf16x8 (&d)[NC], bf16x8 (&o)[NC]) __attribute__((always_inline)) {
    const int n = min(i0 + wave * 32 + m, g.n_pad - 1);
    const int64_t row = (hb + n) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int ch = 16 * c + 8 * gg;
      q[c] = ld8(Q + row + ch);
      d[c] = ld8(dO + row + ch);
      o[c] = ld8(Out + row + ch);
    }
  };
  if (n0 < n1) load_rows(n0, qf, dof, of);
  wait_vmem();
  __syncthreads();

  for (int i0 = n0; i0 < n1; i0 += ROWS) {
    bf16x8 nq[NC], nd[NC], no[NC];
    if (i0 + ROWS < n1) load_rows(i0 + ROWS, nq, nd, no);
    const int n = i0 + wave * 32 + m;
    const bool active = i0 + wave * 32 < n1;  // uniform per wave
    const bool valid = active && n < g.N;
    float su = 0.0f;
    f32x16 u[NT], tt[NT];
    if (active) {
      float den_p = 0.0f, dot_p = 0.0f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const bf16x8 rq = relu8(qf[c]);
        qf[c] = rq;
        const float zz[8] = {zf[c][0].x, zf[c][0].y, zf[c][0].z, zf[c][0].w,
                             zf[c][1].x, zf[c][1].y, zf[c][1].z, zf[c][1].w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          den_p += (float)rq[j] * zz[j];
          dot_p += (float)dof[c][j] * (float)of[c][j];
        }
      }
      const float den = pair_sum(den_p) + eps;
      const float dot_out = pair_sum(dot_p);
      const float inv = 1.0f / den;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        zero(u[t]);
        zero(tt[t]);
        const int r = 32 * t + m;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const int o = TL::off(r, 2 * c + gg);
          const bf16x8 ah = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(smem + o));
          const bf16x8 al = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(smem + MB + o));
          const bf16x8 aw = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(smem + 2 * MB + o));
          u[t] = mfma(ah, qf[c], u[t]);
          u[t] = mfma(al, qf[c], u[t]);
          tt[t] = mfma(aw, dof[c], tt[t]);
        }
      }
      float r = 0.0f;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          u[t][e] *= inv;  // o_l^T
          r += tt[t][e] * u[t][e];
        }
      r = pair_sum(r);
      if (gg == 0) {
        Dq[hb + n] = valid ? dot_out - gv * r : 0.0f;
        dden[hb + n] = valid ? -gv * r * inv : 0.0f;
      }
      float rv = (valid && gg == 0) ? r : 0.0f;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) rv += __shfl_xor(rv, o, 64);
      if (lane == 0) gpart[(int64_t)bh * (g.n_pad / 32) + (i0 + wave * 32) / 32] = rv;
      su = valid ? gv * inv : 0.0f;
    }
    // dU = g t / den and o_l, staged through LDS as [row][channel] for coalesced stores
    const int lr = wave * 32 + m;
    const int nrows = min(ROWS, n1 - i0);
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      if (active) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float x = pass == 0 ? tt[t][e] * su : (valid ? u[t][e] : 0.0f);
            stage[lr * SST + 32 * t + crow(e, gg)] = (__bf16)x;
          }
      }
      __syncthreads();
      __bf16* dst = (pass == 0 ? dU : OL) + (hb + i0) * D;
      for (int e = tid; e < nrows * D / 8; e += 256) {
        const int rr = e / (D / 8), p = e % (D / 8);
        *reinterpret_cast<uint4*>(dst + (int64_t)rr * D + p * 8) =
            *reinterpret_cast<const uint4*>(stage + rr * SST + p * 8);
      }
      __syncthreads();
    }
    if (i0 + ROWS < n1) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        qf[c] = nq[c];
        dof[c] = nd[c];
        of[c] = no[c];
      }
    }
  }
}

// S (fp32, rows c) -> hi + lo bf16 in both orientations.
template <int D>
__global__ void __launch_bounds__(256)
k_split_state(int64_t total, const float* __restrict__ S, __bf16* s_hi, __bf16* s_lo, __bf16* st_hi,
              __bf16* st_lo) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t bh = i / (D * D);
  const int c = (int)(i / D % D), e = (int)(i % D);
  __bf16 hi, lo;
  split_hi_lo(S[i], hi, lo);
  s_hi[i] = hi;
  s_lo[i] = lo;
  const int64_t j = (bh * D + e) * D + c;
  st_hi[j] = hi;
  st_lo[j] = lo;
}

// Zero the slots of tokens at or past `valid` in a transposed fragment (slot
// order rows 16*ks + 8*(j/4) + 4*g + j%4 of the tile).
__device__ inline bf16x8 mask_slots(bf16x8 f, int ks, int valid, int gg) {
  if (16 * ks + 16 <= valid) return f;
  uint4 u = __builtin_bit_cast(uint4, f);
  uint32_t* w = reinterpret_cast<uint32_t*>(&u);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int tok = 16 * ks + 8 * (j >> 2) + 4 * gg + (j & 3);
    if (tok >= valid) w[j >> 1] &= (j & 1) ? 0x0000ffffu : 0xffff0000u;
  }
  return __builtin_bit_cast(bf16x8, u);
}

template <int D>
__global__ void __launch_bounds__(256)
k_lin_bwd_red(Geom g, int chunk, const __bf16* __restrict__ Q, const __bf16* __restrict__ dU,
              const __bf16* __restrict__ OL, const __bf16* __restrict__ dO, const float* __restrict__ dden,
              float* __restrict__ dspart, float* __restrict__ dzpart, float* __restrict__ dwpart) {
  using TL = TileLay<D>;
  constexpr int TD = D / 32, TPW = TD * TD / 4;
  constexpr int TB = kTT * TL::ROW_B;
  __shared__ __align__(16) unsigned char smem[8 * TB];
  __shared__ float dd[2][kTT];
  const int split = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, gg = lane >> 5, m = lane & 31;
  const int n0 = split * chunk, n1 = min(g.N, n0 + chunk);
  const int64_t hb = (int64_t)bh * g.n_pad;
  const int ti = TD == 4 ? wave : wave >> 1;
  const int tj0 = TD == 4 ? 0 : (wave & 1);

  f32x16 as[TPW], aw[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    zero(as[t]);
    zero(aw[t]);
  }
  float zacc = 0.0f;
  // the four token tiles stream HBM -> LDS, double buffered
  TileDma<D, 4> dma;
  dma.init(__builtin_amdgcn_readfirstlane(wave), lane);
  const uint32_t lds0 = lds_addr(smem);
  float dd_r = 0.0f;
  auto issue = [&](int t0, int buf) __attribute__((always_inline)) {
    const uint32_t base = lds0 + buf * 4 * TB;
    dma.issue(base, Q + hb * D, t0, g.N - 1);
    dma.issue(base + TB, dU + hb * D, t0, g.n_pad - 1);
    dma.issue(base + 2 * TB, OL + hb * D, t0, g.n_pad - 1);
    dma.issue(base + 3 * TB, dO + hb * D, t0, g.N - 1);
    if (tid < kTT) dd_r = t0 + tid < n1 ? dden[hb + t0 + tid] : 0.0f;
  };
  if (n0 < n1) {
    issue(n0, 0);
    if (tid < kTT) dd[0][tid] = dd_r;
  }
  wait_vmem();
  __syncthreads();
  int cur = 0;
  for (int t0 = n0; t0 < n1; t0 += kTT) {
    if (t0 + kTT < n1) issue(t0 + kTT, cur ^ 1);
    const unsigned char* Qt = smem + cur * 4 * TB;
    const unsigned char* Ut = Qt + TB;
    const unsigned char* Lt = Qt + 2 * TB;
    const unsigned char* Ot = Qt + 3 * TB;
    const int valid = n1 - t0;
#pragma unroll
    for (int ks = 0; ks < kTT / 16; ++ks) {
      const bf16x8 aq = mask_slots(relu8(frag_tr<D>(Qt, ks, ti, lane)), ks, valid, gg);
      const bf16x8 al = mask_slots(frag_tr<D>(Lt, ks, ti, lane), ks, valid, gg);
      if (tj0 == 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) zacc += (float)aq[j] * dd[cur][16 * ks + 8 * (j >> 2) + 4 * gg + (j & 3)];
      }
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int tj = TD == 4 ? t : tj0;
        as[t] = mfma(aq, frag_tr<D>(Ut, ks, tj, lane), as[t]);
        aw[t] = mfma(al, frag_tr<D>(Ot, ks, tj, lane), aw[t]);
      }
    }
    if (t0 + kTT < n1 && tid < kTT) dd[cur ^ 1][tid] = dd_r;
    wait_vmem();
    __syncthreads();
    cur ^= 1;
  }
  const int64_t po = ((int64_t)split * g.B * g.Hh + bh) * D * D;
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int tj = TD == 4 ? t : tj0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = ti * 32 + crow(i, gg);
      dspart[po + (int64_t)r * D + tj * 32 + m] = as[t][i];
      dwpart[po + (int64_t)r * D + tj * 32 + m] = aw[t][i];
    }
  }
  const float zs = pair_sum(zacc);
  if (tj0 == 0 && gg == 0) dzpart[((int64_t)split * g.B * g.Hh + bh) * D + ti * 32 + m] = zs;
}

// dS_lin, dz_lin: split sums in order; dS as hi + lo bf16, rows c and rows e.
template <int D>
__global__ void __launch_bounds__(256)
k_fold_ds(Geom g, int splits, const float* __restrict__ dspart, const float* __restrict__ dzpart,
          __bf16* ds_hi, __bf16* ds_lo, __bf16* dst_hi, __bf16* dst_lo, float* dz) {
  const int bh = blockIdx.y;
  const int idx = blockIdx.x * 256 + threadIdx.x;  // c * D + e
  const int64_t BH = (int64_t)g.B * g.Hh;
  float s = 0.0f;
  for (int sp = 0; sp < splits; ++sp) s += dspart[((int64_t)sp * BH + bh) * D * D + idx];
  const int c = idx / D, e = idx % D;
  __bf16 hi, lo;
  split_hi_lo(s, hi, lo);
  ds_hi[(int64_t)bh * D * D + idx] = hi;
  ds_lo[(int64_t)bh * D * D + idx] = lo;
  dst_hi[((int64_t)bh * D + e) * D + c] = hi;
  dst_lo[((int64_t)bh * D + e) * D + c] = lo;
  if (blockIdx.x == 0 && threadIdx.x < D) {
    float zz = 0.0f;
    for (int sp = 0; sp < splits; ++sp) zz += dzpart[((int64_t)sp * BH + bh) * D + threadIdx.x];
    dz[(int64_t)bh * D + threadIdx.x] = zz;
  }
}

// dW_lin = sum over heads (in order) of g * (sum over splits, in order): first
// the per-head split sums (one thread per head and element), then the heads.
template <int D>
__global__ void __launch_bounds__(256)
k_fold_dw_heads(Geom g, int splits, const float* __restrict__ dwpart, const float* __restrict__ gate,
                float* __restrict__ dwh) {
  const int bh = blockIdx.y;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  const int64_t BH = (int64_t)g.B * g.Hh;
  float s = 0.0f;
#pragma unroll 8
  for (int sp = 0; sp < splits; ++sp) s += dwpart[((int64_t)sp * BH + bh) * D * D + idx];
  dwh[(int64_t)bh * D * D + idx] = gate[bh] * s;
}

template <int D>
__global__ void __launch_bounds__(256)
k_fold_dw(Geom g, const float* __restrict__ dwh, float* __restrict__ dw) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  const int64_t BH = (int64_t)g.B * g.Hh;
  float acc = 0.0f;
  for (int64_t bh = 0; bh < BH; ++bh) acc += dwh[bh * D * D + idx];
  dw[idx] = acc;
}

// dgate: the head's n_pad/32 partials, strided per thread then a fixed tree.
__global__ void __launch_bounds__(256)
k_fold_dgate(Geom g, const float* __restrict__ gpart, float* __restrict__ dgate) {
  __shared__ float red[256];
  const int bh = blockIdx.x;
  const int parts = g.n_pad / 32;
  float s = 0.0f;
  for (int i = threadIdx.x; i < parts; i += 256) s += gpart[(int64_t)bh * parts + i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) dgate[bh] = red[0];
}

// ---- transposed mask ----------------------------------------------------------

// Transposed mask through a bitmap: one thread per CSR row sets bit qb of word
// qb/32 in its key blocks' columns (atomicOr: order-free), then one thread per
// column counts its bits and, after the scan, lists them in ascending order.
__global__ void __launch_bounds__(256)
k_csc_bits(Geom g, int words, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
           uint32_t* __restrict__ bits) {
  // one wave per CSR row, its lanes over the row's entries
  const int64_t r = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (r >= (int64_t)g.B * g.Hh * g.nb) return;  // uniform per wave
  const int64_t base = r / g.nb * g.nb;
  const int qb = (int)(r - base);
  const uint32_t bit = 1u << (qb & 31);
  for (int e = row_ptr[r] + lane; e < row_ptr[r + 1]; e += 64)
    atomicOr(&bits[(base + col_idx[e]) * words + (qb >> 5)], bit);
}

__global__ void __launch_bounds__(256)
k_csc_count(Geom g, int words, const uint32_t* __restrict__ bits, int32_t* __restrict__ colcnt) {
  const int64_t c = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (c >= (int64_t)g.B * g.Hh * g.nb) return;
  int cnt = 0;
  for (int w = 0; w < words; ++w) cnt += __popc(bits[c * words + w]);
  colcnt[c] = cnt;
}

__global__ void __launch_bounds__(256)
k_csc_fill(Geom g, int words, const uint32_t* __restrict__ bits, const int32_t* __restrict__ colptr,
           int32_t* __restrict__ rowidx) {
  // one wave per column: lanes take 64 words at a time, an exclusive scan of their
  // popcounts gives each lane its output position, bits are emitted in ascending order
  const int64_t c = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (c >= (int64_t)g.B * g.Hh * g.nb) return;  // uniform per wave
  int p = colptr[c];
  for (int w0 = 0; w0 < words; w0 += 64) {
    const int w = w0 + lane;
    uint32_t b = w < words ? bits[c * words + w] : 0u;
    const int cnt = __popc(b);
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    int pos = p + incl - cnt;
    while (b) {
      rowidx[pos++] = w * 32 + (__ffs(b) - 1);
      b &= b - 1;
    }
    p += __shfl(incl, 63, 64);
  }
}

__global__ void k_zero_u32(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// Exclusive scan of n int32 counts into out[0..n] (out[n] = total), one workgroup.
__global__ void __launch_bounds__(1024)
k_scan_counts(const int32_t* __restrict__ in, int64_t n, int32_t* __restrict__ out) {
  __shared__ int64_t part[1024];
  const int t = threadIdx.x;
  const int64_t per = (n + 1023) / 1024;
  const int64_t a = min(n, t * per), b = min(n, a + per);
  int64_t s = 0;
  for (int64_t i = a; i < b; ++i) s += in[i];
  part[t] = s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // inclusive Hillis-Steele scan of the 1024 sums
    const int64_t v = t >= o ? part[t - o] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int64_t run = part[t] - s;
  for (int64_t i = a; i < b; ++i) {
    out[i] = (int32_t)run;
    run += in[i];
  }
  if (t == 1023) out[n] = (int32_t)part[1023];
}

}  // namespace

BwdWorkspace plan_bwd_workspace(const Geom& g, const Cuboid& cu, int dtype) {
  BwdWorkspace L{};
  L.fwd = plan_workspace(g, cu, dtype);
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t BH = (size_t)g.B * g.Hh, D = g.D, nb = g.nb, np = g.n_pad;
  // token reduction: one resident workgroup per CU (128 KiB of LDS), at most 256
  // in all so that it runs in one round
  int splits = (int)std::max<size_t>(1, 256 / BH);
  splits = std::min(splits, (g.N + 63) / 64);
  int chunk = (g.N + splits - 1) / splits;
  chunk = (chunk + 63) / 64 * 64;
  splits = (g.N + chunk - 1) / chunk;
  L.red_splits = splits;
  L.red_chunk = chunk;
  size_t off = al(L.fwd.bytes);
  L.off_s32 = off;    off = al(off + BH * D * D * 4);
  L.off_z = off;      off = al(off + BH * D * 4);
  L.off_s_hi = off;   off = al(off + BH * D * D * 2);
  L.off_s_lo = off;   off = al(off + BH * D * D * 2);
  L.off_st_hi = off;  off = al(off + BH * D * D * 2);
  L.off_st_lo = off;  off = al(off + BH * D * D * 2);
  L.off_dq = off;     off = al(off + BH * np * 4);
  L.off_dden = off;   off = al(off + BH * np * 4);
  L.off_lse = off;    off = al(off + BH * np * 4);
  L.off_du = off;     off = al(off + BH * np * D * 2);
  L.off_ol = off;     off = al(off + BH * np * D * 2);
  L.off_gpart = off;  off = al(off + BH * (np / 32) * 4);
  L.off_dspart = off; off = al(off + (size_t)splits * BH * D * D * 4);
  L.off_dzpart = off; off = al(off + (size_t)splits * BH * D * 4);
  L.off_dwpart = off; off = al(off + (size_t)splits * BH * D * D * 4);
  L.off_ds_hi = off;  off = al(off + BH * D * D * 2);
  L.off_ds_lo = off;  off = al(off + BH * D * D * 2);
  L.off_dst_hi = off; off = al(off + BH * D * D * 2);
  L.off_dst_lo = off; off = al(off + BH * D * D * 2);
  L.off_dz = off;     off = al(off + BH * D * 4);
  L.off_dwh = off;    off = al(off + BH * D * D * 4);
  L.off_colcnt = off; off = al(off + BH * nb * 4);
  L.off_colptr = off; off = al(off + (BH * nb + 1) * 4);
  L.off_rowidx = off; off = al(off + BH * nb * nb * 4);
  L.off_bits = off;   off = al(off + BH * nb * ((nb + 31) / 32) * 4);
  L.off_split_q = off; off = al(off + (9 + kPairModeSlots) * 4);
  L.off_split_k = off; off = al(off + 9 * 4);
  L.bytes = off;
  return L;
}

hipError_t launch_linear_bwd(const Geom& g, const BwdArgs& a, char* ws, const BwdWorkspace& L,
                             hipStream_t st) {
  const int64_t BH = (int64_t)g.B * g.Hh;
  auto B16 = [&](size_t off) { return reinterpret_cast<__bf16*>(ws + off); };
  auto F32 = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  const __bf16* Q = static_cast<const __bf16*>(a.q);
  const __bf16* dO = static_cast<const __bf16*>(a.dout);
  const __bf16* Out = static_cast<const __bf16*>(a.out);
  const __bf16* W = static_cast<const __bf16*>(a.w_lin);
  const int64_t tot = BH * g.D * g.D;
  // row kernel: one workgroup per CU (S^T hi, lo and W_lin in 96 KiB of LDS), chunks of 64-row multiples
  int row_splits = (int)std::max<int64_t>(1, 256 / BH);
  row_splits = std::min(row_splits, g.n_pad / 64);
  int row_chunk = (g.n_pad + row_splits - 1) / row_splits;
  row_chunk = (row_chunk + 63) / 64 * 64;
  row_splits = (g.n_pad + row_chunk - 1) / row_chunk;
  const dim3 tg(row_splits, (unsigned)BH);
  const dim3 rg(L.red_splits, (unsigned)BH);
  const dim3 fg(g.D * g.D / 256, (unsigned)BH);
  if (g.D == 128) {
    hipLaunchKernelGGL(k_split_state<128>, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st, tot,
                       F32(L.off_s32), B16(L.off_s_hi), B16(L.off_s_lo), B16(L.off_st_hi), B16(L.off_st_lo));
    hipLaunchKernelGGL(k_lin_bwd_rows<128>, tg, dim3(256), 0, st, g, row_chunk, Q, dO, Out, B16(L.off_st_hi),
                       B16(L.off_st_lo), F32(L.off_z), W, a.gate, a.eps, F32(L.off_dq), F32(L.off_dden),
                       B16(L.off_du), B16(L.off_ol), F32(L.off_gpart));
    hipLaunchKernelGGL(k_lin_bwd_red<128>, rg, dim3(256), 0, st, g, L.red_chunk, Q, B16(L.off_du),
                       B16(L.off_ol), dO, F32(L.off_dden), F32(L.off_dspart), F32(L.off_dzpart),
                       F32(L.off_dwpart));
    hipLaunchKernelGGL(k_fold_ds<128>, fg, dim3(256), 0, st, g, L.red_splits, F32(L.off_dspart),
                       F32(L.off_dzpart), B16(L.off_ds_hi), B16(L.off_ds_lo), B16(L.off_dst_hi),
                       B16(L.off_dst_lo), F32(L.off_dz));
    hipLaunchKernelGGL(k_fold_dw_heads<128>, fg, dim3(256), 0, st, g, L.red_splits, F32(L.off_dwpart), a.gate,
                       F32(L.off_dwh));
    hipLaunchKernelGGL(k_fold_dw<128>, dim3(128 * 128 / 256), dim3(256), 0, st, g, F32(L.off_dwh), a.dw_lin);
  } else if (g.D == 64) {
    hipLaunchKernelGGL(k_split_state<64>, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st, tot,
                       F32(L.off_s32), B16(L.off_s_hi), B16(L.off_s_lo), B16(L.off_st_hi), B16(L.off_st_lo));
    hipLaunchKernelGGL(k_lin_bwd_rows<64>, tg, dim3(256), 0, st, g, row_chunk, Q, dO, Out, B16(L.off_st_hi),
                       B16(L.off_st_lo), F32(L.off_z), W, a.gate, a.eps, F32(L.off_dq), F32(L.off_dden),
                       B16(L.off_du), B16(L.off_ol), F32(L.off_gpart));
    hipLaunchKernelGGL(k_lin_bwd_red<64>, rg, dim3(256), 0, st, g, L.red_chunk, Q, B16(L.off_du),
                       B16(L.off_ol), dO, F32(L.off_dden), F32(L.off_dspart), F32(L.off_dzpart),
                       F32(L.off_dwpart));
    hipLaunchKernelGGL(k_fold_ds<64>, fg, dim3(256), 0, st, g, L.red_splits, F32(L.off_dspart),
                       F32(L.off_dzpart), B16(L.off_ds_hi), B16(L.off_ds_lo), B16(L.off_dst_hi),
                       B16(L.off_dst_lo), F32(L.off_dz));
    hipLaunchKernelGGL(k_fold_dw_heads<64>, fg, dim3(256), 0, st, g, L.red_splits, F32(L.off_dwpart), a.gate,
                       F32(L.off_dwh));
    hipLaunchKernelGGL(k_fold_dw<64>, dim3(64 * 64 / 256), dim3(256), 0, st, g, F32(L.off_dwh), a.dw_lin);
  } else {
    return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(k_fold_dgate, dim3((unsigned)BH), dim3(256), 0, st, g, F32(L.off_gpart), a.dgate);
  return hipGetLastError();
}

hipError_t launch_mask_transpose(const Geom& g, const int32_t* row_ptr, const int32_t* col_idx, char* ws,
                                 const BwdWorkspace& L, hipStream_t st) {
  const int64_t n = (int64_t)g.B * g.Hh * g.nb;
  int32_t* cnt = reinterpret_cast<int32_t*>(ws + L.off_colcnt);
  int32_t* ptr = reinterpret_cast<int32_t*>(ws + L.off_colptr);
  int32_t* idx = reinterpret_cast<int32_t*>(ws + L.off_rowidx);
  const int words = (g.nb + 31) / 32;
  uint32_t* bits = reinterpret_cast<uint32_t*>(ws + L.off_bits);
  const dim3 grid((unsigned)((n + 255) / 256));
  hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)std::min<int64_t>((n * words + 255) / 256, 4096)), dim3(256), 0, st,
                     bits, n * words);
  const dim3 wave_grid((unsigned)((n * 64 + 255) / 256));  // one wave per row (bits) or column (fill)
  hipLaunchKernelGGL(k_csc_bits, wave_grid, dim3(256), 0, st, g, words, row_ptr, col_idx, bits);
  hipLaunchKernelGGL(k_csc_count, grid, dim3(256), 0, st, g, words, bits, cnt);
  hipLaunchKernelGGL(k_scan_counts, dim3(1), dim3(1024), 0, st, cnt, n, ptr);
  hipLaunchKernelGGL(k_csc_fill, wave_grid, dim3(256), 0, st, g, words, bits, ptr, idx);
  return hipGetLastError();
}

}  // namespace salad
