// attn_f32.hip - fused hybrid attention forward, fp32 in/out, VALU only.
//
// The fp32 path exists for tight-tolerance parity on small layers; it is not
// tuned.  One workgroup per (b, h, query block), one thread per query row.  The
// kept key blocks are walked in 16-key sub-tiles staged in LDS; each thread
// runs the online-softmax recurrence over its row in fp32.  The epilogue adds
// the pre-folded linear branch ReLU(q)^T S'' / (ReLU(q)^T z + eps) with the
// fp32 folded state (same arithmetic as the bf16 kernel, without the hi/lo
// split).
#include "internal.h"

namespace salad {
namespace {

constexpr int kSub = 16;

template <int D>
__global__ void __launch_bounds__(128)
k_attn_f32(Geom g, AttnArgs a, float scale) {
  __shared__ float Ks[kSub][D];
  __shared__ float Vs[kSub][D];
  const int qb = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int row = qb * g.blk + tid;
  const bool valid = row < g.N;
  const float* Qb = static_cast<const float*>(a.q) + (int64_t)bh * g.n_pad * D;
  const float* Kb = static_cast<const float*>(a.k) + (int64_t)bh * g.n_pad * D;
  const float* Vb = static_cast<const float*>(a.v) + (int64_t)bh * g.n_pad * D;

  float q[D], o[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    q[c] = valid ? Qb[(int64_t)row * D + c] : 0.0f;
    o[c] = 0.0f;
  }
  float m_run = -INFINITY, l_run = 0.0f;

  if (a.has_sparse) {
    const int64_t r = (int64_t)bh * g.nb + qb;
    const int beg = a.row_ptr[r], end = a.row_ptr[r + 1];
    for (int e = beg; e < end; ++e) {
      const int kb = a.col_idx[e];
      for (int sub = 0; sub < g.blk / kSub; ++sub) {
        const int key0 = kb * g.blk + sub * kSub;
        if (key0 >= g.N) break;
        __syncthreads();
        for (int i = tid; i < kSub * D; i += blockDim.x) {
          const int j = i / D, c = i % D, n = key0 + j;
          const bool in = (unsigned)n < (unsigned)g.N;
          Ks[j][c] = in ? Kb[(int64_t)n * D + c] : 0.0f;
          Vs[j][c] = in ? Vb[(int64_t)n * D + c] : 0.0f;
        }
        __syncthreads();
        float s[kSub];
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < kSub; ++j) {
          float acc = 0.0f;
#pragma unroll
          for (int c = 0; c < D; ++c) acc = fmaf(q[c], Ks[j][c], acc);
          s[j] = key0 + j < g.N ? acc * scale : -INFINITY;
          mx = fmaxf(mx, s[j]);
        }
        const float m_new = fmaxf(m_run, mx);
        const float alpha = expf(m_run - m_new);
        float rs = 0.0f;
#pragma unroll
        for (int j = 0; j < kSub; ++j) {
          s[j] = expf(s[j] - m_new);
          rs += s[j];
        }
        l_run = l_run * alpha + rs;
        m_run = m_new;
#pragma unroll
        for (int c = 0; c < D; ++c) {
          float acc = o[c] * alpha;
#pragma unroll
          for (int j = 0; j < kSub; ++j) acc = fmaf(s[j], Vs[j][c], acc);
          o[c] = acc;
        }
      }
    }
  }
  const float inv_l = l_run > 0.0f ? 1.0f / l_run : 0.0f;
  bool lin = a.has_lin != 0;
  if (lin && a.gate != nullptr && a.gate[bh] < a.drop_tau) lin = false;
  float inv_den = 0.0f;
  const float* sft = static_cast<const float*>(a.sft) + (int64_t)bh * D * D;
  if (lin) {
    const float* z = a.z + (int64_t)bh * D;
    float den = 0.0f;
#pragma unroll
    for (int c = 0; c < D; ++c) den = fmaf(fmaxf(q[c], 0.0f), z[c], den);
    inv_den = 1.0f / (den + a.eps);
  }
  float* Ob = static_cast<float*>(a.out) + (int64_t)bh * g.n_pad * D;
  if (row >= g.n_pad) return;
  for (int e = 0; e < D; ++e) {
    float v = o[e] * inv_l;
    if (lin) {
      float num = 0.0f;
      for (int c = 0; c < D; ++c) num = fmaf(fmaxf(q[c], 0.0f), sft[e * D + c], num);
      v += num * inv_den;
    }
    Ob[(int64_t)row * D + e] = valid ? v : 0.0f;
  }
}

}  // namespace

hipError_t launch_attn_f32(const Geom& g, const AttnArgs& a, hipStream_t st) {
  dim3 grid(g.nb, g.B * g.Hh);
  if (g.D == 128)
    hipLaunchKernelGGL(k_attn_f32<128>, grid, dim3(g.blk), 0, st, g, a, a.scale);
  else
    hipLaunchKernelGGL(k_attn_f32<64>, grid, dim3(g.blk), 0, st, g, a, a.scale);
  return hipGetLastError();
}

}  // namespace salad
