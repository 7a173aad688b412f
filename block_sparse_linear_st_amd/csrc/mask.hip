// mask.hip - block-mask builder for gfx950: static spatio-temporal window and
// pooled-score top-k, emitted as CSR lists of kept key blocks.
//
// The masks follow the readings stated in include/salad.h (salad_mask_spec).
// Window: every block pair's r* is recomputed on the fly from the horizontal
// runs of the two blocks (a block covers at most ceil(block/W)+1 runs), so no
// r* table is stored.  Selecting the first K pairs in (qb!=kb, r*, |qb-kb|, qb,
// kb) order is done with one histogram over a combined bin (0 for the
// diagonal, 1 + r*·nb + |qb-kb| otherwise), a per-head scan that finds the bin
// holding the K-th pair, and a scan over query blocks inside that bin (a bin
// holds at most two pairs per query block, kb = qb -+ |qb-kb|).  The K-th
// pair's packed key (bin·nb² + qb·nb + kb) is then the keep threshold.
//
// Top-k: block sums in float32, sequential in token order, one division per
// mean, scores as a sequential float32 sum of separately rounded products.
// This file is compiled with floating-point contraction off so that no
// multiply-add is fused: the ranking is reproducible bit for bit.  Each row's
// scores become 64-bit keys (descending score, then ascending kb), are sorted
// in LDS with a bitonic network, and the first k kb's are emitted ascending.
#include <algorithm>

#include "internal.h"

#pragma clang fp contract(off)

namespace salad {

namespace {

constexpr int kScanThreads = 1024;

__device__ inline int rstar_pair(const Geom& g, int qb, int kb, int tw) {
  const int qa0 = qb * g.blk, qa1 = min(qa0 + g.blk, g.N) - 1;
  const int ka0 = kb * g.blk, ka1 = min(ka0 + g.blk, g.N) - 1;
  int best = kRstarInf;
  for (int a = qa0 / g.W; a <= qa1 / g.W; ++a) {
    const int ta = a / g.H, ya = a - ta * g.H;
    const int xa0 = max(qa0, a * g.W) - a * g.W;
    const int xa1 = min(qa1, a * g.W + g.W - 1) - a * g.W;
    for (int c = ka0 / g.W; c <= ka1 / g.W; ++c) {
      const int tc = c / g.H;
      if (abs(ta - tc) > tw) continue;
      const int yc = c - tc * g.H;
      const int xc0 = max(ka0, c * g.W) - c * g.W;
      const int xc1 = min(ka1, c * g.W + g.W - 1) - c * g.W;
      const int gap = max(0, max(xc0 - xa1, xa0 - xc1));
      best = min(best, max(abs(ya - yc), gap));
    }
  }
  return best;
}

__device__ inline bool window_candidate(int r, int r_max) {
  return r < kRstarInf && (r_max < 0 || r <= r_max);
}

// Combined bin of a candidate pair: 0 on the diagonal, else 1 + r*·nb + |qb-kb|.
__device__ inline int64_t pair_bin(int qb, int kb, int r, int nb) {
  return qb == kb ? 0 : 1 + (int64_t)r * nb + abs(qb - kb);
}

__device__ inline int64_t pair_key(int64_t bin, int qb, int kb, int nb) {
  return (bin * nb + qb) * nb + kb;
}

__global__ void k_fill_i32(int32_t* p, int64_t n, int32_t v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// grid (nb, heads): histogram of the candidate pairs of query block qb.
__global__ void k_window_hist(Geom g, HeadTable ht, int32_t* hist, int64_t hist_bins) {
  const int h = blockIdx.y, qb = blockIdx.x;
  if (ht.kind[h] != SALAD_MASK_WINDOW || ht.count[h] < 0) return;
  int32_t* hh = hist + (int64_t)h * hist_bins;
  for (int kb = threadIdx.x; kb < g.nb; kb += blockDim.x) {
    const int r = rstar_pair(g, qb, kb, ht.t_window[h]);
    if (!window_candidate(r, ht.r_max[h])) continue;
    atomicAdd(&hh[pair_bin(qb, kb, r, g.nb)], 1);
  }
}

// Block-wide exclusive scan of one int64 per thread (kScanThreads threads).
__device__ int64_t block_exclusive_scan(int64_t v, int64_t* tmp, int64_t* total) {
  const int t = threadIdx.x;
  tmp[t] = v;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int64_t add = t >= off ? tmp[t - off] : 0;
    __syncthreads();
    tmp[t] += add;
    __syncthreads();
  }
  const int64_t incl = tmp[t];
  if (total) *total = tmp[kScanThreads - 1];
  __syncthreads();
  return incl - v;
}

// grid (heads), kScanThreads threads: the keep threshold of each window head.
__global__ void __launch_bounds__(kScanThreads)
k_window_threshold(Geom g, HeadTable ht, const int32_t* hist, int64_t hist_bins,
                   int64_t* thr, int32_t* flags) {
  __shared__ int64_t tmp[kScanThreads];
  __shared__ int64_t s_bin, s_need;
  const int h = blockIdx.x, t = threadIdx.x;
  if (ht.kind[h] != SALAD_MASK_WINDOW) return;
  const int64_t K = ht.count[h];
  if (K < 0) {  // keep every candidate
    if (t == 0) { thr[h] = INT64_MAX; flags[h] = 0; }
    return;
  }
  if (K == 0) {
    if (t == 0) { thr[h] = -1; flags[h] = 0; }
    return;
  }
  const int32_t* hh = hist + (int64_t)h * hist_bins;
  // 1) the bin that holds the K-th pair
  const int64_t seg = (hist_bins + kScanThreads - 1) / kScanThreads;
  const int64_t lo = min((int64_t)t * seg, hist_bins), hi = min(lo + seg, hist_bins);
  int64_t local = 0;
  for (int64_t b = lo; b < hi; ++b) local += hh[b];
  int64_t total;
  const int64_t excl = block_exclusive_scan(local, tmp, &total);
  if (t == 0) { s_bin = -1; s_need = 0; }
  __syncthreads();
  if (total < K) {  // infeasible: keep all candidates and report it
    if (t == 0) { thr[h] = INT64_MAX; flags[h] = 1; }
    return;
  }
  if (excl < K && K <= excl + local) {
    int64_t cum = excl;
    for (int64_t b = lo; b < hi; ++b) {
      if (cum + hh[b] >= K) { s_bin = b; s_need = K - cum; break; }
      cum += hh[b];
    }
  }
  __syncthreads();
  const int64_t bin = s_bin, need = s_need;
  // 2) inside that bin, pairs run in (qb, kb) order with at most two per qb
  const int tw = ht.t_window[h], rmax = ht.r_max[h];
  const int r = bin == 0 ? 0 : (int)((bin - 1) / g.nb);
  const int dd = bin == 0 ? 0 : (int)((bin - 1) % g.nb);
  auto in_bin = [&](int qb, int kb) -> bool {
    if (kb < 0 || kb >= g.nb) return false;
    const int rr = rstar_pair(g, qb, kb, tw);
    return window_candidate(rr, rmax) && pair_bin(qb, kb, rr, g.nb) == bin;
  };
  const int qseg = (g.nb + kScanThreads - 1) / kScanThreads;
  const int qlo = min(t * qseg, g.nb), qhi = min(qlo + qseg, g.nb);
  int64_t qlocal = 0;
  for (int qb = qlo; qb < qhi; ++qb)
    qlocal += dd == 0 ? (int)in_bin(qb, qb) : (int)in_bin(qb, qb - dd) + (int)in_bin(qb, qb + dd);
  const int64_t qexcl = block_exclusive_scan(qlocal, tmp, nullptr);
  if (qexcl < need && need <= qexcl + qlocal) {
    int64_t cum = qexcl;
    for (int qb = qlo; qb < qhi; ++qb) {
      const bool lo_in = dd == 0 ? in_bin(qb, qb) : in_bin(qb, qb - dd);
      const bool hi_in = dd == 0 ? false : in_bin(qb, qb + dd);
      const int c = (int)lo_in + (int)hi_in;
      if (cum + c >= need) {
        const int64_t rem = need - cum;
        int kb;
        if (dd == 0) kb = qb;
        else if (rem == 1) kb = lo_in ? qb - dd : qb + dd;
        else kb = qb + dd;
        thr[h] = pair_key(bin, qb, kb, g.nb);
        flags[h] = 0;
        break;
      }
      cum += c;
    }
  }
  (void)r;
}

__device__ inline bool window_keep(const Geom& g, int qb, int kb, int tw, int rmax, int64_t thr) {
  const int r = rstar_pair(g, qb, kb, tw);
  if (!window_candidate(r, rmax)) return false;
  if (thr == INT64_MAX) return true;
  return pair_key(pair_bin(qb, kb, r, g.nb), qb, kb, g.nb) <= thr;
}

// grid (nb, heads), one wave: kept blocks per row, replicated over the batch.
__global__ void __launch_bounds__(64)
k_row_counts(Geom g, HeadTable ht, const int64_t* thr, int32_t* rowcnt) {
  const int qb = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  int cnt;
  if (ht.kind[h] == SALAD_MASK_WINDOW) {
    int local = 0;
    const int64_t th = thr[h];
    for (int kb = lane; kb < g.nb; kb += 64)
      local += window_keep(g, qb, kb, ht.t_window[h], ht.r_max[h], th) ? 1 : 0;
    for (int off = 32; off > 0; off >>= 1) local += __shfl_xor(local, off);
    cnt = local;
  } else {
    cnt = ht.count[h];
  }
  if (lane == 0)
    for (int b = 0; b < g.B; ++b) rowcnt[((int64_t)b * g.Hh + h) * g.nb + qb] = cnt;
}

// One workgroup: row_ptr = exclusive scan of the row counts.
__global__ void __launch_bounds__(kScanThreads)
k_scan_rows(const int32_t* rowcnt, int64_t rows, int32_t* row_ptr) {
  __shared__ int64_t tmp[kScanThreads];
  const int t = threadIdx.x;
  const int64_t seg = (rows + kScanThreads - 1) / kScanThreads;
  const int64_t lo = min((int64_t)t * seg, rows), hi = min(lo + seg, rows);
  int64_t local = 0;
  for (int64_t r = lo; r < hi; ++r) local += rowcnt[r];
  int64_t total;
  int64_t run = block_exclusive_scan(local, tmp, &total);
  for (int64_t r = lo; r < hi; ++r) {
    row_ptr[r] = (int32_t)run;
    run += rowcnt[r];
  }
  if (t == 0) row_ptr[rows] = (int32_t)total;
}

// grid (nb, heads), one wave: kept key blocks of window rows, ascending.
__global__ void __launch_bounds__(64)
k_window_emit(Geom g, HeadTable ht, const int64_t* thr, const int32_t* row_ptr,
              int32_t* col_idx, int64_t col_cap) {
  const int qb = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  if (ht.kind[h] != SALAD_MASK_WINDOW) return;
  const int64_t th = thr[h];
  int off = 0;
  for (int kb0 = 0; kb0 < g.nb; kb0 += 64) {
    const int kb = kb0 + lane;
    const bool keep = kb < g.nb && window_keep(g, qb, kb, ht.t_window[h], ht.r_max[h], th);
    const uint64_t m = __ballot(keep);
    const int rank = __popcll(m & ((1ull << lane) - 1ull));
    if (keep) {
      for (int b = 0; b < g.B; ++b) {
        const int64_t pos = (int64_t)row_ptr[((int64_t)b * g.Hh + h) * g.nb + qb] + off + rank;
        if (pos < col_cap) col_idx[pos] = kb;
      }
    }
    off += __popcll(m);
  }
}

// ---- top-k -----------------------------------------------------------------

template <typename T>
struct Load8;
template <>
struct Load8<__bf16> {
  __device__ static void run(const __bf16* p, float* f) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[2 * j] = __uint_as_float(w[j] << 16);
      f[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  }
};
template <>
struct Load8<float> {
  __device__ static void run(const float* p, float* f) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
};

// grid (ceil(B*H*nb*(D/8) / 256), 2): per (b, h, block) sequential float32 sums
// of 8 channels per thread; blockIdx.y selects Q (0) or K (1).
template <typename T>
__global__ void __launch_bounds__(256)
k_pool(Geom g, HeadTable ht, const T* q, const T* k, float* psum_q, float* psum_k) {
  const int which = blockIdx.y;
  const int groups = g.D / 8;
  const int64_t i = blockIdx.x * 256ll + threadIdx.x;
  const int64_t units = (int64_t)g.B * g.Hh * g.nb * groups;
  if (i >= units) return;
  const int cg = (int)(i % groups);
  const int64_t u = i / groups;  // (b*H + h)*nb + blk
  const int blk = (int)(u % g.nb);
  const int64_t bh = u / g.nb;
  const int h = (int)(bh % g.Hh);
  if (!((ht.pool[h] >> which) & 1)) return;
  const T* x = (which == 0 ? q : k) + (bh * g.n_pad + (int64_t)blk * g.blk) * g.D + cg * 8;
  const int nvalid = min(g.blk, g.N - blk * g.blk);
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
  int o = 0;
  for (; o + 8 <= nvalid; o += 8) {
    float f[8][8];
#pragma unroll
    for (int s = 0; s < 8; ++s) Load8<T>::run(x + (int64_t)(o + s) * g.D, f[s]);
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = acc[j] + f[s][j];
  }
  for (; o < nvalid; ++o) {
    float f[8];
    Load8<T>::run(x + (int64_t)o * g.D, f);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = acc[j] + f[j];
  }
  float* dst = (which == 0 ? psum_q : psum_k) + u * g.D + cg * 8;
#pragma unroll
  for (int j = 0; j < 8; ++j) dst[j] = acc[j];
}

__device__ inline uint32_t ordered_bits(float s) {
  const uint32_t u = __float_as_uint(s == 0.0f ? 0.0f : s);  // -0 ranks as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// grid (ceil(nb / rows_per_wg), B*H), 256 threads: scores, top-k and emit for
// rows_per_wg query blocks of one (b, h).  Dynamic LDS layout:
//   pq[rows][D] | scores[rows][nb] | union{ pk[64][D+1], keys[nbp2] u64 + flags[nb] }
__global__ void __launch_bounds__(256)
k_topk(Geom g, HeadTable ht, const float* psum_q, const float* psum_k, int rows_per_wg,
       int nbp2, const int32_t* row_ptr, int32_t* col_idx, int64_t col_cap) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int bh = blockIdx.y, h = bh % g.Hh, t = threadIdx.x;
  if (ht.kind[h] != SALAD_MASK_TOPK) return;
  const int D = g.D, nb = g.nb;
  const int qb0 = blockIdx.x * rows_per_wg;
  const int rows = min(rows_per_wg, nb - qb0);
  float* pq = reinterpret_cast<float*>(smem);
  float* scores = pq + rows_per_wg * D;
  unsigned char* tail = reinterpret_cast<unsigned char*>(scores + (size_t)rows_per_wg * nb);
  float* pk = reinterpret_cast<float*>(tail);
  uint64_t* keys = reinterpret_cast<uint64_t*>(tail);
  int32_t* flags = reinterpret_cast<int32_t*>(keys + nbp2);

  auto nvalid = [&](int b) { return (float)min(g.blk, g.N - b * g.blk); };
  for (int i = t; i < rows * D; i += 256) {
    const int r = i / D, c = i - r * D;
    pq[r * D + c] = __fdiv_rn(psum_q[((int64_t)bh * nb + qb0 + r) * D + c], nvalid(qb0 + r));
  }
  // scores, 64 key blocks at a time
  for (int kb0 = 0; kb0 < nb; kb0 += 64) {
    const int nk = min(64, nb - kb0);
    __syncthreads();
    for (int i = t; i < nk * D; i += 256) {
      const int kk = i / D, c = i - kk * D;
      pk[kk * (D + 1) + c] =
          __fdiv_rn(psum_k[((int64_t)bh * nb + kb0 + kk) * D + c], nvalid(kb0 + kk));
    }
    __syncthreads();
    for (int i = t; i < rows * 64; i += 256) {
      const int r = i / 64, kk = i - r * 64;
      if (kk >= nk) continue;
      float acc = 0.0f;
      const float* a = pq + r * D;
      const float* b = pk + kk * (D + 1);
      for (int c = 0; c < D; ++c) {
        const float prod = a[c] * b[c];
        acc = acc + prod;
      }
      scores[(size_t)r * nb + kb0 + kk] = acc;
    }
  }
  __syncthreads();
  const int kkeep = ht.count[h];
  for (int r = 0; r < rows; ++r) {
    for (int i = t; i < nbp2; i += 256)
      keys[i] = i < nb ? ((uint64_t)(~ordered_bits(scores[(size_t)r * nb + i])) << 32) | (uint32_t)i
                       : ~0ull;
    __syncthreads();
    for (int size = 2; size <= nbp2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = t; i < nbp2 / 2; i += 256) {
          const int lo = 2 * stride * (i / stride) + (i % stride);
          const int hi = lo + stride;
          const bool asc = (lo & size) == 0;
          const uint64_t a = keys[lo], b = keys[hi];
          if ((a > b) == asc) { keys[lo] = b; keys[hi] = a; }
        }
        __syncthreads();
      }
    }
    for (int i = t; i < nb; i += 256) flags[i] = 0;
    __syncthreads();
    for (int i = t; i < kkeep; i += 256) flags[(int)(keys[i] & 0xffffffffu)] = 1;
    __syncthreads();
    // compact ascending: wave 0 walks the flags 64 at a time
    if (t < 64) {
      const int64_t base = row_ptr[(int64_t)bh * nb + qb0 + r];
      int off = 0;
      for (int kb0 = 0; kb0 < nb; kb0 += 64) {
        const int kb = kb0 + t;
        const bool keep = kb < nb && flags[kb];
        const uint64_t m = __ballot(keep);
        if (keep) {
          const int64_t pos = base + off + __popcll(m & ((1ull << t) - 1ull));
          if (pos < col_cap) col_idx[pos] = kb;
        }
        off += __popcll(m);
      }
    }
    __syncthreads();
  }
}

// grid (B*H), 256 threads: gate = sigmoid(mean(Q) . w_g) from the block sums.
__global__ void __launch_bounds__(256)
k_gate(Geom g, const float* psum_q, const float* w_g, float* gate) {
  __shared__ double red[256];
  const int bh = blockIdx.x, t = threadIdx.x;
  double part = 0.0;
  for (int c = t; c < g.D; c += 256) {
    double s = 0.0;
    for (int b = 0; b < g.nb; ++b) s += (double)psum_q[((int64_t)bh * g.nb + b) * g.D + c];
    part += (s / (double)g.N) * (double)w_g[c];
  }
  red[t] = part;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (t < off) red[t] += red[t + off];
    __syncthreads();
  }
  if (t == 0) gate[bh] = (float)(1.0 / (1.0 + exp(-red[0])));
}

__global__ void k_info(const int32_t* flags, HeadTable ht, int32_t* info) {
  if (threadIdx.x != 0) return;
  int n = 0;
  for (int h = 0; h < ht.n_heads; ++h)
    if (ht.kind[h] == SALAD_MASK_WINDOW) n += flags[h];
  info[0] = n;
}

template <typename T>
hipError_t launch_pool(const Geom& g, const HeadTable& ht, const void* q, const void* k,
                       float* pq, float* pk, hipStream_t st) {
  const int64_t units = (int64_t)g.B * g.Hh * g.nb * (g.D / 8);
  dim3 grid((unsigned)((units + 255) / 256), 2);
  hipLaunchKernelGGL(k_pool<T>, grid, dim3(256), 0, st, g, ht, static_cast<const T*>(q),
                     static_cast<const T*>(k), pq, pk);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_build_mask(const Geom& g, int dtype, const HeadTable& ht0, const void* q,
                             const void* k, int32_t* row_ptr, int32_t* col_idx, int64_t col_cap,
                             int32_t* info, const float* w_g, float* gate, char* ws,
                             const Workspace& L, hipStream_t st) {
  HeadTable ht = ht0;
  bool any_window = false, any_topk = false;
  for (int h = 0; h < g.Hh; ++h) {
    ht.pool[h] = 0;
    if (ht.kind[h] == SALAD_MASK_WINDOW) any_window = true;
    else { any_topk = true; ht.pool[h] = 3; }
    if (gate) ht.pool[h] |= 1;
  }
  int32_t* hist = reinterpret_cast<int32_t*>(ws + L.off_hist);
  int64_t* thr = reinterpret_cast<int64_t*>(ws + L.off_thr);
  int32_t* flags = reinterpret_cast<int32_t*>(ws + L.off_flags);
  int32_t* rowcnt = reinterpret_cast<int32_t*>(ws + L.off_rowcnt);
  float* psq = reinterpret_cast<float*>(ws + L.off_psum_q);
  float* psk = reinterpret_cast<float*>(ws + L.off_psum_k);

  hipLaunchKernelGGL(k_fill_i32, dim3(1), dim3(256), 0, st, flags, (int64_t)g.Hh, 0);
  if (any_window) {
    const int64_t nhist = (int64_t)g.Hh * (int64_t)L.hist_bins;
    hipLaunchKernelGGL(k_fill_i32, dim3((unsigned)std::min<int64_t>((nhist + 255) / 256, 65535)),
                       dim3(256), 0, st, hist, nhist, 0);
    hipLaunchKernelGGL(k_window_hist, dim3(g.nb, g.Hh), dim3(256), 0, st, g, ht, hist,
                       (int64_t)L.hist_bins);
    hipLaunchKernelGGL(k_window_threshold, dim3(g.Hh), dim3(kScanThreads), 0, st, g, ht, hist,
                       (int64_t)L.hist_bins, thr, flags);
  }
  if (any_topk || gate) {
    hipError_t e = dtype == SALAD_BF16 ? launch_pool<__bf16>(g, ht, q, k, psq, psk, st)
                                       : launch_pool<float>(g, ht, q, k, psq, psk, st);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_row_counts, dim3(g.nb, g.Hh), dim3(64), 0, st, g, ht, thr, rowcnt);
  const int64_t rows = (int64_t)g.B * g.Hh * g.nb;
  hipLaunchKernelGGL(k_scan_rows, dim3(1), dim3(kScanThreads), 0, st, rowcnt, rows, row_ptr);
  if (any_window)
    hipLaunchKernelGGL(k_window_emit, dim3(g.nb, g.Hh), dim3(64), 0, st, g, ht, thr, row_ptr,
                       col_idx, col_cap);
  if (any_topk) {
    int rpw = g.nb <= 512 ? 16 : g.nb <= 1024 ? 8 : g.nb <= 2048 ? 4 : g.nb <= 4096 ? 2 : 1;
    int nbp2 = 1;
    while (nbp2 < g.nb) nbp2 <<= 1;
    const size_t tail = std::max<size_t>((size_t)64 * (g.D + 1) * 4, (size_t)nbp2 * 8 + (size_t)g.nb * 4);
    const size_t lds = (size_t)rpw * g.D * 4 + (size_t)rpw * g.nb * 4 + tail;
    dim3 grid((g.nb + rpw - 1) / rpw, g.B * g.Hh);
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&k_topk), hipFuncAttributeMaxDynamicSharedMemorySize,
        160 * 1024);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(k_topk, grid, dim3(256), lds, st, g, ht, psq, psk, rpw, nbp2, row_ptr,
                       col_idx, col_cap);
  }
  if (gate) hipLaunchKernelGGL(k_gate, dim3(g.B * g.Hh), dim3(256), 0, st, g, psq, w_g, gate);
  if (info) hipLaunchKernelGGL(k_info, dim3(1), dim3(64), 0, st, flags, ht, info);
  return hipGetLastError();
}

hipError_t launch_gate_from_q(const Geom& g, int dtype, const void* q, const float* w_g,
                              float* gate, char* ws, const Workspace& L, hipStream_t st) {
  HeadTable ht{};
  ht.n_heads = g.Hh;
  for (int h = 0; h < g.Hh; ++h) ht.pool[h] = 1;
  float* psq = reinterpret_cast<float*>(ws + L.off_psum_q);
  float* psk = reinterpret_cast<float*>(ws + L.off_psum_k);
  hipError_t e = dtype == SALAD_BF16 ? launch_pool<__bf16>(g, ht, q, nullptr, psq, psk, st)
                                     : launch_pool<float>(g, ht, q, nullptr, psq, psk, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_gate, dim3(g.B * g.Hh), dim3(256), 0, st, g, psq, w_g, gate);
  return hipGetLastError();
}

}  // namespace salad
