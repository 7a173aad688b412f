// mask.hip - block-mask builder for gfx950: static spatio-temporal window,
// pooled-score top-k and SICS, emitted as CSR lists of kept key blocks.
//
// The masks follow the readings stated in include/salad.h (salad_mask_spec).
// Window: r* of every block pair is computed once per (t_window, r_max) group
// from the horizontal runs of the two blocks (a block covers at most
// ceil(block/W)+1 runs), or in cuboid order from the blocks' box lists, into a
// uint16 table in the workspace.  Selecting the
// first K pairs in (qb!=kb, r*, |qb-kb|, qb, kb) order takes one histogram over
// a combined bin (0 for the diagonal, 1 + r*·nb + |qb-kb| otherwise), a
// per-head scan that finds the bin holding the K-th pair, and a scan over query
// blocks inside that bin (a bin holds at most two pairs per query block,
// kb = qb -+ |qb-kb|).  The K-th pair's packed key (bin·nb² + qb·nb + kb) is
// then the keep threshold; row counts and the CSR emit are table lookups.
//
// Top-k: block sums in float32, sequential in token order, one division per
// mean, scores as a sequential float32 sum of separately rounded products.
// This file is compiled with floating-point contraction off so that no
// multiply-add is fused: the ranking is reproducible bit for bit.  One wave
// per row selects the k largest scores (ties to the lower kb) with a bitwise
// radix search over order-preserving 32-bit keys and emits them ascending.
#include <algorithm>

#include "cuboid.h"
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

constexpr uint16_t kNoCand = 0xffff;

// grid (nb): r* of every (qb, kb) pair for one (t_window, r_max) group, as a
// uint16 table (kNoCand when the pair is no candidate), plus, when `hist` is
// given, the number of candidates in each rank bin.
__global__ void __launch_bounds__(256)
k_window_rstar(Geom g, int tw, int rmax, uint16_t* rt, int32_t* hist) {
  const int qb = blockIdx.x;
  for (int kb = threadIdx.x; kb < g.nb; kb += blockDim.x) {
    const int r = rstar_pair(g, qb, kb, tw);
    const bool cand = window_candidate(r, rmax);
    rt[(int64_t)qb * g.nb + kb] = cand ? (uint16_t)r : kNoCand;
    if (cand && hist) atomicAdd(&hist[pair_bin(qb, kb, r, g.nb)], 1);
  }
}

// Cuboid order: the same table from the blocks' box lists.  Between two boxes
// the least Chebyshev distance over token pairs at most tw frames apart is
// max(y gap, x gap) when the frame gap is <= tw (the three ranges of a box
// vary independently), else infinite; r* is the least over box pairs.
constexpr int kMaxBoxCap = 136;

__global__ void __launch_bounds__(256)
k_window_rstar_boxes(Geom g, int cap, const int32_t* __restrict__ nbox, const Box* __restrict__ boxes,
                     int tw, int rmax, uint16_t* rt, int32_t* hist) {
  __shared__ Box qbx[kMaxBoxCap];
  const int qb = blockIdx.x;
  const int nq = nbox[qb];
  for (int i = threadIdx.x; i < nq; i += blockDim.x) qbx[i] = boxes[(int64_t)qb * cap + i];
  __syncthreads();
  for (int kb = threadIdx.x; kb < g.nb; kb += blockDim.x) {
    const int nk = nbox[kb];
    int best = kRstarInf;
    for (int j = 0; j < nk; ++j) {
      const Box kx = boxes[(int64_t)kb * cap + j];
      for (int i = 0; i < nq; ++i) {
        const Box& qx = qbx[i];
        const int tgap = max(0, max(kx.ty.x - qx.ty.y, qx.ty.x - kx.ty.y));
        if (tgap > tw) continue;
        const int ygap = max(0, max(kx.ty.z - qx.ty.w, qx.ty.z - kx.ty.w));
        const int xgap = max(0, max(kx.x.x - qx.x.y, qx.x.x - kx.x.y));
        best = min(best, max(ygap, xgap));
      }
    }
    const bool cand = window_candidate(best, rmax);
    rt[(int64_t)qb * g.nb + kb] = cand ? (uint16_t)best : kNoCand;
    if (cand && hist) atomicAdd(&hist[pair_bin(qb, kb, best, g.nb)], 1);
  }
}

// r* of one block pair in cuboid order, both box lists read from memory.
__device__ inline int rstar_boxes_pair(int cap, const int32_t* __restrict__ nbox, const Box* __restrict__ boxes,
                                       int qb, int kb, int tw) {
  const int nq = nbox[qb], nk = nbox[kb];
  int best = kRstarInf;
  for (int j = 0; j < nk; ++j) {
    const Box kx = boxes[(int64_t)kb * cap + j];
    for (int i = 0; i < nq; ++i) {
      const Box qx = boxes[(int64_t)qb * cap + i];
      const int tgap = max(0, max(kx.ty.x - qx.ty.y, qx.ty.x - kx.ty.y));
      if (tgap > tw) continue;
      const int ygap = max(0, max(kx.ty.z - qx.ty.w, qx.ty.z - kx.ty.w));
      const int xgap = max(0, max(kx.x.x - qx.x.y, qx.x.x - kx.x.y));
      best = min(best, max(ygap, xgap));
    }
  }
  return best;
}

// The same table, one workgroup per block offset d = kb - qb >= 0, in either
// token order.  r* is symmetric in (qb, kb), so each pair is computed once and
// written to both halves of the table; all pairs of one offset fall in the
// rank bins 1 + r*·nb + d (bin 0 for d = 0), so the workgroup counts them per
// r* in LDS and writes its column of the histogram with plain stores: every
// bin is written, and no clearing pass or global atomics are needed.  Tables
// whose r* range exceeds kMaxRankR use the kernels above.
constexpr int kMaxRankR = 4096;

template <bool BOXES>
__global__ void __launch_bounds__(256)
k_window_rstar_sym(Geom g, int tw, int rmax, uint16_t* rt, int32_t* hist, int cap, const int32_t* nbox,
                   const Box* boxes) {
  __shared__ int cnt[kMaxRankR];
  const int d = blockIdx.x, t = threadIdx.x;
  const int RB = max(g.H, g.W);  // r* < max(H, W)
  if (hist)
    for (int r = t; r < RB; r += blockDim.x) cnt[r] = 0;
  __syncthreads();
  for (int qb = t; qb + d < g.nb; qb += blockDim.x) {
    const int kb = qb + d;
    const int r = BOXES ? rstar_boxes_pair(cap, nbox, boxes, qb, kb, tw) : rstar_pair(g, qb, kb, tw);
    const bool cand = window_candidate(r, rmax);
    const uint16_t v = cand ? (uint16_t)r : kNoCand;
    rt[(int64_t)qb * g.nb + kb] = v;
    if (d > 0) rt[(int64_t)kb * g.nb + qb] = v;
    if (cand && hist) atomicAdd(&cnt[r], d == 0 ? 1 : 2);
  }
  if (!hist) return;
  __syncthreads();
  if (d == 0) {
    // diagonal pairs rank first (bin 0); bins 1 + r*·nb hold nothing
    if (t == 0) {
      int all = 0;
      for (int r = 0; r < RB; ++r) all += cnt[r];
      hist[0] = all;
    }
    for (int r = t; r < RB; r += blockDim.x) hist[1 + (int64_t)r * g.nb] = 0;
  } else {
    for (int r = t; r < RB; r += blockDim.x) hist[1 + (int64_t)r * g.nb + d] = cnt[r];
  }
}

// Block-wide exclusive scan of one int64 per thread (kScanThreads threads):
// shuffle scan inside each wave, then one wave scans the 16 wave totals.
__device__ int64_t block_exclusive_scan(int64_t v, int64_t* tmp, int64_t* total) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int64_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) tmp[w] = x;
  __syncthreads();
  if (w == 0) {
    int64_t s = lane < kScanThreads / 64 ? tmp[lane] : 0;
#pragma unroll
    for (int off = 1; off < kScanThreads / 64; off <<= 1) {
      const int64_t y = __shfl_up(s, off);
      if (lane >= off) s += y;
    }
    if (lane < kScanThreads / 64) tmp[kScanThreads / 64 + lane] = s;
  }
  __syncthreads();
  const int64_t before = w == 0 ? 0 : tmp[kScanThreads / 64 + w - 1];
  if (total) *total = tmp[kScanThreads / 64 + kScanThreads / 64 - 1];
  __syncthreads();
  return before + x - v;
}

__device__ inline int64_t rt_key(const uint16_t* rt, const Geom& g, int qb, int kb, bool* cand) {
  const uint16_t r = rt[(int64_t)qb * g.nb + kb];
  *cand = r != kNoCand;
  return pair_key(pair_bin(qb, kb, r, g.nb), qb, kb, g.nb);
}

// grid (heads), kScanThreads threads: the keep threshold of each window head of
// group `grp` (its r* table and histogram are current).
__global__ void __launch_bounds__(kScanThreads)
k_window_threshold(Geom g, HeadTable ht, int grp, const uint16_t* rt, const int32_t* hist,
                   int64_t hist_bins, int64_t* thr) {
  __shared__ int64_t tmp[2 * kScanThreads / 64];
  __shared__ int64_t s_bin, s_need;
  const int h = blockIdx.x, t = threadIdx.x;
  if (ht.kind[h] != SALAD_MASK_WINDOW || ht.group[h] != grp) return;
  const int64_t K = ht.count[h];
  if (K < 0) {  // keep every candidate
    if (t == 0) thr[h] = INT64_MAX;
    return;
  }
  if (K == 0) {
    if (t == 0) thr[h] = -1;
    return;
  }
  // 1) the bin that holds the K-th pair.  Thread t owns the bins [t*seg, t*seg + seg)
  //    (seg a multiple of 4, so each int4 is aligned; the workspace rounds the
  //    histogram up to 256 bytes, and entries past hist_bins count as 0), read
  //    kVec int4s at a time with every load of a batch in flight.
  constexpr int kVec = 8;
  const int64_t seg = (hist_bins + 4 * kScanThreads - 1) / (4 * kScanThreads) * 4;
  const int64_t lo = min((int64_t)t * seg, hist_bins), hi = min(lo + seg, hist_bins);
  auto load_bins = [&](int64_t b0, int4* x) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kVec; ++u) {
      const int64_t b = min(b0 + 4 * u, (hist_bins - 1) / 4 * 4);  // in bounds, masked below
      x[u] = *reinterpret_cast<const int4*>(hist + b);
    }
  };
  auto bin_at = [&](const int4* x, int64_t b0, int i) __attribute__((always_inline)) -> int {
    const int4 v = x[i >> 2];
    const int e = i & 3;
    const int c = e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
    return b0 + i < hi ? c : 0;
  };
  int64_t local = 0;
  for (int64_t b0 = lo; b0 < hi; b0 += 4 * kVec) {
    int4 x[kVec];
    load_bins(b0, x);
#pragma unroll
    for (int i = 0; i < 4 * kVec; ++i) local += bin_at(x, b0, i);
  }
  int64_t total;
  const int64_t excl = block_exclusive_scan(local, tmp, &total);
  if (total < K) {  // not reached: the host rejects K above the candidate count
    if (t == 0) thr[h] = INT64_MAX;
    return;
  }
  if (excl < K && K <= excl + local) {
    int64_t cum = excl;
    bool found = false;
    for (int64_t b0 = lo; b0 < hi && !found; b0 += 4 * kVec) {
      int4 x[kVec];
      load_bins(b0, x);
#pragma unroll
      for (int i = 0; i < 4 * kVec; ++i) {
        const int c = bin_at(x, b0, i);
        if (!found && b0 + i < hi) {
          if (cum + c >= K) {
            s_bin = b0 + i;
            s_need = K - cum;
            found = true;
          } else {
            cum += c;
          }
        }
      }
    }
  }
  __syncthreads();
  const int64_t bin = s_bin, need = s_need;
  // 2) inside that bin, pairs run in (qb, kb) order with at most two per qb:
  //    (qb, qb - dd) and (qb, qb + dd), or the diagonal alone when dd = 0.  Both
  //    table entries of a qb are read before either is used.
  const int dd = bin == 0 ? 0 : (int)((bin - 1) % g.nb);
  auto pair_in = [&](int qb, bool* lo_in, bool* hi_in) __attribute__((always_inline)) {
    const int kl = qb - dd, kh = qb + dd;
    const bool vl = kl >= 0, vh = dd != 0 && kh < g.nb;
    const uint16_t* row = rt + (int64_t)qb * g.nb;
    const uint16_t rl = row[vl ? kl : qb], rh = row[vh ? kh : qb];
    *lo_in = vl && rl != kNoCand && pair_bin(qb, kl, rl, g.nb) == bin;
    *hi_in = vh && rh != kNoCand && pair_bin(qb, kh, rh, g.nb) == bin;
  };
  const int qseg = (g.nb + kScanThreads - 1) / kScanThreads;
  const int qlo = min(t * qseg, g.nb), qhi = min(qlo + qseg, g.nb);
  int64_t qlocal = 0;
  for (int qb = qlo; qb < qhi; ++qb) {
    bool a, b;
    pair_in(qb, &a, &b);
    qlocal += (int)a + (int)b;
  }
  const int64_t qexcl = block_exclusive_scan(qlocal, tmp, nullptr);
  if (qexcl < need && need <= qexcl + qlocal) {
    int64_t cum = qexcl;
    for (int qb = qlo; qb < qhi; ++qb) {
      bool lo_in, hi_in;
      pair_in(qb, &lo_in, &hi_in);
      const int c = (int)lo_in + (int)hi_in;
      if (cum + c >= need) {
        const int64_t rem = need - cum;
        int kb;
        if (dd == 0) kb = qb;
        else if (rem == 1) kb = lo_in ? qb - dd : qb + dd;
        else kb = qb + dd;
        thr[h] = pair_key(bin, qb, kb, g.nb);
        break;
      }
      cum += c;
    }
  }
}

__device__ inline bool window_keep(const uint16_t* rt, const Geom& g, int qb, int kb, int64_t thr) {
  bool cand;
  const int64_t key = rt_key(rt, g, qb, kb, &cand);
  return cand && (thr == INT64_MAX || key <= thr);
}

// grid (nb, heads), one wave: kept blocks per row, replicated over the batch.
// Window heads of group `grp` count from the r* table; top-k heads (when
// `topk` is set) have k per row.  With direct row pointers the top-k rows
// (closed form) and the final entry go straight to row_ptr instead.
__global__ void __launch_bounds__(64)
k_row_counts(Geom g, HeadTable ht, int grp, int topk, const uint16_t* rt, const int64_t* thr,
             int32_t* rowcnt, int32_t* row_ptr) {
  const int qb = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  if (ht.direct_rows && topk && qb == 0 && h == 0 && lane == 0)
    row_ptr[(int64_t)g.B * g.Hh * g.nb] = g.B * ht.batch_nnz;
  int cnt;
  if (ht.kind[h] == SALAD_MASK_WINDOW) {
    if (ht.group[h] != grp) return;
    int local = 0;
    const int64_t th = thr[h];
    for (int kb = lane; kb < g.nb; kb += 64) local += window_keep(rt, g, qb, kb, th) ? 1 : 0;
    for (int off = 32; off > 0; off >>= 1) local += __shfl_xor(local, off);
    cnt = local;
  } else if (ht.kind[h] == SALAD_MASK_TOPK) {
    if (!topk) return;
    cnt = ht.count[h];
    if (ht.direct_rows) {
      for (int b = lane; b < g.B; b += 64)
        row_ptr[((int64_t)b * g.Hh + h) * g.nb + qb] = b * ht.batch_nnz + ht.base[h] + qb * cnt;
      return;
    }
  } else {
    return;  // SICS heads: k_sics_counts
  }
  if (lane == 0)
    for (int b = 0; b < g.B; ++b) rowcnt[((int64_t)b * g.Hh + h) * g.nb + qb] = cnt;
}

// One workgroup: row_ptr = exclusive scan of the row counts.
__global__ void __launch_bounds__(kScanThreads)
k_scan_rows(const int32_t* rowcnt, int64_t rows, int32_t* row_ptr) {
  __shared__ int64_t tmp[2 * kScanThreads / 64];
  const int t = threadIdx.x;
  const int64_t seg = (rows + kScanThreads - 1) / kScanThreads;
  const int64_t lo = min((int64_t)t * seg, rows), hi = min(lo + seg, rows);
  int64_t local = 0;
#pragma unroll 8
  for (int64_t r = lo; r < hi; ++r) local += rowcnt[r];
  int64_t total;
  int64_t run = block_exclusive_scan(local, tmp, &total);
  // the segment's counts again, 8 loads in flight before their stores
  int64_t r = lo;
  for (; r + 8 <= hi; r += 8) {
    int32_t c[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) c[u] = rowcnt[r + u];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      row_ptr[r + u] = (int32_t)run;
      run += c[u];
    }
  }
  for (; r < hi; ++r) {
    row_ptr[r] = (int32_t)run;
    run += rowcnt[r];
  }
  if (t == 0) row_ptr[rows] = (int32_t)total;
}

// grid (nb, heads), one wave: kept key blocks of the window rows of group `grp`, ascending.
__global__ void __launch_bounds__(64)
k_window_emit(Geom g, HeadTable ht, int grp, const uint16_t* rt, const int64_t* thr,
              int32_t* row_ptr, const int32_t* rowcnt, int32_t* col_idx, int64_t col_cap) {
  const int qb = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  if (ht.kind[h] != SALAD_MASK_WINDOW || ht.group[h] != grp) return;
  const int64_t th = thr[h];
  int64_t first = 0;  // this row's first entry in batch 0 (direct row pointers)
  if (ht.direct_rows) {
    // the head's entries in rows 0 .. qb-1 (the counts are the same in every batch)
    const int32_t* hc = rowcnt + (int64_t)h * g.nb;
    int part = 0;
    for (int r = lane; r < qb; r += 64) part += hc[r];
    for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o);
    first = (int64_t)ht.base[h] + part;
    for (int b = lane; b < g.B; b += 64)
      row_ptr[((int64_t)b * g.Hh + h) * g.nb + qb] = (int32_t)(first + (int64_t)b * ht.batch_nnz);
  }
  int off = 0;
  for (int kb0 = 0; kb0 < g.nb; kb0 += 64) {
    const int kb = kb0 + lane;
    const bool keep = kb < g.nb && window_keep(rt, g, qb, kb, th);
    const uint64_t m = __ballot(keep);
    const int rank = __popcll(m & ((1ull << lane) - 1ull));
    if (keep) {
      for (int b = 0; b < g.B; ++b) {
        const int64_t row0 = ht.direct_rows ? first + (int64_t)b * ht.batch_nnz
                                            : (int64_t)row_ptr[((int64_t)b * g.Hh + h) * g.nb + qb];
        const int64_t pos = row0 + off + rank;
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

// grid (ceil(B*H*nb*(D/8) / 256), 2): per (b, h, block) the float32 mean of 8
// channels per thread (sequential sum in token order, one correctly rounded
// division); blockIdx.y selects Q (0) or K (1).
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
  const float nv = (float)nvalid;
#pragma unroll
  for (int j = 0; j < 8; ++j) dst[j] = __fdiv_rn(acc[j], nv);
}

__device__ inline uint32_t ordered_bits(float s) {
  const uint32_t u = __float_as_uint(s == 0.0f ? 0.0f : s);  // -0 ranks as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Scores of the pooled top-k rule for a batch of heads (bh0 ..): grid
// (ceil(nb / 64) key tiles, ceil(nb / 32) row chunks, heads in the batch),
// 256 threads.  Lane = key block: the tile's 64 key blocks' pooled means sit in
// LDS rows of D + 1 floats (lane l reads row l, channel c: bank (l + c) % 32,
// no conflicts); each wave copies its 8 query blocks' means into its own LDS
// rows and reads them as broadcasts (every lane the same address), 4 rows at a
// time.  Each score is the sequential float32 sum over channels 0..D-1 of
// separately rounded products (this file is compiled without FMA
// contraction), the order the ranking is defined in.  Eight query blocks per
// wave keep the workgroup's LDS at 49 KiB and three workgroups (three waves per
// SIMD, at most 168 registers) fit on a CU: against 16 per wave and two
// workgroups, c4's mask build 2 us and c5's 8 us faster, output bitwise equal.
constexpr int kScoreRowsPerWave = 8;
template <int D>
__global__ void __launch_bounds__(256, 3)
k_topk_scores(Geom g, HeadTable ht, const float* __restrict__ pmean_q, const float* __restrict__ pmean_k,
              float* __restrict__ scores, int bh0) {
  constexpr int KS = D + 1;  // key row stride in LDS (floats)
  constexpr int QR = kScoreRowsPerWave;  // query blocks per wave
  constexpr int RG = 4;      // rows in flight per lane
  __shared__ __align__(16) float keys[64 * KS];
  __shared__ __align__(16) float qrows[4][QR * D];
  const int bh = bh0 + blockIdx.z, h = bh % g.Hh;
  if (ht.kind[h] != SALAD_MASK_TOPK) return;
  const int nb = g.nb, t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int kb0 = blockIdx.x * 64, kb = kb0 + lane;
  const int qb0 = blockIdx.y * 4 * QR + wave * QR;
  const int rows = min(QR, nb - qb0);  // may be <= 0 for the last chunk
#pragma unroll
  for (int i = t; i < 64 * D / 4; i += 256) {  // 16-byte loads, issued together
    const int kk = i / (D / 4), c = (i - kk * (D / 4)) * 4;
    const float4 v = *reinterpret_cast<const float4*>(pmean_k + ((int64_t)bh * nb + min(kb0 + kk, nb - 1)) * D + c);
    float* d = keys + kk * KS + c;
    d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
  }
  float* ql = qrows[wave];
  if (rows > 0) {
    const float4* src = reinterpret_cast<const float4*>(pmean_q + ((int64_t)bh * nb + qb0) * D);
    for (int i = lane; i < rows * D / 4; i += 64) reinterpret_cast<float4*>(ql)[i] = src[i];
  }
  __syncthreads();
  const float* kr = keys + lane * KS;
  float* dst = scores + (int64_t)blockIdx.z * nb * nb;
  for (int r0 = 0; r0 < rows; r0 += RG) {
    float acc[RG];
#pragma unroll
    for (int j = 0; j < RG; ++j) acc[j] = 0.0f;
    const float* qr[RG];
#pragma unroll
    for (int j = 0; j < RG; ++j) qr[j] = ql + min(r0 + j, rows - 1) * D;
#pragma unroll 8
    for (int c4 = 0; c4 < D / 4; ++c4) {
      const float k0 = kr[4 * c4], k1 = kr[4 * c4 + 1], k2 = kr[4 * c4 + 2], k3 = kr[4 * c4 + 3];
#pragma unroll
      for (int j = 0; j < RG; ++j) {
        const float4 q = *reinterpret_cast<const float4*>(qr[j] + 4 * c4);
        acc[j] = acc[j] + q.x * k0;
        acc[j] = acc[j] + q.y * k1;
        acc[j] = acc[j] + q.z * k2;
        acc[j] = acc[j] + q.w * k3;
      }
    }
    if (kb < nb) {
#pragma unroll
      for (int j = 0; j < RG; ++j)
        if (r0 + j < rows) dst[(int64_t)(qb0 + r0 + j) * nb + kb] = acc[j];
    }
  }
}

// Top-k of each row of the scores of a batch of heads: grid (ceil(nb / 4),
// heads in the batch), 256 threads, one wave per query block.  The wave finds
// the k-th largest order-preserving 32-bit key by a bitwise radix search whose
// counts are ballot popcounts over keys held in registers (MAXK per lane),
// keeps every larger key and the first remaining equal keys in kb order, and
// emits the kept kb's ascending.  The search ends at the first bit at which the
// candidates still tied on the bits above are exactly the keys still to take
// (about 15 of 32 bits on 512-block rows of pooled scores).
template <int MAXK>
__global__ void __launch_bounds__(256)
k_topk_select(Geom g, HeadTable ht, const float* __restrict__ scores, int bh0,
              const int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx, int64_t col_cap) {
  const int bh = bh0 + blockIdx.y, h = bh % g.Hh;
  if (ht.kind[h] != SALAD_MASK_TOPK) return;
  const int nb = g.nb, lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= nb) return;
  const float* srow = scores + ((int64_t)blockIdx.y * nb + r) * nb;
  const int kkeep = ht.count[h];
  const int kpl = (nb + 63) / 64;
  const uint64_t lt = (1ull << lane) - 1ull;
  uint32_t key[MAXK];
#pragma unroll
  for (int m = 0; m < MAXK; ++m) {
    if (m < kpl) {
      const int kb = m * 64 + lane;
      key[m] = kb < nb ? ordered_bits(srow[kb]) : 0u;  // real keys are never 0
    }
  }
  // Invariant: every key whose top bits (under `bits`) exceed `prefix` is kept,
  // and krem more are to come from the group of grp real keys whose top bits
  // equal it.  The search stops as soon as that group holds no more keys than
  // are still needed (then all of it is kept); only a group of equal full
  // keys is split, by kb order.
  uint32_t prefix = 0, bits = 0;
  int krem = kkeep, grp = nb;
  for (int bit = 31; bit >= 0 && grp > krem; --bit) {
    const uint32_t bmask = bits | (1u << bit), cand = prefix | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int m = 0; m < MAXK; ++m)
      if (m < kpl) cnt += __popcll(__ballot((key[m] & bmask) == cand));
    if (cnt >= krem) {
      prefix = cand;
      grp = cnt;
    } else {
      krem -= cnt;
      grp -= cnt;
    }
    bits = bmask;
  }
  const int64_t base = row_ptr[(int64_t)bh * nb + r];
  int off = 0, eq_seen = 0;
#pragma unroll
  for (int m = 0; m < MAXK; ++m) {
    if (m < kpl) {
      const int kb = m * 64 + lane;
      const uint32_t top = key[m] & bits;
      const bool eq = top == prefix && kb < nb;
      const uint64_t me = __ballot(eq);
      const bool keep = top > prefix || (eq && eq_seen + __popcll(me & lt) < krem);
      eq_seen += __popcll(me);
      const uint64_t mk = __ballot(keep);
      if (keep) {
        const int64_t pos = base + off + __popcll(mk & lt);
        if (pos < col_cap) col_idx[pos] = kb;
      }
      off += __popcll(mk);
    }
  }
}

// ---- SICS block mask ("SPADE" explainer, scheme generation: blocks whose
// tokens agree, by the sum of intra-block cosine similarities, get attention).
// SICS(b) = sum over valid token pairs of b of cos(k_i, k_j) = || sum_i
// k_i / |k_i| ||^2, in a fixed float32 order (no FMA: this file is compiled
// without contraction): |k_i|^2 sequential over channels; a zero vector
// contributes 0, else khat = k / sqrt(|k|^2) with a correctly rounded square
// root and division; s[c] sequential over the block's tokens in order; SICS =
// sum over channels of s[c]^2, sequential.  Per (b, h) the m =
// max(1, floor(rho * nb + 0.5)) highest blocks (ties to the lower kb) are
// kept for every query block, plus the query block's own block.

// grid (nb, B*H), 256 threads: SICS of one key block of a SICS head.
template <typename T, int D, int BLK>
__global__ void __launch_bounds__(256)
k_sics_scores(Geom g, HeadTable ht, const T* __restrict__ K, float* __restrict__ sics) {
  __shared__ float kl[BLK][D + 1];
  __shared__ float rn[BLK];
  __shared__ float sacc[D];
  const int kb = blockIdx.x, bh = blockIdx.y, h = bh % g.Hh, t = threadIdx.x;
  if (ht.kind[h] != SALAD_MASK_SICS) return;
  const int n0 = kb * BLK, nv = min(BLK, g.N - n0);  // valid tokens, >= 1
  const T* src = K + ((int64_t)bh * g.n_pad + n0) * D;
  // 16-byte loads (all in flight before the LDS stores), converted to float
  constexpr int VE = 16 / sizeof(T);               // elements per 16-byte load
  constexpr int PER = (BLK * D / VE + 255) / 256;  // loads per thread
  uint4 buf[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int i = (u * 256 + t) * VE;
    if (i < nv * D) buf[u] = *reinterpret_cast<const uint4*>(src + i);
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int i = (u * 256 + t) * VE;
    if (i < nv * D) {
      const int r = i / D, c = i - r * D;
      const T* e = reinterpret_cast<const T*>(&buf[u]);
#pragma unroll
      for (int j = 0; j < VE; ++j) kl[r][c + j] = (float)e[j];
    }
  }
  __syncthreads();
  if (t < nv) {
    float n2 = 0.0f;
#pragma unroll  // the reads run ahead of the (ordered) additions
    for (int c = 0; c < D; ++c) n2 = n2 + kl[t][c] * kl[t][c];
    rn[t] = n2 == 0.0f ? 0.0f : __fsqrt_rn(n2);
  }
  __syncthreads();
  // unit keys in place, every element independently (all threads)
  for (int i = t; i < nv * D; i += 256) {
    const int r = i / D, c = i - r * D;
    const float rr = rn[r];
    kl[r][c] = rr == 0.0f ? 0.0f : __fdiv_rn(kl[r][c], rr);
  }
  __syncthreads();
  if (t < D) {
    float sc = 0.0f;
    if (nv == BLK) {
#pragma unroll
      for (int i = 0; i < BLK; ++i) sc = sc + kl[i][t];
    } else {
      for (int i = 0; i < nv; ++i) sc = sc + kl[i][t];
    }
    sacc[t] = sc;
  }
  __syncthreads();
  if (t == 0) {
    float tot = 0.0f;
#pragma unroll
    for (int c = 0; c < D; ++c) tot = tot + sacc[c] * sacc[c];
    sics[(int64_t)bh * g.nb + kb] = tot;
  }
}

// grid (B*H), one wave: the m highest SICS blocks of a head (radix select on
// order-preserving keys, ties to the lower kb).  pack[bh][kb] = 2 * (number
// of kept blocks below kb) + (kb kept).
template <int MAXK>
__global__ void __launch_bounds__(64)
k_sics_select(Geom g, HeadTable ht, const float* __restrict__ sics, int32_t* __restrict__ pack) {
  const int bh = blockIdx.x, h = bh % g.Hh, lane = threadIdx.x;
  if (ht.kind[h] != SALAD_MASK_SICS) return;
  const int nb = g.nb, kpl = (nb + 63) / 64;
  const float* srow = sics + (int64_t)bh * nb;
  const uint64_t lt = (1ull << lane) - 1ull;
  uint32_t key[MAXK];
#pragma unroll
  for (int m = 0; m < MAXK; ++m) {
    if (m < kpl) {
      const int kb = m * 64 + lane;
      key[m] = kb < nb ? ordered_bits(srow[kb]) : 0u;  // real keys are never 0
    }
  }
  uint32_t prefix = 0, bits = 0;
  int krem = ht.count[h];
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t bmask = bits | (1u << bit), cand = prefix | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int m = 0; m < MAXK; ++m)
      if (m < kpl) cnt += __popcll(__ballot((key[m] & bmask) == cand));
    if (cnt >= krem) prefix = cand;
    else krem -= cnt;
    bits = bmask;
  }
  int running = 0, eq_seen = 0;
#pragma unroll
  for (int m = 0; m < MAXK; ++m) {
    if (m < kpl) {
      const int kb = m * 64 + lane;
      const bool eq = key[m] == prefix;
      const uint64_t me = __ballot(eq);
      const bool keep = key[m] > prefix || (eq && eq_seen + __popcll(me & lt) < krem);
      eq_seen += __popcll(me);
      const uint64_t mk = __ballot(keep);
      if (kb < nb) pack[(int64_t)bh * nb + kb] = 2 * (running + __popcll(mk & lt)) + (keep ? 1 : 0);
      running += __popcll(mk);
    }
  }
}

// grid ceil(B*H*nb / 256): row counts of the SICS heads, m or m + 1.
__global__ void __launch_bounds__(256)
k_sics_counts(Geom g, HeadTable ht, const int32_t* __restrict__ pack, int32_t* __restrict__ rowcnt) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)g.B * g.Hh * g.nb) return;
  const int h = (int)((i / g.nb) % g.Hh);
  if (ht.kind[h] != SALAD_MASK_SICS) return;
  rowcnt[i] = ht.count[h] + ((pack[i] & 1) ? 0 : 1);
}

// grid (nb, B*H), one wave: row qb of a SICS head = the kept blocks with qb
// merged in, ascending.
__global__ void __launch_bounds__(64)
k_sics_emit(Geom g, HeadTable ht, const int32_t* __restrict__ pack, const int32_t* __restrict__ row_ptr,
            int32_t* __restrict__ col_idx, int64_t col_cap) {
  const int qb = blockIdx.x, bh = blockIdx.y, h = bh % g.Hh, lane = threadIdx.x;
  if (ht.kind[h] != SALAD_MASK_SICS) return;
  const int nb = g.nb;
  const int32_t* pr = pack + (int64_t)bh * nb;
  const int64_t base = row_ptr[(int64_t)bh * nb + qb];
  const bool qkept = pr[qb] & 1;
  for (int kb = lane; kb < nb; kb += 64) {
    const int v = pr[kb];
    if ((v & 1) || kb == qb) {
      const int64_t pos = base + (v >> 1) + ((!qkept && kb > qb) ? 1 : 0);
      if (pos < col_cap) col_idx[pos] = kb;
    }
  }
}

template <typename T>
hipError_t launch_sics_scores(const Geom& g, const HeadTable& ht, const void* k, float* sics, hipStream_t st) {
  dim3 grid(g.nb, g.B * g.Hh);
  const T* K = static_cast<const T*>(k);
  if (g.D == 128) {
    if (g.blk == 64) hipLaunchKernelGGL((k_sics_scores<T, 128, 64>), grid, dim3(256), 0, st, g, ht, K, sics);
    else hipLaunchKernelGGL((k_sics_scores<T, 128, 128>), grid, dim3(256), 0, st, g, ht, K, sics);
  } else {
    if (g.blk == 64) hipLaunchKernelGGL((k_sics_scores<T, 64, 64>), grid, dim3(256), 0, st, g, ht, K, sics);
    else hipLaunchKernelGGL((k_sics_scores<T, 64, 128>), grid, dim3(256), 0, st, g, ht, K, sics);
  }
  return hipGetLastError();
}

// grid (B*H), 256 threads: gate = sigmoid(mean(Q) . w_g) from the block means,
// each weighted by its valid-token count.  Thread t accumulates channel t % D
// over every (256/D)-th block, in order, in fp64; the partial sums then
// combine in a fixed order.
__global__ void __launch_bounds__(256)
k_gate(Geom g, const float* pmean_q, const float* w_g, float* gate) {
  __shared__ double red[256];
  const int bh = blockIdx.x, t = threadIdx.x;
  const int parts = 256 / g.D, c = t % g.D, part = t / g.D;
  const float* src = pmean_q + (int64_t)bh * g.nb * g.D + c;
  auto nv = [&](int b) { return (double)min(g.blk, g.N - b * g.blk); };
  double s = 0.0;
  int b = part;
  for (; b + 7 * parts < g.nb; b += 8 * parts) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = src[(int64_t)(b + u * parts) * g.D];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += (double)v[u] * nv(b + u * parts);
  }
  for (; b < g.nb; b += parts) s += (double)src[(int64_t)b * g.D] * nv(b);
  red[t] = s;
  __syncthreads();
  if (t < g.D) {
    double tot = 0.0;
    for (int p = 0; p < parts; ++p) tot += red[p * g.D + t];
    red[t] = (tot / (double)g.N) * (double)w_g[t];
  }
  __syncthreads();
  if (t == 0) {
    double dot = 0.0;
    for (int i = 0; i < g.D; ++i) dot += red[i];
    gate[bh] = (float)(1.0 / (1.0 + exp(-dot)));
  }
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

template <int MAXK>
hipError_t launch_topk_select(const Geom& g, const HeadTable& ht, const float* scores, int bh0, int nbh,
                              const int32_t* row_ptr, int32_t* col_idx, int64_t col_cap, hipStream_t st) {
  dim3 grid((g.nb + 3) / 4, nbh);
  hipLaunchKernelGGL(k_topk_select<MAXK>, grid, dim3(256), 0, st, g, ht, scores, bh0, row_ptr, col_idx,
                     col_cap);
  return hipGetLastError();
}

// Scores then selection, for as many heads at a time as the score buffer of
// the workspace holds (topk_heads_per_batch heads).
template <int D>
hipError_t launch_topk(const Geom& g, const HeadTable& ht, const float* pq, const float* pk, float* scores,
                       const int32_t* row_ptr, int32_t* col_idx, int64_t col_cap, hipStream_t st) {
  const int BH = g.B * g.Hh;
  const int per = topk_heads_per_batch(g);
  for (int bh0 = 0; bh0 < BH; bh0 += per) {
    const int nbh = std::min(per, BH - bh0);
    dim3 grid((g.nb + 63) / 64, (g.nb + 4 * kScoreRowsPerWave - 1) / (4 * kScoreRowsPerWave), nbh);
    hipLaunchKernelGGL(k_topk_scores<D>, grid, dim3(256), 0, st, g, ht, pq, pk, scores, bh0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (g.nb <= 512) e = launch_topk_select<8>(g, ht, scores, bh0, nbh, row_ptr, col_idx, col_cap, st);
    else if (g.nb <= 1024) e = launch_topk_select<16>(g, ht, scores, bh0, nbh, row_ptr, col_idx, col_cap, st);
    else if (g.nb <= 2048) e = launch_topk_select<32>(g, ht, scores, bh0, nbh, row_ptr, col_idx, col_cap, st);
    else e = launch_topk_select<64>(g, ht, scores, bh0, nbh, row_ptr, col_idx, col_cap, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_build_mask(const Geom& g, const Cuboid& cu, int dtype, const HeadTable& ht0,
                             const void* q,
                             const void* k, int32_t* row_ptr, int32_t* col_idx, int64_t col_cap,
                             const float* w_g, float* gate, char* ws,
                             const Workspace& L, hipStream_t st) {
  HeadTable ht = ht0;
  bool any_topk = false, any_sics = false;
  // window heads sharing (t_window, r_max) share one r* table and histogram
  int n_groups = 0;
  int grp_tw[SALAD_MAX_HEADS], grp_rmax[SALAD_MAX_HEADS];
  bool grp_ranked[SALAD_MAX_HEADS];
  for (int h = 0; h < g.Hh; ++h) {
    ht.pool[h] = 0;
    ht.group[h] = -1;
    if (ht.kind[h] == SALAD_MASK_WINDOW) {
      int gi = 0;
      while (gi < n_groups && !(grp_tw[gi] == ht.t_window[h] && grp_rmax[gi] == ht.r_max[h])) ++gi;
      if (gi == n_groups) {
        grp_tw[gi] = ht.t_window[h];
        grp_rmax[gi] = ht.r_max[h];
        grp_ranked[gi] = false;
        ++n_groups;
      }
      ht.group[h] = gi;
      if (ht.count[h] >= 0) grp_ranked[gi] = true;
    } else if (ht.kind[h] == SALAD_MASK_TOPK) {
      any_topk = true;
      ht.pool[h] = 3;
    } else {
      any_sics = true;
    }
    if (gate) ht.pool[h] |= 1;
  }
  uint16_t* rt = reinterpret_cast<uint16_t*>(ws + L.off_rt);
  int32_t* hist = reinterpret_cast<int32_t*>(ws + L.off_hist);
  int64_t* thr = reinterpret_cast<int64_t*>(ws + L.off_thr);
  int32_t* rowcnt = reinterpret_cast<int32_t*>(ws + L.off_rowcnt);
  float* psq = reinterpret_cast<float*>(ws + L.off_psum_q);
  float* psk = reinterpret_cast<float*>(ws + L.off_psum_k);

  if (any_topk || gate) {
    hipError_t e = dtype == SALAD_BF16 ? launch_pool<__bf16>(g, ht, q, k, psq, psk, st)
                                       : launch_pool<float>(g, ht, q, k, psq, psk, st);
    if (e != hipSuccess) return e;
  }
  const int32_t* nbox = reinterpret_cast<const int32_t*>(ws + L.off_nbox);
  const Box* boxes = reinterpret_cast<const Box*>(ws + L.off_boxes);
  if (cu.ct != 0 && cu.box_cap > kMaxBoxCap) return hipErrorInvalidValue;
  // tables of moderate r* range come from the symmetric kernels, which also
  // write every histogram bin (no clearing pass)
  const bool sym = std::max(g.H, g.W) <= kMaxRankR;
  auto rstar = [&](int gi, int32_t* h) {
    if (sym && cu.ct == 0)
      hipLaunchKernelGGL(k_window_rstar_sym<false>, dim3(g.nb), dim3(256), 0, st, g, grp_tw[gi], grp_rmax[gi],
                         rt, h, 0, nullptr, nullptr);
    else if (sym)
      hipLaunchKernelGGL(k_window_rstar_sym<true>, dim3(g.nb), dim3(256), 0, st, g, grp_tw[gi], grp_rmax[gi],
                         rt, h, cu.box_cap, nbox, boxes);
    else if (cu.ct == 0)
      hipLaunchKernelGGL(k_window_rstar, dim3(g.nb), dim3(256), 0, st, g, grp_tw[gi], grp_rmax[gi], rt, h);
    else
      hipLaunchKernelGGL(k_window_rstar_boxes, dim3(g.nb), dim3(256), 0, st, g, cu.box_cap, nbox, boxes,
                         grp_tw[gi], grp_rmax[gi], rt, h);
  };
  if (cu.ct != 0 && n_groups > 0) {
    hipError_t e = launch_block_boxes(g, cu, ws, L, st);
    if (e != hipSuccess) return e;
  }
  // counts: every window group in turn (its r* table lives in the workspace)
  for (int gi = 0; gi < n_groups; ++gi) {
    int32_t* h_ptr = nullptr;
    if (grp_ranked[gi]) {
      if (!sym)
        hipLaunchKernelGGL(k_fill_i32, dim3((unsigned)std::min<size_t>((L.hist_bins + 255) / 256, 4096)),
                           dim3(256), 0, st, hist, (int64_t)L.hist_bins, 0);
      h_ptr = hist;
    }
    rstar(gi, h_ptr);
    hipLaunchKernelGGL(k_window_threshold, dim3(g.Hh), dim3(kScanThreads), 0, st, g, ht, gi, rt, hist,
                       (int64_t)L.hist_bins, thr);
    hipLaunchKernelGGL(k_row_counts, dim3(g.nb, g.Hh), dim3(64), 0, st, g, ht, gi, (int)(gi == 0), rt, thr,
                       rowcnt, row_ptr);
  }
  if (n_groups == 0)
    hipLaunchKernelGGL(k_row_counts, dim3(g.nb, g.Hh), dim3(64), 0, st, g, ht, -1, 1, rt, thr, rowcnt, row_ptr);
  const int64_t rows = (int64_t)g.B * g.Hh * g.nb;
  float* sics = reinterpret_cast<float*>(ws + L.off_sics);
  int32_t* pack = reinterpret_cast<int32_t*>(ws + L.off_sics_pack);
  if (any_sics) {
    hipError_t e = dtype == SALAD_BF16 ? launch_sics_scores<__bf16>(g, ht, k, sics, st)
                                       : launch_sics_scores<float>(g, ht, k, sics, st);
    if (e != hipSuccess) return e;
    const dim3 sg(g.B * g.Hh);
    if (g.nb <= 512) hipLaunchKernelGGL(k_sics_select<8>, sg, dim3(64), 0, st, g, ht, sics, pack);
    else if (g.nb <= 1024) hipLaunchKernelGGL(k_sics_select<16>, sg, dim3(64), 0, st, g, ht, sics, pack);
    else if (g.nb <= 2048) hipLaunchKernelGGL(k_sics_select<32>, sg, dim3(64), 0, st, g, ht, sics, pack);
    else hipLaunchKernelGGL(k_sics_select<64>, sg, dim3(64), 0, st, g, ht, sics, pack);
    hipLaunchKernelGGL(k_sics_counts, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, g, ht, pack,
                       rowcnt);
  }
  if (!ht.direct_rows)
    hipLaunchKernelGGL(k_scan_rows, dim3(1), dim3(kScanThreads), 0, st, rowcnt, rows, row_ptr);
  if (any_sics)
    hipLaunchKernelGGL(k_sics_emit, dim3(g.nb, g.B * g.Hh), dim3(64), 0, st, g, ht, pack, row_ptr, col_idx,
                       col_cap);
  // emit: the last group's table is still current; the others are rebuilt
  for (int gi = n_groups - 1; gi >= 0; --gi) {
    if (gi != n_groups - 1) rstar(gi, nullptr);
    hipLaunchKernelGGL(k_window_emit, dim3(g.nb, g.Hh), dim3(64), 0, st, g, ht, gi, rt, thr, row_ptr, rowcnt,
                       col_idx, col_cap);
  }
  if (any_topk) {
    float* scores = reinterpret_cast<float*>(ws + L.off_scores);
    hipError_t e = g.D == 128 ? launch_topk<128>(g, ht, psq, psk, scores, row_ptr, col_idx, col_cap, st)
                              : launch_topk<64>(g, ht, psq, psk, scores, row_ptr, col_idx, col_cap, st);
    if (e != hipSuccess) return e;
  }
  if (gate) hipLaunchKernelGGL(k_gate, dim3(g.B * g.Hh), dim3(256), 0, st, g, psq, w_g, gate);
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
