// sched.hip - work-balanced assignment of attention work items to the XCDs.
//
// Workgroup w of a launch runs on XCD w % 8, and each XCD has its own L2.  The
// attention kernels give every XCD one contiguous run of items (query-block
// groups, or key blocks, in row order), so that neighbouring items, which read
// mostly the same tiles, share an L2.  With equal item counts per XCD, a layer
// whose heads differ in density leaves some XCDs idle while others finish; the
// cut here puts the boundaries where the running work estimate crosses each
// eighth of the total.  An item's work is estimated from the pointer array
// alone: kept blocks of its rows times tiles per block, plus a fixed per-item
// cost (loading its own rows, the epilogue, the stores).
#include "internal.h"

namespace salad {

namespace {

constexpr int kSplitThreads = 1024;
constexpr int kSplitBatch = 16;  // items per thread whose pointer loads are issued together
// Layout modes: up to kModeSamples neighbouring block pairs per head, spread
// evenly over batch 0's query blocks (kModeMaxSamples in all, at least one per
// head), the first kModeCap entries of each list compared.
constexpr int kModeSamples = 2;
constexpr int kModeMaxSamples = kPairModeSlots;
constexpr int kModeCap = 32;
constexpr int kModePerThread = kModeMaxSamples * kModeCap / kSplitThreads;

// One workgroup per job.  Item i = (s, j) covers rows j*per ..
// min(nrows, (j+1)*per)-1 of sequence s.  cum(i), the estimated work of items
// [0, i), grows strictly (ovh > 0), so its eighths e(i) never decrease and
// every x in 1..7 is passed by exactly one i in [0, n_items].
//
// Modes (mode_heads > 0): sample k of head h is the block pair (2j, 2j+1) with
// j = (2k+1)*P / (2S), P = nrows/2 pairs, S samples per head.  The first
// kModeCap entries of each list are compared: the second list is staged in
// LDS, each entry of the first is looked up in it in two rounds of reads
// (every 8th entry, then the 8 entries of its segment), and a ballot counts
// the common entries.  Head h takes mode 1 when 4 * sum(union) >
// 5 * sum(longer list) over its samples.
__global__ void __launch_bounds__(kSplitThreads) k_item_split(ItemSplit j0, ItemSplit j1) {
  __shared__ int s_cut[8];
  __shared__ int s_bnd[kModeMaxSamples][3];       // first-list start, second-list start, second-list end
  __shared__ int s_list[kModeMaxSamples][kModeCap];
  __shared__ int s_inter[kModeMaxSamples];
  const ItemSplit J = blockIdx.x == 0 ? j0 : j1;
  const int t = threadIdx.x;
  const int groups = (J.nrows + J.per - 1) / J.per;
  const int n_items = J.n_seq * groups;
  const int cap = xcd_items_cap(n_items);
  const bool whole = J.nrows % J.per == 0;  // no short last item: first_row(i) = per * i
  auto first_row = [&](int i) -> int64_t {
    if (whole) return (int64_t)J.per * i;
    const int s = i / groups;
    return (int64_t)s * J.nrows + (int64_t)(i - s * groups) * J.per;
  };
  const int npairs = J.nrows / 2;
  const int per_head = J.mode_heads > 0 ? max(1, min(kModeSamples, kModeMaxSamples / J.mode_heads)) : 0;
  const int nsamp = npairs > 0 ? J.mode_heads * per_head : 0;
  if (t < 8) s_cut[t] = n_items;
  if (t < nsamp) {
    const int h = t / per_head, k = t - h * per_head;
    const int j = (int)((int64_t)(2 * k + 1) * npairs / (2 * per_head));
    const int64_t r0 = (int64_t)h * J.nrows + 2 * j;
    s_bnd[t][0] = J.ptr[r0];
    s_bnd[t][1] = J.ptr[r0 + 1];
    s_bnd[t][2] = J.ptr[r0 + 2];
  }
  const int64_t p0 = J.ptr[0];
  const int64_t total = ((int64_t)J.ptr[(int64_t)J.n_seq * J.nrows] - p0) * J.tpb + (int64_t)J.ovh * n_items;
  __syncthreads();
  // sampled lists: entry l of sample s at index s*kModeCap + l, kModePerThread
  // per thread; every load is issued before the first one is used
  int av[kModePerThread], bv[kModePerThread];
#pragma unroll
  for (int u = 0; u < kModePerThread; ++u) {
    const int idx = u * kSplitThreads + t, s = idx / kModeCap, l = idx % kModeCap;
    av[u] = -1;
    bv[u] = -1;
    if (s < nsamp) {
      const int a0 = s_bnd[s][0], a1 = s_bnd[s][1], b1 = s_bnd[s][2];
      if (l < min(a1 - a0, kModeCap)) av[u] = J.col[a0 + l];
      if (l < min(b1 - a1, kModeCap)) bv[u] = J.col[a1 + l];
    }
  }
  // eighths of the estimate, e(i) = floor(8 cum(i) / total) in float (the cuts
  // only steer the work balance): item i starts run x for e(i-1) < x <= e(i).
  // Lanes hold consecutive items, so e(i-1) comes from the lane below; lane 0
  // loads its predecessor's pointer itself.
  const float eighths = 8.0f / (float)total;
  // (no contraction into FMAs, so that two lanes computing e of one item agree)
  auto eighth = [&](int32_t ptr_i, int i) -> int {
    const float c = __fadd_rn(__fmul_rn((float)(ptr_i - (int32_t)p0), (float)J.tpb), __fmul_rn((float)J.ovh, (float)i));
    return min(8, (int)__fmul_rn(c, eighths));
  };
  const int lane = t & 63;
  for (int base = 0; base <= n_items; base += kSplitBatch * kSplitThreads) {
    int32_t pc[kSplitBatch], pl[kSplitBatch];
#pragma unroll
    for (int k = 0; k < kSplitBatch; ++k) {
      const int i = base + k * kSplitThreads + t;
      pc[k] = i <= n_items ? J.ptr[first_row(i)] : 0;
      pl[k] = lane == 0 && i >= 1 && i <= n_items ? J.ptr[first_row(i - 1)] : 0;
    }
#pragma unroll
    for (int k = 0; k < kSplitBatch; ++k) {
      const int i = base + k * kSplitThreads + t;
      const int below = __shfl_up(pc[k], 1);
      if (i > n_items) break;
      const int e = eighth(pc[k], i);
      const int e_prev = i == 0 ? e : eighth(lane == 0 ? pl[k] : below, i - 1);
      for (int x = max(e_prev + 1, 1); x <= min(e, 7); ++x) s_cut[x] = i;
    }
  }
#pragma unroll
  for (int u = 0; u < kModePerThread; ++u) {
    const int idx = u * kSplitThreads + t, s = idx / kModeCap;
    if (s < nsamp && bv[u] >= 0) s_list[s][idx % kModeCap] = bv[u];
  }
  __syncthreads();
  if (nsamp > 0) {
    // half a wave's 32 consecutive indices are one sample's entries
#pragma unroll
    for (int u = 0; u < kModePerThread; ++u) {
      const int idx = u * kSplitThreads + t, s = idx / kModeCap;  // s < kModeMaxSamples
      if (idx - (t & 63) >= nsamp * kModeCap) break;  // uniform per wave
      const int nb2 = s < nsamp ? min(s_bnd[s][2] - s_bnd[s][1], kModeCap) : 0;
      const int a = s < nsamp ? av[u] : -1;
      int first = 0;  // entries 0, 8, 16, 24 of the second list that are <= a
#pragma unroll
      for (int k = 0; k < kModeCap / 8; ++k) first += (8 * k < nb2 && s_list[s][8 * k] <= a) ? 1 : 0;
      bool found = false;
      if (a >= 0 && first > 0) {
        const int seg = 8 * (first - 1);
#pragma unroll
        for (int m = 0; m < 8; ++m) found |= seg + m < nb2 && s_list[s][seg + m] == a;
      }
      const uint64_t bal = __ballot(found);
      const int half = (t & 63) >> 5;
      if ((t & 31) == 0 && s < nsamp) s_inter[s] = __popcll(half ? bal >> 32 : bal & 0xffffffffull);
    }
  }
  __syncthreads();
  // word 9 + x holds the mode of sequence x (head x % mode_heads) for every
  // x < min(n_seq, kPairModeSlots)
  if (J.mode_heads > 0 && t < min(J.n_seq, kPairModeSlots)) {
    const int h = t % J.mode_heads;
    int64_t uni = 0, longer = 0;
    for (int k = 0; k < (nsamp > 0 ? per_head : 0); ++k) {
      const int s = h * per_head + k;
      const int na = min(s_bnd[s][1] - s_bnd[s][0], kModeCap), nb2 = min(s_bnd[s][2] - s_bnd[s][1], kModeCap);
      uni += na + nb2 - s_inter[s];
      longer += max(na, nb2);
    }
    J.split[9 + t] = 4 * uni > 5 * longer ? 1 : 0;
  }
  if (t == 0) {
    // no run longer than cap (the launch has 8*cap workgroups), and what is
    // left after run x always fits in the remaining 7-x runs
    int s = 0;
    J.split[0] = 0;
    for (int x = 1; x < 8; ++x) {
      int v = max(s_cut[x], n_items - (8 - x) * cap);
      v = max(s, min(v, s + cap));
      J.split[x] = v;
      s = v;
    }
    J.split[8] = n_items;
  }
}

}  // namespace

hipError_t launch_item_splits(const ItemSplit* jobs, int n_jobs, hipStream_t st) {
  if (n_jobs < 1 || n_jobs > 2) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_item_split, dim3(n_jobs), dim3(kSplitThreads), 0, st, jobs[0], jobs[n_jobs - 1]);
  return hipGetLastError();
}

}  // namespace salad
