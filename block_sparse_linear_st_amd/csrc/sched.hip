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

// One workgroup per job.  Item i = (s, j) covers rows j*per ..
// min(nrows, (j+1)*per)-1 of sequence s.  cum(i), the estimated work of items
// [0, i), grows strictly (ovh > 0), so each eighth of the total is crossed by
// exactly one i in [0, n_items].
__global__ void __launch_bounds__(kSplitThreads) k_item_split(ItemSplit j0, ItemSplit j1) {
  __shared__ int s_cut[8];
  const ItemSplit J = blockIdx.x == 0 ? j0 : j1;
  const int t = threadIdx.x;
  const int groups = (J.nrows + J.per - 1) / J.per;
  const int n_items = J.n_seq * groups;
  const int cap = xcd_items_cap(n_items);
  auto first_row = [&](int i) -> int64_t {
    const int s = i / groups;
    return (int64_t)s * J.nrows + (int64_t)(i - s * groups) * J.per;
  };
  if (t < 8) s_cut[t] = n_items;
  const int64_t p0 = J.ptr[0];
  const int64_t total = ((int64_t)J.ptr[(int64_t)J.n_seq * J.nrows] - p0) * J.tpb + (int64_t)J.ovh * n_items;
  __syncthreads();
  for (int base = 0; base <= n_items; base += kSplitBatch * kSplitThreads) {
    int32_t pc[kSplitBatch], pp[kSplitBatch];
#pragma unroll
    for (int k = 0; k < kSplitBatch; ++k) {
      const int i = base + k * kSplitThreads + t;
      pc[k] = i <= n_items ? J.ptr[first_row(i)] : 0;
      pp[k] = i >= 1 && i <= n_items ? J.ptr[first_row(i - 1)] : 0;
    }
#pragma unroll
    for (int k = 0; k < kSplitBatch; ++k) {
      const int i = base + k * kSplitThreads + t;
      if (i > n_items) break;
      const int64_t c = ((int64_t)pc[k] - p0) * J.tpb + (int64_t)J.ovh * i;
      const int64_t prev = i == 0 ? -1 : ((int64_t)pp[k] - p0) * J.tpb + (int64_t)J.ovh * (i - 1);
#pragma unroll
      for (int x = 1; x < 8; ++x) {
        const int64_t target = total * x / 8;
        if (c >= target && prev < target) s_cut[x] = i;
      }
    }
  }
  __syncthreads();
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
