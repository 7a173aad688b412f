// check.hip - validation of a caller's CSR block mask (salad_check_mask).
//
// The attention kernels turn every col_idx entry into a key/value tile address
// without checking it, and walk each row's list assuming it ascends (the merge
// of two query blocks' lists needs that order).  This one-workgroup kernel
// checks the structure those kernels rely on and writes a bit set of the
// problems it found; it never reads outside [row_ptr, row_ptr + rows] and
// [col_idx, col_idx + col_cap), whatever the arrays hold.
#include "internal.h"

namespace salad {

namespace {

constexpr int kCheckThreads = 1024;

// One wave per row, rows strided over the workgroup's 16 waves: lanes read
// consecutive entries (coalesced) and compare each with its predecessor.
__global__ void __launch_bounds__(kCheckThreads)
k_check_mask(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int64_t rows,
             int64_t col_cap, int nb, int32_t* out) {
  __shared__ int s_bad;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  if (t == 0) s_bad = 0;
  __syncthreads();
  int bad = 0;
  if (t == 0 && row_ptr[0] != 0) bad |= SALAD_MASK_BAD_START;
  if (t == 0 && (row_ptr[rows] < 0 || (int64_t)row_ptr[rows] > col_cap)) bad |= SALAD_MASK_BAD_ROW_PTR;
  for (int64_t r = wave; r < rows; r += kCheckThreads / 64) {
    const int32_t b = row_ptr[r], e = row_ptr[r + 1];
    if (b < 0 || e < b || (int64_t)e > col_cap) {
      bad |= SALAD_MASK_BAD_ROW_PTR;  // this row's entries are not read
      continue;
    }
    int prev_last = -1;  // last entry of the previous chunk of this row
    for (int32_t i0 = b; i0 < e; i0 += 64) {
      const int32_t i = i0 + lane;
      const int c = i < e ? col_idx[i] : INT32_MAX;
      if (i < e && (c < 0 || c >= nb)) bad |= SALAD_MASK_BAD_COL;
      int before = __shfl_up(c, 1);
      if (lane == 0) before = prev_last;
      if (i < e && c <= before) bad |= SALAD_MASK_BAD_ORDER;
      prev_last = __shfl(c, 63);
    }
  }
  if (bad) atomicOr(&s_bad, bad);
  __syncthreads();
  if (t == 0) out[0] = s_bad;
}

}  // namespace

hipError_t launch_check_mask(const Geom& g, const int32_t* row_ptr, const int32_t* col_idx,
                             int64_t col_cap, int32_t* out, hipStream_t st) {
  const int64_t rows = (int64_t)g.B * g.Hh * g.nb;
  hipLaunchKernelGGL(k_check_mask, dim3(1), dim3(kCheckThreads), 0, st, row_ptr, col_idx, rows, col_cap,
                     g.nb, out);
  return hipGetLastError();
}

}  // namespace salad
