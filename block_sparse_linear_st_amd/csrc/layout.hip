// layout.hip - token storage order: the permutation between frame-major and
// cuboid order of [B][heads][n_pad][head_dim] tensors, and the box lists of the
// blocks' token sets that the window mask measures distances on.
//
// The permutation is pure data movement (HBM bound): a workgroup owns 256/CH
// slots (CH = 16-byte chunks per token row); each thread maps its slot once
// (a handful of integer divisions, closed form) and then copies one 16-byte
// chunk of that slot for every (batch, head), four loads in flight.
#include "cuboid.h"

namespace salad {

namespace {

template <int CH>
__global__ void __launch_bounds__(256)
k_permute(Geom g, Cuboid cu, int inverse, const int4* __restrict__ src, int4* __restrict__ dst) {
  constexpr int SPW = 256 / CH;
  const int p = blockIdx.x * SPW + (int)threadIdx.x / CH;
  const int lane = threadIdx.x % CH;
  if (p >= g.n_pad) return;
  const int tok = p < g.N ? slot_token(g, cu, p) : p;
  const int from = inverse ? p : tok;
  const int to = inverse ? tok : p;
  const int64_t hs = (int64_t)g.n_pad * CH;  // int4s per (batch, head)
  const int4* s = src + (int64_t)from * CH + lane;
  int4* d = dst + (int64_t)to * CH + lane;
  const int BH = g.B * g.Hh;
  int i = 0;
  for (; i + 4 <= BH; i += 4) {
    const int4 v0 = s[(i + 0) * hs];
    const int4 v1 = s[(i + 1) * hs];
    const int4 v2 = s[(i + 2) * hs];
    const int4 v3 = s[(i + 3) * hs];
    d[(i + 0) * hs] = v0;
    d[(i + 1) * hs] = v1;
    d[(i + 2) * hs] = v2;
    d[(i + 3) * hs] = v3;
  }
  for (; i < BH; ++i) d[i * hs] = s[i * hs];
}

// One thread per block: its box list (at most box_cap boxes) and their count.
__global__ void __launch_bounds__(64)
k_block_boxes(Geom g, Cuboid cu, int32_t* nbox, Box* boxes) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= g.nb) return;
  nbox[j] = block_boxes(g, cu, j, boxes + (int64_t)j * cu.box_cap, cu.box_cap);
}

}  // namespace

hipError_t launch_permute_tokens(const Geom& g, const Cuboid& cu, int dtype, int inverse,
                                 const void* src, void* dst, hipStream_t st) {
  const int chunks = g.D * (dtype == SALAD_BF16 ? 2 : 4) / 16;
  const int4* s = static_cast<const int4*>(src);
  int4* d = static_cast<int4*>(dst);
  switch (chunks) {
    case 8:
      hipLaunchKernelGGL(k_permute<8>, dim3((g.n_pad + 31) / 32), dim3(256), 0, st, g, cu, inverse, s, d);
      break;
    case 16:
      hipLaunchKernelGGL(k_permute<16>, dim3((g.n_pad + 15) / 16), dim3(256), 0, st, g, cu, inverse, s, d);
      break;
    case 32:
      hipLaunchKernelGGL(k_permute<32>, dim3((g.n_pad + 7) / 8), dim3(256), 0, st, g, cu, inverse, s, d);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_block_boxes(const Geom& g, const Cuboid& cu, char* ws, const Workspace& L,
                              hipStream_t st) {
  hipLaunchKernelGGL(k_block_boxes, dim3((g.nb + 63) / 64), dim3(64), 0, st, g, cu,
                     reinterpret_cast<int32_t*>(ws + L.off_nbox),
                     reinterpret_cast<Box*>(ws + L.off_boxes));
  return hipGetLastError();
}

}  // namespace salad
