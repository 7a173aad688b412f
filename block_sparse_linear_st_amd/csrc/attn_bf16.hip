// attn_bf16.hip - fused hybrid attention forward for gfx950, bf16 in/out.
//
// One workgroup (4 waves) owns 128 query rows: two 64-token query blocks, or
// one 128-token block.  Each wave owns 32 rows.  The workgroup walks the
// ascending union of its query blocks' kept key-block lists (a two-way merge of
// the CSR rows) in 64-key tiles; a wave computes a tile only when its own
// query block keeps that key block, so dropped blocks cost nothing and shared
// ones are loaded once for both query blocks.
//
// Per tile, with MFMA 32x32x16 bf16 (fp32 accumulate):
//   S^T = K Q^T      A = K tile from LDS, B = Q fragments kept in registers
//   online softmax   per query row; a row's 64 scores sit in one lane pair
//                    (lanes l and l^32), so row max and sum need one exchange
//   O^T += V^T P^T   A = V^T tile from LDS, B = P straight from the S^T
//                    accumulators (bf16), no shuffles
// Working in the transposed orientation keeps every per-query quantity
// (max, sum, rescale factor) in the lane that owns the query.
//
// K/V tiles are double buffered: the next tile's global loads are issued into
// registers before the current tile's MFMAs and written to the other LDS
// buffer after them; one barrier per tile.  V is written transposed, with the
// key order inside every 16-key group permuted so that each MFMA A-fragment is
// one 16-byte LDS read and matches the key order the S^T accumulator hands to
// P.
//
// Epilogue: o_s = O / l; the linear branch ("SALAD" explainer, section 2.1)
// and its gated projection (section 2.2) arrive pre-folded as
// S''^T = (g S W_lin)^T (hi + lo bf16), so g*(o_l W_lin) = (S''^T ReLU(Q)^T) /
// (ReLU(Q) z + eps) is 2*(D/32)*(D/16) more MFMAs on the Q fragments already
// in registers.  Heads whose gate is below drop_tau skip it (section 2.3).
// The 128 x D bf16 result is staged through LDS for 16-byte coalesced stores.
//
// Work items map to workgroups so that each XCD (blockIdx % 8) gets a
// contiguous range of (head, query group) items: neighbouring query blocks,
// whose window lists overlap, share that XCD's L2.
#include "internal.h"

namespace salad {
namespace {

constexpr int kTK = 64;        // keys per LDS tile
constexpr int kVST = kTK + 8;  // V^T row stride (bf16): 144 B keeps A-fragment reads conflict-free

__device__ inline int vt_pos(int key) {
  // position of a key inside its 16-key group so that lane group g's slots
  // j = 0..7 (keys (j/4)*8 + g*4 + j%4) are contiguous
  const int k = key & 15;
  return (key & ~15) | (((k >> 2) & 1) << 3) | ((k >> 3) << 2) | (k & 3);
}

template <int D>
struct Smem {
  static constexpr int KST = D + 8;                         // K row stride (bf16)
  static constexpr int K_ELEMS = kTK * KST;
  static constexpr int V_ELEMS = D * kVST;
  static constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;
  static constexpr int BYTES = 2 * BUF_ELEMS * 2;
  static constexpr int OST = D + 8;                         // output staging stride
  static_assert(128 * OST <= 2 * BUF_ELEMS, "output staging must fit");
};

// Two-way merge over the kept lists of the workgroup's query blocks, expanded
// into 64-key tiles.  All values are uniform across the workgroup.
struct TileIter {
  const int32_t* col;
  int i0, e0, i1, e1, c0, c1;
  int kb, sub, flags;
  bool valid;
  __device__ void init(const int32_t* col_idx, int b0, int en0, int b1, int en1) {
    col = col_idx;
    i0 = b0; e0 = en0; i1 = b1; e1 = en1;
    c0 = i0 < e0 ? col[i0] : INT32_MAX;
    c1 = i1 < e1 ? col[i1] : INT32_MAX;
    sub = 0;
    take();
  }
  __device__ void take() {
    kb = min(c0, c1);
    valid = kb != INT32_MAX;
    flags = (c0 == kb ? 1 : 0) | (c1 == kb ? 2 : 0);
    if (c0 == kb) { ++i0; c0 = i0 < e0 ? col[i0] : INT32_MAX; }
    if (c1 == kb) { ++i1; c1 = i1 < e1 ? col[i1] : INT32_MAX; }
    sub = 0;
  }
  // advance to the next tile; sub-tiles lying wholly in the padding are skipped
  __device__ void next(int blk, int N) {
    if (sub + 1 < blk / kTK && kb * blk + (sub + 1) * kTK < N) { ++sub; return; }
    take();
  }
  __device__ int key0(int blk) const { return kb * blk + sub * kTK; }
};

template <int D>
struct TileRegs {
  static constexpr int CPR = D / 8;               // 16-byte chunks per row
  static constexpr int KCH = kTK * CPR / 256;     // K chunks per thread
  static constexpr int VPR = (kTK / 2) * CPR / 256;  // V key-pair chunks per thread
  uint4 k[KCH];
  uint4 v[VPR][2];

  __device__ void load(const __bf16* Kb, const __bf16* Vb, int key0, int N, int tid) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int ch = tid + 256 * i, key = ch / CPR, dc = ch % CPR;
      const int n = key0 + key;
      k[i] = (unsigned)n < (unsigned)N ? *reinterpret_cast<const uint4*>(Kb + (int64_t)n * D + dc * 8)
                   : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < VPR; ++i) {
      const int pc = tid + 256 * i, kp = pc / CPR, dc = pc % CPR;
      const int n = key0 + 2 * kp;
      v[i][0] = (unsigned)n < (unsigned)N ? *reinterpret_cast<const uint4*>(Vb + (int64_t)n * D + dc * 8)
                      : make_uint4(0, 0, 0, 0);
      v[i][1] = (unsigned)(n + 1) < (unsigned)N ? *reinterpret_cast<const uint4*>(Vb + (int64_t)(n + 1) * D + dc * 8)
                          : make_uint4(0, 0, 0, 0);
    }
  }

  __device__ void store(__bf16* Ks, __bf16* Vt, int tid) const {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int ch = tid + 256 * i, key = ch / CPR, dc = ch % CPR;
      *reinterpret_cast<uint4*>(Ks + key * Smem<D>::KST + dc * 8) = k[i];
    }
#pragma unroll
    for (int i = 0; i < VPR; ++i) {
      const int pc = tid + 256 * i, kp = pc / CPR, dc = pc % CPR;
      const int pos = vt_pos(2 * kp);  // even, and 2kp+1 lands at pos+1
      const uint32_t a[4] = {v[i][0].x, v[i][0].y, v[i][0].z, v[i][0].w};
      const uint32_t b[4] = {v[i][1].x, v[i][1].y, v[i][1].z, v[i][1].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = (a[j] & 0xffffu) | (b[j] << 16);
        const uint32_t hi = (a[j] >> 16) | (b[j] & 0xffff0000u);
        *reinterpret_cast<uint32_t*>(Vt + (dc * 8 + 2 * j) * kVST + pos) = lo;
        *reinterpret_cast<uint32_t*>(Vt + (dc * 8 + 2 * j + 1) * kVST + pos) = hi;
      }
    }
  }
};

__device__ inline bf16x8 load_bf16x8(const __bf16* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__device__ inline bf16x8 relu8(bf16x8 x) {
  uint4 u = __builtin_bit_cast(uint4, x);
  auto r = [](uint32_t w) {
    return ((w & 0x8000u) ? 0u : (w & 0xffffu)) | ((w & 0x80000000u) ? 0u : (w & 0xffff0000u));
  };
  u.x = r(u.x); u.y = r(u.y); u.z = r(u.z); u.w = r(u.w);
  return __builtin_bit_cast(bf16x8, u);
}

template <int D, int BLK>
__global__ void __launch_bounds__(256, 2)
k_attn_bf16(Geom g, AttnArgs a, int n_items, float scale_log2) {
  constexpr int QPW = 128 / BLK;  // query blocks per workgroup
  constexpr int NC = D / 16;      // 16-wide d chunks (QK^T contraction steps)
  constexpr int NT = D / 32;      // 32-wide d tiles of the output
  using SM = Smem<D>;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __bf16* smem = reinterpret_cast<__bf16*>(smem_raw);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g32 = lane >> 5, l32 = lane & 31;

  // XCD-aware item order: workgroup w runs on XCD w % 8; give each XCD a
  // contiguous range of items.
  const int per_xcd = (int)(gridDim.x >> 3);
  const int item = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (item >= n_items) return;
  const int qgroups = (g.nb + QPW - 1) / QPW;
  const int bh = item / qgroups, qg = item - bh * qgroups;
  const int qb_base = qg * QPW;
  const int qsub = QPW == 2 ? (wave >> 1) : 0;
  const int my_qb = qb_base + qsub;
  const bool wave_rows = my_qb < g.nb;
  const int row0 = qb_base * BLK + wave * 32;  // first query row of this wave
  const int my_row = row0 + l32;

  const __bf16* Qb = static_cast<const __bf16*>(a.q) + (int64_t)bh * g.n_pad * D;
  const __bf16* Kb = static_cast<const __bf16*>(a.k) + (int64_t)bh * g.n_pad * D;
  const __bf16* Vb = static_cast<const __bf16*>(a.v) + (int64_t)bh * g.n_pad * D;

  // Q fragments (B operand of S^T = K Q^T): row my_row, d = c*16 + g32*8 .. +7
  bf16x8 qf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (wave_rows && my_row < g.N) qf[c] = load_bf16x8(Qb + (int64_t)my_row * D + c * 16 + g32 * 8);
    else qf[c] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
  }

  f32x16 o[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  if (a.has_sparse) {
    const int64_t rbase = (int64_t)bh * g.nb;
    int b0 = 0, e0 = 0, b1 = 0, e1 = 0;
    if (qb_base < g.nb) { b0 = a.row_ptr[rbase + qb_base]; e0 = a.row_ptr[rbase + qb_base + 1]; }
    if (QPW == 2 && qb_base + 1 < g.nb) { b1 = a.row_ptr[rbase + qb_base + 1]; e1 = a.row_ptr[rbase + qb_base + 2]; }
    TileIter it;
    it.init(a.col_idx, b0, e0, b1, e1);
    TileRegs<D> regs;
    int buf = 0;
    if (it.valid) {
      regs.load(Kb, Vb, it.key0(BLK), g.N, tid);
      regs.store(smem, smem + SM::K_ELEMS, tid);
    }
    __syncthreads();
    while (it.valid) {
      const int key0 = it.key0(BLK);
      const int flags = it.flags;
      TileIter nx = it;
      nx.next(BLK, g.N);
      if (nx.valid) regs.load(Kb, Vb, nx.key0(BLK), g.N, tid);

      const __bf16* Ks = smem + buf * SM::BUF_ELEMS;
      const __bf16* Vt = Ks + SM::K_ELEMS;
      if (wave_rows && ((flags >> qsub) & 1)) {
        f32x16 s[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
          for (int i = 0; i < 16; ++i) s[kt][i] = 0.0f;
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            const bf16x8 kf = load_bf16x8(Ks + (kt * 32 + l32) * SM::KST + c * 16 + g32 * 8);
            s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], s[kt], 0, 0, 0);
          }
        }
        // scale, mask padded keys, row max
        float mx = -INFINITY;
        const bool tail = key0 + kTK > g.N;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float x = s[kt][i] * scale_log2;
            if (tail) {
              const int key = key0 + kt * 32 + (i >> 2) * 8 + g32 * 4 + (i & 3);
              if (key >= g.N) x = -INFINITY;
            }
            s[kt][i] = x;
            mx = fmaxf(mx, x);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.0f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        float rs = 0.0f;
        bf16x8 pf[4];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float p = __builtin_amdgcn_exp2f(s[kt][i] - m_use);
            rs += p;
            pf[kt * 2 + (i >> 3)][i & 7] = (__bf16)p;
          }
        rs += __shfl_xor(rs, 32);
        l_run = l_run * alpha + rs;
        m_run = m_new;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[t][i] *= alpha;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 vf = load_bf16x8(Vt + (t * 32 + l32) * kVST + ks * 16 + g32 * 8);
            o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks], o[t], 0, 0, 0);
          }
      }
      if (nx.valid) regs.store(smem + (buf ^ 1) * SM::BUF_ELEMS,
                               smem + (buf ^ 1) * SM::BUF_ELEMS + SM::K_ELEMS, tid);
      __syncthreads();
      buf ^= 1;
      it = nx;
    }
  }

  // ---- epilogue -------------------------------------------------------------
  const float inv_l = l_run > 0.0f ? 1.0f / l_run : 0.0f;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] *= inv_l;

  bool lin = a.has_lin != 0;
  if (lin && a.gate != nullptr && a.gate[bh] < a.drop_tau) lin = false;
  if (lin && wave_rows) {
    const __bf16* hi = static_cast<const __bf16*>(a.sft_hi) + (int64_t)bh * D * D;
    const __bf16* lo = static_cast<const __bf16*>(a.sft_lo) + (int64_t)bh * D * D;
    const float* z = a.z + (int64_t)bh * D;
    bf16x8 rq[NC];
    float den = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      rq[c] = relu8(qf[c]);
#pragma unroll
      for (int j = 0; j < 8; ++j) den += (float)rq[c][j] * z[c * 16 + g32 * 8 + j];
    }
    den += __shfl_xor(den, 32);
    const float inv_den = 1.0f / (den + a.eps);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f32x16 la;
#pragma unroll
      for (int i = 0; i < 16; ++i) la[i] = 0.0f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int64_t off = (int64_t)(t * 32 + l32) * D + c * 16 + g32 * 8;
        la = __builtin_amdgcn_mfma_f32_32x32x16_bf16(load_bf16x8(hi + off), rq[c], la, 0, 0, 0);
        la = __builtin_amdgcn_mfma_f32_32x32x16_bf16(load_bf16x8(lo + off), rq[c], la, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) o[t][i] += la[i] * inv_den;
    }
  }

  // stage [128 rows][D] bf16 through LDS, then 16-byte coalesced stores
  __syncthreads();
  __bf16* ost = smem;
  const bool row_ok = wave_rows && my_row < g.N;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = t * 32 + i4 * 8 + g32 * 4;
      uint32_t w0, w1;
      if (row_ok) {
        const uint32_t b0 = __builtin_bit_cast(uint16_t, (__bf16)o[t][i4 * 4 + 0]);
        const uint32_t b1 = __builtin_bit_cast(uint16_t, (__bf16)o[t][i4 * 4 + 1]);
        const uint32_t b2 = __builtin_bit_cast(uint16_t, (__bf16)o[t][i4 * 4 + 2]);
        const uint32_t b3 = __builtin_bit_cast(uint16_t, (__bf16)o[t][i4 * 4 + 3]);
        w0 = b0 | (b1 << 16);
        w1 = b2 | (b3 << 16);
      } else {
        w0 = 0; w1 = 0;
      }
      *reinterpret_cast<uint2*>(ost + (wave * 32 + l32) * SM::OST + d0) = make_uint2(w0, w1);
    }
  __syncthreads();
  __bf16* Ob = static_cast<__bf16*>(a.out) + (int64_t)bh * g.n_pad * D;
  constexpr int CPR = D / 8;
  for (int ch = tid; ch < 128 * CPR; ch += 256) {
    const int r = ch / CPR, dc = ch % CPR;
    const int row = qb_base * BLK + r;
    if (row < g.n_pad)
      *reinterpret_cast<uint4*>(Ob + (int64_t)row * D + dc * 8) =
          *reinterpret_cast<const uint4*>(ost + r * SM::OST + dc * 8);
  }
}

template <int D, int BLK>
hipError_t launch(const Geom& g, const AttnArgs& a, hipStream_t st) {
  constexpr int QPW = 128 / BLK;
  const int qgroups = (g.nb + QPW - 1) / QPW;
  const int n_items = g.B * g.Hh * qgroups;
  const int grid = (n_items + 7) / 8 * 8;
  const float scale_log2 = a.scale * 1.4426950408889634f;
  // more than 64 KiB of dynamic LDS must be opted into once per kernel
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&k_attn_bf16<D, BLK>),
      hipFuncAttributeMaxDynamicSharedMemorySize, Smem<D>::BYTES);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((k_attn_bf16<D, BLK>), dim3(grid), dim3(256), Smem<D>::BYTES, st, g, a,
                     n_items, scale_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const Geom& g, const AttnArgs& a, hipStream_t st) {
  if (g.D == 128) return g.blk == 64 ? launch<128, 64>(g, a, st) : launch<128, 128>(g, a, st);
  return g.blk == 64 ? launch<64, 64>(g, a, st) : launch<64, 128>(g, a, st);
}

}  // namespace salad
