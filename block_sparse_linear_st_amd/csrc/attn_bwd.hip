// attn_bwd.hip - backward of the block-sparse softmax branch on gfx950, with
// the linear branch's dq, dk, dv terms folded into the same kernels.
//
// With x = scale * q.k, P = softmax over the kept keys, D_i = <dout_i, o_s,i>
// (from linear_bwd.hip):  dS = P * (dout V^T - D),  dQ = scale dS K,
// dK = scale dS^T Q,  dV = P^T dout.  The row statistic (log2-sum-exp of the
// scaled scores) comes from the forward when it kept it, else it is recomputed
// by the dQ kernel in a first pass.
//
// All kernels stream their 64-row tiles HBM -> LDS with global_load_lds_dwordx4,
// double buffered (the next tile's loads are issued before the current tile's
// MFMAs).
//
// k_attn_bwd_dq2 (the forward kept its statistic): the forward kernel's shape,
// 128 queries per workgroup over the union of two query blocks' kept lists; per
// tile S^T, P^T, dP^T, dS^T and dQ^T += K^T dS^T as below.
//
// k_attn_bwd_dq (statistic recomputed): one query block per workgroup, one wave
// per 32 queries, queries in lanes (the forward's transposed orientation).
// Pass 1 over the kept key tiles: S^T = K Q^T and the running max / sum -> log2-sum-exp per
// query (written for the key-side kernel).  Pass 2: S^T, P^T, dP^T = V dO^T,
// dS^T, and dQ^T += K^T dS^T with K^T read by LDS transpose reads and dS^T
// taken straight from the accumulators.  The epilogue adds the linear term
// (S dU^T + z dden^T) * [q > 0] on MFMAs (S as hi + lo bf16).
//
// k_attn_bwd_dkdv_pair: one key block per workgroup, keys in lanes, each 32-key
// group served by a pair of waves.  It walks the transposed mask (the query
// blocks that keep this key block, ascending) in 64-query tiles: wave A forms
// S = Q K^T, P and dV^T += dO^T P; wave B forms dP = dO V^T, takes P from A
// through LDS, and accumulates dK^T += Q^T dS, with dO^T and Q^T by transpose
// reads.  The linear terms dS_lin^T phi(K)^T (dV) and (dS_lin V^T + dz) * [k > 0]
// (dK) seed the accumulators.
//
// Every tile row past the last valid token is a copy of token N-1 (finite), so
// no NaN from padding can reach an MFMA; padded keys and queries are masked by
// index and their output rows are written as 0.
#include <cmath>
#include <type_traits>

#include "bwd_common.h"

namespace salad {

using namespace bwd;

namespace {

constexpr int kT = 64;  // keys (dQ kernels) or queries (dK/dV kernel) per LDS tile

__device__ inline bf16x8 ld8(const __bf16* p) { return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p)); }

template <int D, int BLK>
struct BwdSmem {
  static constexpr int TB = kT * TileLay<D>::ROW_B;
  static constexpr int SST = D + 8;                 // staging row stride (bf16)
  static constexpr int STAGE = BLK * SST * 2;
  static constexpr int BYTES = 4 * TB > STAGE ? 4 * TB : STAGE;  // two buffers of two tiles
};

// Stage a C-layout [channel][row-in-lane] result of NT tiles per wave as
// [row][channel] bf16 in LDS and store BLK rows to dst (rows >= nvalid as 0).
template <int D, int BLK>
__device__ inline void store_rows(unsigned char* smem, const f32x16 (&acc)[D / 32], __bf16* dst, int nvalid,
                                  int wave, int lane, int tid, int nrows = BLK) {
  using SM = BwdSmem<D, BLK>;
  __bf16* st = reinterpret_cast<__bf16*>(smem);
  const int gg = lane >> 5, m = lane & 31;
  const int lr = wave * 32 + m;
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) st[lr * SM::SST + 32 * t + crow(i, gg)] = (__bf16)(lr < nvalid ? acc[t][i] : 0.0f);
  __syncthreads();
  for (int i = tid; i < nrows * D / 8; i += BLK * 2) {
    const int r = i / (D / 8), p = i % (D / 8);
    *reinterpret_cast<uint4*>(dst + (int64_t)r * D + p * 8) = *reinterpret_cast<const uint4*>(st + r * SM::SST + p * 8);
  }
  __syncthreads();
}

template <int D, int BLK>
__global__ void __launch_bounds__(BLK * 2)
k_attn_bwd_dq(Geom g, BwdArgs a, const float* __restrict__ Dq, const float* __restrict__ dden,
              const __bf16* __restrict__ dU, const __bf16* __restrict__ s_hi, const __bf16* __restrict__ s_lo,
              const float* __restrict__ z, float* __restrict__ lse_out, float c_log2) {
  constexpr int NT = D / 32, NC = D / 16;
  using SM = BwdSmem<D, BLK>;
  __shared__ __align__(16) unsigned char smem[SM::BYTES];
  const int qb = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, gg = lane >> 5, m = lane & 31;
  const int n = qb * BLK + wave * 32 + m;
  const bool valid = n < g.N;
  const int nrow = min(n, g.N - 1);
  const int64_t hb = (int64_t)bh * g.n_pad;
  const __bf16* Q = static_cast<const __bf16*>(a.q) + hb * D;
  const __bf16* K = static_cast<const __bf16*>(a.k) + hb * D;
  const __bf16* V = static_cast<const __bf16*>(a.v) + hb * D;
  const __bf16* dO = static_cast<const __bf16*>(a.dout) + hb * D;

  bf16x8 qf[NC], dof[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    qf[c] = ld8(Q + (int64_t)nrow * D + 16 * c + 8 * gg);
    dof[c] = ld8(dO + (int64_t)nrow * D + 16 * c + 8 * gg);
  }
  const float Dn = Dq[hb + n];
  const int64_t r = (int64_t)bh * g.nb + qb;
  const int e0 = a.row_ptr[r], e1 = a.row_ptr[r + 1];
  constexpr int SUB = BLK / kT;
  constexpr int NW = BLK / 32;

  // The kept key tiles are visited twice: pass 1 (tiles 0 .. T-1, K only)
  // accumulates the log2-sum-exp, pass 2 (tiles T .. 2T-1, K and V) dQ.  Each
  // tile's DMA is issued one tile ahead into the other buffer.
  const int T = (e1 - e0) * SUB;
  const uint32_t lds0 = lds_addr(smem);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  TileDma<D, NW> dma;
  dma.init(wave_u, lane);
  auto issue = [&](int i, int buf) __attribute__((always_inline)) {
    const int ii = i < T ? i : i - T;
    const int key0 = a.col_idx[e0 + ii / SUB] * BLK + (ii % SUB) * kT;
    const uint32_t base = lds0 + buf * 2 * SM::TB;
    dma.issue(base, K, key0, g.N - 1);
    if (i >= T) dma.issue(base + SM::TB, V, key0, g.N - 1);
  };
  float mrun = -INFINITY, lrun = 0.0f, lse = INFINITY;
  f32x16 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) zero(acc[t]);
  if (T > 0) issue(0, 0);
  wait_vmem();
  __syncthreads();
  for (int i = 0; i < 2 * T; ++i) {
    const int cur = i & 1;
    if (i + 1 < 2 * T) issue(i + 1, cur ^ 1);
    const unsigned char* Kt = smem + cur * 2 * SM::TB;
    const unsigned char* Vt = Kt + SM::TB;
    const int ii = i < T ? i : i - T;
    const int key0 = a.col_idx[e0 + ii / SUB] * BLK + (ii % SUB) * kT;
    if (i < T) {
      f32x16 s[2];
      zero(s[0]);
      zero(s[1]);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        s[0] = mfma(frag_direct<D>(Kt, 0, c, lane), qf[c], s[0]);
        s[1] = mfma(frag_direct<D>(Kt, 32, c, lane), qf[c], s[1]);
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = key0 + 32 * kt + crow(j, gg);
          const float x = key < g.N ? s[kt][j] * c_log2 : -INFINITY;
          s[kt][j] = x;
          mx = fmaxf(mx, x);
        }
      mx = pair_max(mx);
      const float mnew = fmaxf(mrun, mx);
      if (mnew > -INFINITY) {
        lrun *= __builtin_amdgcn_exp2f(mrun - mnew);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int j = 0; j < 16; ++j) lrun += __builtin_amdgcn_exp2f(s[kt][j] - mnew);
        mrun = mnew;
      }
    } else {
      if (i == T) {
        const float lt = pair_sum(lrun);
        lse = (valid && lt > 0.0f) ? mrun + log2f(lt) : INFINITY;
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        // every LDS fragment of a phase is read before its MFMAs, so each
        // MFMA waits for its own operand only
        bf16x8 ka[NC], va[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          ka[c] = frag_direct<D>(Kt, 32 * kt, c, lane);
          va[c] = frag_direct<D>(Vt, 32 * kt, c, lane);
        }
        f32x16 s, dp;
        zero(s);
        zero(dp);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          s = mfma(ka[c], qf[c], s);
          dp = mfma(va[c], dof[c], dp);
        }
        SG_DSREAD(2 * NC);
        SG_MFMA(2 * NC);
        bf16x8 kt_f[2][NT];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) kt_f[h2][tt] = frag_tr<D>(Kt, 2 * kt + h2, tt, lane);
        // key0 + 32 kt + crow(j, gg) < N, tested against a per-lane limit
        const int klim = g.N - key0 - 32 * kt - 4 * gg;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float p = 8 * (j >> 2) + (j & 3) < klim ? __builtin_amdgcn_exp2f(s[j] * c_log2 - lse) : 0.0f;
          s[j] = p * (dp[j] - Dn);
        }
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const bf16x8 b = c_to_b(s, h2);
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) acc[tt] = mfma(kt_f[h2][tt], b, acc[tt]);
        }
        SG_DSREAD(4 * NT);
        SG_MFMA(2 * NT);
      }
    }
    wait_vmem();
    __syncthreads();
  }
  if (gg == 0) lse_out[hb + n] = lse;

  // linear term: (S dU^T + z dden^T) * [q > 0], S rows c as hi + lo bf16
  bf16x8 duf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) duf[c] = ld8(dU + (hb + n) * D + 16 * c + 8 * gg);
  const float ddn = dden[hb + n];
  const __bf16* sh = s_hi + (int64_t)bh * D * D;
  const __bf16* sl = s_lo + (int64_t)bh * D * D;
  float zr[NT][16];
  rows_f32<D>(z + (int64_t)bh * D, gg, zr);
  const uint64_t qpos = positive_rows<D>(Q + (int64_t)nrow * D, gg);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    f32x16 lt2;
    zero(lt2);
    const int64_t ro = (int64_t)(32 * t + m) * D + 8 * gg;
    bf16x8 ah[NC], al[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      ah[c] = ld8(sh + ro + 16 * c);
      al[c] = ld8(sl + ro + 16 * c);
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      lt2 = mfma(ah[c], duf[c], lt2);
      lt2 = mfma(al[c], duf[c], lt2);
    }
    SG_VMREAD(2 * NC);
    SG_MFMA(2 * NC);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float lin = ((qpos >> (16 * t + i)) & 1) ? lt2[i] + zr[t][i] * ddn : 0.0f;
      acc[t][i] = a.scale * acc[t][i] + lin;
    }
  }
  __syncthreads();
  store_rows<D, BLK>(smem, acc, static_cast<__bf16*>(a.dq) + (hb + (int64_t)qb * BLK) * D, g.N - qb * BLK, wave,
                     lane, tid);
}

// dQ with the forward's log2-sum-exp, in the forward kernel's shape: a
// workgroup of 4 waves owns 128 query rows (two 64-token query blocks, or one
// 128-token block) and walks the ascending union of their kept lists in
// 64-key tiles (K and V streamed HBM -> LDS, double buffered); a wave works on
// a tile only when its own query block keeps it.  The per-lane LDS read
// offsets are computed once and the loop is unrolled over the two buffers.
// Two workgroups share a CU.
template <int D, int BLK>
__global__ void __launch_bounds__(256, 2)
k_attn_bwd_dq2(Geom g, BwdArgs a, int n_items, const int32_t* __restrict__ cuts, const float* __restrict__ Dq,
               const float* __restrict__ dden,
               const __bf16* __restrict__ dU, const __bf16* __restrict__ s_hi, const __bf16* __restrict__ s_lo,
               const float* __restrict__ z, float c_log2) {
  using TL = TileLay<D>;
  constexpr int QPW = 128 / BLK;
  constexpr int NC = D / 16, NT = D / 32;
  constexpr int TPB = BLK / kT;
  constexpr int TB = kT * TL::ROW_B;      // one K or V tile
  constexpr int BUF = 2 * TB;             // K then V
  using SM = BwdSmem<D, 128>;
  constexpr int SMEM = 2 * BUF > SM::STAGE ? 2 * BUF : SM::STAGE;
  __shared__ __align__(1024) unsigned char smem[SMEM];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, gg = lane >> 5, m = lane & 31;
  // workgroup w runs on XCD w % 8, which takes its own contiguous run of items
  const int xcd = (int)(blockIdx.x & 7);
  const int item = cuts[xcd] + (int)(blockIdx.x >> 3);
  if (item >= cuts[xcd + 1] || item >= n_items) return;
  const int qgroups = (g.nb + QPW - 1) / QPW;
  const int bh = item / qgroups, qg = item - bh * qgroups;
  const int qb_base = qg * QPW;
  const int qsub = QPW == 2 ? (wave >> 1) : 0;
  const bool wave_rows = qb_base + qsub < g.nb;
  const int n = qb_base * BLK + wave * 32 + m;  // this lane's query (rows past n_pad only when !wave_rows)
  const bool valid = wave_rows && n < g.N;
  const int nrow = min(n, g.N - 1);
  const int64_t hb = (int64_t)bh * g.n_pad;
  const __bf16* Q = static_cast<const __bf16*>(a.q) + hb * D;
  const __bf16* K = static_cast<const __bf16*>(a.k) + hb * D;
  const __bf16* V = static_cast<const __bf16*>(a.v) + hb * D;
  const __bf16* dO = static_cast<const __bf16*>(a.dout) + hb * D;

  bf16x8 qf[NC], dof[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    qf[c] = ld8(Q + (int64_t)nrow * D + 16 * c + 8 * gg);
    dof[c] = ld8(dO + (int64_t)nrow * D + 16 * c + 8 * gg);
  }
  const float Dn = wave_rows ? Dq[hb + n] : 0.0f;
  const float lse = valid ? a.lse[hb + n] : INFINITY;
  f32x16 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) zero(acc[t]);

  // kept lists of the workgroup's query blocks
  const int64_t rbase = (int64_t)bh * g.nb + qb_base;
  int i0 = 0, e0 = 0, i1 = 0, e1 = 0;
  if (qb_base < g.nb) { i0 = a.row_ptr[rbase]; e0 = a.row_ptr[rbase + 1]; }
  if (QPW == 2 && qb_base + 1 < g.nb) { i1 = e0; e1 = a.row_ptr[rbase + 2]; }
  // this head's layout (as the forward kernel's): 0 walks the union of the two
  // lists, 1 gives each wave pair its own block's list
  const bool own_lists = QPW == 2 && cuts[9 + (bh < kPairModeSlots ? bh : bh % g.Hh)] != 0;
  const int i0s = i0, e0s = e0, i1s = i1, e1s = e1;
  int c0 = i0 < e0 ? a.col_idx[i0] : INT32_MAX;
  int c1 = i1 < e1 ? a.col_idx[i1] : INT32_MAX;
  int kb = 0, sub = 0, flags = 0;
  bool more = false;
  auto advance = [&](int& nkb, int& nsub, int& nflags, bool& nmore) __attribute__((always_inline)) {
    if (more && sub + 1 < TPB && kb * BLK + (sub + 1) * kT < g.N) {
      nkb = kb; nsub = sub + 1; nflags = flags; nmore = true;
      return;
    }
    nkb = min(c0, c1);
    nmore = nkb != INT32_MAX;
    nflags = (c0 == nkb ? 1 : 0) | (c1 == nkb ? 2 : 0);
    nsub = 0;
    if (c0 == nkb) { ++i0; c0 = i0 < e0 ? a.col_idx[i0] : INT32_MAX; }
    if (c1 == nkb) { ++i1; c1 = i1 < e1 ? a.col_idx[i1] : INT32_MAX; }
  };
  advance(kb, sub, flags, more);
  const uint32_t lds0 = lds_addr(smem);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  TileDma<D, 4> dma;
  dma.init(wave_u, lane);
  auto issue = [&](int key0, int buf) __attribute__((always_inline)) {
    dma.issue(lds0 + buf * BUF, K, key0, g.N - 1);
    dma.issue(lds0 + buf * BUF + TB, V, key0, g.N - 1);
  };
  if (more && !own_lists) issue(kb * BLK + sub * kT, 0);
  wait_vmem();
  __syncthreads();

  // per-lane read offsets inside a tile.  The swizzle only XORs chunk bits, so
  // one base per read kind covers every chunk: direct reads of row m (and of
  // row 32 + m, which has the same swizzle) at chunk 2c + gg are od ^ (c << 5);
  // transposed K reads for output tile tt are otr ^ (tt << 6), and the second
  // 8-row half adds 8 rows with chunk bit 1 flipped.
  uint32_t od = (uint32_t)TL::off(m, gg), otr;
  {
    const int sl = lane & 15, dh = (lane >> 4) & 1;
    otr = (uint32_t)(TL::off(4 * gg + (sl >> 2), 2 * dh + ((sl & 3) >> 1)) + (sl & 1) * 8);
  }
  asm volatile("" : "+v"(od), "+v"(otr));
  static_assert(TL::xor_rebuild_holds(), "swizzle rebuild assumed below");

  // the products of one K/V tile of KH 32-key halves at Kt, Vt
  auto compute_at = [&](const unsigned char* Kt, const unsigned char* Vt, auto kh_c, int key0)
                        __attribute__((always_inline)) {
    constexpr int KH = decltype(kh_c)::value;
    auto rd = [&](const unsigned char* base, int c, int kt) __attribute__((always_inline)) {
      return __builtin_bit_cast(bf16x8,
                                *reinterpret_cast<const uint4*>(base + (od ^ (c << 5)) + kt * 32 * TL::ROW_B));
    };
    auto ktr = [&](int tt, int ks) __attribute__((always_inline)) {
      uint2 tr[2];
      const uint32_t o0 = otr ^ (tt << 6);
#pragma unroll
      for (int h = 0; h < 2; ++h)
        tr[h] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                              (__attribute__((address_space(3))) s16x4*)(
                                                  Kt + (h ? (o0 ^ 32) : o0) + (16 * ks + 8 * h) * TL::ROW_B)));
      return __builtin_bit_cast(bf16x8, make_uint4(tr[0].x, tr[0].y, tr[1].x, tr[1].y));
    };
#pragma unroll
    for (int kt = 0; kt < KH; ++kt) {
      // S^T and dP^T of 32 keys: two chains, fragments read one contraction step ahead
      f32x16 s, dp;
      zero(s);
      zero(dp);
      bf16x8 ka = rd(Kt, 0, kt), va = rd(Vt, 0, kt);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        bf16x8 kn = ka, vn = va;
        if (c + 1 < NC) { kn = rd(Kt, c + 1, kt); vn = rd(Vt, c + 1, kt); }
        s = mfma(ka, qf[c], s);
        dp = mfma(va, dof[c], dp);
        ka = kn; va = vn;
      }
      bf16x8 kf = ktr(0, 2 * kt);
      // key = key0 + 32 kt + crow(j, gg) < N, with the lane's part moved to the
      // right-hand side so that each test compares a constant
      const int klim = g.N - key0 - 32 * kt - 4 * gg;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float p = 8 * (j >> 2) + (j & 3) < klim ? __builtin_amdgcn_exp2f(s[j] * c_log2 - lse) : 0.0f;
        s[j] = p * (dp[j] - Dn);
      }
      // dQ^T += K^T dS^T over the 32 keys (two 16-key steps)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const bf16x8 b = c_to_b(s, h2);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          bf16x8 kn = kf;
          if (tt + 1 < NT) kn = ktr(tt + 1, 2 * kt + h2);
          else if (h2 == 0) kn = ktr(0, 2 * kt + 1);
          acc[tt] = mfma(kf, b, acc[tt]);
          kf = kn;
        }
      }
    }
  };
  auto compute = [&](auto cur_c, int key0) __attribute__((always_inline)) {
    constexpr int CUR = decltype(cur_c)::value;
    compute_at(smem + CUR * BUF, smem + CUR * BUF + TB, std::integral_constant<int, 2>{}, key0);
  };
  auto step = [&](auto cur_c) __attribute__((always_inline)) {
    constexpr int CUR = decltype(cur_c)::value;
    int nkb, nsub, nflags;
    bool nmore;
    advance(nkb, nsub, nflags, nmore);
    if (nmore) issue(nkb * BLK + nsub * kT, CUR ^ 1);
    if (wave_rows && ((flags >> qsub) & 1)) compute(cur_c, kb * BLK + sub * kT);
    wait_vmem();
    __syncthreads();
    kb = nkb; sub = nsub; flags = nflags; more = nmore;
  };
  if (own_lists) {
    // each wave pair walks its own block's list in 32-key tiles through its
    // own half of the LDS (two buffers of K then V), the pairs in step
    constexpr int TB32 = 32 * TL::ROW_B, BUF32 = 2 * TB32;
    const int wp = wave_u & 1, qs = wave_u >> 1;
    const uint32_t pbase = lds0 + qs * 2 * BUF32;
    const unsigned char* psmem = smem + qs * 2 * BUF32;
    TileDma<D, 2, 32> pdma;
    pdma.init(wp, lane);
    constexpr int TP = BLK / 32;  // 32-key tiles per key block
    const int ib = qs == 0 ? i0s : i1s;
    const int len = qs == 0 ? e0s - i0s : e1s - i1s;
    const int nsteps = max(e0s - i0s, e1s - i1s) * TP;
    auto tile_at = [&](int s_, int& kb_) __attribute__((always_inline)) -> bool {
      const int e = s_ / TP;
      if (e >= len) return false;
      kb_ = a.col_idx[ib + e];
      return kb_ * BLK + (s_ % TP) * 32 < g.N;
    };
    auto pissue = [&](int key0, int buf) __attribute__((always_inline)) {
      pdma.issue(pbase + buf * BUF32, K, key0, g.N - 1);
      pdma.issue(pbase + buf * BUF32 + TB32, V, key0, g.N - 1);
    };
    int s = 0, kb_c = 0;
    bool v_c = nsteps > 0 && tile_at(0, kb_c);
    if (v_c) pissue(kb_c * BLK, 0);
    wait_vmem();
    __syncthreads();
    auto ostep = [&](auto cur_c) __attribute__((always_inline)) {
      constexpr int CUR = decltype(cur_c)::value;
      int kb_n = 0;
      const bool v_n = s + 1 < nsteps && tile_at(s + 1, kb_n);
      if (v_n) pissue(kb_n * BLK + ((s + 1) % TP) * 32, CUR ^ 1);
      if (wave_rows && v_c)
        compute_at(psmem + CUR * BUF32, psmem + CUR * BUF32 + TB32, std::integral_constant<int, 1>{},
                   kb_c * BLK + (s % TP) * 32);
      wait_vmem();      // the next tile has landed in LDS ...
      __syncthreads();  // ... for both waves of the pair, and nobody still reads the current one
      kb_c = kb_n; v_c = v_n; ++s;
    };
    while (s < nsteps) {
      ostep(std::integral_constant<int, 0>{});
      if (s >= nsteps) break;
      ostep(std::integral_constant<int, 1>{});
    }
  } else {
    while (more) {
      step(std::integral_constant<int, 0>{});
      if (!more) break;
      step(std::integral_constant<int, 1>{});
    }
  }

  // linear term: (S dU^T + z dden^T) * [q > 0], S rows c as hi + lo bf16
  if (wave_rows) {
    bf16x8 duf[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) duf[c] = ld8(dU + (hb + n) * D + 16 * c + 8 * gg);
    const float ddn = dden[hb + n];
    const __bf16* sh = s_hi + (int64_t)bh * D * D;
    const __bf16* sl = s_lo + (int64_t)bh * D * D;
    const float* zh = z + (int64_t)bh * D;
    const uint64_t qpos = positive_rows<D>(Q + (int64_t)nrow * D, gg);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f32x16 lt2;
      zero(lt2);
      const int64_t ro = (int64_t)(32 * t + m) * D + 8 * gg;
      bf16x8 ah[NC], al[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        ah[c] = ld8(sh + ro + 16 * c);
        al[c] = ld8(sl + ro + 16 * c);
      }
      float4 zw[4];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) zw[q4] = *reinterpret_cast<const float4*>(zh + 32 * t + 8 * q4 + 4 * gg);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        lt2 = mfma(ah[c], duf[c], lt2);
        lt2 = mfma(al[c], duf[c], lt2);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float4 w4 = zw[i >> 2];
        const float zi = (i & 3) == 0 ? w4.x : (i & 3) == 1 ? w4.y : (i & 3) == 2 ? w4.z : w4.w;
        const float lin = ((qpos >> (16 * t + i)) & 1) ? lt2[i] + zi * ddn : 0.0f;
        acc[t][i] = a.scale * acc[t][i] + lin;
      }
    }
  }
  const int row0 = qb_base * BLK;
  store_rows<D, 128>(smem, acc, static_cast<__bf16*>(a.dq) + (hb + row0) * D, g.N - row0, wave, lane, tid,
                     min(128, g.n_pad - row0));
}

// dK and dV with the work of each 32-key group split over a pair of waves, so
// that two waves share each SIMD: wave A of pair p forms S = Q K^T and P for
// keys 32p .. 32p+31 and accumulates dV^T += dO^T P; wave B forms dP = dO V^T
// and accumulates dK^T += Q^T dS with dS = P (dP - D), P reaching it through
// LDS in bf16 (the operand form A already built for its own product).  Each
// wave runs 16 MFMAs per 32-query half, the fused kernel's 32 split in two, and
// holds only its own 32 keys' K (A) or V (B) fragments and one accumulator set.
// One key block per workgroup walks its CSC list in 64-query tiles: Q, dO and
// the tile's lse and D rows stream HBM -> LDS double buffered; two barriers per
// tile (tile landed, P written).  The linear branch's terms seed the
// accumulators; the softmax scale is folded into dS.
template <int D, int BLK>
__global__ void __launch_bounds__(BLK * 4, BLK == 64 ? 2 : 1)
k_attn_bwd_dkdv_pair(Geom g, BwdArgs a, int n_items, const int32_t* __restrict__ cuts,
                     const int32_t* __restrict__ colptr,
                     const int32_t* __restrict__ rowidx, const float* __restrict__ Dq, const float* __restrict__ lse,
                     const __bf16* __restrict__ ds_hi, const __bf16* __restrict__ ds_lo,
                     const __bf16* __restrict__ dst_hi, const __bf16* __restrict__ dst_lo,
                     const float* __restrict__ dz, float c_log2) {
  using TL = TileLay<D>;
  constexpr int NP = BLK / 32;            // wave pairs
  constexpr int NW = 2 * NP, NTH = NW * 64;
  constexpr int NC = D / 16, NT = D / 32;
  constexpr int TB = kT * TL::ROW_B;      // one Q or dO tile
  constexpr int ST = 2 * kT * 4;          // the tile's lse, then D
  constexpr int PX = NP * 2 * 2048;       // P of every pair and 32-query half, bf16 operand form
  constexpr int OFF_ST = 4 * TB, OFF_P = OFF_ST + 2 * ST;
  constexpr int SST = D + 8;              // output staging stride (bf16)
  constexpr int STAGE = 2 * BLK * SST * 2;
  constexpr int SMEM = OFF_P + PX > STAGE ? OFF_P + PX : STAGE;
  __shared__ __align__(1024) unsigned char smem[SMEM];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, gg = lane >> 5, m = lane & 31;
  // workgroup w runs on XCD w % 8, which takes its own contiguous run of items
  const int xcd = (int)(blockIdx.x & 7);
  const int item = cuts[xcd] + (int)(blockIdx.x >> 3);
  if (item >= cuts[xcd + 1] || item >= n_items) return;
  const int bh = item / g.nb, kb = item - bh * g.nb;
  const int pair = wave >> 1;
  const bool role_b = (wave & 1) != 0;  // uniform per wave
  const int j = kb * BLK + pair * 32 + m;  // this lane's key
  const int jrow = min(j, g.N - 1);
  const int64_t hb = (int64_t)bh * g.n_pad;
  const __bf16* Q = static_cast<const __bf16*>(a.q) + hb * D;
  const __bf16* K = static_cast<const __bf16*>(a.k) + hb * D;
  const __bf16* V = static_cast<const __bf16*>(a.v) + hb * D;
  const __bf16* dO = static_cast<const __bf16*>(a.dout) + hb * D;

  // A: K fragments of its keys; B: V fragments
  bf16x8 kv[NC];
  {
    const __bf16* src = (role_b ? V : K) + (int64_t)jrow * D + 8 * gg;
#pragma unroll
    for (int c = 0; c < NC; ++c) kv[c] = ld8(src + 16 * c);
  }

  const int64_t col = (int64_t)bh * g.nb + kb;
  const int p0 = colptr[col], p1 = colptr[col + 1];
  constexpr int SUB = BLK / kT;
  const int T = (p1 - p0) * SUB;
  const uint32_t lds0 = lds_addr(smem);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  TileDma<D, NW> dma;
  dma.init(wave_u, lane);
  auto q0_of = [&](int i) __attribute__((always_inline)) { return rowidx[p0 + i / SUB] * BLK + (i % SUB) * kT; };
  auto issue = [&](int i, int buf) __attribute__((always_inline)) {
    const int q0 = q0_of(i);
    dma.issue(lds0 + buf * 2 * TB, Q, q0, g.N - 1);
    dma.issue(lds0 + buf * 2 * TB + TB, dO, q0, g.N - 1);
    // lanes 0-15 of wave 0 bring the 64 lse values, lanes 16-31 the 64 D values
    if (wave_u == 0 && lane < 32)
      lds_dma16(lane < 16 ? lse + hb + q0 + 4 * lane : Dq + hb + q0 + 4 * (lane - 16), lds0 + OFF_ST + buf * ST);
  };
  if (T > 0) issue(0, 0);

  // linear terms first: A: dV^T = dS_lin^T phi(K)^T; B: dK^T = (dS_lin V^T + dz) [k > 0]
  f32x16 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) zero(acc[t]);
  {
    const int64_t mb = (int64_t)bh * D * D;
    const __bf16* mh = (role_b ? ds_hi : dst_hi) + mb;
    const __bf16* ml = (role_b ? ds_lo : dst_lo) + mb;
    bf16x8 bop[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) bop[c] = role_b ? kv[c] : relu8(kv[c]);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int64_t ro = (int64_t)(32 * t + m) * D + 8 * gg;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        acc[t] = mfma(ld8(mh + ro + 16 * c), bop[c], acc[t]);
        acc[t] = mfma(ld8(ml + ro + 16 * c), bop[c], acc[t]);
      }
    }
    if (role_b) {
      const uint64_t kpos = positive_rows<D>(K + (int64_t)jrow * D, gg);
      const float* dzh = dz + (int64_t)bh * D;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        float4 zw[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) zw[q4] = *reinterpret_cast<const float4*>(dzh + 32 * t + 8 * q4 + 4 * gg);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float4 w4 = zw[i >> 2];
          const float zi = (i & 3) == 0 ? w4.x : (i & 3) == 1 ? w4.y : (i & 3) == 2 ? w4.z : w4.w;
          acc[t][i] = ((kpos >> (16 * t + i)) & 1) ? acc[t][i] + zi : 0.0f;
        }
      }
    }
  }
  wait_vmem();
  __syncthreads();

  const float neg_inv_c = -1.0f / c_log2;
  const float sc = a.scale;
  unsigned char* pslot = smem + OFF_P + pair * 2 * 2048;
  for (int i = 0; i < T; ++i) {
    const int cur = i & 1;
    if (i + 1 < T) issue(i + 1, cur ^ 1);
    const unsigned char* Qt = smem + cur * 2 * TB;
    const unsigned char* Ot = Qt + TB;
    const float* stat = reinterpret_cast<const float*>(smem + OFF_ST + cur * ST);
    bf16x8 pb[2][2];
    f32x16 dp[2];
    if (!role_b) {
      // A: S (from -lse / c), P = exp2(c S), P to LDS in operand form
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        f32x16 s;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 l4 = *reinterpret_cast<const float4*>(stat + 32 * qs + 8 * q4 + 4 * gg);
          s[4 * q4 + 0] = l4.x * neg_inv_c; s[4 * q4 + 1] = l4.y * neg_inv_c;
          s[4 * q4 + 2] = l4.z * neg_inv_c; s[4 * q4 + 3] = l4.w * neg_inv_c;
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) s = mfma(frag_direct<D>(Qt, 32 * qs, c, lane), kv[c], s);
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = __builtin_amdgcn_exp2f(s[e] * c_log2);  // 0 for padded queries
        pb[qs][0] = c_to_b(s, 0);
        pb[qs][1] = c_to_b(s, 1);
        *reinterpret_cast<uint4*>(pslot + qs * 2048 + lane * 16) = __builtin_bit_cast(uint4, pb[qs][0]);
        *reinterpret_cast<uint4*>(pslot + qs * 2048 + 1024 + lane * 16) = __builtin_bit_cast(uint4, pb[qs][1]);
      }
    } else {
      // B: dP - D
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 d4 = *reinterpret_cast<const float4*>(stat + kT + 32 * qs + 8 * q4 + 4 * gg);
          dp[qs][4 * q4 + 0] = -d4.x; dp[qs][4 * q4 + 1] = -d4.y;
          dp[qs][4 * q4 + 2] = -d4.z; dp[qs][4 * q4 + 3] = -d4.w;
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) dp[qs] = mfma(frag_direct<D>(Ot, 32 * qs, c, lane), kv[c], dp[qs]);
      }
    }
    __syncthreads();  // P of this tile is in LDS
    if (!role_b) {
#pragma unroll
      for (int qs = 0; qs < 2; ++qs)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) acc[tt] = mfma(frag_tr<D>(Ot, 2 * qs + h2, tt, lane), pb[qs][h2], acc[tt]);
    } else {
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        f32x16 ds;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const bf16x8 pp = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(pslot + qs * 2048 + h2 * 1024 + lane * 16));
#pragma unroll
          for (int e = 0; e < 8; ++e) ds[8 * h2 + e] = (float)pp[e] * sc * dp[qs][8 * h2 + e];
        }
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const bf16x8 bd = c_to_b(ds, h2);
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) acc[tt] = mfma(frag_tr<D>(Qt, 2 * qs + h2, tt, lane), bd, acc[tt]);
        }
      }
    }
    wait_vmem();
    __syncthreads();  // next tile landed; this tile's buffers and P slots are free
  }

  // stage dK rows [0, BLK) and dV rows [BLK, 2 BLK) as bf16, then coalesced stores
  __bf16* st = reinterpret_cast<__bf16*>(smem);
  const int nvalid = g.N - kb * BLK;
  const int lr = (role_b ? 0 : BLK) + pair * 32 + m;
  const bool ok = pair * 32 + m < nvalid;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) st[lr * SST + 32 * t + crow(e, gg)] = (__bf16)(ok ? acc[t][e] : 0.0f);
  __syncthreads();
  __bf16* dkd = static_cast<__bf16*>(a.dk) + (hb + (int64_t)kb * BLK) * D;
  __bf16* dvd = static_cast<__bf16*>(a.dv) + (hb + (int64_t)kb * BLK) * D;
  for (int e = tid; e < 2 * BLK * D / 8; e += NTH) {
    const int r = e / (D / 8), c8 = e % (D / 8);
    __bf16* dst = r < BLK ? dkd + (int64_t)r * D : dvd + (int64_t)(r - BLK) * D;
    *reinterpret_cast<uint4*>(dst + c8 * 8) = *reinterpret_cast<const uint4*>(st + r * SST + c8 * 8);
  }
}

template <int D, int BLK>
hipError_t launch_bwd_t(const Geom& g, const BwdArgs& a, char* ws, const BwdWorkspace& L, hipStream_t st) {
  auto B16 = [&](size_t off) { return reinterpret_cast<const __bf16*>(ws + off); };
  auto F32 = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  const float c_log2 = a.scale * 1.4426950408889634f;
  const dim3 grid(g.nb, g.B * g.Hh);
  // XCD runs of both kernels' items, from one launch: query-block groups over
  // the CSR rows (the one-pass dQ kernel), key blocks over the CSC columns
  constexpr int QPW = 128 / BLK;
  const int32_t* colptr = reinterpret_cast<const int32_t*>(ws + L.off_colptr);
  int32_t* qcuts = reinterpret_cast<int32_t*>(ws + L.off_split_q);
  int32_t* kcuts = reinterpret_cast<int32_t*>(ws + L.off_split_k);
  ItemSplit jobs[2] = {{colptr, kcuts, g.B * g.Hh, g.nb, 1, BLK / kT, 2 * 64 / kT},
                       {a.row_ptr, qcuts, g.B * g.Hh, g.nb, QPW, BLK / kT, 3 * 64 / kT}};
  if (QPW == 2) {  // the dQ kernel's per-head list layout, as in the forward
    jobs[1].col = a.col_idx;
    jobs[1].mode_heads = g.Hh;
  }
  hipError_t e = launch_item_splits(jobs, a.lse != nullptr ? 2 : 1, st);
  if (e != hipSuccess) return e;
  if (a.lse != nullptr) {
    const int n_items = g.B * g.Hh * ((g.nb + QPW - 1) / QPW);
    hipLaunchKernelGGL((k_attn_bwd_dq2<D, BLK>), dim3(8 * xcd_items_cap(n_items)), dim3(256), 0, st, g, a,
                       n_items, qcuts, F32(L.off_dq), F32(L.off_dden), B16(L.off_du), B16(L.off_s_hi),
                       B16(L.off_s_lo), F32(L.off_z), c_log2);
  } else
    hipLaunchKernelGGL((k_attn_bwd_dq<D, BLK>), grid, dim3(BLK * 2), 0, st, g, a, F32(L.off_dq),
                       F32(L.off_dden), B16(L.off_du), B16(L.off_s_hi), B16(L.off_s_lo), F32(L.off_z),
                       F32(L.off_lse), c_log2);
  const float* lse = a.lse != nullptr ? a.lse : F32(L.off_lse);
  // key-block items: the query blocks that keep a key block (its CSC column) are its work
  const int k_items = g.B * g.Hh * g.nb;
  hipLaunchKernelGGL((k_attn_bwd_dkdv_pair<D, BLK>), dim3(8 * xcd_items_cap(k_items)), dim3(BLK * 4), 0, st, g,
                     a, k_items, kcuts, colptr,
                     reinterpret_cast<const int32_t*>(ws + L.off_rowidx), F32(L.off_dq), lse,
                     B16(L.off_ds_hi), B16(L.off_ds_lo), B16(L.off_dst_hi), B16(L.off_dst_lo), F32(L.off_dz),
                     c_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd(const Geom& g, const BwdArgs& a, char* ws, const BwdWorkspace& L, hipStream_t st) {
  if (g.D == 128 && g.blk == 64) return launch_bwd_t<128, 64>(g, a, ws, L, st);
  if (g.D == 128 && g.blk == 128) return launch_bwd_t<128, 128>(g, a, ws, L, st);
  if (g.D == 64 && g.blk == 64) return launch_bwd_t<64, 64>(g, a, ws, L, st);
  if (g.D == 64 && g.blk == 128) return launch_bwd_t<64, 128>(g, a, ws, L, st);
  return hipErrorInvalidValue;
}

}  // namespace salad
