// api.hip - the extern "C" entry points of libsalad (declared in include/salad.h):
// argument validation, workspace planning and the launch sequence of each call.
#include <algorithm>
#include <cmath>
#include <mutex>

#include "cuboid.h"
#include "internal.h"

// The allocation-free forward's scratch (salad_attn_fwd_noalloc): one static
// device array per GPU; each device that loads the library holds its own copy
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not the device address: the address comes from hipGetSymbolAddress, once per
// device, with that device current (scratch_of_current_device).
static constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace salad {

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int shape_status(const salad_shape* s) {
  if (s == nullptr) return SALAD_EINVAL;
  if (s->batch < 1 || s->heads < 1 || s->T < 1 || s->H < 1 || s->W < 1 || s->block < 1 ||
      s->head_dim < 1)
    return SALAD_EINVAL;
  if (s->dtype != SALAD_F32 && s->dtype != SALAD_BF16) return SALAD_EINVAL;
  if (s->head_dim != 64 && s->head_dim != 128) return SALAD_EUNSUPPORTED;
  if (s->block != 64 && s->block != 128) return SALAD_EUNSUPPORTED;
  if (s->heads > SALAD_MAX_HEADS) return SALAD_EUNSUPPORTED;
  const int64_t N = (int64_t)s->T * s->H * s->W;
  if (N > INT32_MAX / 2) return SALAD_EUNSUPPORTED;
  const int64_t nb = (N + s->block - 1) / s->block;
  if ((int64_t)s->n_pad != nb * s->block) return SALAD_EINVAL;
  if (nb > 46340) return SALAD_EUNSUPPORTED;  // nb*nb must fit int32
  if (s->H > 65534 || s->W > 65534) return SALAD_EUNSUPPORTED;  // r* is stored in 16 bits
  if ((int64_t)s->batch * s->heads * nb + 1 > INT32_MAX) return SALAD_EUNSUPPORTED;
  const bool raster = s->cuboid_t == 0 && s->cuboid_h == 0 && s->cuboid_w == 0;
  if (!raster) {
    if (s->cuboid_t < 1 || s->cuboid_h < 1 || s->cuboid_w < 1) return SALAD_EINVAL;
    if ((int64_t)s->cuboid_t * s->cuboid_h * s->cuboid_w != s->block) return SALAD_EINVAL;
  }
  return SALAD_OK;
}

int spec_status(const salad_shape* s, const salad_mask_spec* specs) {
  if (specs == nullptr) return SALAD_EINVAL;
  const int64_t nb = s->n_pad / s->block;
  for (int h = 0; h < s->heads; ++h) {
    const salad_mask_spec& sp = specs[h];
    if (sp.kind == SALAD_MASK_WINDOW) {
      if (sp.t_window < 0) return SALAD_EINVAL;
    } else if (sp.kind == SALAD_MASK_TOPK || sp.kind == SALAD_MASK_SICS) {
      if (nb > 4096) return SALAD_EUNSUPPORTED;  // the selection holds a row's nb keys in one wave
    } else {
      return SALAD_EINVAL;
    }
    if (!std::isfinite(sp.density)) return SALAD_EINVAL;
  }
  return SALAD_OK;
}

int64_t topk_count(float density, int64_t nb) {
  const double k = std::floor((double)density * (double)nb + 0.5);
  if (!(k >= 1.0)) return 1;
  return k >= (double)nb ? nb : (int64_t)k;
}

// Per-head entry counts of one (b, h) (host).  count[h] receives the window K
// (-1 = keep every candidate) or the top-k / SICS k; per[h] the CSR entries of
// one (b, h): exact for window and top-k heads, the upper bound (m + 1) * nb for
// SICS heads.  SALAD_EINFEASIBLE when a window head asks for more pairs than it
// has candidates.
int head_counts(const salad_shape* s, const salad_mask_spec* specs, int64_t* count, int64_t* per) {
  Geom g;
  make_geom(s, &g);
  Cuboid cu;
  make_cuboid(s, &cu);
  const int64_t nb = g.nb;
  // window heads sharing (t_window, r_max) share one candidate count
  int64_t cand[SALAD_MAX_HEADS];
  for (int h = 0; h < s->heads; ++h) {
    const salad_mask_spec& sp = specs[h];
    if (sp.kind == SALAD_MASK_WINDOW) {
      cand[h] = -1;
      for (int j = 0; j < h; ++j)
        if (specs[j].kind == SALAD_MASK_WINDOW && specs[j].t_window == sp.t_window &&
            specs[j].r_max == sp.r_max) {
          cand[h] = cand[j];
          break;
        }
      if (cand[h] < 0) cand[h] = window_candidates(g, cu, sp.t_window, sp.r_max);
      if (sp.density <= 0.0f) {
        count[h] = -1;
        per[h] = cand[h];
      } else {
        // K = floor(density * nb^2 + 0.5), compared in double before any cast
        const double K = std::floor((double)sp.density * (double)nb * (double)nb + 0.5);
        if (K > (double)cand[h]) return SALAD_EINFEASIBLE;
        count[h] = per[h] = (int64_t)K;
      }
    } else {
      count[h] = topk_count(sp.density, nb);
      per[h] = (sp.kind == SALAD_MASK_TOPK ? count[h] : std::min<int64_t>(count[h] + 1, nb)) * nb;
    }
  }
  return SALAD_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? SALAD_OK : SALAD_EHIP; }

// Device address of `scratch` on the current device, looked up on the first
// call on each device and kept (write-once per device, under a lock).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SALAD_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return SALAD_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SALAD_EHIP;
    g_scratch_ptr[dev] = static_cast<char*>(p);
  }
  *out = g_scratch_ptr[dev];
  return SALAD_OK;
}

}  // namespace

bool make_geom(const salad_shape* s, Geom* g) {
  if (shape_status(s) != SALAD_OK) return false;
  g->B = s->batch;
  g->Hh = s->heads;
  g->D = s->head_dim;
  g->T = s->T;
  g->H = s->H;
  g->W = s->W;
  g->N = s->T * s->H * s->W;
  g->n_pad = s->n_pad;
  g->blk = s->block;
  g->nb = s->n_pad / s->block;
  return true;
}

void make_cuboid(const salad_shape* s, Cuboid* c) {
  *c = Cuboid{};
  if (s->cuboid_t == 0) return;  // frame-major order
  c->ct = s->cuboid_t;
  c->ch = s->cuboid_h;
  c->cw = s->cuboid_w;
  c->nt = (s->T + c->ct - 1) / c->ct;
  c->ny = (s->H + c->ch - 1) / c->ch;
  c->nx = (s->W + c->cw - 1) / c->cw;
  c->Ft = s->T / c->ct;
  c->Fy = s->H / c->ch;
  c->Fx = s->W / c->cw;
  c->rt = s->T - (c->nt - 1) * c->ct;
  c->ry = s->H - (c->ny - 1) * c->ch;
  c->rx = s->W - (c->nx - 1) * c->cw;
  c->F = c->Ft * c->Fy * c->Fx;
  // Smallest partial cuboid: each axis takes its full extent (if any cuboid is
  // full on it) or its remainder (if one is short), at least one remainder.
  // An interval of `block` slots meets at most ceil(block / smallest) + 1
  // pieces; each inner piece is one box and the two cut ones at most three.
  int smallest = 0;
  const int et[2] = {c->Ft > 0 ? c->ct : 0, c->rt < c->ct ? c->rt : 0};
  const int ey[2] = {c->Fy > 0 ? c->ch : 0, c->ry < c->ch ? c->ry : 0};
  const int ex[2] = {c->Fx > 0 ? c->cw : 0, c->rx < c->cw ? c->rx : 0};
  for (int m = 1; m < 8; ++m) {
    const int v = et[m & 1] * ey[(m >> 1) & 1] * ex[(m >> 2) & 1];
    if (v > 0 && (smallest == 0 || v < smallest)) smallest = v;
  }
  c->box_cap = smallest == 0 ? 1 : (s->block + smallest - 1) / smallest + 1 + 4;
}

Workspace plan_workspace(const Geom& g, const Cuboid& cu, int dtype) {
  Workspace L{};
  const size_t BH = (size_t)g.B * g.Hh, D = g.D, nb = g.nb;
  // mask build
  size_t off = 0;
  L.hist_bins = 1 + (size_t)std::max(g.H, g.W) * nb;
  L.off_rt = off;     off = align_up(off + nb * nb * 2);
  L.off_hist = off;   off = align_up(off + L.hist_bins * 4);
  L.off_thr = off;    off = align_up(off + (size_t)g.Hh * 8);
  L.off_rowcnt = off; off = align_up(off + BH * nb * 4);
  L.off_psum_q = off; off = align_up(off + BH * nb * D * 4);
  L.off_psum_k = off; off = align_up(off + BH * nb * D * 4);
  L.off_scores = off; off = align_up(off + (size_t)topk_heads_per_batch(g) * nb * nb * 4);
  L.off_sics = off;   off = align_up(off + BH * nb * 4);
  L.off_sics_pack = off; off = align_up(off + BH * nb * 4);
  const size_t boxes = cu.ct == 0 ? 0 : nb;
  L.off_nbox = off;   off = align_up(off + boxes * 4);
  L.off_boxes = off;  off = align_up(off + boxes * (size_t)cu.box_cap * sizeof(Box));
  L.mask_end = off;
  // linear state: at most 256 workgroups in all (one resident per CU, each
  // with a four-tile ring of 128 KiB LDS), so that the split reduction runs in
  // one round; 64-token chunks
  int splits = (int)std::max<size_t>(1, 256 / BH);
  splits = std::min(splits, (g.N + 63) / 64);
  int chunk = (g.N + splits - 1) / splits;
  chunk = (chunk + 63) / 64 * 64;
  splits = (g.N + chunk - 1) / chunk;
  L.lin_splits = splits;
  L.lin_chunk = chunk;
  off = 0;  // the two phases never overlap in time on one stream
  L.off_spart = off;  off = align_up(off + (size_t)splits * BH * D * D * 4);
  L.off_zpart = off;  off = align_up(off + (size_t)splits * BH * D * 4);
  L.off_z = off;      off = align_up(off + BH * D * 4);
  const size_t esz = dtype == SALAD_BF16 ? 2 : 4;
  L.off_sft = off;    off = align_up(off + BH * D * D * esz);
  L.off_split = off;  off = align_up(off + (9 + kPairModeSlots) * 4);
  L.lin_end = off;
  L.bytes = std::max(L.mask_end, L.lin_end);
  return L;
}

namespace {

Workspace plan_for(const salad_shape* s, const Geom& g) {
  Cuboid cu;
  make_cuboid(s, &cu);
  return plan_workspace(g, cu, s->dtype);
}

}  // namespace

}  // namespace salad

using namespace salad;

extern "C" {

int salad_version(void) { return SALAD_VERSION; }

const char* salad_status_str(int status) {
  switch (status) {
    case SALAD_OK: return "ok";
    case SALAD_EINVAL: return "invalid argument";
    case SALAD_EUNSUPPORTED: return "unsupported shape (head_dim/block not 64 or 128, too many heads or blocks)";
    case SALAD_ENOSPACE: return "workspace or col_idx capacity too small";
    case SALAD_EINFEASIBLE: return "window density exceeds the candidate block pairs";
    case SALAD_EHIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int64_t salad_mask_nnz(const salad_shape* shape, const salad_mask_spec* specs) {
  int st = shape_status(shape);
  if (st != SALAD_OK) return st;
  st = spec_status(shape, specs);
  if (st != SALAD_OK) return st;
  int64_t count[SALAD_MAX_HEADS], per[SALAD_MAX_HEADS];
  st = head_counts(shape, specs, count, per);
  if (st != SALAD_OK) return st;
  int64_t total = 0;
  for (int h = 0; h < shape->heads; ++h) total += per[h] * shape->batch;
  return total;
}

size_t salad_workspace_bytes(const salad_shape* shape) {
  Geom g;
  if (!make_geom(shape, &g)) return 0;
  return plan_for(shape, g).bytes;
}

int salad_build_mask(const salad_shape* shape, const salad_mask_spec* specs, const void* q,
                     const void* k, int32_t* row_ptr, int32_t* col_idx, int64_t col_cap,
                     const float* w_g, float* gate, void* ws, size_t ws_bytes, void* stream) {
  Geom g;
  int st = shape_status(shape);
  if (st != SALAD_OK) return st;
  make_geom(shape, &g);
  st = spec_status(shape, specs);
  if (st != SALAD_OK) return st;
  bool any_topk = false, any_k = false;
  for (int h = 0; h < g.Hh; ++h) {
    any_topk |= specs[h].kind == SALAD_MASK_TOPK;
    any_k |= specs[h].kind != SALAD_MASK_WINDOW;
  }
  if ((w_g == nullptr) != (gate == nullptr)) return SALAD_EINVAL;
  const bool want_gate = gate != nullptr;
  if (!row_ptr || !col_idx || !ws) return SALAD_EINVAL;
  if ((any_topk || want_gate) && (!q || !aligned16(q))) return SALAD_EINVAL;
  if (any_k && (!k || !aligned16(k))) return SALAD_EINVAL;
  if (!aligned16(ws)) return SALAD_EINVAL;
  const Workspace L = plan_for(shape, g);
  if (ws_bytes < L.bytes) return SALAD_ENOSPACE;
  int64_t count[SALAD_MAX_HEADS], per[SALAD_MAX_HEADS];
  st = head_counts(shape, specs, count, per);
  if (st != SALAD_OK) return st;
  int64_t need = 0;
  for (int h = 0; h < g.Hh; ++h) need += per[h] * g.B;
  if (need > INT32_MAX) return SALAD_EUNSUPPORTED;  // row_ptr is int32
  if (col_cap < need) return SALAD_ENOSPACE;
  HeadTable ht{};
  ht.n_heads = g.Hh;
  for (int h = 0; h < g.Hh; ++h) {
    ht.kind[h] = specs[h].kind;
    ht.t_window[h] = specs[h].t_window;
    ht.r_max[h] = specs[h].r_max;
    ht.count[h] = (int)count[h];  // <= nb * nb < 2^31, or -1
  }
  // per[h] is exact for window and top-k heads (a bound for SICS heads)
  bool any_sics = false;
  for (int h = 0; h < g.Hh; ++h) any_sics |= specs[h].kind == SALAD_MASK_SICS;
  ht.direct_rows = !any_sics && g.nb <= kDirectRowsMaxNb;
  int64_t run = 0;
  for (int h = 0; h < g.Hh; ++h) {
    ht.base[h] = (int)run;  // need <= INT32_MAX, checked above
    run += per[h];
  }
  ht.batch_nnz = (int)run;
  Cuboid cu;
  make_cuboid(shape, &cu);
  return hip_status(launch_build_mask(g, cu, shape->dtype, ht, q, k, row_ptr, col_idx, col_cap, w_g,
                                      gate, static_cast<char*>(ws), L,
                                      static_cast<hipStream_t>(stream)));
}

int salad_check_mask(const salad_shape* shape, const int32_t* row_ptr, const int32_t* col_idx,
                     int64_t col_cap, int32_t* result, void* stream) {
  Geom g;
  const int st = shape_status(shape);
  if (st != SALAD_OK) return st;
  if (!row_ptr || !result || col_cap < 0 || (col_cap > 0 && !col_idx)) return SALAD_EINVAL;
  make_geom(shape, &g);
  return hip_status(launch_check_mask(g, row_ptr, col_idx, col_cap, result, static_cast<hipStream_t>(stream)));
}

int salad_token_order(const salad_shape* shape, int32_t* order) {
  Geom g;
  const int st = shape_status(shape);
  if (st != SALAD_OK) return st;
  if (!order) return SALAD_EINVAL;
  make_geom(shape, &g);
  Cuboid cu;
  make_cuboid(shape, &cu);
  for (int p = 0; p < g.n_pad; ++p) order[p] = p < g.N ? slot_token(g, cu, p) : p;
  return SALAD_OK;
}

int salad_permute_tokens(const salad_shape* shape, int inverse, const void* src, void* dst,
                         void* stream) {
  Geom g;
  const int st = shape_status(shape);
  if (st != SALAD_OK) return st;
  if (!src || !dst || !aligned16(src) || !aligned16(dst) || (inverse != 0 && inverse != 1))
    return SALAD_EINVAL;
  make_geom(shape, &g);
  const size_t bytes = (size_t)g.B * g.Hh * g.n_pad * g.D * (shape->dtype == SALAD_BF16 ? 2 : 4);
  const char* s = static_cast<const char*>(src);
  const char* d = static_cast<const char*>(dst);
  if (s < d + bytes && d < s + bytes) return SALAD_EINVAL;  // overlapping buffers
  Cuboid cu;
  make_cuboid(shape, &cu);
  return hip_status(launch_permute_tokens(g, cu, shape->dtype, inverse, src, dst,
                                          static_cast<hipStream_t>(stream)));
}

int salad_gate_from_q(const salad_shape* shape, const void* q, const float* w_g, float* gate,
                      void* ws, size_t ws_bytes, void* stream) {
  Geom g;
  const int st = shape_status(shape);
  if (st != SALAD_OK) return st;
  make_geom(shape, &g);
  if (!q || !w_g || !gate || !ws || !aligned16(q) || !aligned16(ws)) return SALAD_EINVAL;
  const Workspace L = plan_for(shape, g);
  if (ws_bytes < L.bytes) return SALAD_ENOSPACE;
  return hip_status(launch_gate_from_q(g, shape->dtype, q, w_g, gate, static_cast<char*>(ws), L,
                                       static_cast<hipStream_t>(stream)));
}

int salad_linear_state(const salad_shape* shape, const void* k, const void* v, float* S, float* z,
                       void* ws, size_t ws_bytes, void* stream) {
  Geom g;
  const int st = shape_status(shape);
  if (st != SALAD_OK) return st;
  make_geom(shape, &g);
  if (!k || !v || !S || !z || !ws || !aligned16(k) || !aligned16(v) || !aligned16(ws))
    return SALAD_EINVAL;
  const Workspace L = plan_for(shape, g);
  if (ws_bytes < L.bytes) return SALAD_ENOSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  hipError_t e = launch_linear_state(g, shape->dtype, k, v, nullptr, 0.0f, nullptr, w, L, s);
  if (e != hipSuccess) return SALAD_EHIP;
  return hip_status(launch_linear_fold(g, shape->dtype, nullptr, nullptr, 2, 0.0f, S, z, w, L, s));
}

namespace {

int attn_common(const salad_shape* shape, const void* q, const void* k, const void* v,
                const int32_t* row_ptr, const int32_t* col_idx, void* ws, size_t ws_bytes,
                Geom* g, Workspace* L) {
  const int st = shape_status(shape);
  if (st != SALAD_OK) return st;
  make_geom(shape, g);
  if (!q || !k || !v || !row_ptr || !col_idx || !ws) return SALAD_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(ws)) return SALAD_EINVAL;
  *L = plan_for(shape, *g);
  if (ws_bytes < L->bytes) return SALAD_ENOSPACE;
  return SALAD_OK;
}

hipError_t run_attn(const Geom& g, int dtype, const AttnArgs& a, hipStream_t s) {
  return dtype == SALAD_BF16 ? launch_attn_bf16(g, a, s) : launch_attn_f32(g, a, s);
}

// Arguments of the fused forward beyond q, k, v and the mask.
int fwd_args_status(const salad_shape* shape, const float* gate, const void* w_lin, float eps, float scale,
                    float drop_tau, void* out, float* lse) {
  if (!gate || !w_lin || !aligned16(w_lin) || !out || !aligned16(out) || !(eps >= 0.0f) ||
      !std::isfinite(scale) || std::isnan(drop_tau))
    return SALAD_EINVAL;
  if (lse != nullptr && shape->dtype != SALAD_BF16) return SALAD_EUNSUPPORTED;
  return SALAD_OK;
}

// The fused forward's launches (validated arguments): linear-state partials,
// fold, attention with the linear epilogue.  Only the linear-phase part of the
// workspace layout (up to L.lin_end) is touched.
int fwd_run(const salad_shape* shape, const Geom& g, const Workspace& L, const void* q, const void* k,
            const void* v, const int32_t* row_ptr, const int32_t* col_idx, const float* gate,
            const void* w_lin, float eps, float scale, float drop_tau, void* out, float* lse, char* w,
            hipStream_t s) {
  hipError_t e = launch_linear_state(g, shape->dtype, k, v, gate, drop_tau, w_lin, w, L, s);
  if (e == hipSuccess)
    e = launch_linear_fold(g, shape->dtype, gate, w_lin, 0, drop_tau, nullptr, nullptr, w, L, s);
  if (e != hipSuccess) return SALAD_EHIP;
  AttnArgs a{};
  a.q = q; a.k = k; a.v = v; a.out = out;
  a.row_ptr = row_ptr; a.col_idx = col_idx;
  a.sft = w + L.off_sft;
  a.split = reinterpret_cast<int32_t*>(w + L.off_split);
  a.z = reinterpret_cast<const float*>(w + L.off_z);
  a.gate = gate; a.drop_tau = drop_tau; a.eps = eps;
  a.scale = scale > 0.0f ? scale : 1.0f / std::sqrt((float)g.D);
  a.has_sparse = 1; a.has_lin = 1;
  a.lse = lse;
  return hip_status(run_attn(g, shape->dtype, a, s));
}

}  // namespace

int salad_linear_prepare(const salad_shape* shape, const void* k, const void* v,
                         const float* gate, const void* w_lin, float drop_tau, void* ws,
                         size_t ws_bytes, void* stream) {
  Geom g;
  const int st = shape_status(shape);
  if (st != SALAD_OK) return st;
  make_geom(shape, &g);
  if (!k || !v || !gate || !w_lin || !ws || !aligned16(k) || !aligned16(v) || !aligned16(ws) ||
      !aligned16(w_lin) || std::isnan(drop_tau))
    return SALAD_EINVAL;
  const Workspace L = plan_for(shape, g);
  if (ws_bytes < L.bytes) return SALAD_ENOSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  hipError_t e = launch_linear_state(g, shape->dtype, k, v, gate, drop_tau, w_lin, w, L, s);
  if (e == hipSuccess)
    e = launch_linear_fold(g, shape->dtype, gate, w_lin, 0, drop_tau, nullptr, nullptr, w, L, s);
  return hip_status(e);
}

int salad_attn_apply(const salad_shape* shape, const void* q, const void* k, const void* v,
                     const int32_t* row_ptr, const int32_t* col_idx, const float* gate, float eps,
                     float scale, float drop_tau, void* out, float* lse, void* ws, size_t ws_bytes,
                     void* stream) {
  Geom g;
  Workspace L;
  int st = attn_common(shape, q, k, v, row_ptr, col_idx, ws, ws_bytes, &g, &L);
  if (st != SALAD_OK) return st;
  if (!gate || !out || !aligned16(out) || !(eps >= 0.0f) || !std::isfinite(scale) ||
      std::isnan(drop_tau))
    return SALAD_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  AttnArgs a{};
  a.q = q; a.k = k; a.v = v; a.out = out;
  a.row_ptr = row_ptr; a.col_idx = col_idx;
  a.sft = w + L.off_sft;
  a.split = reinterpret_cast<int32_t*>(w + L.off_split);
  a.z = reinterpret_cast<const float*>(w + L.off_z);
  a.gate = gate; a.drop_tau = drop_tau; a.eps = eps;
  a.scale = scale > 0.0f ? scale : 1.0f / std::sqrt((float)g.D);
  a.has_sparse = 1; a.has_lin = 1;
  if (lse != nullptr && shape->dtype != SALAD_BF16) return SALAD_EUNSUPPORTED;
  a.lse = lse;
  return hip_status(run_attn(g, shape->dtype, a, s));
}

int salad_attn_fwd(const salad_shape* shape, const void* q, const void* k, const void* v,
                   const int32_t* row_ptr, const int32_t* col_idx, const float* gate,
                   const void* w_lin, float eps, float scale, float drop_tau, void* out, float* lse,
                   void* ws, size_t ws_bytes, void* stream) {
  Geom g;
  Workspace L;
  int st = attn_common(shape, q, k, v, row_ptr, col_idx, ws, ws_bytes, &g, &L);
  if (st != SALAD_OK) return st;
  st = fwd_args_status(shape, gate, w_lin, eps, scale, drop_tau, out, lse);
  if (st != SALAD_OK) return st;
  return fwd_run(shape, g, L, q, k, v, row_ptr, col_idx, gate, w_lin, eps, scale, drop_tau, out, lse,
                 static_cast<char*>(ws), static_cast<hipStream_t>(stream));
}

int salad_attn_fwd_noalloc(const salad_shape* shape, const void* q, const void* k, const void* v,
                           const int32_t* row_ptr, const int32_t* col_idx, const float* gate,
                           const void* w_lin, float eps, float scale, float drop_tau, void* out,
                           float* lse, void* stream) {
  Geom g;
  int st = shape_status(shape);
  if (st != SALAD_OK) return st;
  make_geom(shape, &g);
  if (!q || !k || !v || !row_ptr || !col_idx) return SALAD_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return SALAD_EINVAL;
  st = fwd_args_status(shape, gate, w_lin, eps, scale, drop_tau, out, lse);
  if (st != SALAD_OK) return st;
  const Workspace L = plan_for(shape, g);
  if (L.lin_end > kScratchBytes) return SALAD_ENOSPACE;  // the forward uses the linear-phase part only
  char* w = nullptr;
  st = scratch_of_current_device(&w);
  if (st != SALAD_OK) return st;
  return fwd_run(shape, g, L, q, k, v, row_ptr, col_idx, gate, w_lin, eps, scale, drop_tau, out, lse, w,
                 static_cast<hipStream_t>(stream));
}

int salad_attn_fwd_branches(const salad_shape* shape, const void* q, const void* k, const void* v,
                            const int32_t* row_ptr, const int32_t* col_idx, float eps, float scale,
                            void* out_sparse, void* out_lin, void* ws, size_t ws_bytes,
                            void* stream) {
  Geom g;
  Workspace L;
  int st = attn_common(shape, q, k, v, row_ptr, col_idx, ws, ws_bytes, &g, &L);
  if (st != SALAD_OK) return st;
  if ((out_sparse && !aligned16(out_sparse)) || (out_lin && !aligned16(out_lin)) ||
      !(eps >= 0.0f) || !std::isfinite(scale))
    return SALAD_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  AttnArgs a{};
  a.q = q; a.k = k; a.v = v;
  a.row_ptr = row_ptr; a.col_idx = col_idx;
  a.sft = w + L.off_sft;
  a.split = reinterpret_cast<int32_t*>(w + L.off_split);
  a.z = reinterpret_cast<const float*>(w + L.off_z);
  a.gate = nullptr; a.drop_tau = 0.0f; a.eps = eps;
  a.scale = scale > 0.0f ? scale : 1.0f / std::sqrt((float)g.D);
  if (out_sparse) {
    a.out = out_sparse; a.has_sparse = 1; a.has_lin = 0;
    if (run_attn(g, shape->dtype, a, s) != hipSuccess) return SALAD_EHIP;
  }
  if (out_lin) {
    hipError_t e = launch_linear_state(g, shape->dtype, k, v, nullptr, 0.0f, nullptr, w, L, s);
    if (e == hipSuccess)
      e = launch_linear_fold(g, shape->dtype, nullptr, nullptr, 1, 0.0f, nullptr, nullptr, w, L, s);
    if (e != hipSuccess) return SALAD_EHIP;
    a.out = out_lin; a.has_sparse = 0; a.has_lin = 1;
    if (run_attn(g, shape->dtype, a, s) != hipSuccess) return SALAD_EHIP;
  }
  return SALAD_OK;
}

size_t salad_bwd_workspace_bytes(const salad_shape* shape) {
  Geom g;
  if (!make_geom(shape, &g)) return 0;
  Cuboid cu;
  make_cuboid(shape, &cu);
  return plan_bwd_workspace(g, cu, shape->dtype).bytes;
}

int salad_attn_bwd(const salad_shape* shape, const void* q, const void* k, const void* v,
                   const int32_t* row_ptr, const int32_t* col_idx, const float* gate,
                   const void* w_lin, float eps, float scale, const void* out, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, float* dw_lin, float* dgate,
                   void* ws, size_t ws_bytes, void* stream) {
  Geom g;
  const int st = shape_status(shape);
  if (st != SALAD_OK) return st;
  if (shape->dtype != SALAD_BF16) return SALAD_EUNSUPPORTED;
  make_geom(shape, &g);
  const void* ptrs[] = {q, k, v, out, dout, dq, dk, dv, ws, w_lin};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return SALAD_EINVAL;
  if (!row_ptr || !col_idx || !gate || !dw_lin || !dgate) return SALAD_EINVAL;
  if (lse && !aligned16(lse)) return SALAD_EINVAL;  // read in 16-byte rows by the dK/dV kernel
  if (!(eps >= 0.0f) || !std::isfinite(scale)) return SALAD_EINVAL;
  Cuboid cu;
  make_cuboid(shape, &cu);
  const BwdWorkspace L = plan_bwd_workspace(g, cu, shape->dtype);
  if (ws_bytes < L.bytes) return SALAD_ENOSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.row_ptr = row_ptr; a.col_idx = col_idx; a.gate = gate;
  a.w_lin = w_lin; a.out = out; a.dout = dout; a.dq = dq; a.dk = dk; a.dv = dv;
  a.dw_lin = dw_lin; a.dgate = dgate; a.lse = lse; a.eps = eps;
  a.scale = scale > 0.0f ? scale : 1.0f / std::sqrt((float)g.D);
  hipError_t e = launch_linear_state(g, shape->dtype, k, v, nullptr, 0.0f, nullptr, w, L.fwd, s);
  if (e == hipSuccess)
    e = launch_linear_fold(g, shape->dtype, nullptr, nullptr, 2, 0.0f,
                           reinterpret_cast<float*>(w + L.off_s32), reinterpret_cast<float*>(w + L.off_z),
                           w, L.fwd, s);
  if (e == hipSuccess) e = launch_linear_bwd(g, a, w, L, s);
  if (e == hipSuccess) e = launch_mask_transpose(g, row_ptr, col_idx, w, L, s);
  if (e == hipSuccess) e = launch_attn_bwd(g, a, w, L, s);
  return hip_status(e);
}

}  // extern "C"
