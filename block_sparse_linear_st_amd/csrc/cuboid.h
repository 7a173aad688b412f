// cuboid.h - slot -> token map of the cuboid storage order, and the boxes a
// block's token set splits into.  Closed forms shared by the host entry point
// that lists the order, the permutation kernel and the window-mask kernels.
//
// Storage order (for cuboid extents ct, ch, cw with ct*ch*cw = block): every
// full cuboid in lexicographic (a, b, c) order, then every partial cuboid (one
// that meets the far edge of an axis the extent does not divide) in
// lexicographic order; frame-major inside each cuboid.  Reading of the SPADE
// explainer's vDiT-SSR blueprint part (a 3-D grid of video blocks cut into
// flat, tall or mixed shapes).
//
// Tail arithmetic.  Let xr = W - Fx*cw (width of the x-edge band).  In a slab
// a < Ft (all ct frames present) the partial cuboids are the x-edge piece of
// each full row b < Fy (ct*ch*xr tokens) and then every piece of the partial
// row b = Fy, so the slab holds ct*(H*W - Fy*ch*Fx*cw) tail tokens.  In the
// partial slab a = Ft every cuboid is partial and row b holds et*ey(b)*W.
#pragma once

#include "internal.h"

namespace salad {

__host__ __device__ inline int imin(int a, int b) { return a < b ? a : b; }

// Where slot p (< N) lives: cuboid (a, b, c) with extents (et, ey, ex), offset u
// inside it (frame-major).
struct Piece {
  int a, b, c;
  int et, ey, ex;
  int u;
};

__host__ __device__ inline Piece locate_slot(const Geom& g, const Cuboid& cu, int p) {
  Piece r;
  const int blk = g.blk;
  if (p < cu.F * blk) {
    const int f = p / blk;
    r.u = p - f * blk;
    r.a = f / (cu.Fy * cu.Fx);
    const int rem = f - r.a * cu.Fy * cu.Fx;
    r.b = rem / cu.Fx;
    r.c = rem - r.b * cu.Fx;
    r.et = cu.ct;
    r.ey = cu.ch;
    r.ex = cu.cw;
    return r;
  }
  int s = p - cu.F * blk;
  const int xr = g.W - cu.Fx * cu.cw;
  const int slab_tail = cu.ct * (g.H * g.W - cu.Fy * cu.ch * cu.Fx * cu.cw);
  if (s < cu.Ft * slab_tail) {
    r.a = s / slab_tail;
    s -= r.a * slab_tail;
  } else {
    r.a = cu.Ft;
    s -= cu.Ft * slab_tail;
  }
  r.et = r.a < cu.nt - 1 ? cu.ct : cu.rt;
  if (r.a < cu.Ft) {
    const int row_tail = cu.ct * cu.ch * xr;
    if (s < cu.Fy * row_tail) {
      r.b = s / row_tail;
      s -= r.b * row_tail;
    } else {
      r.b = cu.Fy;
      s -= cu.Fy * row_tail;
    }
  } else {
    const int row_all = r.et * cu.ch * g.W;
    r.b = imin(s / row_all, cu.ny - 1);
    s -= r.b * row_all;
  }
  r.ey = r.b < cu.ny - 1 ? cu.ch : cu.ry;
  if (r.a < cu.Ft && r.b < cu.Fy) {
    r.c = cu.Fx;  // the x-edge piece, = nx - 1
    r.ex = xr;
  } else {
    const int piece = r.et * r.ey * cu.cw;
    r.c = imin(s / piece, cu.nx - 1);
    s -= r.c * piece;
    r.ex = r.c < cu.nx - 1 ? cu.cw : cu.rx;
  }
  r.u = s;
  return r;
}

// Frame-major index of the token stored at slot p (< N).
__host__ __device__ inline int slot_token(const Geom& g, const Cuboid& cu, int p) {
  if (cu.ct == 0) return p;
  const Piece r = locate_slot(g, cu, p);
  const int plane = r.ey * r.ex;
  const int dt = r.u / plane;
  const int rem = r.u - dt * plane;
  const int dy = rem / r.ex;
  const int dx = rem - dy * r.ex;
  const int t = r.a * cu.ct + dt, y = r.b * cu.ch + dy, x = r.c * cu.cw + dx;
  return (t * g.H + y) * g.W + x;
}

// Boxes of block j's token set (cuboid order): one per full cuboid; a tail
// block walks its pieces and splits each covered range [u0, u1) of a piece into
// at most five boxes (a partial row, rows of one frame, whole frames, rows, a
// partial row).  Writes at most `cap` boxes; returns how many it wrote.
__host__ __device__ inline int block_boxes(const Geom& g, const Cuboid& cu, int j, Box* out,
                                           int cap) {
  int n = 0;
  const int s1 = imin((j + 1) * g.blk, g.N);
  int p = j * g.blk;
  while (p < s1 && n < cap) {
    const Piece r = locate_slot(g, cu, p);
    const int len = imin(r.et * r.ey * r.ex - r.u, s1 - p);
    const int t0 = r.a * cu.ct, y0 = r.b * cu.ch, x0 = r.c * cu.cw;
    const int plane = r.ey * r.ex;
    int u = r.u;
    const int u1 = r.u + len;
    while (u < u1 && n < cap) {
      const int dt = u / plane;
      const int rem = u - dt * plane;
      const int dy = rem / r.ex;
      const int dx = rem - dy * r.ex;
      Box b;
      if (dx != 0 || u1 - u < r.ex) {  // part of one row
        const int w = imin(r.ex - dx, u1 - u);
        b.ty = make_int4(t0 + dt, t0 + dt, y0 + dy, y0 + dy);
        b.x = make_int4(x0 + dx, x0 + dx + w - 1, 0, 0);
        u += w;
      } else if (dy != 0 || u1 - u < plane) {  // whole rows of one frame
        const int rows = imin(r.ey - dy, (u1 - u) / r.ex);
        b.ty = make_int4(t0 + dt, t0 + dt, y0 + dy, y0 + dy + rows - 1);
        b.x = make_int4(x0, x0 + r.ex - 1, 0, 0);
        u += rows * r.ex;
      } else {  // whole frames
        const int frames = (u1 - u) / plane;
        b.ty = make_int4(t0 + dt, t0 + dt + frames - 1, y0, y0 + r.ey - 1);
        b.x = make_int4(x0, x0 + r.ex - 1, 0, 0);
        u += frames * plane;
      }
      out[n++] = b;
    }
    p += len;
  }
  return n;
}

}  // namespace salad
