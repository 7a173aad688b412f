// window_count.hip - host-side count of the candidate block pairs of a static
// spatio-temporal window ("SALAD" explainer, section 5: static sliding-window
// masks; sciencestack Figure 1, ST-SWA), so that the entry points can give the
// exact number of CSR entries and reject an infeasible request before any
// launch.
//
// A pair (qb, kb) is a candidate when some token of qb and some token of kb
// are at most t_window frames apart (r* finite) and, when r_max >= 0, r* <=
// r_max, with r* the least Chebyshev distance max(|dy|, |dx|) over such token
// pairs.  Each block's token set is a short list of axis-aligned boxes (the
// frame-major run of a block, or the cuboid pieces of cuboid order); between
// two boxes the least distance over token pairs at most t_window frames apart
// is max(y gap, x gap) when their frame gap is <= t_window, else infinite.
//
// Cost.  Without a spatial cap and when every block's frames form one
// interval (always so for frame-major runs), the count needs only the blocks'
// frame intervals: O(nb log nb).  Otherwise each query block visits the boxes
// of the frames within t_window of its own: O(nb * boxes per frame * frames
// spanned), a few milliseconds on the grids used here, more on single-frame
// grids with many blocks.
#include <algorithm>
#include <vector>

#include "cuboid.h"
#include "internal.h"

namespace salad {

namespace {

struct HBox {
  int t0, t1, y0, y1, x0, x1;
};

// Boxes of the frame-major run of block j: a partial row, whole rows of one
// frame, whole frames, whole rows, a partial row (at most five).
int run_boxes(const Geom& g, int j, HBox* out) {
  const int plane = g.H * g.W;
  const int p1 = std::min((j + 1) * g.blk, g.N);
  int u = j * g.blk, n = 0;
  while (u < p1) {
    const int t = u / plane, rem = u - t * plane;
    const int y = rem / g.W, x = rem - y * g.W;
    if (x != 0 || p1 - u < g.W) {
      const int w = std::min(g.W - x, p1 - u);
      out[n++] = HBox{t, t, y, y, x, x + w - 1};
      u += w;
    } else if (y != 0 || p1 - u < plane) {
      const int rows = std::min(g.H - y, (p1 - u) / g.W);
      out[n++] = HBox{t, t, y, y + rows - 1, 0, g.W - 1};
      u += rows * g.W;
    } else {
      const int frames = (p1 - u) / plane;
      out[n++] = HBox{t, t + frames - 1, 0, g.H - 1, 0, g.W - 1};
      u += frames * plane;
    }
  }
  return n;
}

int gap(int a0, int a1, int b0, int b1) { return std::max(0, std::max(b0 - a1, a0 - b1)); }

}  // namespace

int64_t window_candidates(const Geom& g, const Cuboid& cu, int t_window, int r_max) {
  const int nb = g.nb;
  // every block's boxes, flattened
  std::vector<int> first(nb + 1, 0);
  std::vector<HBox> boxes;
  boxes.reserve((size_t)nb * 3);
  if (cu.ct == 0) {
    HBox tmp[8];
    for (int j = 0; j < nb; ++j) {
      first[j] = (int)boxes.size();
      const int n = run_boxes(g, j, tmp);
      boxes.insert(boxes.end(), tmp, tmp + n);
    }
  } else {
    std::vector<Box> tmp(cu.box_cap);
    for (int j = 0; j < nb; ++j) {
      first[j] = (int)boxes.size();
      const int n = block_boxes(g, cu, j, tmp.data(), cu.box_cap);
      for (int i = 0; i < n; ++i)
        boxes.push_back(HBox{tmp[i].ty.x, tmp[i].ty.y, tmp[i].ty.z, tmp[i].ty.w, tmp[i].x.x, tmp[i].x.y});
    }
  }
  first[nb] = (int)boxes.size();

  // frames of each block: one interval?
  std::vector<int> f0(nb), f1(nb);
  bool intervals = true;
  for (int j = 0; j < nb; ++j) {
    std::vector<std::pair<int, int>> fr;
    for (int i = first[j]; i < first[j + 1]; ++i) fr.emplace_back(boxes[i].t0, boxes[i].t1);
    std::sort(fr.begin(), fr.end());
    int lo = fr[0].first, hi = fr[0].second;
    for (size_t i = 1; i < fr.size(); ++i) {
      if (fr[i].first > hi + 1) intervals = false;
      hi = std::max(hi, fr[i].second);
    }
    f0[j] = lo;
    f1[j] = hi;
  }
  const int64_t tw = t_window;
  if (r_max < 0 && intervals) {
    // candidates of q: nb - #{k : f0[k] > f1[q] + tw} - #{k : f1[k] < f0[q] - tw}
    // (disjoint sets, since f0[k] <= f1[k])
    std::vector<int> s0(f0), s1(f1);
    std::sort(s0.begin(), s0.end());
    std::sort(s1.begin(), s1.end());
    int64_t total = 0;
    for (int q = 0; q < nb; ++q) {
      const int64_t hi = f1[q] + tw, lo = (int64_t)f0[q] - tw;
      const int64_t above = s0.end() - std::upper_bound(s0.begin(), s0.end(), (int)std::min<int64_t>(hi, INT32_MAX));
      const int64_t below = std::lower_bound(s1.begin(), s1.end(), (int)std::max<int64_t>(lo, INT32_MIN)) - s1.begin();
      total += nb - above - below;
    }
    return total;
  }
  // general case: per frame, the boxes that touch it; each query block marks
  // the key blocks one of whose boxes is close enough to one of its own
  std::vector<std::vector<int>> by_frame(g.T);
  std::vector<int> owner(boxes.size());
  for (int j = 0; j < nb; ++j)
    for (int i = first[j]; i < first[j + 1]; ++i) {
      owner[i] = j;
      for (int t = boxes[i].t0; t <= boxes[i].t1; ++t) by_frame[t].push_back(i);
    }
  std::vector<int> seen(nb, -1);
  int64_t total = 0;
  for (int q = 0; q < nb; ++q) {
    for (int i = first[q]; i < first[q + 1]; ++i) {
      const HBox& a = boxes[i];
      const int t_lo = (int)std::max<int64_t>(0, a.t0 - tw);
      const int t_hi = (int)std::min<int64_t>(g.T - 1, a.t1 + tw);
      for (int t = t_lo; t <= t_hi; ++t)
        for (int bi : by_frame[t]) {
          const int k = owner[bi];
          if (seen[k] == q) continue;
          if (r_max >= 0) {
            const HBox& b = boxes[bi];
            if (std::max(gap(a.y0, a.y1, b.y0, b.y1), gap(a.x0, a.x1, b.x0, b.x1)) > r_max) continue;
          }
          seen[k] = q;
          ++total;
        }
    }
  }
  return total;
}

}  // namespace salad
