// Window geometry of TEmporal Swin Attention, shared by the forward and
// backward window kernels (page "LinGen：基于Mamba机制的线性复杂度高清长视频生成框架",
// section 关键算法创新 > TESA: fixed small 3D windows, plain and shifted
// partitions alternating between layers).
//
// Windows are enumerated on the grid offset by the shift, wrapping around
// each axis, so every window has wt*wh*ww slots.  A slot whose coordinate
// wrapped along an axis gets that axis's bit in its wrap class: with masking
// on (Swin's cut border windows) only slots of equal class attend to each
// other; with masking off the enumeration is the cyclic partition.
#pragma once

#include <hip/hip_runtime.h>

#include "lingen_mate.h"

namespace lingen {

struct WinGeom {
  int T, H, W;
  int wt, wh, ww;
  int st, sh, sw;   // grid offset per axis, 0 <= shift < window (0 on unshifted layers)
  int nwt, nwh, nww;  // windows per axis (T/wt, ...)
  int masked;         // 1: wrapped tokens form windows of their own (Swin); 0: cyclic windows
};

inline WinGeom make_wingeom(const lingen_mate_shape* s, const int shift[3], int masked) {
  WinGeom g;
  g.T = s->T; g.H = s->H; g.W = s->W;
  g.wt = s->win_t; g.wh = s->win_h; g.ww = s->win_w;
  g.st = shift[0]; g.sh = shift[1]; g.sw = shift[2];
  g.nwt = s->T / s->win_t; g.nwh = s->H / s->win_h; g.nww = s->W / s->win_w;
  g.masked = masked;
  return g;
}

// Canonical token of slot (a, b, c) of window (wi, wj, wk), and its wrap
// class (bit 2: t wrapped, bit 1: h, bit 0: w).
__device__ __forceinline__ int window_token(const WinGeom& g, int wi, int wj, int wk, int a, int b, int c, int& cls) {
  int t = wi * g.wt + a + g.st, hh = wj * g.wh + b + g.sh, w = wk * g.ww + c + g.sw;
  int cl = 0;
  if (t >= g.T) { t -= g.T; cl |= 4; }
  if (hh >= g.H) { hh -= g.H; cl |= 2; }
  if (w >= g.W) { w -= g.W; cl |= 1; }
  cls = cl;
  return (t * g.H + hh) * g.W + w;
}

// A window holds wrapped slots iff it is the last one along a shifted axis.
__device__ __forceinline__ bool window_wrapped(const WinGeom& g, int wi, int wj, int wk) {
  return (g.st > 0 && wi == g.nwt - 1) || (g.sh > 0 && wj == g.nwh - 1) || (g.sw > 0 && wk == g.nww - 1);
}

}  // namespace lingen
