// Scan position -> canonical token for the four Rotary Major Scan orders
// (page "LinGen：基于Mamba机制的线性复杂度高清长视频生成框架", section 关键算法创新 >
// Rotary Major Scan): 0 W fastest then H then T, 1 H then W then T, 2 T then
// W then H, 3 T then H then W.  Canonical order is (t, h, w) row-major.  Used
// by the kernels around the scan; the scan kernels carry the same map.
#pragma once

#include <hip/hip_runtime.h>

namespace lingen {

struct ScanOrder {
  int mode, T, H, W;
  __device__ __forceinline__ int canon(int s) const {
    int t, h, w;
    switch (mode) {
      case 0: return s;
      case 1: { h = s % H; const int r = s / H; w = r % W; t = r / W; break; }
      case 2: { t = s % T; const int r = s / T; w = r % W; h = r / W; break; }
      default: { t = s % T; const int r = s / T; h = r % H; w = r / H; break; }
    }
    return (t * H + h) * W + w;
  }
};

}  // namespace lingen
