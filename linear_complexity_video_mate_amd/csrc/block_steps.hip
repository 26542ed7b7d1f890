// The elementwise steps either side of the MA branch's scan, in the Mamba2
// block's conventions (LinGen builds its MA branch from a bidirectional Mamba2
// block; the block layout follows "Transformers are SSMs", Dao & Gu 2024,
// section 7 on the Mamba-2 architecture): before the scan the x, B, C channels
// pass a short depthwise causal convolution and SiLU, and dt is
// softplus(dt_raw + dt_bias); after it, y is gated by SiLU(z) and normalised
// by its root mean square per channel group, times a weight.  Each kernel is
// one streaming pass over HBM.  The convolution runs along the scan order of
// the Rotary Major Scan and reads its taps through the scan map, so no
// permuted copy of the tensor is ever formed; both scan directions come out
// of the same pass.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "lingen_device.h"
#include "lingen_internal.h"

namespace lingen {

namespace {

// Scan position -> canonical token for the four Rotary Major Scan orders
// (t-major 0, h-fastest 1, t-fastest w-major 2, t-fastest h-major 3; the same
// four maps the scan kernels use).
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

__device__ __forceinline__ float silu(float v) { return v / (1.f + __expf(-v)); }

// 16 bytes of channels: 8 bf16 or 4 fp32, widened to fp32 in registers.
template <typename TS> struct Unit16;
template <> struct Unit16<__bf16> {
  static constexpr int n = 8;
  __device__ static void load(const __bf16* p, float (&v)[8]) {
    const bf16x8 u = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = static_cast<float>(u[e]);
  }
  __device__ static void store(__bf16* p, const float (&v)[8]) {
    bf16x8 u;
#pragma unroll
    for (int e = 0; e < 8; ++e) u[e] = static_cast<__bf16>(v[e]);
    *reinterpret_cast<bf16x8*>(p) = u;
  }
};
template <> struct Unit16<float> {
  static constexpr int n = 4;
  __device__ static void load(const float* p, float (&v)[4]) {
    const float4 u = *reinterpret_cast<const float4*>(p);
    v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
  }
  __device__ static void store(float* p, const float (&v)[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

struct PrepOut {
  void* x[2];   // [L][d] per direction (forward, backward)
  void* b[2];   // [L][gn]
  void* c[2];   // [L][gn]
};

// One thread per (run of S consecutive scan positions, 16-byte unit of
// channels); consecutive threads take consecutive units of the same rows, so
// every row is read and written in whole coalesced lines.  For scan position
// s and channel c, with K taps,
//   forward:  silu(bf[c] + sum_k wf[c][k] in[canon(s - K + 1 + k)][c])
//   backward: silu(bb[c] + sum_k wb[c][k] in[canon(s + K - 1 - k)][c])
// (the backward direction is the same convolution along the reversed order),
// taps outside [0, L) read as zero.  Each thread loads the S + 2(K-1) rows its
// outputs touch once, and its 2*K*V weights once.
template <typename TS, int K, int S>
__global__ __launch_bounds__(256) void scan_conv_silu_kernel(const TS* __restrict__ in, const float* __restrict__ wf,
                                                             const float* __restrict__ bf,
                                                             const float* __restrict__ wb,
                                                             const float* __restrict__ bb, ScanOrder so, int L,
                                                             int ch, int d, int gn, PrepOut out) {
  using U = Unit16<TS>;
  constexpr int V = U::n;
  const int units = ch / V;
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t runs = (int64_t(L) + S - 1) / S;
  if (i >= runs * units) return;
  const int s0 = int(i / units) * S, c0 = int(i % units) * V;

  float w_f[V][K], w_b[V][K];
  {
    const float4* pf = reinterpret_cast<const float4*>(wf + int64_t(c0) * K);
    const float4* pb = reinterpret_cast<const float4*>(wb + int64_t(c0) * K);
#pragma unroll
    for (int q = 0; q < V * K / 4; ++q) {
      const float4 a = pf[q], b = pb[q];
      const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        w_f[(4 * q + r) / K][(4 * q + r) % K] = av[r];
        w_b[(4 * q + r) / K][(4 * q + r) % K] = bv[r];
      }
    }
  }
  float acc_f[S][V], acc_b[S][V];
#pragma unroll
  for (int e = 0; e < V; ++e) {
    const float b0 = bf[c0 + e], b1 = bb[c0 + e];
#pragma unroll
    for (int j = 0; j < S; ++j) { acc_f[j][e] = b0; acc_b[j][e] = b1; }
  }
  // Row at scan position s0 + r feeds forward output j with tap
  // k = r - j + K - 1 and backward output j with tap k = j - r + K - 1.
#pragma unroll
  for (int r = -(K - 1); r < S + K - 1; ++r) {
    const int p = s0 + r;
    if (p < 0 || p >= L) continue;
    float v[V];
    U::load(in + int64_t(so.canon(p)) * ch + c0, v);
#pragma unroll
    for (int j = 0; j < S; ++j) {
      const int kf = r - j + K - 1, kb = j - r + K - 1;
      if (kf >= 0 && kf < K) {
#pragma unroll
        for (int e = 0; e < V; ++e) acc_f[j][e] = fmaf(w_f[e][kf], v[e], acc_f[j][e]);
      }
      if (kb >= 0 && kb < K) {
#pragma unroll
        for (int e = 0; e < V; ++e) acc_b[j][e] = fmaf(w_b[e][kb], v[e], acc_b[j][e]);
      }
    }
  }
  // Channel unit -> destination tensor (x: first d channels, then B, then C).
  int sec, col, width;
  if (c0 < d) { sec = 0; col = c0; width = d; }
  else if (c0 < d + gn) { sec = 1; col = c0 - d; width = gn; }
  else { sec = 2; col = c0 - d - gn; width = gn; }
  TS* df = static_cast<TS*>(sec == 0 ? out.x[0] : sec == 1 ? out.b[0] : out.c[0]);
  TS* db = static_cast<TS*>(sec == 0 ? out.x[1] : sec == 1 ? out.b[1] : out.c[1]);
#pragma unroll
  for (int j = 0; j < S; ++j) {
    const int p = s0 + j;
    if (p >= L) break;
    const int64_t tok = so.canon(p);
#pragma unroll
    for (int e = 0; e < V; ++e) { acc_f[j][e] = silu(acc_f[j][e]); acc_b[j][e] = silu(acc_b[j][e]); }
    U::store(df + tok * width + col, acc_f[j]);
    U::store(db + tok * width + col, acc_b[j]);
  }
}

// dt = softplus(dt_raw + dt_bias[head]) in the overflow-safe form
// max(a, 0) + log1p(exp(-|a|)).
__global__ __launch_bounds__(256) void softplus_bias_kernel(const float* __restrict__ raw,
                                                            const float* __restrict__ bias, int64_t n, int heads,
                                                            float* __restrict__ out) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  const float a = raw[i] + bias[i % heads];
  out[i] = fmaxf(a, 0.f) + log1pf(expf(-fabsf(a)));
}

constexpr int kNormThreads = 256;
constexpr int kNormUnits = 4;   // 16-byte units per thread: dim <= 256 * 4 * V

// One workgroup per row: g = y * silu(z); each group of `group` channels is
// divided by sqrt(mean(g^2) + eps) and multiplied by the weight.  Sums of
// squares go through LDS per 16-byte unit; each wave then reduces whole
// groups (lanes stride over the group's units, then a butterfly).
template <typename TS>
__global__ __launch_bounds__(kNormThreads) void gated_rmsnorm_kernel(const TS* __restrict__ y,
                                                                     const TS* __restrict__ z,
                                                                     const float* __restrict__ wt, float eps,
                                                                     int dim, int group, TS* __restrict__ out) {
  using U = Unit16<TS>;
  constexpr int V = U::n;
  __shared__ float part[kNormThreads * kNormUnits];
  __shared__ float inv[kNormThreads * kNormUnits];
  const int64_t row = blockIdx.x;
  const int units = dim / V, upg = group / V, ngroups = units / upg;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float g[kNormUnits][V];
#pragma unroll
  for (int m = 0; m < kNormUnits; ++m) {
    const int u = threadIdx.x + m * kNormThreads;
    if (u < units) {
      float yv[V], zv[V];
      U::load(y + row * dim + u * V, yv);
      U::load(z + row * dim + u * V, zv);
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        g[m][e] = yv[e] * silu(zv[e]);
        ss = fmaf(g[m][e], g[m][e], ss);
      }
      part[u] = ss;
    }
  }
  __syncthreads();
  for (int gi = wave; gi < ngroups; gi += kNormThreads / 64) {
    float ss = 0.f;
    for (int u = gi * upg + lane; u < (gi + 1) * upg; u += 64) ss += part[u];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
    if (lane == 0) inv[gi] = rsqrtf(ss / float(group) + eps);
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < kNormUnits; ++m) {
    const int u = threadIdx.x + m * kNormThreads;
    if (u < units) {
      const float r = inv[u / upg];
      const float4* wp = reinterpret_cast<const float4*>(wt + u * V);
      float o[V];
#pragma unroll
      for (int q = 0; q < V / 4; ++q) {
        const float4 w4 = wp[q];
        o[4 * q + 0] = g[m][4 * q + 0] * r * w4.x;
        o[4 * q + 1] = g[m][4 * q + 1] * r * w4.y;
        o[4 * q + 2] = g[m][4 * q + 2] * r * w4.z;
        o[4 * q + 3] = g[m][4 * q + 3] * r * w4.w;
      }
      U::store(out + row * dim + u * V, o);
    }
  }
}

constexpr int kConvRun = 4;   // scan positions per thread

template <typename TS, int K>
int launch_conv(const TS* in, const float* wf, const float* bf, const float* wb, const float* bb, ScanOrder so,
                int L, int ch, int d, int gn, PrepOut o, hipStream_t st) {
  const int64_t threads = (int64_t(L) + kConvRun - 1) / kConvRun * (ch / Unit16<TS>::n);
  scan_conv_silu_kernel<TS, K, kConvRun><<<unsigned((threads + 255) / 256), 256, 0, st>>>(in, wf, bf, wb, bb, so, L,
                                                                                          ch, d, gn, o);
  return hipGetLastError() == hipSuccess ? LINGEN_OK : LINGEN_ERR_HIP;
}

template <typename TS>
int launch_prep(const lingen_mate_shape* s, const void* xbc, const float* dt_raw, const float* wf, const float* bf,
                const float* wb, const float* bb, const float* dt_bias, int K, int mode, void* const outs[6],
                float* dt, hipStream_t st) {
  const int L = int(tokens(s));
  const int d = s->ssd_heads * s->headdim, gn = s->ngroups * s->d_state, ch = d + 2 * gn;
  const int64_t eb = sizeof(TS);
  const ScanOrder so{mode, s->T, s->H, s->W};
  for (int b = 0; b < s->batch; ++b) {
    const TS* in = reinterpret_cast<const TS*>(static_cast<const char*>(xbc) + int64_t(b) * L * ch * eb);
    PrepOut o;
    for (int dir = 0; dir < 2; ++dir) {
      o.x[dir] = static_cast<char*>(outs[3 * dir]) + int64_t(b) * L * d * eb;
      o.b[dir] = static_cast<char*>(outs[3 * dir + 1]) + int64_t(b) * L * gn * eb;
      o.c[dir] = static_cast<char*>(outs[3 * dir + 2]) + int64_t(b) * L * gn * eb;
    }
    int rc;
    switch (K) {
      case 1: rc = launch_conv<TS, 1>(in, wf, bf, wb, bb, so, L, ch, d, gn, o, st); break;
      case 2: rc = launch_conv<TS, 2>(in, wf, bf, wb, bb, so, L, ch, d, gn, o, st); break;
      case 3: rc = launch_conv<TS, 3>(in, wf, bf, wb, bb, so, L, ch, d, gn, o, st); break;
      default: rc = launch_conv<TS, 4>(in, wf, bf, wb, bb, so, L, ch, d, gn, o, st); break;
    }
    if (rc) return rc;
  }
  const int64_t n = int64_t(s->batch) * L * s->ssd_heads;
  softplus_bias_kernel<<<unsigned((n + 255) / 256), 256, 0, st>>>(dt_raw, dt_bias, n, s->ssd_heads, dt);
  return hipGetLastError() == hipSuccess ? LINGEN_OK : LINGEN_ERR_HIP;
}

}  // namespace
}  // namespace lingen

using namespace lingen;

extern "C" int lingen_ma_prep(const void* xbc, const float* dt_raw, const float* conv_w_f, const float* conv_b_f,
                              const float* conv_w_b, const float* conv_b_b, const float* dt_bias, int32_t conv_k,
                              int32_t mode, const lingen_mate_shape* shape, void* x_f, void* B_f, void* C_f,
                              void* x_b, void* B_b, void* C_b, float* dt, hipStream_t stream) {
  if (int rc = validate_shape(shape)) return rc;
  const int v = shape->dtype == LINGEN_BF16 ? 8 : 4;
  if (mode < 0 || mode > 3 || conv_k < 1 || conv_k > 4) return LINGEN_ERR_SHAPE;
  if ((shape->ssd_heads * shape->headdim) % v || (shape->ngroups * shape->d_state) % v) return LINGEN_ERR_SHAPE;
  const void* ptrs[] = {xbc, dt_raw, conv_w_f, conv_b_f, conv_w_b, conv_b_b, dt_bias, x_f, B_f, C_f, x_b, B_b, C_b, dt};
  for (const void* p : ptrs)
    if (int rc = check_ptr(p)) return rc;
  void* const outs[6] = {x_f, B_f, C_f, x_b, B_b, C_b};
  if (shape->dtype == LINGEN_BF16)
    return launch_prep<__bf16>(shape, xbc, dt_raw, conv_w_f, conv_b_f, conv_w_b, conv_b_b, dt_bias, conv_k, mode,
                               outs, dt, stream);
  return launch_prep<float>(shape, xbc, dt_raw, conv_w_f, conv_b_f, conv_w_b, conv_b_b, dt_bias, conv_k, mode, outs,
                            dt, stream);
}

extern "C" int lingen_gated_rmsnorm(const void* y, const void* z, const float* weight, float eps, int64_t rows,
                                    int32_t dim, int32_t group, int32_t dtype, void* out, hipStream_t stream) {
  if (dtype != LINGEN_F32 && dtype != LINGEN_BF16) return LINGEN_ERR_DTYPE;
  const int v = dtype == LINGEN_BF16 ? 8 : 4;
  if (rows < 0 || rows > int64_t(0x7fffffff) || dim < 1 || group < 1 || dim % group || group % v ||
      dim > kNormThreads * kNormUnits * v || !(eps >= 0.f))
    return LINGEN_ERR_SHAPE;
  if (rows == 0) return LINGEN_OK;
  const void* ptrs[] = {y, z, weight, out};
  for (const void* p : ptrs)
    if (int rc = check_ptr(p)) return rc;
  if (dtype == LINGEN_BF16)
    gated_rmsnorm_kernel<__bf16><<<unsigned(rows), kNormThreads, 0, stream>>>(
        static_cast<const __bf16*>(y), static_cast<const __bf16*>(z), weight, eps, dim, group,
        static_cast<__bf16*>(out));
  else
    gated_rmsnorm_kernel<float><<<unsigned(rows), kNormThreads, 0, stream>>>(
        static_cast<const float*>(y), static_cast<const float*>(z), weight, eps, dim, group,
        static_cast<float*>(out));
  return hipGetLastError() == hipSuccess ? LINGEN_OK : LINGEN_ERR_HIP;
}
