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
#include "lingen_scan_map.h"

namespace lingen {

namespace {

// 16 bytes of channels: 8 bf16 or 4 fp32, widened to fp32 in registers.
template <typename TS> struct Unit16;
template <> struct Unit16<__bf16> {
  static constexpr int n = 8;
  using raw = bf16x8;
  __device__ static raw load_raw(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
  __device__ static raw zero_raw() { return raw{}; }
  __device__ static void widen(const raw& u, float (&v)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = static_cast<float>(u[e]);
  }
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
  using raw = float4;
  __device__ static raw load_raw(const float* p) { return *reinterpret_cast<const float4*>(p); }
  __device__ static raw zero_raw() { return make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ static void widen(const raw& u, float (&v)[4]) { v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w; }
  __device__ static void load(const float* p, float (&v)[4]) {
    const float4 u = *reinterpret_cast<const float4*>(p);
    v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
  }
  __device__ static void store(float* p, const float (&v)[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

// s_waitcnt immediate waiting for at most n outstanding vector-memory
// operations (vmcnt split over bits 3:0 and 15:14; expcnt and lgkmcnt left
// at their maxima, i.e. not waited for).
constexpr int vmcnt_imm(int n) { return 0x0f70 | (n & 15) | ((n >> 4) << 14); }

struct PrepOut {
  void* x[2];   // [L][d] per direction (forward, backward)
  void* b[2];   // [L][gn]
  void* c[2];   // [L][gn]
};

constexpr int kConvMaxTaps = 4;
constexpr int kConvSegMax = 128;  // scan positions per wave, at most

// Four 16-byte LDS reads at addr, addr + 1 KiB, + 2 KiB, + 3 KiB, waited for
// inside the same statement.  Written as one asm statement so that the
// compiler, which cannot tell the ring buffers apart from the LDS targets of
// loads still in flight, does not add a wait for every outstanding global
// load before them; the waits the data needs are issued explicitly.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void lds_read4x16(unsigned addr, i32x4& a, i32x4& b, i32x4& c, i32x4& d) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:1024\n\t"
      "ds_read_b128 %2, %4 offset:2048\n\t"
      "ds_read_b128 %3, %4 offset:3072\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a), "=&v"(b), "=&v"(c), "=&v"(d)
      : "v"(addr)
      : "memory");
}

// One wave per (segment of consecutive scan positions, tile of 64 16-byte
// channel units): lane l owns unit 64*tile + l, so every row access of the
// wave is one contiguous KiB.  For scan position s and channel c, K taps,
//   forward:  silu(bf[c] + sum_k wf[c][k] in[canon(s - K + 1 + k)][c])
//   backward: silu(bb[c] + sum_k wb[c][k] in[canon(s + K - 1 - k)][c])
// (the backward direction is the same convolution along the reversed order),
// taps outside [0, L) read as zero.  The wave walks its segment 4 positions
// per step, keeping rows s-K+1 .. s+K+2 in registers; the 4 new rows of each
// step arrive by direct global-to-LDS loads issued D steps earlier into a
// ring of D+1 LDS buffers (read back with lds_read4x16), which keeps 4*D KiB
// per wave in flight without holding registers for it.  Each row is fetched once per segment, plus
// 2(K-1) halo rows; weights once per segment.  The scan map of every
// position the segment touches is computed once, one position per lane, and
// broadcast from its lane when needed.
//
// Wait accounting (vector-memory operations of one wave complete in issue
// order): step s issues the 4 loads of step s+D, then its own loads' data is
// complete once at most 4*D + 8*min(s, D) newer operations are pending -- the
// later loads and the 8 stores of every step in between.  Every step issues
// exactly 4 loads and 8 stores (L and the segment length are multiples of 4,
// and the loads of the D steps past the end re-read a valid row), so the
// count is exact; the first D steps use the smaller bound 4*D.
template <typename TS, int K, int D>
__global__ __launch_bounds__(256) void scan_conv_silu_kernel(const TS* __restrict__ in, const float* __restrict__ wf,
                                                             const float* __restrict__ bf,
                                                             const float* __restrict__ wb,
                                                             const float* __restrict__ bb, ScanOrder so, int L,
                                                             int seg, int ch, int d, int gn, PrepOut out) {
  using U = Unit16<TS>;
  using Raw = typename U::raw;
  constexpr int V = U::n;
  constexpr int R = 4;                    // positions per step (the four-row LDS read)
  constexpr int H = 2 * (K - 1);          // halo rows carried from step to step
  constexpr int NW = H + R;               // window rows
  constexpr int NB = D + 1;               // LDS ring buffers
  static_assert(K >= 1 && K <= kConvMaxTaps && NB >= 2 && NB <= 4, "compiled tap counts and ring depths");
  static_assert(3 * R * D <= 63, "vmcnt field");
  static_assert(kConvSegMax + 2 * (kConvMaxTaps - 1) <= 192, "three positions per lane in the token table");
  constexpr int WBUF = R * 64 * 16;       // bytes per wave and buffer: R rows x 64 lanes x 16 B
  __shared__ __attribute__((aligned(16))) char ring[NB][4][WBUF];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int units = ch / V, tiles = (units + 63) / 64;
  const int64_t item = int64_t(blockIdx.x) * 4 + wave;
  const int64_t nseg = (int64_t(L) + seg - 1) / seg;
  if (item >= nseg * tiles) return;
  const int s_begin = int(item / tiles) * seg, tile = int(item % tiles);
  const int s_end = min(L, s_begin + seg);
  const int nsteps = (s_end - s_begin) / R;
  const int u = tile * 64 + lane;
  const bool valid = u < units;
  const int c0 = min(u, units - 1) * V;   // lanes past the last unit load the last unit and store nothing

  // Stream row j sits at scan position s_begin - (K-1) + j (rows outside
  // [0, L) are loaded clamped; their data is replaced by zeros); its token
  // is held by lane j % 64 in tok0, tok1 or tok2 (j / 64).
  const int p0 = s_begin - (K - 1) + lane;
  const int tok0 = so.canon(min(max(p0, 0), L - 1));
  const int tok1 = so.canon(min(max(p0 + 64, 0), L - 1));
  const int tok2 = so.canon(min(max(p0 + 128, 0), L - 1));
  auto token = [&](int j) -> int {   // j is the same in every lane
    const int a = __builtin_amdgcn_readlane(tok0, j & 63);
    const int b = __builtin_amdgcn_readlane(tok1, j & 63);
    const int c = __builtin_amdgcn_readlane(tok2, j & 63);
    return j < 64 ? a : (j < 128 ? b : c);
  };

  float w_f[V][K], w_b[V][K], b_f[V], b_b[V];
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
#pragma unroll
    for (int e = 0; e < V; ++e) { b_f[e] = bf[c0 + e]; b_b[e] = bb[c0 + e]; }
  }
  const TS* src = in + c0;
  const int last_row = s_end - s_begin + H - 1;   // last stream row the segment needs
  // Loads of step `step` into ring buffer step % NB.
  auto issue = [&](int step) {
    char* base = ring[step % NB][wave];
#pragma unroll
    for (int r = 0; r < R; ++r)
      lds_load16(src + int64_t(token(min(H + step * R + r, last_row))) * ch, base + r * 1024);
  };
  // Channel unit -> destination tensor (x: first d channels, then B, then C).
  int col, width;
  void *pf_, *pb_;
  if (c0 < d) { col = c0; width = d; pf_ = out.x[0]; pb_ = out.x[1]; }
  else if (c0 < d + gn) { col = c0 - d; width = gn; pf_ = out.b[0]; pb_ = out.b[1]; }
  else { col = c0 - d - gn; width = gn; pf_ = out.c[0]; pb_ = out.c[1]; }
  TS* df = static_cast<TS*>(pf_) + col;
  TS* db = static_cast<TS*>(pb_) + col;

  // win[r] holds stream row s*R + r during step s.
  float win[NW][V];
  {
    Raw first[H > 0 ? H : 1];
#pragma unroll
    for (int j = 0; j < H; ++j) first[j] = *reinterpret_cast<const Raw*>(src + int64_t(token(j)) * ch);
#pragma unroll
    for (int t = 0; t < D; ++t) issue(t);
#pragma unroll
    for (int j = 0; j < H; ++j) {
      U::widen(first[j], win[R + j]);
      const int q = s_begin - (K - 1) + j;
      if (q < 0 || q >= L)
#pragma unroll
        for (int e = 0; e < V; ++e) win[R + j][e] = 0.f;
    }
  }
  for (int s = 0; s < nsteps; ++s) {
    issue(s + D);
    if (s < D) __builtin_amdgcn_s_waitcnt(vmcnt_imm(R * D));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * R * D));
#pragma unroll
    for (int r = 0; r < H; ++r)
#pragma unroll
      for (int e = 0; e < V; ++e) win[r][e] = win[r + R][e];
    {
      const unsigned addr = unsigned(reinterpret_cast<uintptr_t>(ring[s % NB][wave])) + unsigned(lane * 16);
      i32x4 raw[R];
      lds_read4x16(addr, raw[0], raw[1], raw[2], raw[3]);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        U::widen(__builtin_bit_cast(Raw, raw[r]), win[H + r]);
        const int q = s_begin - (K - 1) + H + s * R + r;
        if (q >= L)
#pragma unroll
          for (int e = 0; e < V; ++e) win[H + r][e] = 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < R; ++j) {
      float o_f[V], o_b[V];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        float af = b_f[e], ab = b_b[e];
#pragma unroll
        for (int k = 0; k < K; ++k) {
          af = fmaf(w_f[e][k], win[j + k][e], af);
          ab = fmaf(w_b[e][k], win[j + H - k][e], ab);
        }
        o_f[e] = silu(af);
        o_b[e] = silu(ab);
      }
      const int64_t off = int64_t(token(K - 1 + s * R + j)) * width;
      if (valid) {
        U::store(df + off, o_f);
        U::store(db + off, o_b);
      }
    }
  }
  wait_vmem();   // the loads issued past the end are still landing in LDS
}

// dt = softplus(dt_raw + dt_bias[head]) in the overflow-safe form
// max(a, 0) + log1p(exp(-|a|)).
__global__ __launch_bounds__(256) void softplus_bias_kernel(const float* __restrict__ raw,
                                                            const float* __restrict__ bias, int64_t n, int heads,
                                                            float* __restrict__ out) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  out[i] = softplus(raw[i] + bias[i % heads]);
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
    ss = sum64(ss);
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

constexpr int kConvStep = 4;      // scan positions per step of a wave
constexpr int kConvAhead = 2;     // steps of loads in flight per wave

template <typename TS, int K>
int launch_conv(const TS* in, const float* wf, const float* bf, const float* wb, const float* bb, ScanOrder so,
                int L, int ch, int d, int gn, PrepOut o, hipStream_t st) {
  const int64_t tiles = (ch / Unit16<TS>::n + 63) / 64;
  // Longest segment that still gives every compute unit several waves per
  // SIMD: long segments load fewer halo rows and weights, short ones fill the
  // chip.
  const int cus = compute_units();
  const int64_t want_waves = 32LL * (cus > 0 ? cus : 256);
  int seg = kConvSegMax;
  while (seg > kConvStep && ((int64_t(L) + seg - 1) / seg) * tiles < want_waves) seg /= 2;
  const int64_t waves = ((int64_t(L) + seg - 1) / seg) * tiles;
  scan_conv_silu_kernel<TS, K, kConvAhead><<<unsigned((waves + 3) / 4), 256, 0, st>>>(in, wf, bf, wb, bb, so, L, seg,
                                                                                      ch, d, gn, o);
  return launch_status(__func__);
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
  return launch_status(__func__);
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
  // the convolution walks whole steps of kConvStep positions (every compiled
  // chunk length is a multiple of it, so every valid shape passes)
  if (tokens(shape) % kConvStep) return LINGEN_ERR_SHAPE;
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
  return launch_status(__func__);
}
