// HIP kernels (gfx950 / CDNA4) of the MATE token mixer and the C-ABI entry
// points that launch them.
//
// Pipeline of one forward call (per batch element, all on the caller's
// stream):
//   review_pool, review_state  (only with review tokens)
//   ssd_chunk_state            phase A: per (chunk, head) the decay-weighted
//                              chunk states of both scan directions, on MFMA
//   ssd_state_pass             inter-chunk recurrence, forward and backward
//                              (the backward walk is the same loop with the
//                              chunk index reflected)
//   ssd_chunk_out              phase B: per (chunk, head) the in-chunk
//                              quadratic form plus both inter-chunk terms plus
//                              the skip, scattered to canonical token order
//   tesa_window                per (window, head) masked softmax attention on
//                              MFMA with an online softmax, adding the MA
//                              output (fused branch sum)
//
// The Rotary Major Scan never materialises a permuted copy: every scan-order
// access goes through RmsMap::canon, which turns a scan position into the
// canonical token index with mixed-radix arithmetic.
//
// Chunked form of the bidirectional scan used by phases A and B (Mamba2's SSD
// chunking, extended to the reversed direction).  Inside a chunk of Q scan
// positions, with a_s = dt_s*A, cum_t = sum_{tau<=t} a_tau and
// exc_t = cum_t - a_t (both taken within the chunk; the kernels keep them in
// log2 units, i.e. multiplied by log2(e), and exponentiate with v_exp_f32):
//   forward  state out of the chunk   = e^{cum_end} h_in + sum_s e^{cum_end-cum_s} dt_s x_s B_s^T
//   backward state out of the chunk   = e^{cum_end} h_in + sum_s e^{exc_s} dt_s x_s B_s^T
//   y_t = sum_s Lambda[t,s] (C_t.B_s) dt_s x_s + e^{cum_t} C_t.h_fwd_in
//         + e^{cum_end-exc_t} C_t.h_bwd_in + 2 D x_t,
//   Lambda[t,s] = e^{cum_t-cum_s} (s<t), e^{exc_s-exc_t} (s>t), 2 (s=t).
// Only differences of partial sums that are <= 0 are exponentiated.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "lingen_device.h"
#include "lingen_internal.h"
#include "lingen_window.h"

namespace lingen {

// ---------------------------------------------------------------------------
// Small device helpers
// ---------------------------------------------------------------------------

// Element padding of k-contiguous LDS rows (keeps 16-byte alignment and
// spreads the 16 rows one fragment load touches over different banks).
template <typename MT> struct LdsPad { static constexpr int v = 8; };
template <> struct LdsPad<float> { static constexpr int v = 4; };

// LDS tile with COLS elements per row, read by MFMA fragment loads (16 rows
// x one 16-byte chunk per lane group).  bf16 rows that are a whole number of
// 128-byte lines are stored unpadded with the 16-byte chunks of row r
// permuted as chunk ^ (r mod 16) (mod 8 for 128-byte rows) ^ 4 [bit 3 of r]:
// fragment loads and row-contiguous stores touch distinct banks, and so do
// the transposed token-pair stores of the chunk-state kernel, whose 32
// lanes write rows r and r + 8 at once (with chunk ^ (r mod 16) alone those
// two rows' chunks meet in the same banks, 128 bytes of banks per cycle).
// Other tiles are padded by LdsPad.
template <typename MT, int COLS>
struct Tile {
  static constexpr bool kSwz = sizeof(MT) == 2 && COLS % 64 == 0;
  static constexpr int LD = kSwz ? COLS : COLS + LdsPad<MT>::v;
  static constexpr int kMask = (COLS / 8 >= 16 ? 16 : COLS / 8) - 1;
  __device__ static __forceinline__ int at(int row, int col) {
    if constexpr (kSwz) return row * COLS + ((((col >> 3) ^ (row & kMask) ^ ((row >> 1) & 4)) << 3) | (col & 7));
    else return row * LD + col;
  }
  // Operand fragment of row `row` for k = k0 + the lane group's k values.
  __device__ static __forceinline__ typename Frag<MT>::type frag(const MT* base, int row, int k0, int lane) {
    if constexpr (sizeof(MT) == 2) return *reinterpret_cast<const bf16x8*>(base + at(row, k0 + (lane >> 4) * 8));
    else return base[at(row, k0 + (lane >> 4))];
  }
};

// 16-byte global vector, viewed as elements.
template <typename T> struct Vec16 {
  static constexpr int n = 16 / sizeof(T);
  union { uint4 u; T e[16 / sizeof(T)]; };
};

// Staging of TOTAL 16-byte units by NTHR threads (unit u -> thread u % NTHR)
// in two steps, so that all of a thread's global loads are in flight before
// the first one is consumed: load() issues them into registers, use() hands
// each to the caller (typically to be written to LDS).
template <int TOTAL, int NTHR>
struct Stage16 {
  static constexpr int IT = (TOTAL + NTHR - 1) / NTHR;
  uint4 v[IT];
  template <typename Load>
  __device__ __forceinline__ void load(Load f) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int u = int(threadIdx.x) + it * NTHR;
      if (TOTAL % NTHR == 0 || u < TOTAL) v[it] = f(u);
    }
  }
  template <typename Use>
  __device__ __forceinline__ void use(Use f) const {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int u = int(threadIdx.x) + it * NTHR;
      if (TOTAL % NTHR == 0 || u < TOTAL) f(u, v[it]);
    }
  }
};

// Transposing stage of a [ROWS tokens][COLS] block of T into an LDS block
// laid out [COLS][ld]: unit u covers the token pair (2i, 2i+1) and VEC
// consecutive columns; both rows are loaded before any is consumed, and the
// consumer writes each column's pair of values with one store (for bf16 one
// 32-bit LDS word, so no two lanes touch the same word).  LPT consecutive
// units take consecutive 16-byte pieces of the same pair of rows.
template <typename T, int ROWS, int COLS, int NTHR, int LPT = 1>
struct StageT {
  static constexpr int VEC = Vec16<T>::n;
  static constexpr int UNITS = (ROWS / 2) * (COLS / VEC);
  static constexpr int IT = (UNITS + NTHR - 1) / NTHR;
  static_assert(ROWS % 2 == 0 && COLS % VEC == 0, "token pairs and 16-byte columns");
  static_assert((COLS / VEC) % LPT == 0, "whole groups of pieces per row");
  __device__ static __forceinline__ int pair_of(int u) { return (u / LPT) % (ROWS / 2); }
  __device__ static __forceinline__ int col_of(int u) { return ((u / LPT) / (ROWS / 2) * LPT + u % LPT) * VEC; }
  uint4 a[IT], b[IT];
  template <typename RowPtr>   // RowPtr(token) -> const T* to the start of that token's row
  __device__ __forceinline__ void load(RowPtr row) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int u = int(threadIdx.x) + it * NTHR;
      if (UNITS % NTHR == 0 || u < UNITS) {
        const int i = pair_of(u), c0 = col_of(u);
        a[it] = *reinterpret_cast<const uint4*>(row(2 * i) + c0);
        b[it] = *reinterpret_cast<const uint4*>(row(2 * i + 1) + c0);
      }
    }
  }
  template <typename Use>      // Use(s0 = even token, c0 = first column, values of s0, values of s0 + 1)
  __device__ __forceinline__ void use(Use f) const {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int u = int(threadIdx.x) + it * NTHR;
      if (UNITS % NTHR == 0 || u < UNITS) {
        Vec16<T> va, vb;
        va.u = a[it];
        vb.u = b[it];
        f(2 * pair_of(u), col_of(u), va, vb);
      }
    }
  }
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// Two consecutive elements of one LDS row (4-byte aligned for bf16, 8 for
// fp32): from values already in the element type, or rounded from fp32.
__device__ __forceinline__ void st_pair(__bf16* dst, __bf16 lo, __bf16 hi) {
  *reinterpret_cast<bf16x2*>(dst) = bf16x2{lo, hi};
}
__device__ __forceinline__ void st_pair_f32(__bf16* dst, float lo, float hi) {
  *reinterpret_cast<bf16x2*>(dst) = bf16x2{static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
}
__device__ __forceinline__ void st_pair(float* dst, float lo, float hi) {
  *reinterpret_cast<float2*>(dst) = make_float2(lo, hi);
}
__device__ __forceinline__ void st_pair_f32(float* dst, float lo, float hi) { st_pair(dst, lo, hi); }

// Scan position -> canonical token index for the four Rotary Major Scan
// orders (page "LinGen：基于Mamba机制的线性复杂度高清长视频生成框架", section
// 关键算法创新 > Rotary Major Scan):
//   mode 0: s = (t*H + h)*W + w   W first, then H, then T
//   mode 1: s = (t*W + w)*H + h   H first, then W, then T
//   mode 2: s = (h*W + w)*T + t   T first, then W, then H
//   mode 3: s = (w*H + h)*T + t   T first, then H, then W
// rev = 1 walks the order backwards (scan position s is position L-1-s of
// the mode's order): the backward scan of a direction-specific parameter set.
struct RmsMap {
  int mode, T, H, W;
  int rev = 0;
  __device__ __forceinline__ int canon(int s) const {
    if (rev) s = T * H * W - 1 - s;
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

// Workgroups are dispatched round-robin over the 8 XCDs of the chip.  Give
// every XCD a contiguous range of work ids so that the workgroups of all
// heads of one chunk share one L2 (B, C and dt rows are shared by heads).
__device__ __forceinline__ int xcd_work_id(int bid, int nblocks) {
  if (nblocks % 8) return bid;
  return (bid % 8) * (nblocks / 8) + bid / 8;
}

// Order in which the chunk workgroups take their chunks (chunks are
// independent in the chunk-state and output kernels, so any bijection will
// do).  In scan order 3 (T fastest, then H, then W) consecutive chunks step
// along h at fixed w, so workgroups that run at the same time would read
// rows H*W apart in every frame (different pages); taking the chunks w
// first instead gives them the locality of order 2, rows one apart.  With
// M = H*T/Q chunks per w-column (a whole number in every workload), the
// j-th chunk taken is c = (j mod W) * M + j / W.
template <int Q>
__device__ __forceinline__ int chunk_order(const RmsMap& m, int j) {
  if (m.mode != 3 || (m.H * m.T) % Q) return j;
  const int M = m.H * m.T / Q;
  return (j % m.W) * M + j / m.W;
}

// Inclusive and exclusive prefix sums of a_s = dt_s * A * log2(e) over one
// chunk of Q scan positions (Q <= 256), computed by the calling wave alone
// (all 64 lanes call it; no block barrier inside).
template <int Q, bool WITH_EXC = true>
__device__ __forceinline__ void wave_chunk_prefix(const float* sdt, float Ah, float* scum, float* sexc) {
  constexpr int E = (Q + 63) / 64;
  const int lane = threadIdx.x & 63;
  const float a2 = Ah * kLog2e;
  float v[E];
  float run = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int idx = lane * E + e;
    v[e] = idx < Q ? sdt[idx] * a2 : 0.f;
    run += v[e];
  }
  float base = wave_scan_incl(run) - run;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int idx = lane * E + e;
    if (idx < Q) {
      if (WITH_EXC) sexc[idx] = base;
      base += v[e];
      scum[idx] = base;
    }
  }
}

// Heads handled by one chunk workgroup (the largest divisor of Hs up to 16
// for the output kernel; up to 8 for the chunk-state kernel, whose LDS then
// still fits twice per CU).
constexpr int kHeadGroupMax = 16;
constexpr int kStateHeadGroup = 8;

// Per-chunk schedule shared by the heads of one workgroup: the canonical
// token of every scan position, and per head the step sizes and their
// inclusive / exclusive prefix sums of dt*A in log2 units.
template <int Q, int HGM = kHeadGroupMax, bool WITH_EXC = true>
struct __attribute__((aligned(16))) ChunkSched {
  static_assert(Q % 4 == 0, "rows are read as float4");
  int tok[Q];
  float dt[HGM][Q];
  float cum[HGM][Q];
  float exc[WITH_EXC ? HGM : 1][WITH_EXC ? Q : 4];   // exc = cum - a when not kept
};

// The chunk schedule in steps, so that a kernel can issue its token-row loads
// (which need only the token map) between the dt loads and their use:
// load_chunk_tokens fills cs.tok; ChunkDt::load fetches the heads' dt into
// registers (with A of the heads whose prefix sums the wave forms) and
// ChunkDt::finish stores them (dt_bias, when not null: as
// softplus(dt + dt_bias[h])) and forms the prefix sums.
template <int Q, int NTHR, int HGM, bool WITH_EXC>
__device__ __forceinline__ void load_chunk_tokens(ChunkSched<Q, HGM, WITH_EXC>& cs, RmsMap rms, int c) {
  for (int i = threadIdx.x; i < Q; i += NTHR) cs.tok[i] = rms.canon(c * Q + i);
  lds_barrier();
}

template <int Q, int NTHR, int HGM>
struct ChunkDt {
  static constexpr int IT = (Q * HGM + NTHR - 1) / NTHR;
  static constexpr int NWAVE = NTHR / 64, JT = (HGM + NWAVE - 1) / NWAVE;
  float v[IT];    // dt of the chunk's tokens and heads
  float av[JT];   // A of the heads whose prefix sums this wave forms
  template <bool WITH_EXC>
  __device__ __forceinline__ void load(const ChunkSched<Q, HGM, WITH_EXC>& cs, const float* __restrict__ dt,
                                       const float* __restrict__ A, int Hs, int h0, int hg) {
    // (vector loads for A too: a scalar load would join the LDS reads' wait
    // counter, which the token-row loads issued behind these wait on)
    const int tid = threadIdx.x, wave = tid >> 6;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int u = tid + it * NTHR;
      if (u < Q * hg) v[it] = dt[int64_t(cs.tok[u / hg]) * Hs + h0 + u % hg];
    }
#pragma unroll
    for (int k = 0; k < JT; ++k) {
      const int j = wave + k * NWAVE;
      av[k] = A[h0 + (j < hg ? j : hg - 1)];   // (no branch around the load)
    }
  }
  template <bool WITH_EXC>
  __device__ __forceinline__ void finish(ChunkSched<Q, HGM, WITH_EXC>& cs, int h0, int hg,
                                         const float* __restrict__ dt_bias = nullptr) {
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int u = tid + it * NTHR;
      if (u < Q * hg) cs.dt[u % hg][u / hg] = dt_bias ? softplus(v[it] + dt_bias[h0 + u % hg]) : v[it];
    }
    lds_barrier();
#pragma unroll
    for (int k = 0; k < JT; ++k) {
      const int j = wave + k * NWAVE;
      if (j < hg) wave_chunk_prefix<Q, WITH_EXC>(cs.dt[j], av[k], cs.cum[j], cs.exc[WITH_EXC ? j : 0]);
    }
    lds_barrier();
  }
};

template <int Q, int NTHR, int HGM, bool WITH_EXC>
__device__ __forceinline__ void load_chunk_dt(ChunkSched<Q, HGM, WITH_EXC>& cs, const float* __restrict__ dt,
                                              const float* __restrict__ A, int Hs, int h0, int hg,
                                              const float* __restrict__ dt_bias = nullptr) {
  ChunkDt<Q, NTHR, HGM> d;
  d.load(cs, dt, A, Hs, h0, hg);
  d.finish(cs, h0, hg, dt_bias);
}

// ---------------------------------------------------------------------------
// RMS probe kernels: the index map and a scan-order copy.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void rms_index_kernel(RmsMap m, int L, int* __restrict__ perm) {
  const int s = blockIdx.x * 256 + threadIdx.x;
  if (s < L) perm[s] = m.canon(s);
}

// Scan position of the r-th row copied.  Rows are taken in scan order,
// except in order 3 (T fastest, then H, then W): consecutive positions there
// step along h, so the rows read at the same time would sit W rows apart in
// every frame; taking the (h, w) sites w first, as order 2 does, reads
// neighbouring rows instead.  Any bijection of the rows gives the same copy.
__device__ __forceinline__ int gather_row_order(const RmsMap& m, int r) {
  if (m.mode != 3) return r;
  const int t = r % m.T, q = r / m.T;
  return ((q % m.W) * m.H + q / m.W) * m.T + t;
}

// One workgroup per row: the row's source and destination offsets are
// uniform over the workgroup, and each element is touched once, so loads and
// stores are streaming (non-temporal).  Measured on the 4 KiB rows of the
// minute-length 128x64x64 grid: 61-77% of 8 TB/s with per-lane index
// arithmetic and cached accesses, 74-82% in this form.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void rms_gather_kernel(const u32x4* __restrict__ src, int64_t row16, RmsMap m,
                                                         u32x4* __restrict__ dst) {
  const int s = gather_row_order(m, blockIdx.x);
  const u32x4* from = src + int64_t(m.canon(s)) * row16;
  u32x4* to = dst + int64_t(s) * row16;
  for (int64_t off = threadIdx.x; off < row16; off += 256)
    __builtin_nontemporal_store(__builtin_nontemporal_load(from + off), to + off);
}

// ---------------------------------------------------------------------------
// Review tokens: block means at the sampled block positions, then the state
// the review tokens leave behind.
// ---------------------------------------------------------------------------

struct ReviewGeom {
  int pt, ph, pw;   // pooling block
  int rt, rh, rw;   // points per axis
  int st, sh, sw;   // stride between sampled blocks, in blocks
};

// Block (r, y): the mean over review block r of head y's x row slice (and
// of dt for that head) for y < Hs, of group y - Hs's B rows for y >= Hs.  Each thread
// sums the 16-byte chunk c of every RP-th token row, with several rows'
// loads in flight, and the RP partial sums are reduced through LDS.
template <typename TS>
__global__ __launch_bounds__(256) void review_pool_kernel(const TS* __restrict__ x, const float* __restrict__ dt,
                                                          const TS* __restrict__ B, int T, int H, int W, int Hs,
                                                          int P, int N, int G, ReviewGeom g, float* __restrict__ rx,
                                                          float* __restrict__ rdt, float* __restrict__ rb) {
  constexpr int VEC = Vec16<TS>::n;
  constexpr int UNROLL = 4;
  __shared__ float red[256 * VEC];
  const int r = blockIdx.x;
  const int y = blockIdx.y;
  const int tid = threadIdx.x;
  const int i = r / (g.rh * g.rw), j = (r / g.rw) % g.rh, k = r % g.rw;
  const int t0 = i * g.st * g.pt, h0 = j * g.sh * g.ph, w0 = k * g.sw * g.pw;
  const int cnt = g.pt * g.ph * g.pw;
  const float inv = 1.f / float(cnt);
  auto token = [&](int tl) {
    const int a = tl / (g.ph * g.pw), b = (tl / g.pw) % g.ph, c = tl % g.pw;
    return ((t0 + a) * H + (h0 + b)) * W + (w0 + c);
  };
  const int width = (y < Hs) ? P : N;   // P, N in {16, 32, 64, 128} in every compiled family, so
                                        // width / VEC divides 256
  const int cpr = width / VEC, rp = 256 / cpr;
  const int c = tid % cpr, ro = tid / cpr;
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  for (int tl0 = ro; tl0 < cnt; tl0 += rp * UNROLL) {
    Vec16<TS> v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int tl = tl0 + u * rp;
      v[u].u = make_uint4(0, 0, 0, 0);
      if (tl < cnt) {
        const int64_t tok = token(tl);
        const TS* src = (y < Hs) ? x + (tok * Hs + y) * P : B + (tok * G + (y - Hs)) * N;
        v[u].u = *reinterpret_cast<const uint4*>(src + c * VEC);
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] += to_f32(v[u].e[e]);
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) red[ro * width + c * VEC + e] = acc[e];
  lds_barrier();
  if (tid < width) {
    float sum = 0.f;
    for (int q = 0; q < rp; ++q) sum += red[q * width + tid];
    if (y < Hs) rx[(int64_t(r) * Hs + y) * P + tid] = sum * inv;
    else rb[(int64_t(r) * G + (y - Hs)) * N + tid] = sum * inv;
  }
  if (y < Hs) {
    lds_barrier();
    float d = 0.f;
    for (int tl = tid; tl < cnt; tl += 256) d += dt[int64_t(token(tl)) * Hs + y];
    red[tid] = d;
    lds_barrier();
    for (int off = 128; off > 0; off >>= 1) {
      if (tid < off) red[tid] += red[tid + off];
      lds_barrier();
    }
    if (tid == 0) rdt[int64_t(r) * Hs + y] = red[0] * inv;
  }
}

// h_R[h][p][n] = sum_r exp(sum_{tau>r} a_tau) dt_r x_r[p] B_r[n], from zero.
__global__ __launch_bounds__(256) void review_state_kernel(const float* __restrict__ rx, const float* __restrict__ rdt,
                                                           const float* __restrict__ rb, const float* __restrict__ A,
                                                           int R, int Hs, int P, int N, int G, float* __restrict__ hR) {
  // Block (h, slice) computes elements slice*1024 .. +1023 of head h's P x N
  // state, four per thread.  Review tokens are taken RT at a time: their
  // weighted x rows and B rows are staged in LDS, then every thread
  // accumulates its elements.
  constexpr int RT = 64, MAXP = 128, MAXN = 128, MAXE = 4;
  __shared__ float w[256];
  __shared__ float sx[RT * MAXP];
  __shared__ float sb[RT * MAXN];
  const int h = blockIdx.x, tid = threadIdx.x;
  const int grp = h / (Hs / G);   // B group of head h
  for (int r = tid; r < R; r += 256) w[r] = rdt[r * Hs + h];
  lds_barrier();
  if (tid == 0) {   // w_r = e^{sum_{tau > r} a_tau} dt_r, from the last review token back
    float suf = 0.f;
    for (int r = R - 1; r >= 0; --r) {
      const float d = w[r];
      w[r] = expf(suf) * d;
      suf += d * A[h];
    }
  }
  lds_barrier();
  const int e0 = int(blockIdx.y) * 1024 + tid;
  float acc[MAXE];
#pragma unroll
  for (int k = 0; k < MAXE; ++k) acc[k] = 0.f;
  for (int r0 = 0; r0 < R; r0 += RT) {
    const int rn = R - r0 < RT ? R - r0 : RT;
    for (int u = tid; u < rn * P; u += 256) sx[u] = rx[((r0 + u / P) * Hs + h) * P + u % P] * w[r0 + u / P];
    for (int u = tid; u < rn * N; u += 256) sb[u] = rb[((r0 + u / N) * G + grp) * N + u % N];
    lds_barrier();
    int pk[MAXE], nk[MAXE];
#pragma unroll
    for (int k = 0; k < MAXE; ++k) {
      const int e = e0 + k * 256 < P * N ? e0 + k * 256 : 0;
      pk[k] = e / N;
      nk[k] = e % N;
    }
    for (int rr = 0; rr < rn; ++rr)
#pragma unroll
      for (int k = 0; k < MAXE; ++k) acc[k] += sx[rr * P + pk[k]] * sb[rr * N + nk[k]];
    lds_barrier();
  }
#pragma unroll
  for (int k = 0; k < MAXE; ++k)
    if (e0 + k * 256 < P * N) hR[int64_t(h) * P * N + e0 + k * 256] = acc[k];
}

// ---------------------------------------------------------------------------
// Phase A: chunk states of both directions.  One workgroup per (chunk, group
// of heads); B^T is staged once and reused by every head of the group.
//   S_f^T[p][n] = sum_s (x_s[p] wf_s) B_s[n],  wf_s = e^{cum_end - cum_s} dt_s
//   S_b^T[p][n] = sum_s (x_s[p] wb_s) B_s[n],  wb_s = e^{exc_s} dt_s
// Stored in the input element type as states[dir][chunk][head][p][n], plus
// decay[chunk][head] = e^{cum_end}.
// ---------------------------------------------------------------------------

template <int P, int N>
struct StateCfg {
  static constexpr int PT = P / 16, NT = N / 16;
  static constexpr int NWAVE = PT * NT >= 16 ? 8 : 4;
  static constexpr int WP = PT >= 4 ? 4 : PT;       // waves along p
  static constexpr int WN = NWAVE / WP;               // waves along n
  static constexpr int PT_PER = PT / WP;
  static constexpr int NT_PER = (NT + WN - 1) / WN;
};

// Pieces of one token-pair row taken by consecutive lanes when staging x
// and B: one load instruction then touches 32 token rows instead of 64,
// which halves its address translations when the scan order puts
// consecutive tokens far apart, while the transposed LDS stores stay
// spread over the banks.
constexpr int kLptX = 2, kLptB = 2;

// ---------------------------------------------------------------------------
// The Mamba-2 steps between the input projection and the scan, fused into the
// scan kernels of a scan with a parameter set per direction (page
// "视频生成模子太贵太慢如何办？", section 要领: the MA branch is a
// bidirectional Mamba2 block).  x, B and C are SiLU of a causal depthwise
// convolution of the xBC channels along the scan order of the direction, and
// dt = softplus(dt_raw + dt_bias).  A chunk's Q positions read the
// kConvTaps - 1 positions before it as well (its halo).  Fewer taps than
// kConvTaps run as kConvTaps with leading zero weights: fma(0, v, a) = a for
// the finite inputs here, so every tap count takes the same roundings as the
// standalone convolution (bias first, then the taps oldest first, SiLU,
// rounding to the storage type).
// ---------------------------------------------------------------------------
constexpr int kConvTaps = 4;
constexpr int kConvHalo = kConvTaps - 1;
constexpr int kConvW = kConvTaps + 1;   // rows of a weight table: the padded taps, then the bias

// The thread index through an empty asm statement: values formed from it
// inside a loop are formed again on every pass instead of being kept in
// registers across the loop (the fused kernels' per-head staging addresses
// otherwise outgrow the register budget and spill).
__device__ __forceinline__ int fresh_tid() {
  int t = int(threadIdx.x);
  asm volatile("" : "+v"(t));
  return t;
}

struct ConvIn {
  const float* w = nullptr;        // [ch][K] taps per channel
  const float* b = nullptr;        // [ch] biases
  const float* dt_bias = nullptr;  // [Hs]; null: dt is taken as given
  int K = 0;                       // taps, 1 .. kConvTaps
  int ch = 0;                      // channels of an xBC row (its stride in elements)
  int coff_b = 0, coff_c = 0;      // first channel of B and of C (x starts at 0)
};

// Token of row j of a chunk's raw rows: rows 0 .. kConvHalo - 1 are the halo
// (scan positions c*Q - kConvHalo + j), the others the chunk's own
// positions.  Halo rows before the sequence (chunk 0 only) give the chunk's
// first token instead, a valid row whose data the staging replaces by
// zeros: every load is then issued unconditionally (no branch around a
// load, which would make the wait counters drain at the join).
// The halo's tokens are formed once per chunk (halo_tokens, before the
// schedule's barrier) and read from LDS with the chunk's own.
template <int Q>
__device__ __forceinline__ void halo_tokens(int* htok, const RmsMap& m, int c) {
  const int j = int(threadIdx.x);
  if (j < kConvHalo) htok[j] = m.canon(c > 0 ? c * Q - kConvHalo + j : 0);
}
template <typename Sched>
__device__ __forceinline__ int raw_row_token(const Sched& cs, const int* htok, int j) {
  return j >= kConvHalo ? cs.tok[j - kConvHalo] : htok[j];
}

// Conv weights of COLS channels from channel c0, as [kConvW][COLS] (the taps
// padded at the front, then the bias): fetched into registers, then written
// to LDS by the caller's workgroup of NTHR threads.
template <int COLS, int NTHR>
struct ConvWeights {
  static constexpr int PER = COLS * kConvW;
  static constexpr int IT = (PER + NTHR - 1) / NTHR;
  float w[IT], b[IT];
  int pad;   // taps of the table before the caller's first
  // Both candidates are loaded from clamped, valid indices and the entry is
  // chosen when it is stored (no branch around a load).
  __device__ __forceinline__ void load(const ConvIn& cv, int c0) {
    const int t = fresh_tid();
    pad = kConvTaps - cv.K;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int i = PER % NTHR == 0 ? t + it * NTHR : min(t + it * NTHR, PER - 1);
      const int k = i / COLS, col = i % COLS;
      w[it] = cv.w[int64_t(c0 + col) * cv.K + min(max(k - pad, 0), cv.K - 1)];
      b[it] = cv.b[c0 + col];
    }
  }
  __device__ __forceinline__ void store(float* dst) const {
    const int t = fresh_tid();
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int i = t + it * NTHR, k = i / COLS;
      if (PER % NTHR == 0 || i < PER) dst[i] = k == kConvTaps ? b[it] : (k < pad ? 0.f : w[it]);
    }
  }
};

// A chunk's raw rows (halo first) of COLS channels, each row from `row(j)`,
// staged through registers: the chunk's own rows go to `main` (tile layout
// TL), the halo rows to `halo` ([kConvHalo][COLS]), as zeros when zero_halo
// (chunk 0: the halo lies before the sequence).  Lanes past the last piece
// load the last piece again and store nothing.
template <typename TS, int Q, int COLS, int NTHR>
struct RawRows {
  static constexpr int VEC = Vec16<TS>::n, PR = COLS / VEC;
  static constexpr int TOTAL = (Q + kConvHalo) * PR;
  static constexpr int IT = (TOTAL + NTHR - 1) / NTHR;
  uint4 v[IT];
  template <typename Row>
  __device__ __forceinline__ void load(Row row) {
    const int t = fresh_tid();
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int u = TOTAL % NTHR == 0 ? t + it * NTHR : min(t + it * NTHR, TOTAL - 1);
      v[it] = *reinterpret_cast<const uint4*>(row(u / PR) + (u % PR) * VEC);
    }
  }
  template <typename TL>
  __device__ __forceinline__ void store(TS* main, TS* halo, bool zero_halo) const {
    const int t = fresh_tid();
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int u = t + it * NTHR;
      if (TOTAL % NTHR == 0 || u < TOTAL) {
        const int j = u / PR, col = (u % PR) * VEC;
        if (j < kConvHalo) *reinterpret_cast<uint4*>(&halo[j * COLS + col]) = zero_halo ? uint4{0u, 0u, 0u, 0u} : v[it];
        else *reinterpret_cast<uint4*>(&main[TL::at(j - kConvHalo, col)]) = v[it];
      }
    }
  }
};

// 16 bytes of raw row r (0 .. Q + kConvHalo - 1) at column col, widened.
template <typename TS, typename TL, int COLS>
__device__ __forceinline__ void raw_read(const TS* main, const TS* halo, int r, int col, float (&v)[Vec16<TS>::n]) {
  Vec16<TS> u;
  u.u = *reinterpret_cast<const uint4*>(r < kConvHalo ? &halo[r * COLS + col] : &main[TL::at(r - kConvHalo, col)]);
#pragma unroll
  for (int e = 0; e < Vec16<TS>::n; ++e) v[e] = to_f32(u.e[e]);
}

// Convolution + SiLU of R consecutive positions s0 .. s0 + R - 1 of the
// chunk for the VEC channels at column col (raw rows s0 .. s0 + R + 2), with
// the weights wt ([kConvW][COLS] in LDS); out in the storage type.  Taps
// outermost, so one tap's weights are live at a time.
template <typename TS, typename TL, int COLS, int R>
__device__ __forceinline__ void conv_rows(const TS* main, const TS* halo, const float* wt, int s0, int col,
                                          TS (&out)[R][Vec16<TS>::n]) {
  constexpr int V = Vec16<TS>::n;
  static_assert(V % 4 == 0, "whole float4 pieces of the weight rows");
  auto weights = [&](int k, float (&w)[V]) {
#pragma unroll
    for (int q = 0; q < V / 4; ++q) {
      const float4 a = *reinterpret_cast<const float4*>(&wt[k * COLS + col + 4 * q]);
      w[4 * q + 0] = a.x; w[4 * q + 1] = a.y; w[4 * q + 2] = a.z; w[4 * q + 3] = a.w;
    }
  };
  float acc[R][V];
  {
    float bias[V];
    weights(kConvTaps, bias);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int e = 0; e < V; ++e) acc[r][e] = bias[e];
  }
#pragma unroll
  for (int k = 0; k < kConvTaps; ++k) {
    float w[V];
    weights(k, w);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float v[V];
      raw_read<TS, TL, COLS>(main, halo, s0 + r + k, col, v);   // tap k of position s0 + r
#pragma unroll
      for (int e = 0; e < V; ++e) acc[r][e] = fmaf(w[e], v[e], acc[r][e]);
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int e = 0; e < V; ++e) out[r][e] = from_f32<TS>(silu(acc[r][e]));
}

// BIDIR = false: the forward direction's chunk states only (a scan whose
// backward direction has parameters of its own).
// CONV: x and B are the convolved xBC channels (the fused steps above): x
// and B both point at the xBC rows, cv gives the convolution and dt_bias.
// Two workgroups share a compute unit (at most 128 VGPRs).
template <typename TS, int P, int N, int Q, bool BIDIR = true, int WM = kWeightDt, bool CONV = false>
__global__ __launch_bounds__((StateCfg<P, N>::NWAVE * 64), 4) void ssd_chunk_state_kernel(const TS* __restrict__ x, const float* __restrict__ dt,
                                                              const float* __restrict__ A, const TS* __restrict__ B,
                                                              RmsMap rms, int Hs, int G, int hg, int n_chunks,
                                                              TS* __restrict__ states, float* __restrict__ decay,
                                                              ConvIn cv) {
  using MT = TS;
  using F = Frag<MT>;
  constexpr int KI = F::K;
  using TQ = Tile<MT, Q>;     // rows of Q tokens: B^T and the weighted x^T
  using TO = Tile<TS, N>;     // output staging, rows of N
  constexpr int QP = TQ::LD;
  constexpr int VEC = Vec16<TS>::n;
  static_assert(Q % KI == 0 && P % 16 == 0 && N % 16 == 0 && P % VEC == 0 && N % VEC == 0, "tile shape");
  constexpr int XBYTES = 2 * P * QP * int(sizeof(MT));
  constexpr int OBYTES = 2 * P * N * int(sizeof(TS));
  constexpr int UBYTES = XBYTES > OBYTES ? XBYTES : OBYTES;
  __shared__ __attribute__((aligned(16))) MT sBt[N * QP];
  __shared__ __attribute__((aligned(16))) char sU[UBYTES];   // x staging, then output staging
  __shared__ ChunkSched<Q, kStateHeadGroup, false> cs;
  __shared__ float sW[2][Q];
  MT* sXf = reinterpret_cast<MT*>(sU);
  MT* sXb = sXf + P * QP;
  TS* sOut = reinterpret_cast<TS*>(sU);
  using SC = StateCfg<P, N>;
  constexpr int NTHR = SC::NWAVE * 64;
  // CONV: the raw rows of B (chunk rows in sU, before any x staging) and of
  // each head's x (chunk rows in the second half of sU, unused by one
  // direction), the halo rows and the weight table.
  static_assert(!CONV || (!BIDIR && WM == kWeightDt && sizeof(TS) == 2), "fused steps: one direction, bf16");
  static_assert(!CONV || Q * N * int(sizeof(TS)) <= UBYTES, "raw B rows fit the x / output staging");
  constexpr int CW = N > P ? N : P;
  __shared__ __attribute__((aligned(16))) MT sHalo[CONV ? kConvHalo * CW : 1];
  __shared__ __attribute__((aligned(16))) float sCw[CONV ? kConvW * CW : 1];
  __shared__ int sHtok[kConvHalo];
  using TRB = Tile<MT, N>;
  using TRX = Tile<MT, P>;

  const int ngrp = Hs / hg;
  const int work = xcd_work_id(blockIdx.x, gridDim.x);
  const int c = chunk_order<Q>(rms, work / ngrp), h0 = (work % ngrp) * hg;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t xstride = CONV ? cv.ch : int64_t(Hs) * P;   // elements per token row of x

  if constexpr (CONV) halo_tokens<Q>(sHtok, rms, c);
  // The token map, then the dt loads, then the chunk's B rows and the first
  // head's x; the prefix sums run while the rows are in flight (1.55 -> 1.53 ms
  // at the minute-length workload; issuing the rows before the dt loads, as
  // the output kernel does, was 1% slower here, where two workgroups share a
  // CU and cover each other's schedule).
  load_chunk_tokens<Q, NTHR>(cs, rms, c);
  ChunkDt<Q, NTHR, kStateHeadGroup> cdt;
  cdt.load(cs, dt, A, Hs, h0, hg);
  if constexpr (CONV) cdt.finish(cs, h0, hg, cv.dt_bias);
  // x of the next head is loaded while the current head is computed.
  StageT<TS, Q, P, NTHR, kLptX> xs;
  RawRows<TS, Q, P, NTHR> xr;
  ConvWeights<P, NTHR> xw;
  auto load_x = [&](int h) {
    if constexpr (CONV) {
      xr.load([&](int j) { return x + int64_t(raw_row_token(cs, sHtok, j)) * xstride + int64_t(h) * P; });
      xw.load(cv, h * P);
    } else {
      xs.load([&](int s) { return x + int64_t(cs.tok[s]) * xstride + int64_t(h) * P; });
    }
  };
  {
    // the hg heads of the workgroup share one B group
    const int g = h0 / (Hs / G);
    if constexpr (CONV) {
      RawRows<TS, Q, N, NTHR> br;
      ConvWeights<N, NTHR> bw;
      const TS* Bg = x + cv.coff_b + int64_t(g) * N;
      br.load([&](int j) { return Bg + int64_t(raw_row_token(cs, sHtok, j)) * cv.ch; });
      bw.load(cv, cv.coff_b + g * N);
      load_x(h0);
      MT* rawB = reinterpret_cast<MT*>(sU);
      br.template store<TRB>(rawB, sHalo, c == 0);
      bw.store(sCw);
      lds_barrier();
      // B^T of the chunk, two positions (a token pair) per unit, the units
      // spread over pairs as in the unfused staging (transposed stores to
      // distinct banks)
      constexpr int UNITS = (Q / 2) * (N / VEC);
#pragma unroll 1
      for (int u = tid; u < UNITS; u += NTHR) {
        const int i = (u / kLptB) % (Q / 2), n0 = ((u / kLptB) / (Q / 2) * kLptB + u % kLptB) * VEC;
        TS o[2][VEC];
        conv_rows<TS, TRB, N, 2>(rawB, sHalo, sCw, 2 * i, n0, o);
#pragma unroll
        for (int e = 0; e < VEC; ++e) st_pair(&sBt[TQ::at(n0 + e, 2 * i)], o[0][e], o[1][e]);
      }
      lds_barrier();   // the raw rows and the weight table are free for x
    } else {
      const TS* Bg = B + int64_t(g) * N;
      StageT<TS, Q, N, NTHR, kLptB> bs;
      bs.load([&](int s) { return Bg + int64_t(cs.tok[s]) * G * N; });
      load_x(h0);
      cdt.finish(cs, h0, hg);
      bs.use([&](int s0, int n0, const Vec16<TS>& va, const Vec16<TS>& vb) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) st_pair(&sBt[TQ::at(n0 + e, s0)], va.e[e], vb.e[e]);
      });
    }
  }

  constexpr int NT = SC::NT, WP = SC::WP, WN = SC::WN, PT_PER = SC::PT_PER, NT_PER = SC::NT_PER;
  const int wp = wave % WP, wn = wave / WP;
  const int r16 = lane & 15, g4 = (lane >> 4) * 4;
  const int64_t per = int64_t(P) * N;
  // Output staging is unpadded [P][N] per direction (chunk-permuted for bf16).
  auto out_at = [](int row, int col) { return TO::kSwz ? TO::at(row, col) : row * N + col; };

#pragma unroll 1
  for (int hh = 0; hh < hg; ++hh) {
    const int h = h0 + hh;
    const float cum_end = cs.cum[hh][Q - 1];
    const float a2 = A[h] * kLog2e;
    // token weights by WeightMode (the weighted x^T of each direction)
    for (int i = CONV ? fresh_tid() : tid; i < Q; i += NTHR) {
      const float d = cs.dt[hh][i];
      const float cum_i = cs.cum[hh][i];
      if constexpr (WM == kWeightAdjoint) {
        sW[0][i] = fast_exp2(cum_end - cum_i + d * a2);   // e^{cum_end - exc_i}
        sW[1][i] = fast_exp2(cum_i);                      // e^{exc_i + a_i}
      } else {
        sW[0][i] = fast_exp2(cum_end - cum_i) * d;
        sW[1][i] = fast_exp2(cum_i - d * a2) * d;     // exc_i = cum_i - a_i
      }
    }
    if (tid == 0) decay[int64_t(c) * Hs + h] = fast_exp2(cum_end);
    if constexpr (CONV) {
      // raw rows of x_h into the second half of sU (free with one direction)
      xr.template store<TRX>(sXb, sHalo, c == 0);
      xw.store(sCw);
    }
    lds_barrier();
    if constexpr (CONV) {
      const int u0 = fresh_tid();
      constexpr int UNITS = (Q / 2) * (P / VEC);
#pragma unroll 1
      for (int u = u0; u < UNITS; u += NTHR) {
        const int i = (u / kLptX) % (Q / 2), p0 = ((u / kLptX) / (Q / 2) * kLptX + u % kLptX) * VEC, s0 = 2 * i;
        TS o[2][VEC];
        conv_rows<TS, TRX, P, 2>(sXb, sHalo, sCw, s0, p0, o);
        const float wf0 = sW[0][s0], wf1 = sW[0][s0 + 1];
#pragma unroll
        for (int e = 0; e < VEC; ++e)
          st_pair_f32(&sXf[TQ::at(p0 + e, s0)], to_f32(o[0][e]) * wf0, to_f32(o[1][e]) * wf1);
      }
    } else {
      xs.use([&](int s0, int p0, const Vec16<TS>& va, const Vec16<TS>& vb) {
        const float wf0 = sW[0][s0], wf1 = sW[0][s0 + 1], wb0 = sW[1][s0], wb1 = sW[1][s0 + 1];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float x0 = to_f32(va.e[e]), x1 = to_f32(vb.e[e]);
          st_pair_f32(&sXf[TQ::at(p0 + e, s0)], x0 * wf0, x1 * wf1);
          if constexpr (BIDIR) st_pair_f32(&sXb[TQ::at(p0 + e, s0)], x0 * wb0, x1 * wb1);
        }
      });
    }
    lds_barrier();
    if (hh + 1 < hg) load_x(h + 1);
    f32x4 accf[PT_PER][NT_PER], accb[PT_PER][NT_PER];
#pragma unroll
    for (int i = 0; i < PT_PER; ++i)
#pragma unroll
      for (int j = 0; j < NT_PER; ++j) {
        accf[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        accb[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int ks = 0; ks < Q / KI; ++ks) {
      typename F::type af[PT_PER], ab[PT_PER];
#pragma unroll
      for (int i = 0; i < PT_PER; ++i) {
        const int pt = wp + i * WP;
        af[i] = TQ::frag(sXf, pt * 16 + r16, ks * KI, lane);
        if constexpr (BIDIR) ab[i] = TQ::frag(sXb, pt * 16 + r16, ks * KI, lane);
      }
#pragma unroll
      for (int j = 0; j < NT_PER; ++j) {
        const int nt = wn + j * WN;
        if (nt < NT) {
          const typename F::type bf = TQ::frag(sBt, nt * 16 + r16, ks * KI, lane);
#pragma unroll
          for (int i = 0; i < PT_PER; ++i) {
            accf[i][j] = mma(af[i], bf, accf[i][j]);
            if constexpr (BIDIR) accb[i][j] = mma(ab[i], bf, accb[i][j]);
          }
        }
      }
    }
    lds_barrier();   // x staging (aliased by the output staging) fully read
#pragma unroll
    for (int i = 0; i < PT_PER; ++i)
#pragma unroll
      for (int j = 0; j < NT_PER; ++j) {
        const int nt = wn + j * WN;
        if (nt < NT) {
          const int pbase = (wp + i * WP) * 16 + g4, n = nt * 16 + r16;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            sOut[out_at(pbase + r, n)] = from_f32<TS>(accf[i][j][r]);
            if constexpr (BIDIR) sOut[per + out_at(pbase + r, n)] = from_f32<TS>(accb[i][j][r]);
          }
        }
      }
    lds_barrier();
    constexpr int VPD = P * N / VEC;   // 16-byte vectors per direction
    for (int u = tid; u < (BIDIR ? 2 : 1) * VPD; u += NTHR) {
      const int dir = u / VPD, off = u % VPD;
      uint4* dst = reinterpret_cast<uint4*>(states + ((int64_t(dir) * n_chunks + c) * Hs + h) * per);
      dst[off] = reinterpret_cast<const uint4*>(sOut)[dir * VPD + out_at(off / (N / VEC), (off % (N / VEC)) * VEC) / VEC];
    }
  }
}

// ---------------------------------------------------------------------------
// State pass: turns chunk states into the state entering each chunk, in
// place.  dir 0 walks chunks upward, dir 1 downward; h0 (review state, fp32,
// or zero) starts both walks.  Each thread owns 8 elements of one head's
// P x N state and carries them in fp32.  h_last (optional, fp32
// [dir][Hs][P][N]) receives the state each walk carries out of its last
// chunk: for the adjoint states of the backward pass, the adjoints of the
// two directions' initial states.
// ---------------------------------------------------------------------------

template <typename TS, int U, int E>
__global__ __launch_bounds__(256) void ssd_state_pass_kernel(TS* __restrict__ states, const float* __restrict__ decay,
                                                             const float* __restrict__ h0, int Hs, int PN,
                                                             int n_chunks, float* __restrict__ h_last) {
  // E elements per thread (16-byte accesses for bf16 at E = 8), U chunks'
  // loads in flight.  A block (blockDim.x threads, dividing PN/E) covers
  // consecutive elements of one head, so the head index and its chunk
  // decays are wave-uniform.  Every state is read and written exactly once,
  // so the accesses are marked non-temporal (they need not stay in cache).
  using VT = TS __attribute__((ext_vector_type(E)));
  const int dir = blockIdx.y;
  const int blocks_per_head = (PN / E) / int(blockDim.x);
  const int h = __builtin_amdgcn_readfirstlane(int(blockIdx.x) / blocks_per_head);
  const int64_t ev = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  float hv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) hv[e] = h0 ? h0[ev * E + e] : 0.f;
  const int64_t cstride = int64_t(Hs) * PN / E;
  VT* base = reinterpret_cast<VT*>(states) + int64_t(dir) * n_chunks * cstride + ev;
  const float* dec = decay + h;
  for (int step = 0; step < n_chunks; step += U) {
    VT buf[U];
    float g[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = step + u;
      if (k < n_chunks) {
        const int c = dir ? n_chunks - 1 - k : k;
        buf[u] = __builtin_nontemporal_load(&base[int64_t(c) * cstride]);
        g[u] = dec[int64_t(c) * Hs];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = step + u;
      if (k < n_chunks) {
        const int c = dir ? n_chunks - 1 - k : k;
        VT o;
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = from_f32<TS>(hv[e]);
        __builtin_nontemporal_store(o, &base[int64_t(c) * cstride]);
#pragma unroll
        for (int e = 0; e < E; ++e) hv[e] = g[u] * hv[e] + to_f32(buf[u][e]);
      }
    }
  }
  if (h_last) {
#pragma unroll
    for (int e = 0; e < E; ++e) h_last[int64_t(dir) * Hs * PN + ev * E + e] = hv[e];
  }
}

// Scan states in the workspace -> fp32 output (lingen_ssd_chunk_states).
template <typename TS>
__global__ __launch_bounds__(256) void states_to_f32_kernel(const TS* __restrict__ src, float* __restrict__ dst,
                                                            int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) dst[i] = to_f32(src[i]);
}

// ---------------------------------------------------------------------------
// Phase B: chunk outputs.  One workgroup per (chunk, group of heads); wave w
// owns output positions t of t-tile w.  Per chunk (head independent):
//   G^T[s][t] = B_s . C_t   (MFMA, fragments straight from global memory)
// and the C_t fragments are kept in registers.  Per head:
//   M^T[s][t] = G^T[s][t] Lambda[t,s] dt_s        (registers)
//   Y^T[p][t] = sum_s x_s[p] M^T[s][t]             (MFMA, k = s)
//             + e^{cum_t}         sum_n Hf[p][n] C_t[n]
//             + e^{cum_end-exc_t} sum_n Hb[p][n] C_t[n]
//             + 2 D x_t[p]
// and y[canon(t)][h*P + p] = Y^T[p][t].
// ---------------------------------------------------------------------------

template <typename TS, int P, int N, int Q>
struct OutCfg {
  static constexpr int QT = Q / 16, PT = P / 16;
  static constexpr int NW = QT >= 8 ? 8 : 4;               // waves per workgroup
  static constexpr int WT = NW < QT ? NW : QT;              // waves along t
  static constexpr int WPW = NW / WT;                       // waves along p
  static constexpr int P_PER = (PT + WPW - 1) / WPW;
  static_assert(QT <= NW, "one t-tile per wave");
};

// BIDIR = false: the forward direction alone (lower triangle and diagonal
// weight 1, the forward inter-chunk term, D x once), for a scan whose
// backward direction has parameters of its own; ACC adds the result to y.
// With bf16 storage the one-direction passes also use ylo (laid out like y):
// the first pass (ACC = false) writes its fp32 result v as y = bf16(v) and
// ylo = bf16(v - y), and the second pass (ACC = true) adds y + ylo, so the
// first direction's result reaches the sum with about 16 significant bits
// instead of 8 (where the two directions nearly cancel, a rounded first
// term would dominate the error of the row).
// UNIT: no dt factor on the tokens (the input carries its own token
// weights), and no skip term (D is not read).
// TRANS (with BIDIR and UNIT): the transposed scan (M_f^T + M_b^T) u of the
// bidirectional one, which the backward pass needs: pairs s < t decay by
// e^{exc_t - exc_s} and pairs s > t by e^{cum_s - cum_t} (the roles of the
// inclusive and exclusive prefix sums exchanged), the entering states apply
// e^{exc_t} and e^{cum_end - cum_t}, and the caller exchanges B and C and
// passes the states of u with the adjoint token weights (kWeightAdjoint),
// whose chunk-local weights e^{cum_end - exc_s} and e^{cum_s} are exactly
// the transposed scan's.
// CONV (one direction): x, B and C are the convolved xBC channels (x, B and
// C all point at the xBC rows; cv gives the convolution and dt_bias).
template <typename TS, int P, int N, int Q, bool BIDIR = true, bool ACC = false, bool UNIT = false,
          bool TRANS = false, bool CONV = false>
__global__ __launch_bounds__((OutCfg<TS, P, N, Q>::NW * 64)) void ssd_chunk_out_kernel(
    const TS* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A, const TS* __restrict__ B,
    const TS* __restrict__ C, const float* __restrict__ D, RmsMap rms, int Hs, int G, int hg, int n_chunks,
    const TS* __restrict__ states, TS* __restrict__ y, TS* __restrict__ ylo, ConvIn cv) {
  using MT = TS;
  using F = Frag<MT>;
  using Cfg = OutCfg<TS, P, N, Q>;
  static_assert(!TRANS || (BIDIR && UNIT), "the transposed scan is bidirectional with unit token weights");
  constexpr int NTHR = Cfg::NW * 64;
  constexpr int KI = F::K;
  using TN = Tile<MT, N>;     // rows of N: B rows and the entering states
  constexpr int NP = TN::LD;
  constexpr int VEC = Vec16<TS>::n;
  constexpr bool kBf16 = std::is_same<MT, __bf16>::value;
  static_assert((N % KI == 0 && Q % 32 == 0) || !kBf16, "bf16 tiles need Q multiple of 32");
  // One LDS region, used first for the B rows of the chunk (to form G^T)
  // and then, per head, for x (row-major [Q][P], read transposed for the
  // MFMA A operand) and the two entering states.
  using TX = KvTile<MT, P>;
  constexpr int HEAD_ELEMS = Q * P + 2 * P * NP;
  constexpr int U_ELEMS = HEAD_ELEMS > Q * NP ? HEAD_ELEMS : Q * NP;
  __shared__ __attribute__((aligned(16))) MT sU[U_ELEMS];
  MT* sX = sU;
  MT* sHf = sX + Q * P;
  MT* sHb = sHf + P * NP;
  MT* sBr = sU;
  __shared__ ChunkSched<Q> cs;
  __shared__ __attribute__((aligned(16))) float sV[Cfg::NW][Q];   // per-wave decay factors of s
  // CONV: raw rows of the chunk (B, then C, then each head's x), the halo
  // rows and the weight table.
  static_assert(!CONV || (!BIDIR && !UNIT && !TRANS && kBf16), "fused steps: one direction, bf16");
  constexpr int CW = N > P ? N : P;
  __shared__ __attribute__((aligned(16))) MT sRaw[CONV ? Q * CW : 1];
  __shared__ __attribute__((aligned(16))) MT sHalo[CONV ? kConvHalo * CW : 1];
  __shared__ __attribute__((aligned(16))) float sCw[CONV ? kConvW * CW : 1];
  __shared__ int sHtok[kConvHalo];
  using TRN = Tile<MT, N>;   // raw B and C rows
  using TRX = Tile<MT, P>;   // raw x rows
  constexpr int RB = Q * (N / VEC) / NTHR, RX = Q * (P / VEC) / NTHR;   // conv rows per thread
  static_assert(!CONV || (RB * NTHR == Q * (N / VEC) && RX * NTHR == Q * (P / VEC) && NTHR % (N / VEC) == 0 &&
                          NTHR % (P / VEC) == 0), "conv rows tile the chunk");

  const int ngrp = Hs / hg;
  const int work = xcd_work_id(blockIdx.x, gridDim.x);
  const int c = chunk_order<Q>(rms, work / ngrp), h0 = (work % ngrp) * hg;
  // The wave index as a scalar in [0, NW): the tests on the wave's t-tile
  // (the diagonal M^T tile, the p-tiles it owns) are then branches of the
  // whole wave rather than per-lane masks.
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6) & (Cfg::NW - 1);
  const int r16 = lane & 15, grp = lane >> 4;
  const int64_t xstride = CONV ? cv.ch : int64_t(Hs) * P;   // elements per token row of x
  const int64_t bstride = CONV ? cv.ch : int64_t(G) * N;    // ... of B and C

  if constexpr (CONV) halo_tokens<Q>(sHtok, rms, c);
  // The token map first; the first head's x and states and the chunk's B and
  // C rows are issued before the dt loads and prefix sums, so that they are in
  // flight while the schedule forms (one workgroup per CU: nothing else covers
  // the prologue).  Measured: 2.20 -> 2.03 ms at the minute-length workload.
  // Issuing the dt loads first and waiting for them alone was slower (2.17 ms):
  // their addresses need the token map from LDS, which delays the row loads.
  load_chunk_tokens<Q, NTHR>(cs, rms, c);

  // x and the two entering states of the next head are loaded while the
  // current head is computed.
  const int64_t per = int64_t(P) * N;
  struct HeadBuf {
    Stage16<Q * (P / VEC), NTHR> xs;
    RawRows<TS, Q, P, NTHR> xr;
    ConvWeights<P, NTHR> xw;
    Stage16<P * (N / VEC), NTHR> hfs, hbs;
  };
  HeadBuf buf0;
  auto load_head = [&](HeadBuf& hb_, int h) {
    // Consecutive lanes take consecutive 16-byte pieces of one token row, so
    // one load instruction touches few rows (and pages) even when the scan
    // order puts consecutive tokens far apart.
    if constexpr (CONV) {
      hb_.xr.load([&](int j) { return x + int64_t(raw_row_token(cs, sHtok, j)) * xstride + int64_t(h) * P; });
      hb_.xw.load(cv, h * P);
    } else {
      hb_.xs.load([&](int u) {
        return *reinterpret_cast<const uint4*>(x + int64_t(cs.tok[u / (P / VEC)]) * xstride + int64_t(h) * P +
                                               (u % (P / VEC)) * VEC);
      });
    }
    const uint4* hf = reinterpret_cast<const uint4*>(states + (int64_t(c) * Hs + h) * per);
    const uint4* hb = reinterpret_cast<const uint4*>(states + ((int64_t(n_chunks) + c) * Hs + h) * per);
    hb_.hfs.load([&](int u) { return hf[u]; });
    if constexpr (BIDIR) hb_.hbs.load([&](int u) { return hb[u]; });
  };
  load_head(buf0, h0);

  const int wt = wave % Cfg::WT, wpw = wave / Cfg::WT;
  const int t = wt * 16 + r16;            // this lane's output position
  const int64_t tok_t = cs.tok[t];
  // the hg heads of the workgroup share one B, C group
  const int grp_bc = h0 / (Hs / G);
  const TS* Bg = (CONV ? x + cv.coff_b : B) + int64_t(grp_bc) * N;
  const TS* Cg = (CONV ? x + cv.coff_c : C) + int64_t(grp_bc) * N;
  // C_t fragments (B operand, k = n) for the inter-chunk terms, and G^T.
  typename F::type cfr[N / KI];
  // G^T is accumulated in fp32 and kept in the operand type (bf16 for bf16
  // data: the M^T values built from it are rounded to bf16 anyway).
  using GT = typename std::conditional<kBf16, bf16x4, f32x4>::type;
  // The B rows of the chunk are staged once (coalesced, row-major) and every
  // wave reads its MFMA fragments from LDS.
  if constexpr (CONV) {
    load_chunk_dt<Q, NTHR>(cs, dt, A, Hs, h0, hg, cv.dt_bias);
    // Raw B and C rows (with the halo) and their weights are fetched
    // together; B is convolved into sBr by whole tiles (each thread one
    // column piece over RB consecutive rows), C straight into each lane's
    // fragments.
    RawRows<TS, Q, N, NTHR> br, cr;
    ConvWeights<N, NTHR> bw, cw;
    auto rows_of = [&](const TS* base) {
      return [&, base](int j) { return base + int64_t(raw_row_token(cs, sHtok, j)) * bstride; };
    };
    br.load(rows_of(Bg));
    bw.load(cv, cv.coff_b + grp_bc * N);
    cr.load(rows_of(Cg));
    cw.load(cv, cv.coff_c + grp_bc * N);
    br.template store<TRN>(sRaw, sHalo, c == 0);
    bw.store(sCw);
    lds_barrier();
    {
      constexpr int PR = N / VEC;
      const int col = (tid % PR) * VEC, s0 = (tid / PR) * RB;
      TS o[RB][VEC];
      conv_rows<TS, TRN, N, RB>(sRaw, sHalo, sCw, s0, col, o);
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        Vec16<TS> v;
#pragma unroll
        for (int e = 0; e < VEC; ++e) v.e[e] = o[r][e];
        *reinterpret_cast<uint4*>(&sBr[TN::at(s0 + r, col)]) = v.u;
      }
    }
    lds_barrier();
    cr.template store<TRN>(sRaw, sHalo, c == 0);
    cw.store(sCw);
    lds_barrier();
#pragma unroll
    for (int ks = 0; ks < N / KI; ++ks) {
      TS o[1][VEC];
      conv_rows<TS, TRN, N, 1>(sRaw, sHalo, sCw, t, ks * KI + (lane >> 4) * VEC, o);
#pragma unroll
      for (int e = 0; e < VEC; ++e) cfr[ks][e] = o[0][e];
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < N / KI; ++ks) cfr[ks] = F::load(Cg + tok_t * bstride + ks * KI, lane);
    Stage16<Q * (N / VEC), NTHR> bs;
    bs.load([&](int u) {
      return *reinterpret_cast<const uint4*>(Bg + int64_t(cs.tok[u / (N / VEC)]) * bstride + (u % (N / VEC)) * VEC);
    });
    load_chunk_dt<Q, NTHR>(cs, dt, A, Hs, h0, hg);
    bs.use([&](int u, uint4 raw) {
      *reinterpret_cast<uint4*>(&sBr[TN::at(u / (N / VEC), (u % (N / VEC)) * VEC)]) = raw;
    });
  }
  lds_barrier();
  GT g[Cfg::QT];
#pragma unroll
  for (int st = 0; st < Cfg::QT; ++st) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < N / KI; ++ks) acc = mma(TN::frag(sBr, st * 16 + r16, ks * KI, lane), cfr[ks], acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) g[st][r] = from_f32<MT>(acc[r]);
  }
  lds_barrier();   // the region now takes the per-head staging

  auto do_head = [&](int hh, HeadBuf& buf) {
    const int h = h0 + hh;
    // Stage x_h and the two entering states of this head.
    if constexpr (CONV) {
      buf.xr.template store<TRX>(sRaw, sHalo, c == 0);
      buf.xw.store(sCw);
    } else {
      buf.xs.use([&](int u, uint4 raw) {
        *reinterpret_cast<uint4*>(&sX[TX::at(u / (P / VEC), (u % (P / VEC)) * VEC)]) = raw;
      });
    }
    buf.hfs.use([&](int u, uint4 raw) {
      *reinterpret_cast<uint4*>(&sHf[TN::at(u / (N / VEC), (u % (N / VEC)) * VEC)]) = raw;
    });
    if constexpr (BIDIR)
      buf.hbs.use([&](int u, uint4 raw) {
        *reinterpret_cast<uint4*>(&sHb[TN::at(u / (N / VEC), (u % (N / VEC)) * VEC)]) = raw;
      });
    // Off the wave's own t-tile [ts, te] the decay splits at the tile edge
    // into two factors that are both <= 1:
    //   s < ts: e^{cum_t - cum_s}  = e^{cum_t - exc_ts} * e^{exc_ts - cum_s}
    //   s > te: e^{exc_s - exc_t}  = e^{cum_te - exc_t} * e^{exc_s - cum_te}
    // The s-side factor (times dt_s) goes to sV; the t-side one stays in a
    // register, so each off-diagonal element costs two multiplies.
    {
      const float* cum = cs.cum[hh];
      const float* exc = cs.exc[hh];
      const int ts = wt * 16, te = ts + 15;
      const float ref_lo = exc[ts], ref_hi = cum[te];
      for (int s = lane; s < Q; s += 64) {
        float vs = 0.f;
        const float w = UNIT ? 1.f : cs.dt[hh][s];
        // (TRANS: the same references, the other prefix sum at s)
        if (s < ts) vs = fast_exp2(ref_lo - (TRANS ? exc[s] : cum[s])) * w;
        else if (s > te) vs = fast_exp2((TRANS ? cum[s] : exc[s]) - ref_hi) * w;
        sV[wave][s] = vs;
      }
    }
    lds_barrier();
    if (hh + 1 < hg) load_head(buf, h + 1);
    if constexpr (CONV) {
      // x_h from its raw rows: each thread one column piece over RX
      // consecutive rows
      constexpr int PR = P / VEC;
      const int u0 = fresh_tid();
      const int col = (u0 % PR) * VEC, s0 = (u0 / PR) * RX;
      TS o[RX][VEC];
      conv_rows<TS, TRX, P, RX>(sRaw, sHalo, sCw, s0, col, o);
#pragma unroll
      for (int r = 0; r < RX; ++r) {
        Vec16<TS> v;
#pragma unroll
        for (int e = 0; e < VEC; ++e) v.e[e] = o[r][e];
        *reinterpret_cast<uint4*>(&sX[TX::at(s0 + r, col)]) = v.u;
      }
      lds_barrier();
    }

    const float* cum = cs.cum[hh];
    const float* exc = cs.exc[hh];
    const float* dth = cs.dt[hh];
    const float cum_t = cum[t], exc_t = exc[t];
    const float fac_lo = fast_exp2((TRANS ? exc_t : cum_t) - exc[wt * 16]);   // t-side factor, s before the tile
    const float fac_hi = fast_exp2(cum[wt * 16 + 15] - (TRANS ? cum_t : exc_t));   // t-side factor, s after the tile

    // M^T values of this lane for s-tile st (s = 16*st + 4*grp + r).  On the
    // diagonal tile: s < t forward decay e^{cum_t - cum_s}, s > t backward
    // decay e^{exc_s - exc_t}, s = t both directions see the token (weight 2).
    auto m_tile = [&](int st, float (&mv)[4]) {
      const int sb = st * 16 + grp * 4;
      if (st == wt) {
        const float4 cum4 = *reinterpret_cast<const float4*>(&cum[sb]);
        const float4 exc4 = *reinterpret_cast<const float4*>(&exc[sb]);
        const float4 dt4 = *reinterpret_cast<const float4*>(&dth[sb]);
        const float cv[4] = {cum4.x, cum4.y, cum4.z, cum4.w};
        const float xv[4] = {exc4.x, exc4.y, exc4.z, exc4.w};
        const float dv[4] = {dt4.x, dt4.y, dt4.z, dt4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s = sb + r;
          const float arg = TRANS ? (s < t ? exc_t - xv[r] : cv[r] - cum_t) : (s < t ? cum_t - cv[r] : xv[r] - exc_t);
          const float lam = s == t ? (BIDIR ? 2.f : 1.f) : (BIDIR || s < t ? fast_exp2(arg) : 0.f);
          mv[r] = to_f32(g[st][r]) * lam * (UNIT ? 1.f : dv[r]);
        }
      } else {
        const float4 v4 = *reinterpret_cast<const float4*>(&sV[wave][sb]);
        const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
        const float fac = st < wt ? fac_lo : (BIDIR ? fac_hi : 0.f);
#pragma unroll
        for (int r = 0; r < 4; ++r) mv[r] = to_f32(g[st][r]) * vv[r] * fac;
      }
    };

    // Intra-chunk term, s-tiles outermost so one M^T pair is live at a time.
    f32x4 acc[Cfg::P_PER];
#pragma unroll
    for (int pj = 0; pj < Cfg::P_PER; ++pj) acc[pj] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (kBf16) {
      // k = s in pairs of s-tiles: lane group g covers s = 32k + 4g + {0..3}
      // and 32k + 16 + 4g + {0..3}, matching the M^T values it holds.
#pragma unroll
      for (int k2 = 0; k2 < Cfg::QT / 2; ++k2) {
        float m0[4], m1[4];
        m_tile(2 * k2, m0);
        m_tile(2 * k2 + 1, m1);
        bf16x8 bm;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          bm[r] = static_cast<__bf16>(m0[r]);
          bm[4 + r] = static_cast<__bf16>(m1[r]);
        }
#pragma unroll
        for (int pj = 0; pj < Cfg::P_PER; ++pj) {
          const int pt = wpw + pj * Cfg::WPW;
          if (pt < Cfg::PT) {
            // x^T fragment (row p = pt*16 + r16) by transposing reads of the
            // row-major tile: lane group g gets s = 32k + 4g + {0..3} and
            // 32k + 16 + 4g + {0..3}.
            lds_bf16* xr = (lds_bf16*)(sX) + TX::at(k2 * 32 + 4 * grp + (r16 >> 2), pt * 16 + 4 * (r16 & 3));
            const bf16x4 lo = lds_read_tr(xr);
            const bf16x4 hi = lds_read_tr(xr + 16 * P);
            acc[pj] = mma(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), bm, acc[pj]);
          }
        }
      }
    } else {
#pragma unroll
      for (int st = 0; st < Cfg::QT; ++st) {
        float mv[4];
        m_tile(st, mv);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int pj = 0; pj < Cfg::P_PER; ++pj) {
            const int pt = wpw + pj * Cfg::WPW;
            if (pt < Cfg::PT)
              acc[pj] = mma(to_f32(sX[TX::at(st * 16 + grp * 4 + r, pt * 16 + r16)]), mv[r], acc[pj]);
          }
      }
    }

    // Inter-chunk terms, the skip, and the store.
    const float ef = fast_exp2(TRANS ? exc_t : cum_t);
    const float eb = BIDIR ? fast_exp2(cum[Q - 1] - (TRANS ? cum_t : exc_t)) : 0.f;
    const float twoD = UNIT ? 0.f : (BIDIR ? 2.f : 1.f) * D[h];
    // bf16 rows of 64 owned by one wave: the four p-tiles are stored together
    // in 16-byte pieces (see below).
    constexpr bool kP16 = kBf16 && Cfg::PT == 4 && Cfg::P_PER == 4 && Cfg::WPW == 1;
    constexpr bool kSplit = kBf16 && !BIDIR;   // hi / lo halves of the one-direction passes (ylo)
    static_assert(!kSplit || kP16, "the split sum is stored in 16-byte pieces");
    float ob[4][4];
#pragma unroll
    for (int pj = 0; pj < Cfg::P_PER; ++pj) {
      const int pt = wpw + pj * Cfg::WPW;
      if (pt >= Cfg::PT) break;
      const int prow = pt * 16 + r16;      // A-operand row of this lane
      f32x4 zf = f32x4{0.f, 0.f, 0.f, 0.f}, zb = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < N / KI; ++ks) {
        zf = mma(TN::frag(sHf, prow, ks * KI, lane), cfr[ks], zf);
        if constexpr (BIDIR) zb = mma(TN::frag(sHb, prow, ks * KI, lane), cfr[ks], zb);
      }
      // Lane holds Y^T[p][t] for p = pt*16 + 4*grp + r.
      const int p0 = pt * 16 + grp * 4;
      float o[4];
      const MT* xt = &sX[TX::at(t, p0)];    // x_t[p0 .. p0+3]
#pragma unroll
      for (int r = 0; r < 4; ++r)
        o[r] = acc[pj][r] + ef * zf[r] + eb * zb[r] + twoD * to_f32(xt[r]);
      if constexpr (kP16) {
#pragma unroll
        for (int r = 0; r < 4; ++r) ob[pj][r] = o[r];
        continue;
      }
      TS* dst = y + tok_t * (int64_t(Hs) * P) + int64_t(h) * P + p0;
      if constexpr (kBf16) {
        bf16x4 ov;
        if constexpr (ACC) {
          const bf16x4 old = *reinterpret_cast<const bf16x4*>(dst);
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] += static_cast<float>(old[r]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) ov[r] = static_cast<__bf16>(o[r]);
        *reinterpret_cast<bf16x4*>(dst) = ov;
      } else {
        if constexpr (ACC) {
          const float4 old = *reinterpret_cast<const float4*>(dst);
          o[0] += old.x; o[1] += old.y; o[2] += old.z; o[3] += old.w;
        }
        *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
      }
    }
    if constexpr (kP16) {
      // Exchange the 4-element pieces of p-tiles 2 r1 and 2 r1 + 1 between
      // lane groups g and g ^ 1 (v_permlane16_swap): the lane then holds
      // p0 .. p0 + 7, p0 = 32 r1 + 16 (g & 1) + 8 (g >> 1), and a wave's
      // 16-byte stores cover 64 contiguous bytes of each row.
      const int64_t roff = tok_t * (int64_t(Hs) * P) + int64_t(h) * P + 16 * (grp & 1) + 8 * (grp >> 1);
      TS* row = y + roff;
#pragma unroll
      for (int r1 = 0; r1 < 2; ++r1) {
        bf16x8 old, oldlo;
        if constexpr (ACC) old = *reinterpret_cast<const bf16x8*>(row + 32 * r1);
        if constexpr (ACC && kSplit) oldlo = *reinterpret_cast<const bf16x8*>(ylo + roff + 32 * r1);
        float v[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(ob[2 * r1][r]),
                                                           __float_as_uint(ob[2 * r1 + 1][r]), false, false);
          v[r] = __uint_as_float(sw[0]);
          v[4 + r] = __uint_as_float(sw[1]);
        }
        if constexpr (ACC) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            v[e] += static_cast<float>(old[e]);
            if constexpr (kSplit) v[e] += static_cast<float>(oldlo[e]);
          }
        }
        bf16x8 res, rlo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          res[e] = static_cast<__bf16>(v[e]);
          rlo[e] = static_cast<__bf16>(v[e] - static_cast<float>(res[e]));
        }
        *reinterpret_cast<bf16x8*>(row + 32 * r1) = res;
        if constexpr (kSplit && !ACC) *reinterpret_cast<bf16x8*>(ylo + roff + 32 * r1) = rlo;
      }
    }
    lds_barrier();   // staging buffers free for the next head
  };
#pragma unroll 1
  for (int hh = 0; hh < hg; ++hh) do_head(hh, buf0);
}

// ---------------------------------------------------------------------------
// TESA.  Windows are enumerated on the rolled grid (offset by the shift,
// wrapping), so every window has n_w tokens; a token that wrapped along an
// axis belongs to a different window of the unrolled partition than one
// that did not, which the kernel enforces by masking scores between tokens
// of different wrap classes.  This is the border-cut partition of page
// "LinGen：基于Mamba机制的线性复杂度高清长视频生成框架", section 关键算法创新 >
// TESA (plain and shifted windows alternate), in Swin's roll-and-mask form.
// Windows with no wrapped token skip the mask.  With masking off the same
// enumeration gives the cyclic reading of shifted windows (wrapped tokens
// join the window they rolled into).  Window sizes that are not a multiple
// of 32 tokens (3x3x3 on the same page) are padded to the next 32 slots.
//
// Work item = (window, head).  The grid is persistent (one workgroup per
// CU for 256-token windows); a workgroup walks its items in sequence with the K and V tiles of the
// next item streaming into the second of two LDS buffers (direct
// global-to-LDS loads, no registers) while the current one is computed, and
// the next item's Q fragments in registers.  Per item and block of 64 keys
// (32 for fp32):
//   S^T[j][i] = K_j . Q_i            (MFMA, A = K from LDS, B = Q in registers)
//   m_i <- max(m_i, max_j S[i][j])   (running maximum; each lane owns one query)
//   P^T = 2^((S^T - m) log2(e)/sqrt(d)); output and row sums rescaled by
//         2^(m_old - m_new) and accumulated:
//   O^T[e][i] += V^T[e][j] P^T[j][i] (MFMA, B = P^T in registers; A = V^T
//         read from the row-major V tile with LDS transpose loads)
// ---------------------------------------------------------------------------

template <typename TS, int DH, int NWIN>
struct AttnCfg {
  static constexpr int QTILES = NWIN / 16;
  static constexpr int NWAVE = QTILES >= 16 ? 16 : QTILES;
  static constexpr int QT_PER = QTILES / NWAVE;       // query tiles per wave
  static constexpr int VEC = 16 / int(sizeof(TS));     // elements per 16-byte chunk
  static constexpr int CPR = DH / VEC;                 // chunks per K / V row
  static constexpr int UNITS = NWIN * CPR;             // 16-byte chunks per tile
  static constexpr int DMA_PER_WAVE = UNITS / (NWAVE * 64);
  static_assert(CPR == 8, "K / V rows of 128 bytes");
  static_assert(UNITS % (NWAVE * 64) == 0, "whole wave-wide LDS loads per tile");
};

// NVALID = wt*wh*ww tokens of a window occupy the first NVALID of NWIN slots;
// the remaining slots (odd window sizes) repeat the window's first token, and
// their keys are masked and their query rows not stored.
template <typename TS, int DH, int NWIN, int NVALID, bool ACCUMULATE>
__global__ __launch_bounds__((AttnCfg<TS, DH, NWIN>::NWAVE * 64)) void tesa_window_kernel(
    const TS* __restrict__ q, const TS* __restrict__ k, const TS* __restrict__ v, WinGeom wg, int Ha,
    int n_items, TS* __restrict__ y) {
  using MT = TS;
  using F = Frag<MT>;
  using Cfg = AttnCfg<TS, DH, NWIN>;
  using KT = KvTile<TS, DH>;
  constexpr int NTHR = Cfg::NWAVE * 64;
  constexpr int QTP = Cfg::QT_PER;
  constexpr int KI = F::K;
  constexpr int VEC = Cfg::VEC;
  constexpr bool kBf16 = std::is_same<MT, __bf16>::value;
  constexpr int ET = DH / 16;
  constexpr int NKS = DH / KI;
  static_assert(NWIN % 32 == 0 && DH % 16 == 0 && DH % KI == 0, "attention tile shape");
  // Two buffers per tile, as separate arrays so that reads of the current
  // buffer need not wait for the loads streaming into the other one.
  __shared__ __attribute__((aligned(16))) MT sK0[NWIN * DH];
  __shared__ __attribute__((aligned(16))) MT sK1[NWIN * DH];
  __shared__ __attribute__((aligned(16))) MT sV0[NWIN * DH];
  __shared__ __attribute__((aligned(16))) MT sV1[NWIN * DH];
  __shared__ int sTok[2][NWIN];   // token index of each window slot (item parity)
  __shared__ int sCls[3][NWIN];   // wrap class of each window slot (item mod 3)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, grp = lane >> 4;
  const int64_t rowstride = int64_t(Ha) * DH;
  const int nwin_hw = wg.nwh * wg.nww;
  // scores stay in raw units; p = 2^((s - max) * sc) with sc = log2(e)/sqrt(d)
  const float sc = kLog2e * rsqrtf(float(DH));

  // Position of an item: head and window coordinates.  Items advance by the
  // grid size, which is added in mixed radix (no divisions per item).
  struct ItemPos { int item, h, wi, wj, wk; };
  auto decompose = [&](int it) {
    const int win = it / Ha;
    return ItemPos{it, it % Ha, win / nwin_hw, (win / wg.nww) % wg.nwh, win % wg.nww};
  };
  const ItemPos step_pos = decompose(int(gridDim.x));   // item offset of one step, as (h, wi, wj, wk)
  auto advance = [&](ItemPos p) {
    p.item += int(gridDim.x);
    p.h += step_pos.h;
    int c = p.h >= Ha;
    if (c) p.h -= Ha;
    p.wk += step_pos.wk + c;
    c = p.wk >= wg.nww;
    if (c) p.wk -= wg.nww;
    p.wj += step_pos.wj + c;
    c = p.wj >= wg.nwh;
    if (c) p.wj -= wg.nwh;
    p.wi += step_pos.wi + c;
    return p;
  };
  // Offsets of this thread's window slot (tid < NWIN) inside the window.
  static_assert(NWIN <= NTHR, "one window slot per thread");
  static_assert(NVALID <= NWIN && NVALID > NWIN - 32, "padding below one 32-key block");
  constexpr bool kPadded = NVALID < NWIN;
  const int slot = tid < NVALID ? tid : 0;
  const int slot_a = slot / (wg.wh * wg.ww), slot_b = (slot / wg.ww) % wg.wh, slot_c = slot % wg.ww;
  // Token index and wrap class of every slot of an item's window.
  auto item_tokens = [&](const ItemPos& p, int* tok, int* cls) {
    if (tid < NWIN) {
      int cl;
      tok[tid] = window_token(wg, p.wi, p.wj, p.wk, slot_a, slot_b, slot_c, cl);
      // Class 8 (padding) matches no query of the window; cyclic windows
      // (masking off) put every real slot in class 0.
      cls[tid] = (kPadded && tid >= NVALID) ? 8 : (wg.masked ? cl : 0);
    }
  };
  auto item_wrapped = [&](const ItemPos& p) { return window_wrapped(wg, p.wi, p.wj, p.wk); };
  // Direct global-to-LDS loads of an item's K and V tiles.
  auto issue_kv = [&](MT* dK, MT* dV, const int* tok, int h) {
#pragma unroll
    for (int d = 0; d < Cfg::DMA_PER_WAVE; ++d) {
      const int base = (wave * Cfg::DMA_PER_WAVE + d) * 64;    // first chunk of this instruction
      const int u = base + lane, row = u / Cfg::CPR, ch = (u % Cfg::CPR) ^ (row & 7);
      const int64_t goff = int64_t(tok[row]) * rowstride + int64_t(h) * DH + ch * VEC;
      lds_load16(k + goff, dK + base * VEC);
      lds_load16(v + goff, dV + base * VEC);
    }
  };
  using YV = typename std::conditional<kBf16, bf16x4, f32x4>::type;
  // bf16 rows of 64: y is read and written in 16-byte pieces (see the epilogue)
  constexpr bool kY16 = kBf16 && ET == 4;
  const int y16_off = 16 * (grp & 1) + 8 * (grp >> 1);
  // Per-lane registers of an item, loaded one item ahead: Q fragments and
  // the query tokens.
  struct QState {
    typename F::type qf[QTP][NKS];
    int tokq[QTP];
  };
  auto load_q = [&](QState& qs, const int* tok, int h) {
#pragma unroll
    for (int qi = 0; qi < QTP; ++qi) {
      const int iq = (wave + qi * Cfg::NWAVE) * 16 + r16;
      qs.tokq[qi] = tok[iq];
      const TS* qrow = q + int64_t(qs.tokq[qi]) * rowstride + int64_t(h) * DH;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qs.qf[qi][ks] = F::load(qrow + ks * KI, lane);
    }
  };

  if (int(blockIdx.x) >= n_items) return;
  ItemPos pos = decompose(int(blockIdx.x));
  item_tokens(pos, sTok[0], sCls[0]);
  lds_barrier();
  QState nxt;
  issue_kv(sK0, sV0, sTok[0], pos.h);
  load_q(nxt, sTok[0], pos.h);

  // Per-lane LDS offsets of the operand fragments in rows 0..15 of a tile.
  // A fragment 8m rows further down is m*8*DH elements further on (the
  // chunk permutation repeats every 8 rows), a compile-time offset.
  int offk[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) offk[ks] = KT::at(r16, ks * KI + grp * (kBf16 ? 8 : 1));
  int offv[kBf16 ? ET : 1];
  if constexpr (kBf16) {
#pragma unroll
    for (int et = 0; et < ET; ++et) offv[et] = KT::at(4 * grp + (r16 >> 2), et * 16 + 4 * (r16 & 3));
  }

  // One item whose K / V tiles are in (cK, cV); the next item's go to (nK, nV).
  auto step = [&](int n, const MT* cK, const MT* cV, MT* nK, MT* nV) -> bool {
    const int h = pos.h;
    const ItemPos npos = advance(pos);
    const bool has_next = npos.item < n_items;
    if (has_next) item_tokens(npos, sTok[(n + 1) & 1], sCls[(n + 1) % 3]);
    wait_vmem();        // this wave's loads for the item (and earlier stores) are done
    lds_barrier();      // ... and every wave's; the other buffers are free
    const QState cur = nxt;
    if (has_next) {
      issue_kv(nK, nV, sTok[(n + 1) & 1], npos.h);
      load_q(nxt, sTok[(n + 1) & 1], npos.h);
    }
    // The MA output this item adds to (fused branch sum) arrives while the
    // two passes run.
    YV yp[QTP][ET];
    bf16x8 yq[QTP][2];
    if constexpr (ACCUMULATE && kY16) {
#pragma unroll
      for (int qi = 0; qi < QTP; ++qi) {
        const TS* yrow = y + int64_t(cur.tokq[qi]) * rowstride + int64_t(h) * DH + y16_off;
#pragma unroll
        for (int r1 = 0; r1 < 2; ++r1) yq[qi][r1] = *reinterpret_cast<const bf16x8*>(yrow + 32 * r1);
      }
    } else if constexpr (ACCUMULATE) {
#pragma unroll
      for (int qi = 0; qi < QTP; ++qi) {
        const TS* yrow = y + int64_t(cur.tokq[qi]) * rowstride + int64_t(h) * DH;
#pragma unroll
        for (int et = 0; et < ET; ++et) yp[qi][et] = *reinterpret_cast<const YV*>(yrow + et * 16 + grp * 4);
      }
    }
    const bool wrapped = kPadded || (wg.masked && item_wrapped(pos));
    const int* cls = sCls[n % 3];
    int qcls[QTP];
#pragma unroll
    for (int qi = 0; qi < QTP; ++qi) qcls[qi] = cls[(wave + qi * Cfg::NWAVE) * 16 + r16];

    // One pass over the key blocks with a running maximum per query: the
    // block's scores are exponentiated against max(running, block) and the
    // earlier output and sums are rescaled when the maximum grows.
    float msc[QTP];
    f32x4 o[QTP][ET];
    float l[QTP];
#pragma unroll
    for (int qi = 0; qi < QTP; ++qi) {
      msc[qi] = -INFINITY;
      l[qi] = 0.f;
#pragma unroll
      for (int et = 0; et < ET; ++et) o[qi][et] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    constexpr int SB = (kBf16 && NWIN % 64 == 0) ? 2 : 1;     // 32-key sub-blocks per block
#pragma unroll 1
    for (int jb = 0; jb < NWIN; jb += 32 * SB) {
#pragma unroll
      for (int qi = 0; qi < QTP; ++qi) {
        f32x4 s[SB][2];
#pragma unroll
        for (int sb = 0; sb < SB; ++sb) {
          const MT* kb = cK + jb * DH;
#pragma unroll
          for (int jt = 0; jt < 2; ++jt) {
            s[sb][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
              typename F::type kf;
              const MT* kp = kb + offk[ks] + (32 * sb + 16 * jt) * DH;
              if constexpr (kBf16) kf = *reinterpret_cast<const bf16x8*>(kp);
              else kf = *kp;
              s[sb][jt] = mma(kf, cur.qf[qi][ks], s[sb][jt]);
            }
          }
          if (wrapped) {
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) {
              const int4 kc = *reinterpret_cast<const int4*>(&cls[jb + 32 * sb + jt * 16 + grp * 4]);
              const int kcv[4] = {kc.x, kc.y, kc.z, kc.w};
#pragma unroll
              for (int r = 0; r < 4; ++r) s[sb][jt][r] = kcv[r] != qcls[qi] ? -INFINITY : s[sb][jt][r];
            }
          }
        }
        float bm = -INFINITY;
#pragma unroll
        for (int sb = 0; sb < SB; ++sb)
          bm = fmaxf(bm, fmaxf(fmaxf(fmaxf(s[sb][0][0], s[sb][0][1]), fmaxf(s[sb][0][2], s[sb][0][3])),
                               fmaxf(fmaxf(s[sb][1][0], s[sb][1][1]), fmaxf(s[sb][1][2], s[sb][1][3]))));
        bm = max_rows(bm);
        const float mnew = fmaxf(msc[qi], bm * sc);
        const float mref = mnew == -INFINITY ? 0.f : mnew;
        const float alpha = fast_exp2(msc[qi] - mref);
        msc[qi] = mnew;
        float lsum = 0.f;
#pragma unroll
        for (int sb = 0; sb < SB; ++sb)
#pragma unroll
          for (int jt = 0; jt < 2; ++jt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float p = fast_exp2(fmaf(s[sb][jt][r], sc, -mref));
              s[sb][jt][r] = p;
              lsum += p;
            }
        l[qi] = fmaf(l[qi], alpha, lsum);
#pragma unroll
        for (int et = 0; et < ET; ++et)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[qi][et][r] *= alpha;
#pragma unroll
        for (int sb = 0; sb < SB; ++sb) {
          if constexpr (kBf16) {
            bf16x8 pb;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              pb[r] = static_cast<__bf16>(s[sb][0][r]);
              pb[4 + r] = static_cast<__bf16>(s[sb][1][r]);
            }
            lds_bf16* vb = (lds_bf16*)(cV) + jb * DH;
#pragma unroll
            for (int et = 0; et < ET; ++et) {
              const bf16x4 lo = lds_read_tr(vb + offv[et] + (32 * sb) * DH);
              const bf16x4 hi = lds_read_tr(vb + offv[et] + (32 * sb + 16) * DH);
              o[qi][et] = mma(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pb, o[qi][et]);
            }
          } else {
#pragma unroll
            for (int jt = 0; jt < 2; ++jt)
#pragma unroll
              for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int et = 0; et < ET; ++et) {
                  const float av = to_f32(cV[KT::at(jb + jt * 16 + grp * 4 + r, et * 16 + r16)]);
                  o[qi][et] = mma(av, s[sb][jt][r], o[qi][et]);
                }
          }
        }
      }
    }

#pragma unroll
    for (int qi = 0; qi < QTP; ++qi) {
      float lt = l[qi];
      lt = sum_rows(lt);
      const float inv = __builtin_amdgcn_rcpf(lt);
      if (kPadded && (wave + qi * Cfg::NWAVE) * 16 + r16 >= NVALID) continue;   // padding slot
      TS* yrow = y + int64_t(cur.tokq[qi]) * rowstride + int64_t(h) * DH;
      if constexpr (kY16) {
        // Exchange the 4-element pieces of the d-tiles 2 r1 and 2 r1 + 1
        // between lane groups g and g ^ 1 (v_permlane16_swap): the lane then
        // holds d0 .. d0 + 7, d0 = 32 r1 + 16 (g & 1) + 8 (g >> 1), and a
        // wave's 16-byte stores cover 64 contiguous bytes of each row.
#pragma unroll
        for (int r1 = 0; r1 < 2; ++r1) {
          float ov[8];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(o[qi][2 * r1][r]),
                                                             __float_as_uint(o[qi][2 * r1 + 1][r]), false, false);
            ov[r] = __uint_as_float(sw[0]);
            ov[4 + r] = __uint_as_float(sw[1]);
          }
          bf16x8 res;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float val = ov[e] * inv;
            res[e] = static_cast<__bf16>(ACCUMULATE ? to_f32(yq[qi][r1][e]) + val : val);
          }
          *reinterpret_cast<bf16x8*>(yrow + y16_off + 32 * r1) = res;
        }
        continue;
      }
#pragma unroll
      for (int et = 0; et < ET; ++et) {
        YV res;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float ov = o[qi][et][r] * inv;
          res[r] = from_f32<TS>(ACCUMULATE ? to_f32(yp[qi][et][r]) + ov : ov);
        }
        *reinterpret_cast<YV*>(yrow + et * 16 + grp * 4) = res;
      }
    }
    pos = npos;
    return has_next;
  };

#pragma unroll 1
  for (int n = 0;; n += 2) {
    if (!step(n, sK0, sV0, sK1, sV1)) break;
    if (!step(n + 1, sK1, sV1, sK0, sV0)) break;
  }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------

namespace {

struct Args {
  const void* x; const float* dt; const float* A; const void* B; const void* C; const float* D;
  const void* q; const void* k; const void* v;
};

int64_t elem_bytes(const lingen_mate_shape* s) { return s->dtype == LINGEN_BF16 ? 2 : 4; }



RmsMap make_rms(const lingen_mate_shape* s, int mode, int rev = 0) { return RmsMap{mode, s->T, s->H, s->W, rev}; }


// Heads per chunk workgroup: the largest divisor of Hs not above `cap`.
int head_group(int Hs, int cap = kHeadGroupMax) {
  for (int g = cap; g > 1; --g)
    if (Hs % g == 0) return g;
  return 1;
}

// Optional stage markers (lingen_mate_fwd_events): ev[i] is recorded on the
// stream when stage boundary i is reached.
int mark(const hipEvent_t* ev, int i, hipStream_t st) {
  if (ev == nullptr) return LINGEN_OK;
  return hipEventRecord(ev[i], st) == hipSuccess ? LINGEN_OK : LINGEN_ERR_HIP;
}

template <typename TS>
int launch_review(const lingen_mate_shape* s, const TS* x, const float* dt, const float* A, const TS* B,
                  char* ws, const WsLayout& lay, hipStream_t st) {
  ReviewGeom g;
  g.pt = s->rpool_t; g.ph = s->rpool_h; g.pw = s->rpool_w;
  g.rt = s->rgrid_t; g.rh = s->rgrid_h; g.rw = s->rgrid_w;
  g.st = (s->T / g.pt) / g.rt; g.sh = (s->H / g.ph) / g.rh; g.sw = (s->W / g.pw) / g.rw;
  float* rx = reinterpret_cast<float*>(ws + lay.review_x);
  float* rdt = reinterpret_cast<float*>(ws + lay.review_dt);
  float* rb = reinterpret_cast<float*>(ws + lay.review_b);
  float* hR = reinterpret_cast<float*>(ws + lay.review_h);
  review_pool_kernel<TS><<<dim3(s->n_review, s->ssd_heads + s->ngroups), 256, 0, st>>>(
      x, dt, B, s->T, s->H, s->W, s->ssd_heads, s->headdim, s->d_state, s->ngroups, g, rx, rdt, rb);
  if (launch_status(__func__)) return LINGEN_ERR_HIP;
  review_state_kernel<<<dim3(s->ssd_heads, (s->headdim * s->d_state + 1023) / 1024), 256, 0, st>>>(rx, rdt, rb, A, s->n_review, s->ssd_heads, s->headdim,
                                                    s->d_state, s->ngroups, hR);
  return launch_status(__func__);
}

// Phase A + state pass (+ review state) for one batch element.  BIDIR =
// false: the forward direction of the (possibly reversed, rev = 1) order only.
// CONV: x is the xBC rows and the convolution of cv is fused (no review).
template <typename TS, int P, int N, int Q, bool BIDIR = true, int WM = kWeightDt, bool CONV = false>
int launch_states(const lingen_mate_shape* s, int mode, const TS* x, const float* dt, const float* A, const TS* B,
                  char* ws, hipStream_t st, const hipEvent_t* ev = nullptr, int rev = 0, float* h_last = nullptr,
                  const ConvIn& cv = ConvIn{}) {
  const WsLayout lay = ws_layout(s);
  const int L = int(tokens(s));
  const int nc = L / Q;
  const int Hs = s->ssd_heads;
  TS* states = reinterpret_cast<TS*>(ws + lay.states);
  float* decay = reinterpret_cast<float*>(ws + lay.decay);
  // heads per workgroup: a divisor of the heads per B group
  const int hg = head_group(Hs / s->ngroups, kStateHeadGroup);
  const float* h0 = nullptr;
  if (s->n_review > 0) {
    if (CONV) return LINGEN_ERR_UNSUPPORTED;
    if (int rc = launch_review<TS>(s, x, dt, A, B, ws, lay, st)) return rc;
    h0 = reinterpret_cast<const float*>(ws + lay.review_h);
  }
  if (int rc = mark(ev, 1, st)) return rc;
  ssd_chunk_state_kernel<TS, P, N, Q, BIDIR, WM, CONV><<<nc * (Hs / hg), StateCfg<P, N>::NWAVE * 64, 0, st>>>(
      x, dt, A, B, make_rms(s, mode, rev), Hs, s->ngroups, hg, nc, states, decay, cv);
  if (launch_status(__func__)) return LINGEN_ERR_HIP;
  if (int rc = mark(ev, 2, st)) return rc;
  // P*N/E threads per head, in blocks of up to 256.  Both directions: E = 8
  // elements per thread, 8 chunks' loads in flight.  One direction has half
  // the work, so it takes E = 4 (twice the threads) with 16 chunks in flight
  // (measured: 0.25 -> 0.21 ms per one-direction pass at the 512p-like
  // workload; 16 in flight slows the two-direction pass).
  constexpr int E = BIDIR ? 8 : 4, U = BIDIR ? 8 : 16, BS = 256;
  static_assert((P * N / E) % 64 == 0 && ((P * N / E) < BS || (P * N / E) % BS == 0), "state pass blocking");
  const int bs = (P * N / E) < BS ? (P * N / E) : BS;
  const int64_t thr = int64_t(Hs) * P * N / E;
  ssd_state_pass_kernel<TS, U, E><<<dim3(unsigned(thr / bs), BIDIR ? 2 : 1), bs, 0, st>>>(states, decay, h0, Hs,
                                                                                           P * N, nc, h_last);
  if (launch_status(__func__)) return LINGEN_ERR_HIP;
  return mark(ev, 3, st);
}

template <typename TS, int P, int N, int Q>
int launch_ma(const lingen_mate_shape* s, int mode, const Args& a, void* y, char* ws, hipStream_t st,
              const hipEvent_t* ev) {
  const int L = int(tokens(s));
  const int nc = L / Q;
  const int Hs = s->ssd_heads;
  const WsLayout lay = ws_layout(s);
  const int64_t eb = elem_bytes(s);
  for (int b = 0; b < s->batch; ++b) {
    const TS* x = reinterpret_cast<const TS*>(static_cast<const char*>(a.x) + int64_t(b) * L * Hs * P * eb);
    const float* dt = a.dt + int64_t(b) * L * Hs;
    const int64_t bc = int64_t(b) * L * s->ngroups * N * eb;
    const TS* B = reinterpret_cast<const TS*>(static_cast<const char*>(a.B) + bc);
    const TS* C = reinterpret_cast<const TS*>(static_cast<const char*>(a.C) + bc);
    TS* yb = reinterpret_cast<TS*>(static_cast<char*>(y) + int64_t(b) * L * Hs * P * eb);
    if (int rc = launch_states<TS, P, N, Q>(s, mode, x, dt, a.A, B, ws, st, ev)) return rc;
    using Cfg = OutCfg<TS, P, N, Q>;
    const int hg = head_group(Hs / s->ngroups);   // a divisor of the heads per B, C group
    ssd_chunk_out_kernel<TS, P, N, Q><<<nc * (Hs / hg), Cfg::NW * 64, 0, st>>>(
        x, dt, a.A, B, C, a.D, make_rms(s, mode), Hs, s->ngroups, hg, nc, reinterpret_cast<const TS*>(ws + lay.states),
        yb, nullptr, ConvIn{});
    if (launch_status(__func__)) return LINGEN_ERR_HIP;
    if (int rc = mark(ev, 4, st)) return rc;
  }
  return LINGEN_OK;
}

// MA branch with a parameter set per direction: the forward direction of
// the scan order with af, then the forward direction of the reversed order
// (the backward scan) with ab, added to the first result.  CONV: both
// directions read the xBC rows (a.x; a.B and a.C unused) and dt_raw (a.dt),
// with the convolution and dt bias of cv[dir] fused into their kernels.
template <typename TS, int P, int N, int Q, bool CONV = false>
int launch_ma_dirs(const lingen_mate_shape* s, int mode, const Args& af, const Args& ab, void* y, char* ws,
                   hipStream_t st, const ConvIn* cv = nullptr) {
  const int L = int(tokens(s));
  const int nc = L / Q;
  const int Hs = s->ssd_heads;
  const WsLayout lay = ws_layout(s);
  const int64_t eb = elem_bytes(s);
  using Cfg = OutCfg<TS, P, N, Q>;
  const int hg = head_group(Hs / s->ngroups);
  // elements per token row of x and of B, C
  const int64_t xrow = CONV ? cv[0].ch : int64_t(Hs) * P, brow = CONV ? cv[0].ch : int64_t(s->ngroups) * N;
  for (int b = 0; b < s->batch; ++b) {
    TS* yb = reinterpret_cast<TS*>(static_cast<char*>(y) + int64_t(b) * L * Hs * P * eb);
    for (int dir = 0; dir < 2; ++dir) {
      const Args& a = dir ? ab : af;
      const ConvIn cvd = CONV ? cv[dir] : ConvIn{};
      const TS* x = reinterpret_cast<const TS*>(static_cast<const char*>(a.x) + int64_t(b) * L * xrow * eb);
      const float* dt = a.dt + int64_t(b) * L * Hs;
      const int64_t bc = int64_t(b) * L * brow * eb;
      const TS* B = CONV ? x : reinterpret_cast<const TS*>(static_cast<const char*>(a.B) + bc);
      const TS* C = CONV ? x : reinterpret_cast<const TS*>(static_cast<const char*>(a.C) + bc);
      if (int rc = launch_states<TS, P, N, Q, false, kWeightDt, CONV>(s, mode, x, dt, a.A, B, ws, st, nullptr, dir,
                                                                      nullptr, cvd))
        return rc;
      const TS* states = reinterpret_cast<const TS*>(ws + lay.states);
      // The one-direction passes fill only the first half of the states
      // region; the second half (nc*Hs*P*N elements, at least L*Hs*P since
      // N >= Q in the bf16 families) holds the low half of the first
      // direction's result for the second pass.
      static_assert(std::is_same<TS, float>::value || N >= Q, "room for the low half of y");
      TS* ylo = std::is_same<TS, float>::value ? nullptr
                                               : reinterpret_cast<TS*>(ws + lay.states) + int64_t(nc) * Hs * P * N;
      if (dir == 0)
        ssd_chunk_out_kernel<TS, P, N, Q, false, false, false, false, CONV><<<nc * (Hs / hg), Cfg::NW * 64, 0, st>>>(
            x, dt, a.A, B, C, a.D, make_rms(s, mode, 0), Hs, s->ngroups, hg, nc, states, yb, ylo, cvd);
      else
        ssd_chunk_out_kernel<TS, P, N, Q, false, true, false, false, CONV><<<nc * (Hs / hg), Cfg::NW * 64, 0, st>>>(
            x, dt, a.A, B, C, a.D, make_rms(s, mode, 1), Hs, s->ngroups, hg, nc, states, yb, ylo, cvd);
      if (launch_status(__func__)) return LINGEN_ERR_HIP;
    }
  }
  return LINGEN_OK;
}

int dispatch_ma_dirs(const lingen_mate_shape* s, int mode, const Args& af, const Args& ab, void* y, char* ws,
                     hipStream_t st) {
  switch (scan_family(s)) {
    case SCAN_F32_P32_N16_Q16: return launch_ma_dirs<float, 32, 16, 16>(s, mode, af, ab, y, ws, st);
    case SCAN_BF16_P64_N64_Q64: return launch_ma_dirs<__bf16, 64, 64, 64>(s, mode, af, ab, y, ws, st);
    case SCAN_BF16_P64_N128_Q128: return launch_ma_dirs<__bf16, 64, 128, 128>(s, mode, af, ab, y, ws, st);
    default: return LINGEN_ERR_UNSUPPORTED;
  }
}

// The fused form: bf16 families only (the fp32 family runs the standalone
// steps and then dispatch_ma_dirs).
int dispatch_ma_dirs_conv(const lingen_mate_shape* s, int mode, const Args& af, const Args& ab, const ConvIn* cv,
                          void* y, char* ws, hipStream_t st) {
  switch (scan_family(s)) {
    case SCAN_BF16_P64_N64_Q64: return launch_ma_dirs<__bf16, 64, 64, 64, true>(s, mode, af, ab, y, ws, st, cv);
    case SCAN_BF16_P64_N128_Q128: return launch_ma_dirs<__bf16, 64, 128, 128, true>(s, mode, af, ab, y, ws, st, cv);
    default: return LINGEN_ERR_UNSUPPORTED;
  }
}

// The transposed bidirectional scan of one batch element (TRANS above): the
// states are those of u against C with the adjoint token weights, left by
// scan_states_one in `ws`; B and C are exchanged for the output kernel.
template <typename TS, int P, int N, int Q>
int launch_transposed(const lingen_mate_shape* s, int mode, const TS* u, const float* dt, const float* A,
                      const TS* B, const TS* C, const char* ws, TS* y, hipStream_t st) {
  const int nc = int(tokens(s)) / Q;
  const int Hs = s->ssd_heads;
  using Cfg = OutCfg<TS, P, N, Q>;
  const int hg = head_group(Hs / s->ngroups);
  const TS* states = reinterpret_cast<const TS*>(ws + ws_layout(s).states);
  ssd_chunk_out_kernel<TS, P, N, Q, true, false, true, true><<<nc * (Hs / hg), Cfg::NW * 64, 0, st>>>(
      u, dt, A, C, B, nullptr, make_rms(s, mode), Hs, s->ngroups, hg, nc, states, y, nullptr, ConvIn{});
  if (launch_status(__func__)) return LINGEN_ERR_HIP;
  return LINGEN_OK;
}

int dispatch_ma(const lingen_mate_shape* s, int mode, const Args& a, void* y, char* ws, hipStream_t st,
                const hipEvent_t* ev = nullptr) {
  switch (scan_family(s)) {
    case SCAN_F32_P32_N16_Q16: return launch_ma<float, 32, 16, 16>(s, mode, a, y, ws, st, ev);
    case SCAN_BF16_P64_N64_Q64: return launch_ma<__bf16, 64, 64, 64>(s, mode, a, y, ws, st, ev);
    case SCAN_BF16_P64_N128_Q128: return launch_ma<__bf16, 64, 128, 128>(s, mode, a, y, ws, st, ev);
    default: return LINGEN_ERR_UNSUPPORTED;
  }
}

template <typename TS, int DH, int NWIN, int NVALID>
int launch_te(const lingen_mate_shape* s, const int shift[3], int masked, const void* q, const void* k,
              const void* v, void* y, int accumulate, hipStream_t st) {
  const WinGeom g = make_wingeom(s, shift, masked);
  const int64_t L = tokens(s);
  const int nwin = g.nwt * g.nwh * g.nww;
  const int64_t per = L * s->attn_heads * DH * elem_bytes(s);
  using Cfg = AttnCfg<TS, DH, NWIN>;
  // Persistent grid: 16 waves per compute unit (one workgroup of the
  // 256-slot windows, several of the small ones).
  const int ncu = compute_units();
  if (ncu < 1) return LINGEN_ERR_HIP;
  const int64_t slots = int64_t(ncu) * (Cfg::NWAVE >= 16 ? 1 : 16 / Cfg::NWAVE);
  for (int b = 0; b < s->batch; ++b) {
    const int64_t off = int64_t(b) * per;
    const TS* qb = reinterpret_cast<const TS*>(static_cast<const char*>(q) + off);
    const TS* kb = reinterpret_cast<const TS*>(static_cast<const char*>(k) + off);
    const TS* vb = reinterpret_cast<const TS*>(static_cast<const char*>(v) + off);
    TS* yb = reinterpret_cast<TS*>(static_cast<char*>(y) + off);
    const int items = nwin * s->attn_heads;
    const int grid = int(items < slots ? items : slots);
    if (accumulate)
      tesa_window_kernel<TS, DH, NWIN, NVALID, true><<<grid, Cfg::NWAVE * 64, 0, st>>>(qb, kb, vb, g, s->attn_heads,
                                                                                      items, yb);
    else
      tesa_window_kernel<TS, DH, NWIN, NVALID, false><<<grid, Cfg::NWAVE * 64, 0, st>>>(qb, kb, vb, g, s->attn_heads,
                                                                                       items, yb);
    if (launch_status(__func__)) return LINGEN_ERR_HIP;
  }
  return LINGEN_OK;
}

// shift: grid offset per axis (0 <= shift < window); masked: 1 for Swin's
// cut border windows, 0 for cyclic windows.
int dispatch_te(const lingen_mate_shape* s, const int shift[3], int masked, const void* q, const void* k,
                const void* v, void* y, int accumulate, hipStream_t st) {
  switch (attn_family(s)) {
    case ATTN_F32_D32_W32: return launch_te<float, 32, 32, 32>(s, shift, masked, q, k, v, y, accumulate, st);
    case ATTN_BF16_D64_W256: return launch_te_win256(s, shift, masked, q, k, v, y, accumulate, st);
    case ATTN_BF16_D64_W27: return launch_te<__bf16, 64, 32, 27>(s, shift, masked, q, k, v, y, accumulate, st);
    default: return LINGEN_ERR_UNSUPPORTED;
  }
}

// Half-window offsets (floored) on shifted layers, none otherwise.
void layer_shift(const lingen_mate_shape* s, int shifted, int shift[3]) {
  shift[0] = shifted ? s->win_t / 2 : 0;
  shift[1] = shifted ? s->win_h / 2 : 0;
  shift[2] = shifted ? s->win_w / 2 : 0;
}

int check_all(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (int rc = check_ptr(p)) return rc;
  return LINGEN_OK;
}

int check_ws(const lingen_mate_shape* s, const void* ws, size_t ws_bytes) {
  if (int rc = check_ptr(ws)) return rc;
  if (ws_bytes < ws_layout(s).total) return LINGEN_ERR_WORKSPACE;
  return LINGEN_OK;
}

}  // namespace
}  // namespace lingen

using namespace lingen;

namespace lingen {
// Chunk states and scan states of one batch element into the workspace (at
// ws_layout().states, [2][n_chunks][Hs][P][N] in the storage dtype: the
// state entering each chunk of the forward scan, then of the reverse scan).
// wmode: kWeightDt or kWeightAdjoint.
int scan_states_one(const lingen_mate_shape* s, int mode, const void* xb, const float* dtb, const float* A,
                    const void* Bb, void* workspace, hipStream_t stream, int wmode, float* h_last) {
  char* ws = static_cast<char*>(workspace);
  if (wmode != kWeightDt && wmode != kWeightAdjoint) return LINGEN_ERR_UNSUPPORTED;
  const bool adj = wmode == kWeightAdjoint;
  switch (scan_family(s)) {
    case SCAN_F32_P32_N16_Q16: {
      const float* x = static_cast<const float*>(xb);
      const float* B = static_cast<const float*>(Bb);
      return adj ? launch_states<float, 32, 16, 16, true, kWeightAdjoint>(s, mode, x, dtb, A, B, ws, stream, nullptr,
                                                                          0, h_last)
                 : launch_states<float, 32, 16, 16>(s, mode, x, dtb, A, B, ws, stream, nullptr, 0, h_last);
    }
    case SCAN_BF16_P64_N64_Q64: {
      const __bf16* x = static_cast<const __bf16*>(xb);
      const __bf16* B = static_cast<const __bf16*>(Bb);
      return adj ? launch_states<__bf16, 64, 64, 64, true, kWeightAdjoint>(s, mode, x, dtb, A, B, ws, stream, nullptr,
                                                                           0, h_last)
                 : launch_states<__bf16, 64, 64, 64>(s, mode, x, dtb, A, B, ws, stream, nullptr, 0, h_last);
    }
    case SCAN_BF16_P64_N128_Q128: {
      const __bf16* x = static_cast<const __bf16*>(xb);
      const __bf16* B = static_cast<const __bf16*>(Bb);
      return adj ? launch_states<__bf16, 64, 128, 128, true, kWeightAdjoint>(s, mode, x, dtb, A, B, ws, stream,
                                                                             nullptr, 0, h_last)
                 : launch_states<__bf16, 64, 128, 128>(s, mode, x, dtb, A, B, ws, stream, nullptr, 0, h_last);
    }
    default:
      return LINGEN_ERR_UNSUPPORTED;
  }
}

int ma_transposed_one(const lingen_mate_shape* s, int mode, const void* ub, const float* dtb, const float* A,
                      const void* Bb, const void* Cb, const void* workspace, void* yb, hipStream_t stream) {
  if (s->n_review != 0) return LINGEN_ERR_UNSUPPORTED;
  const char* ws = static_cast<const char*>(workspace);
  switch (scan_family(s)) {
    case SCAN_F32_P32_N16_Q16:
      return launch_transposed<float, 32, 16, 16>(s, mode, static_cast<const float*>(ub), dtb, A,
                                                  static_cast<const float*>(Bb), static_cast<const float*>(Cb), ws,
                                                  static_cast<float*>(yb), stream);
    case SCAN_BF16_P64_N64_Q64:
      return launch_transposed<__bf16, 64, 64, 64>(s, mode, static_cast<const __bf16*>(ub), dtb, A,
                                                   static_cast<const __bf16*>(Bb), static_cast<const __bf16*>(Cb), ws,
                                                   static_cast<__bf16*>(yb), stream);
    case SCAN_BF16_P64_N128_Q128:
      return launch_transposed<__bf16, 64, 128, 128>(s, mode, static_cast<const __bf16*>(ub), dtb, A,
                                                     static_cast<const __bf16*>(Bb), static_cast<const __bf16*>(Cb),
                                                     ws, static_cast<__bf16*>(yb), stream);
    default:
      return LINGEN_ERR_UNSUPPORTED;
  }
}
}  // namespace lingen

extern "C" {

int lingen_rms_index_device(int32_t mode, int32_t T, int32_t H, int32_t W, int32_t* perm_dev, hipStream_t stream) {
  if (mode < 0 || mode > 3 || T < 1 || H < 1 || W < 1) return LINGEN_ERR_SHAPE;
  const int64_t L = int64_t(T) * H * W;
  if (L > (int64_t(1) << 31) - 1) return LINGEN_ERR_SHAPE;
  if (int rc = check_ptr(perm_dev)) return rc;
  rms_index_kernel<<<unsigned((L + 255) / 256), 256, 0, stream>>>(RmsMap{mode, T, H, W}, int(L), perm_dev);
  return launch_status(__func__);
}

int lingen_rms_gather(const void* src, int64_t row_bytes, int32_t mode, int32_t T, int32_t H, int32_t W, void* dst,
                      hipStream_t stream) {
  if (mode < 0 || mode > 3 || T < 1 || H < 1 || W < 1) return LINGEN_ERR_SHAPE;
  const int64_t L = int64_t(T) * H * W;
  if (L > (int64_t(1) << 31) - 1) return LINGEN_ERR_SHAPE;
  if (row_bytes < 16 || row_bytes % 16) return LINGEN_ERR_SHAPE;
  if (int rc = check_all({src, dst})) return rc;
  const int64_t row16 = row_bytes / 16;
  rms_gather_kernel<<<unsigned(L), 256, 0, stream>>>(static_cast<const u32x4*>(src), row16, RmsMap{mode, T, H, W},
                                                     static_cast<u32x4*>(dst));
  return launch_status(__func__);
}

int lingen_ssd_chunk_states(const void* x, const float* dt, const float* A, const void* B, int32_t mode,
                            const lingen_mate_shape* shape, float* h_fwd, float* h_bwd, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  if (int rc = validate_shape(shape)) return rc;
  if (mode < 0 || mode > 3) return LINGEN_ERR_SHAPE;
  if (int rc = check_all({x, dt, A, B, h_fwd, h_bwd})) return rc;
  if (int rc = check_ws(shape, workspace, workspace_bytes)) return rc;
  const lingen_mate_shape* s = shape;
  const int64_t L = tokens(s);
  const int64_t Hs = s->ssd_heads, P = s->headdim, N = s->d_state, nc = L / s->chunk;
  const int64_t eb = elem_bytes(s);
  const int64_t per = nc * Hs * P * N;       // floats per direction per batch element
  char* ws = static_cast<char*>(workspace);
  const WsLayout lay = ws_layout(s);
  for (int b = 0; b < s->batch; ++b) {
    const char* xb = static_cast<const char*>(x) + b * L * Hs * P * eb;
    const float* dtb = dt + b * L * Hs;
    const char* Bb = static_cast<const char*>(B) + b * L * s->ngroups * N * eb;
    if (int rc = scan_states_one(s, mode, xb, dtb, A, Bb, ws, stream, kWeightDt, nullptr)) return rc;
    const unsigned blocks = unsigned((per + 255) / 256);
    if (s->dtype == LINGEN_BF16) {
      const __bf16* st = reinterpret_cast<const __bf16*>(ws + lay.states);
      states_to_f32_kernel<__bf16><<<blocks, 256, 0, stream>>>(st, h_fwd + b * per, per);
      states_to_f32_kernel<__bf16><<<blocks, 256, 0, stream>>>(st + per, h_bwd + b * per, per);
    } else {
      const float* st = reinterpret_cast<const float*>(ws + lay.states);
      states_to_f32_kernel<float><<<blocks, 256, 0, stream>>>(st, h_fwd + b * per, per);
      states_to_f32_kernel<float><<<blocks, 256, 0, stream>>>(st + per, h_bwd + b * per, per);
    }
    if (launch_status(__func__)) return LINGEN_ERR_HIP;
  }
  return LINGEN_OK;
}

int lingen_ma_fwd(const void* x, const float* dt, const float* A, const void* B, const void* C, const float* D,
                  int32_t mode, const lingen_mate_shape* shape, void* y_ma, void* workspace, size_t workspace_bytes,
                  hipStream_t stream) {
  if (int rc = validate_shape(shape)) return rc;
  if (mode < 0 || mode > 3) return LINGEN_ERR_SHAPE;
  if (int rc = check_all({x, dt, A, B, C, D, y_ma})) return rc;
  if (int rc = check_ws(shape, workspace, workspace_bytes)) return rc;
  Args a{x, dt, A, B, C, D, nullptr, nullptr, nullptr};
  return dispatch_ma(shape, mode, a, y_ma, static_cast<char*>(workspace), stream);
}

int lingen_ma_fwd_dirs(const void* x_f, const float* dt_f, const float* A_f, const void* B_f, const void* C_f,
                       const float* D_f, const void* x_b, const float* dt_b, const float* A_b, const void* B_b,
                       const void* C_b, const float* D_b, int32_t mode, const lingen_mate_shape* shape, void* y_ma,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (int rc = validate_shape(shape)) return rc;
  if (mode < 0 || mode > 3) return LINGEN_ERR_SHAPE;
  if (int rc = check_all({x_f, dt_f, A_f, B_f, C_f, D_f, x_b, dt_b, A_b, B_b, C_b, D_b, y_ma})) return rc;
  if (int rc = check_ws(shape, workspace, workspace_bytes)) return rc;
  Args af{x_f, dt_f, A_f, B_f, C_f, D_f, nullptr, nullptr, nullptr};
  Args ab{x_b, dt_b, A_b, B_b, C_b, D_b, nullptr, nullptr, nullptr};
  return dispatch_ma_dirs(shape, mode, af, ab, y_ma, static_cast<char*>(workspace), stream);
}

int lingen_ma_fwd_dirs_conv(const void* xbc, const float* dt_raw, const float* dt_bias, int32_t conv_k,
                            const float* conv_w_f, const float* conv_b_f, const float* A_f, const float* D_f,
                            const float* conv_w_b, const float* conv_b_b, const float* A_b, const float* D_b,
                            int32_t mode, const lingen_mate_shape* shape, void* y_ma, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  if (int rc = validate_shape(shape)) return rc;
  if (mode < 0 || mode > 3 || conv_k < 1 || conv_k > kConvTaps) return LINGEN_ERR_SHAPE;
  if (int rc = check_all({xbc, dt_raw, dt_bias, conv_w_f, conv_b_f, A_f, D_f, conv_w_b, conv_b_b, A_b, D_b, y_ma}))
    return rc;
  if (int rc = check_ws(shape, workspace, workspace_bytes)) return rc;
  if (shape->dtype != LINGEN_BF16 || shape->n_review > 0) return LINGEN_ERR_UNSUPPORTED;
  const int d = shape->ssd_heads * shape->headdim, gn = shape->ngroups * shape->d_state;
  // 16-byte pieces of every row: x, B, C all start on a piece
  if (d % 8 || gn % 8) return LINGEN_ERR_SHAPE;
  ConvIn cv[2];
  cv[0] = ConvIn{conv_w_f, conv_b_f, dt_bias, conv_k, d + 2 * gn, d, d + gn};
  cv[1] = ConvIn{conv_w_b, conv_b_b, dt_bias, conv_k, d + 2 * gn, d, d + gn};
  Args af{xbc, dt_raw, A_f, xbc, xbc, D_f, nullptr, nullptr, nullptr};
  Args ab{xbc, dt_raw, A_b, xbc, xbc, D_b, nullptr, nullptr, nullptr};
  return dispatch_ma_dirs_conv(shape, mode, af, ab, cv, y_ma, static_cast<char*>(workspace), stream);
}

int lingen_te_fwd(const void* q, const void* k, const void* v, int32_t shifted, const lingen_mate_shape* shape,
                  void* y_te, hipStream_t stream) {
  if (int rc = validate_shape(shape)) return rc;
  if (int rc = check_all({q, k, v, y_te})) return rc;
  int shift[3];
  layer_shift(shape, shifted ? 1 : 0, shift);
  return dispatch_te(shape, shift, 1, q, k, v, y_te, 0, stream);
}

int lingen_te_fwd_shift(const void* q, const void* k, const void* v, int32_t shift_t, int32_t shift_h,
                        int32_t shift_w, int32_t masked, const lingen_mate_shape* shape, void* y_te,
                        hipStream_t stream) {
  if (int rc = validate_shape(shape)) return rc;
  if (shift_t < 0 || shift_t >= shape->win_t || shift_h < 0 || shift_h >= shape->win_h || shift_w < 0 ||
      shift_w >= shape->win_w || (masked != 0 && masked != 1))
    return LINGEN_ERR_SHAPE;
  if (int rc = check_all({q, k, v, y_te})) return rc;
  const int shift[3] = {shift_t, shift_h, shift_w};
  return dispatch_te(shape, shift, masked, q, k, v, y_te, 0, stream);
}

static int mate_fwd_impl(const void* x, const float* dt, const float* A, const void* B, const void* C,
                         const float* D, const void* q, const void* k, const void* v, int32_t layer_idx,
                         const lingen_mate_shape* shape, void* y, void* workspace, size_t workspace_bytes,
                         hipStream_t stream, const hipEvent_t* ev) {
  if (int rc = validate_shape(shape)) return rc;
  if (layer_idx < 0) return LINGEN_ERR_SHAPE;
  if (int rc = check_all({x, dt, A, B, C, D, q, k, v, y})) return rc;
  if (int rc = check_ws(shape, workspace, workspace_bytes)) return rc;
  const int mode = layer_idx % 4;
  int shift[3];
  layer_shift(shape, layer_idx % 2, shift);
  Args a{x, dt, A, B, C, D, q, k, v};
  if (int rc = mark(ev, 0, stream)) return rc;
  if (int rc = dispatch_ma(shape, mode, a, y, static_cast<char*>(workspace), stream, ev)) return rc;
  if (int rc = dispatch_te(shape, shift, 1, q, k, v, y, 1, stream)) return rc;
  return mark(ev, 5, stream);
}

int lingen_mate_fwd(const void* x, const float* dt, const float* A, const void* B, const void* C, const float* D,
                    const void* q, const void* k, const void* v, int32_t layer_idx, const lingen_mate_shape* shape,
                    void* y, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return mate_fwd_impl(x, dt, A, B, C, D, q, k, v, layer_idx, shape, y, workspace, workspace_bytes, stream, nullptr);
}

int lingen_mate_fwd_events(const void* x, const float* dt, const float* A, const void* B, const void* C,
                           const float* D, const void* q, const void* k, const void* v, int32_t layer_idx,
                           const lingen_mate_shape* shape, void* y, void* workspace, size_t workspace_bytes,
                           hipStream_t stream, hipEvent_t* events) {
  if (events == nullptr) return LINGEN_ERR_NULL;
  if (shape != nullptr && shape->batch != 1) return LINGEN_ERR_SHAPE;
  for (int i = 0; i < 6; ++i)
    if (events[i] == nullptr) return LINGEN_ERR_NULL;
  return mate_fwd_impl(x, dt, A, B, C, D, q, k, v, layer_idx, shape, y, workspace, workspace_bytes, stream, events);
}

}  // extern "C"
