// Backward pass of the MA branch: gradients of sum(dy * y_MA) for the
// shared-parameter bidirectional scan (Mamba2's scalar-A recurrence, "Transformers
// are SSMs", Dao & Gu 2024; run along the Rotary Major Scan order and its
// reverse, page "视频生成模子太贵太慢如何办？", section 要领：线性复杂度的 MATE 模块)
// with respect to x, dt, A, B, C and D.
//
// Per direction write M for the scan's matrix (y = M x), L_ts for the decay
// product between scan positions and W_ts = M_ts (dy_t . x_s).  Every
// gradient is built from scans the library already runs, with transformed
// operands, plus the kernels of this file:
//   * dx = dt yhat + 2 D dy with yhat = (M_f^T + M_b^T) dy / dt.  Inside a
//     chunk, M_f^T + M_b^T is the bidirectional scan with B and C exchanged,
//     unit token weights and the inclusive and exclusive prefix sums of
//     dt A trading places in the decays; its chunk states are those of dy
//     against C with the token weights exp(dt A), i.e. the adjoint states
//     below, so yhat is one output-kernel launch over them;
//   * dB and dC are, per chunk, products of the same chunk-local matrices the
//     crossing sums need (E = dt (dy x^T) weighted by the decays) with C and
//     B, plus products of the chunk-boundary states with x and dy;
//   * the chunk-boundary adjoint states are the scan states of x' = dy
//     exp(dt A) / dt with C in place of B, taken from dy with the token
//     weights exp(dt A) in place of dt (x' itself is never formed; read in
//     bf16 from the chunk-state pass's workspace, one batch element at a
//     time);
//   * ddt and dA need, at every position r, the crossing sum
//     R_r = sum_{s < r <= t} W_ts: the pairs inside r's chunk come from the
//     chunk's W (row minus column sums, then a suffix sum), the pairs with
//     one end outside from products of the chunk-boundary states with the
//     chunk's rows, the pairs with both ends outside from one inner product
//     of states; ddt = x . (yhat_f + yhat_b) + A (R_f + R_b) with yhat the
//     transposed outputs before the dt factor, dA = sum dt (R_f + R_b).
//     (Forming the in-chunk part instead from the difference of the bf16
//     forward and transposed outputs cancels, and loses dA.)
// All sums are formed chunk by chunk, in fp32 from the bf16 inputs, so no
// sum runs over the whole sequence.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "lingen_device.h"
#include "lingen_internal.h"
#include "lingen_scan_map.h"

namespace lingen {
namespace {

constexpr int kThreads = 256;

unsigned blocks_for(int64_t n) { return unsigned((n + kThreads - 1) / kThreads); }

// Zero two arrays of n floats each (the accumulated gradients dA, dD).
__global__ __launch_bounds__(kThreads) void zero_floats_kernel(float* __restrict__ a, float* __restrict__ b, int n) {
  for (int i = threadIdx.x; i < n; i += kThreads) {
    a[i] = 0.f;
    b[i] = 0.f;
  }
}

constexpr int kCrossThreads = 512;

// Block-wide sum over the 512 threads of a workgroup.
__device__ __forceinline__ float block_sum512(float v, float* red) {
  v = sum64(v);
  lds_barrier();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  lds_barrier();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < kCrossThreads / 64; ++w) t += red[w];
  return t;
}

// Inclusive prefix sums of Q = 64 V values held V per lane (lane l holds
// positions V l .. V l + V - 1), within one wave (all lanes active).
template <int V>
__device__ __forceinline__ void wave_prefix(float (&v)[V]) {
#pragma unroll
  for (int e = 1; e < V; ++e) v[e] += v[e - 1];
  const float run = wave_scan_incl(v[V - 1]);
  const float before = run - v[V - 1];
#pragma unroll
  for (int e = 0; e < V; ++e) v[e] += before;
}

// Two 4-element transposing LDS reads (rows k and k + 16 of a row-major
// bf16 tile, 16 columns from `col`), giving lane group g the contraction
// indices {4g..4g+3, 16+4g..16+4g+3} of a 32-block for column (lane & 15):
// the operand order of the 16x16x32 MFMA with its k axis permuted.
__device__ __forceinline__ bf16x8 tr_frag(const __bf16* tile, int ld, int k0, int col0, int lane) {
  const int r16 = lane & 15, grp = lane >> 4;
  lds_bf16* p = (lds_bf16*)(tile + (k0 + 4 * grp + (r16 >> 2)) * ld + col0 + 4 * (r16 & 3));
  const bf16x4 lo = lds_read_tr(p);
  const bf16x4 hi = lds_read_tr(p + 16 * ld);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
// The matching operand from a k-contiguous row: k = {4g..4g+3, 16+4g..16+4g+3}.
__device__ __forceinline__ bf16x8 perm_frag(const __bf16* row, int k0, int lane) {
  const int grp = lane >> 4;
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + k0 + 4 * grp);
  const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + k0 + 16 + 4 * grp);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Per (chunk, group, batch element), looping over the group's heads (head
// size 64): the crossing sums R_r behind ddt and dA, and from them and the
// transposed outputs yhat = (M_f^T + M_b^T) dy / dt the per-token gradients
//   dx = dt yhat + 2 D dy,   ddt = x . yhat + A R,   dA += dt R,   dD += 2 dy . x
// (dx [batch, L, Hs, P], ddt [batch, L, Hs]; dA and dD [Hs], added to), and
// the gradients dB, dC of the chunk's tokens, written to [batch, L, G, N]
// fp32.  With cs the chunk-local inclusive cumulative sum of dt*A
// along the scan order and csx its exclusive form:
//   forward pairs s <= t:  decay exp(cs_t - cs_s),   backward pairs s >= t:
//   decay exp(csx_s - csx_t); E_ts = dt_s (dy_t . x_s) (sum of the decays that
//   apply); W_ts = E_ts (C_t . B_s) split by direction (s = t excluded).
// Crossing sums (forward: s < r <= t; backward: t <= r < s):
//   R_r = suffix_{t >= r}(d_f + U_f + V_b) + prefix_{t <= r}(d_b + U_b + V_f)
//         - V_f(r) - V_b(r) + K,
// d_f, d_b the row minus column sums of W per direction, and the pairs with
// an end outside the chunk from the four chunk-boundary states (hf1: forward
// state entering the chunk; hb1: reverse state entering it from the right;
// hf2, hb2: adjoint states of the reverse / forward scan):
//   U_f(t) = exp(cs_t) dy_t . (hf1 C_t)      V_f(s) = dt_s exp(cs_last - cs_s) x_s . (hb2 B_s)
//   U_b(t) = exp(cs_last - csx_t) dy_t . (hb1 C_t)   V_b(s) = dt_s exp(csx_s) x_s . (hf2 B_s)
//   K = exp(cs_last) (<hf1, hb2> + <hb1, hf2>)
// and, summed over the heads of the group,
//   dC_t = sum_s E_ts B_s + exp(cs_t) hf1^T dy_t + exp(cs_last - csx_t) hb1^T dy_t
//   dB_s = sum_t E_ts C_t + dt_s exp(cs_last - cs_s) hb2^T x_s + dt_s exp(csx_s) hf2^T x_s.
// Products on 16x16x32 bf16 MFMA tiles from padded LDS rows (C B^T, dy x^T,
// E B, E^T C and the state products, per head), fp32 everywhere after them;
// no sum runs across the sequence.  The states are the bf16 scan states the
// chunk-state pass leaves in its workspace (st1: of (x, B); st2: of
// (dy exp(dt A) / dt, C); each [2][n_chunks][Hs][P][N], forward then reverse),
// for batch element b.  512
// threads (8 waves); wave w owns row block w of every Q x N result.
template <int Q, int N>
__global__ __launch_bounds__(kCrossThreads) void ma_bwd_cross_kernel(
    const __bf16* __restrict__ x, const __bf16* __restrict__ dy, const float* __restrict__ dt,
    const float* __restrict__ A, const __bf16* __restrict__ B, const __bf16* __restrict__ C,
    const __bf16* __restrict__ st1, const __bf16* __restrict__ st2, int64_t per, ScanOrder so, int L, int Hs,
    int G, int b, const __bf16* __restrict__ yh, const float* __restrict__ D, float* __restrict__ dx,
    float* __restrict__ ddt, float* __restrict__ dA, float* __restrict__ dD, float* __restrict__ dB,
    float* __restrict__ dC) {
  constexpr int P = 64, NT = kCrossThreads, NW = NT / 64;
  constexpr int LDB = N + 8, LDX = P + 8, LDE = Q + 8;   // padded bf16 row strides
  constexpr int QT = Q / 16, NTL = N / 16;
  constexpr int CBT = (QT * QT + NW - 1) / NW;           // Q x Q tiles per wave
  constexpr int M_ELEMS = P * LDB, E_ELEMS = Q * LDE;
  constexpr int U_ELEMS = 2 * M_ELEMS > E_ELEMS ? 2 * M_ELEMS : E_ELEMS;
  constexpr int SCH = P * N / 8 / NT;                    // 16-byte state chunks per thread
  static_assert(Q % 32 == 0 && Q <= NT && N % 32 == 0 && QT <= NW && (P * N) % (8 * NT) == 0 &&
                (Q * P) % (8 * NT) == 0 && (Q * N) % (8 * NT) == 0, "tiles");
  __shared__ __attribute__((aligned(16))) __bf16 sB[Q * LDB], sC[Q * LDB], sX[Q * LDX], sDY[Q * LDX];
  __shared__ __attribute__((aligned(16))) __bf16 sU[U_ELEMS];   // E^T (Q x Q, row s), then a state (P x N rows)
  __shared__ float s_cs[Q], s_csx[Q], s_dt[Q], s_fw[Q], s_bw[Q], s_sub[Q], red[NW], s_hsum[2];
  __shared__ int s_tok[Q];
  __bf16* const sE = sU;
  __bf16* const sM0 = sU;
  __bf16* const sM1 = sU + M_ELEMS;

  const int c = blockIdx.x, g = blockIdx.y;
  const int hpg = Hs / G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int64_t bl = int64_t(b) * L;

  for (int i = tid; i < Q; i += NT) s_tok[i] = so.canon(c * Q + i);
  lds_barrier();
  {
    // every load is issued before the first LDS store
    constexpr int UB = Q * (N / 8) / NT;
    bf16x8 vb[UB], vc[UB];
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int i = tid + u * NT, row = i / (N / 8), k8 = (i % (N / 8)) * 8;
      const int64_t src = ((bl + s_tok[row]) * G + g) * N + k8;
      vb[u] = *reinterpret_cast<const bf16x8*>(B + src);
      vc[u] = *reinterpret_cast<const bf16x8*>(C + src);
    }
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int i = tid + u * NT, row = i / (N / 8), k8 = (i % (N / 8)) * 8;
      *reinterpret_cast<bf16x8*>(sB + row * LDB + k8) = vb[u];
      *reinterpret_cast<bf16x8*>(sC + row * LDB + k8) = vc[u];
    }
  }
  lds_barrier();
  // dC, dB of row block `wave`, summed over the group's heads, transposed:
  // the lane holds columns 16 j + 4 lg + r of row r0 + lr
  f32x4 gC[NTL], gB[NTL];
#pragma unroll
  for (int j = 0; j < NTL; ++j) { gC[j] = f32x4{0.f, 0.f, 0.f, 0.f}; gB[j] = f32x4{0.f, 0.f, 0.f, 0.f}; }
  const bool owns_rows = wave < QT;
  const int r0 = wave * 16;   // the row block this wave owns in the Q x N results

  // C B^T on the wave's pair tiles (the same for every head of the group),
  // formed once and kept in registers as bf16, in the order the pair loop
  // below walks the tiles: that loop takes each tile's four values from the
  // front of the vector and rotates the next tile's to the front.
  static_assert(QT * QT == CBT * NW, "every wave walks CBT pair tiles, so the rotation comes full circle");
  typedef __bf16 bf16xcb __attribute__((ext_vector_type(4 * CBT)));
  bf16xcb cbq;
  auto rotate_tiles = [](const bf16xcb& v) {
    bf16xcb o;
#pragma unroll
    for (int i = 0; i < 4 * CBT; ++i) o[i] = v[(i + 4) % (4 * CBT)];
    return o;
  };
#pragma unroll
  for (int q = 0; q < CBT; ++q) {
    const int tile = wave + q * NW;
    const int t0 = (wave % QT) * 16, s0 = ((tile / QT + wave % QT) % QT) * 16;
    f32x4 cb = {0.f, 0.f, 0.f, 0.f};
    if (tile < QT * QT) {
#pragma unroll
      for (int k = 0; k < N; k += 32) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(sC + (t0 + lr) * LDB + k + 8 * lg);
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(sB + (s0 + lr) * LDB + k + 8 * lg);
        cb = mma(a, v, cb);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) cbq[4 * q + r] = static_cast<__bf16>(cb[r]);
  }

#pragma unroll 1
  for (int hh = 0; hh < hpg; ++hh) {
    const int h = g * hpg + hh;
    const float a_h = A[h];
    lds_barrier();   // the previous head is done with every shared array
    if (tid == 0) {   // the previous head's dA, dD shares of this chunk
      if (hh > 0) {
        atomicAdd(dA + h - 1, s_hsum[0]);
        atomicAdd(dD + h - 1, s_hsum[1]);
      }
      s_hsum[0] = 0.f;
      s_hsum[1] = 0.f;
    }
    {
      // dt, x and dy rows: every load is issued before the first LDS store
      constexpr int UX = Q * (P / 8) / NT;
      const float dt_i = tid < Q ? dt[(bl + s_tok[tid]) * Hs + h] : 0.f;
      bf16x8 vx[UX], vd[UX];
#pragma unroll
      for (int u = 0; u < UX; ++u) {
        const int i = tid + u * NT, row = i / (P / 8), k8 = (i % (P / 8)) * 8;
        const int64_t src = ((bl + s_tok[row]) * Hs + h) * P + k8;
        vx[u] = *reinterpret_cast<const bf16x8*>(x + src);
        vd[u] = *reinterpret_cast<const bf16x8*>(dy + src);
      }
      if (tid < Q) {
        s_dt[tid] = dt_i;
        s_fw[tid] = 0.f;
        s_bw[tid] = 0.f;
        s_sub[tid] = 0.f;
      }
#pragma unroll
      for (int u = 0; u < UX; ++u) {
        const int i = tid + u * NT, row = i / (P / 8), k8 = (i % (P / 8)) * 8;
        *reinterpret_cast<bf16x8*>(sX + row * LDX + k8) = vx[u];
        *reinterpret_cast<bf16x8*>(sDY + row * LDX + k8) = vd[u];
      }
    }
    lds_barrier();
    if (wave == 0) {   // chunk-local cumulative sums of dt*A, inclusive and exclusive
      constexpr int V = Q / 64;
      float v[V], d0[V];
#pragma unroll
      for (int e = 0; e < V; ++e) { d0[e] = s_dt[V * lane + e] * a_h; v[e] = d0[e]; }
      wave_prefix<V>(v);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        s_cs[V * lane + e] = v[e];
        s_csx[V * lane + e] = v[e] - d0[e];
      }
    }
    lds_barrier();
    const float cs_last = s_cs[Q - 1];

    // the four chunk-boundary states of this head (hf1, hb2, hb1, hf2); the
    // first one is fetched now, each next one while the previous is in use
    const int64_t st_off = (int64_t(c) * Hs + h) * int64_t(P) * N;
    // (chosen by selects on the kernel's own pointers, so the loads stay
    // global loads rather than generic ones, which the LDS waits would drain)
    auto state = [&](int term) {
      const __bf16* base = (term == 0 || term == 2) ? st1 : st2;
      return reinterpret_cast<const bf16x8*>(base + ((term == 1 || term == 2) ? per : 0) + st_off);
    };
    bf16x8 cur0[SCH], cur1[SCH];
#pragma unroll
    for (int q = 0; q < SCH; ++q) {
      cur0[q] = state(0)[tid + q * NT];
      cur1[q] = state(1)[tid + q * NT];
    }

    // pairs inside the chunk: dy x^T tiles -> W (crossing sums) and E (dB, dC
    // weights).  Wave w keeps the t rows of tile w mod QT, so its row sums of
    // W stay in registers until the end; it walks the s tiles from a start
    // that differs from the other waves', so their column sums land on
    // different LDS words at any one time.
    {
      const int t0 = (wave % QT) * 16;
      float cs_t[4], csx_t[4], rf[4] = {0.f, 0.f, 0.f, 0.f}, rb[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        cs_t[r] = s_cs[t0 + 4 * lg + r];
        csx_t[r] = s_csx[t0 + 4 * lg + r];
      }
#pragma unroll 1
      for (int q = 0; q < CBT; ++q) {
        const int tile = wave + q * NW;
        if (tile >= QT * QT) break;
        const int s0 = ((tile / QT + wave % QT) % QT) * 16;
        f32x4 cb, dx = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r) cb[r] = static_cast<float>(cbq[r]);
        cbq = rotate_tiles(cbq);
#pragma unroll
        for (int k = 0; k < P; k += 32) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(sDY + (t0 + lr) * LDX + k + 8 * lg);
          const bf16x8 v = *reinterpret_cast<const bf16x8*>(sX + (s0 + lr) * LDX + k + 8 * lg);
          dx = mma(a, v, dx);
        }
        const int s2 = s0 + lr;
        const float ds = s_dt[s2], cs_s = s_cs[s2], csx_s = s_csx[s2];
        bf16x4 e4;
        // A tile below the diagonal holds forward pairs only (s < t), one
        // above it backward pairs only: one decay each, and one column sum.
        if (s0 < t0) {
          float cf = 0.f;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float df = __expf(cs_t[r] - cs_s);
            const float e = ds * dx[r];
            e4[r] = static_cast<__bf16>(e * df);
            const float wf = df * (e * cb[r]);
            rf[r] += wf;
            cf += wf;
          }
          cf = sum_rows(cf);
          if (lg == 0) atomicAdd(s_fw + s2, -cf);
        } else if (s0 > t0) {
          float cbk = 0.f;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float db = __expf(csx_s - csx_t[r]);
            const float e = ds * dx[r];
            e4[r] = static_cast<__bf16>(e * db);
            const float wb = db * (e * cb[r]);
            rb[r] += wb;
            cbk += wb;
          }
          cbk = sum_rows(cbk);
          if (lg == 0) atomicAdd(s_bw + s2, -cbk);
        } else {
          float cf = 0.f, cbk = 0.f;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = t0 + 4 * lg + r;
            const float df = s2 <= t ? __expf(cs_t[r] - cs_s) : 0.f;
            const float db = s2 >= t ? __expf(csx_s - csx_t[r]) : 0.f;
            const float e = ds * dx[r];
            e4[r] = static_cast<__bf16>(e * (df + db));
            const float v = e * cb[r];
            const float wf = s2 < t ? df * v : 0.f;
            const float wb = s2 > t ? db * v : 0.f;
            rf[r] += wf;
            rb[r] += wb;
            cf += wf;
            cbk += wb;
          }
          cf = sum_rows(cf);
          cbk = sum_rows(cbk);
          if (lg == 0) {
            atomicAdd(s_fw + s2, -cf);
            atomicAdd(s_bw + s2, -cbk);
          }
        }
        // E is stored transposed (row s, column t): the lane's four t are one 8-byte piece
        *reinterpret_cast<bf16x4*>(sE + s2 * LDE + t0 + 4 * lg) = e4;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        rf[r] = sum16(rf[r]);
        rb[r] = sum16(rb[r]);
      }
      if (lr < 4) {
        float f = rf[0], bk = rb[0];
#pragma unroll
        for (int r = 1; r < 4; ++r)
          if (lr == r) { f = rf[r]; bk = rb[r]; }
        atomicAdd(s_fw + t0 + 4 * lg + lr, f);
        atomicAdd(s_bw + t0 + 4 * lg + lr, bk);
      }
    }
    lds_barrier();   // E is complete
    // dC^T += B^T E^T (columns t = row block), dB^T += C^T E (columns s = row block)
    if (owns_rows) {
#pragma unroll 1
      for (int kb = 0; kb < Q; kb += 32) {
        const bf16x8 ea = tr_frag(sE, LDE, kb, r0, lane);                  // E rows r0.., k = s
        const bf16x8 et = perm_frag(sE + (r0 + lr) * LDE, kb, lane);     // E^T rows r0.., k = t
#pragma unroll
        for (int j = 0; j < NTL; ++j) {
          gC[j] = mma(tr_frag(sB, LDB, kb, 16 * j, lane), ea, gC[j]);
          gB[j] = mma(tr_frag(sC, LDB, kb, 16 * j, lane), et, gB[j]);
        }
      }
    }

    // pairs with one end outside the chunk, and their share of dC, dB: the
    // four terms in two rounds, each round the two states whose inner
    // product enters K ((hf1, hb2), then (hb1, hf2)), staged side by side
    float k = 0.f;
    // The round's two terms on one loop over the column tiles, so that each
    // tile carries two independent product chains: a U term (dy, C, into dC)
    // with the state in sM0 and a V term (x, B, into dB) with the state in
    // sM1.  Round 0: U_f with hf1, V_f with hb2; round 1: U_b with hb1, V_b
    // with hf2.
    auto do_terms = [&](int round) {
      // rows of dy and x as the MFMA's columns, k = p
      bf16x8 au[P / 32], av[P / 32];
#pragma unroll
      for (int kk = 0; kk < P / 32; ++kk) {
        au[kk] = perm_frag(sDY + (r0 + lr) * LDX, 32 * kk, lane);
        av[kk] = perm_frag(sX + (r0 + lr) * LDX, 32 * kk, lane);
      }
      // the terms' row scales for the lane's row t
      const int t = r0 + lr;
      const float su = round == 0 ? __expf(s_cs[t]) : __expf(cs_last - s_csx[t]);
      const float sv = round == 0 ? s_dt[t] * __expf(cs_last - s_cs[t]) : s_dt[t] * __expf(s_csx[t]);
      const __bf16* crow = sC + t * LDB + 4 * lg;
      const __bf16* brow = sB + t * LDB + 4 * lg;
      float pu = 0.f, pv = 0.f;
#pragma unroll
      for (int nt = 0; nt < NTL; ++nt) {
        const int n0 = nt * 16;
        // (state^T a^T)[n][t] for n = n0 + 4 lg + r
        f32x4 accu = {0.f, 0.f, 0.f, 0.f}, accv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < P / 32; ++kk) {
          accu = mma(tr_frag(sM0, LDB, 32 * kk, n0, lane), au[kk], accu);
          accv = mma(tr_frag(sM1, LDB, 32 * kk, n0, lane), av[kk], accv);
        }
        const bf16x4 c4 = *reinterpret_cast<const bf16x4*>(crow + n0);
        const bf16x4 b4 = *reinterpret_cast<const bf16x4*>(brow + n0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pu = fmaf(accu[r], static_cast<float>(c4[r]), pu);
          pv = fmaf(accv[r], static_cast<float>(b4[r]), pv);
          gC[nt][r] = fmaf(su, accu[r], gC[nt][r]);
          gB[nt][r] = fmaf(sv, accv[r], gB[nt][r]);
        }
      }
      pu = sum_rows(pu);
      pv = sum_rows(pv);
      if (lg == 0) {
        const float vu = su * pu, vv = sv * pv;
        if (round == 0) {
          s_fw[t] += vu;    // U_f
          s_bw[t] += vv;    // V_f
        } else {
          s_bw[t] += vu;    // U_b
          s_fw[t] += vv;    // V_b
        }
        s_sub[t] += vv;
      }
    };
#pragma unroll
    for (int round = 0; round < 2; ++round) {
      lds_barrier();   // E (and the previous states) are no longer read; the pair sums have landed
#pragma unroll
      for (int q = 0; q < SCH; ++q) {
        const int i = tid + q * NT;
#pragma unroll
        for (int e = 0; e < 8; ++e) k = fmaf(static_cast<float>(cur0[q][e]), static_cast<float>(cur1[q][e]), k);
        const int pp = (i * 8) / N, n = (i * 8) % N;
        *reinterpret_cast<bf16x8*>(sM0 + pp * LDB + n) = cur0[q];
        *reinterpret_cast<bf16x8*>(sM1 + pp * LDB + n) = cur1[q];
      }
      if (round == 0) {
#pragma unroll
        for (int q = 0; q < SCH; ++q) {
          cur0[q] = state(2)[tid + q * NT];
          cur1[q] = state(3)[tid + q * NT];
        }
      }
      lds_barrier();
      if (owns_rows) do_terms(round);
    }
    // this head's yhat rows, used at the end of the head.  The thread index
    // goes through an empty asm statement, so the addresses of this part are
    // formed anew in every head rather than kept in registers across the loop.
    constexpr int UT = Q * (P / 8) / NT;
    int tidh = tid;
    asm volatile("" : "+v"(tidh));
    bf16x8 yv[UT];
#pragma unroll
    for (int u = 0; u < UT; ++u) {
      const int i = tidh + u * NT, row = i / (P / 8), k8 = (i % (P / 8)) * 8;
      yv[u] = *reinterpret_cast<const bf16x8*>(yh + ((bl + s_tok[row]) * Hs + h) * P + k8);
    }
    k = __expf(cs_last) * block_sum512(k, red);   // its barriers also order the boundary terms before the scans

    // suffix sums of s_fw, prefix sums of s_bw, by wave 0 (the suffix sums as
    // prefix sums of the reversed order)
    if (wave == 0) {
      constexpr int V = Q / 64;
      float f[V], bk[V];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        f[e] = s_fw[Q - 1 - (V * lane + e)];
        bk[e] = s_bw[V * lane + e];
      }
      wave_prefix<V>(f);
      wave_prefix<V>(bk);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const int rf = Q - 1 - (V * lane + e), rb = V * lane + e;
        s_fw[rf] = f[e];
        s_bw[rb] = bk[e];
      }
    }
    lds_barrier();
    // the per-token gradients of this head: eight lanes per token row
    {
      const float two_d = 2.f * D[h];
      float da = 0.f, dd = 0.f;
#pragma unroll
      for (int u = 0; u < UT; ++u) {
        const int i = tidh + u * NT, row = i / (P / 8), k8 = (i % (P / 8)) * 8;
        const float dtr = s_dt[row];
        const float r = s_fw[row] + s_bw[row] - s_sub[row] + k;
        const bf16x8 xv = *reinterpret_cast<const bf16x8*>(sX + row * LDX + k8);
        const bf16x8 dv = *reinterpret_cast<const bf16x8*>(sDY + row * LDX + k8);
        float gx[8], xyh = 0.f, dyx = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float vx = static_cast<float>(xv[e]), vd = static_cast<float>(dv[e]);
          const float vh = static_cast<float>(yv[u][e]);
          xyh = fmaf(vx, vh, xyh);
          dyx = fmaf(vd, vx, dyx);
          gx[e] = fmaf(dtr, vh, two_d * vd);
        }
        const int64_t rh = (bl + s_tok[row]) * Hs + h;
        float4* o = reinterpret_cast<float4*>(dx + rh * P + k8);
        o[0] = make_float4(gx[0], gx[1], gx[2], gx[3]);
        o[1] = make_float4(gx[4], gx[5], gx[6], gx[7]);
        xyh = sum8(xyh);
        dyx = sum8(dyx);
        if (k8 == 0) {
          ddt[rh] = xyh + a_h * r;
          da += dtr * r;
          dd += 2.f * dyx;
        }
      }
      da = sum64(da);
      dd = sum64(dd);
      if (lane == 0) {
        atomicAdd(&s_hsum[0], da);
        atomicAdd(&s_hsum[1], dd);
      }
    }
  }
  lds_barrier();
  if (tid == 0) {   // the last head's dA, dD shares
    atomicAdd(dA + g * hpg + hpg - 1, s_hsum[0]);
    atomicAdd(dD + g * hpg + hpg - 1, s_hsum[1]);
  }

  // dB, dC of the chunk's tokens (row r0 + lr, columns 16 j + 4 lg .. + 3)
  if (owns_rows) {
    const int64_t row = ((bl + s_tok[r0 + lr]) * G + g) * N;
#pragma unroll
    for (int j = 0; j < NTL; ++j) {
      *reinterpret_cast<float4*>(dC + row + 16 * j + 4 * lg) = make_float4(gC[j][0], gC[j][1], gC[j][2], gC[j][3]);
      *reinterpret_cast<float4*>(dB + row + 16 * j + 4 * lg) = make_float4(gB[j][0], gB[j][1], gB[j][2], gB[j][3]);
    }
  }
}


// The same crossing sums and dB, dC for fp32 storage (the small family: head
// size 32, N = Q = 16), every product a plain fp32 loop over LDS rows: the
// chunk's Q x Q pairs and the P x N states are a few thousand
// multiply-adds per head.  One workgroup of 256 threads per (chunk, group,
// batch element); the states are the fp32 ones the chunk-state pass leaves.
template <int Q, int N, int P>
__global__ __launch_bounds__(256) void ma_bwd_cross_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ dy, const float* __restrict__ dt,
    const float* __restrict__ A, const float* __restrict__ B, const float* __restrict__ C,
    const float* __restrict__ st1, const float* __restrict__ st2, int64_t per, ScanOrder so, int L, int Hs, int G,
    int b, float* __restrict__ R, float* __restrict__ dB, float* __restrict__ dC) {
  constexpr int NT = 256, LQ = Q + 1, LN = N + 1, LP = P + 1;
  static_assert(Q <= 64 && Q * Q <= 4 * NT, "pairs per thread");
  __shared__ float sB[Q * LN], sC[Q * LN], sX[Q * LP], sDY[Q * LP], sE[Q * LQ];
  __shared__ float sS[4][P * LN];   // hf1, hb2, hb1, hf2 of the head
  __shared__ float gB[Q * LN], gC[Q * LN];
  __shared__ float s_cs[Q], s_csx[Q], s_dt[Q], s_fw[Q], s_bw[Q], s_sub[Q], s_k;
  __shared__ int s_tok[Q];
  const int c = blockIdx.x, g = blockIdx.y;
  const int hpg = Hs / G;
  const int tid = threadIdx.x;
  const int64_t bl = int64_t(b) * L;
  for (int i = tid; i < Q; i += NT) s_tok[i] = so.canon(c * Q + i);
  __syncthreads();
  for (int u = tid; u < Q * N; u += NT) {
    const int i = u / N, n = u % N;
    const int64_t src = ((bl + s_tok[i]) * G + g) * N + n;
    sB[i * LN + n] = B[src];
    sC[i * LN + n] = C[src];
    gB[i * LN + n] = 0.f;
    gC[i * LN + n] = 0.f;
  }
#pragma unroll 1
  for (int hh = 0; hh < hpg; ++hh) {
    const int h = g * hpg + hh;
    const float a_h = A[h];
    __syncthreads();   // the previous head is done with every shared array
    for (int u = tid; u < Q * P; u += NT) {
      const int i = u / P, p = u % P;
      const int64_t src = ((bl + s_tok[i]) * Hs + h) * P + p;
      sX[i * LP + p] = x[src];
      sDY[i * LP + p] = dy[src];
    }
    const int64_t st_off = (int64_t(c) * Hs + h) * int64_t(P) * N;
    for (int u = tid; u < P * N; u += NT) {
      const int p = u / N, n = u % N;
      sS[0][p * LN + n] = st1[st_off + u];          // hf1: forward state entering the chunk
      sS[1][p * LN + n] = st2[per + st_off + u];    // hb2: adjoint state of the forward scan
      sS[2][p * LN + n] = st1[per + st_off + u];    // hb1: reverse state entering from the right
      sS[3][p * LN + n] = st2[st_off + u];          // hf2: adjoint state of the reverse scan
    }
    if (tid < Q) {
      s_dt[tid] = dt[(bl + s_tok[tid]) * Hs + h];
      s_fw[tid] = s_bw[tid] = s_sub[tid] = 0.f;
    }
    if (tid == 0) s_k = 0.f;
    __syncthreads();
    if (tid == 0) {   // chunk-local cumulative sums of dt*A, inclusive and exclusive
      float run = 0.f;
      for (int i = 0; i < Q; ++i) {
        const float a = s_dt[i] * a_h;
        run += a;
        s_cs[i] = run;
        s_csx[i] = run - a;
      }
    }
    __syncthreads();
    const float cs_last = s_cs[Q - 1];
    // pairs inside the chunk: E (dB, dC weights) and W's row and column sums
    for (int u = tid; u < Q * Q; u += NT) {
      const int t = u / Q, s2 = u % Q;
      float dx = 0.f, cb = 0.f;
      for (int p = 0; p < P; ++p) dx = fmaf(sDY[t * LP + p], sX[s2 * LP + p], dx);
      for (int n = 0; n < N; ++n) cb = fmaf(sC[t * LN + n], sB[s2 * LN + n], cb);
      const float df = s2 <= t ? __expf(s_cs[t] - s_cs[s2]) : 0.f;
      const float db = s2 >= t ? __expf(s_csx[s2] - s_csx[t]) : 0.f;
      const float e = s_dt[s2] * dx;
      sE[t * LQ + s2] = e * (df + db);
      const float v = e * cb;
      const float wf = s2 < t ? df * v : 0.f;
      const float wb = s2 > t ? db * v : 0.f;
      atomicAdd(s_fw + t, wf);
      atomicAdd(s_bw + t, wb);
      atomicAdd(s_fw + s2, -wf);
      atomicAdd(s_bw + s2, -wb);
    }
    __syncthreads();
    // dC_t += sum_s E_ts B_s,  dB_s += sum_t E_ts C_t
    for (int u = tid; u < Q * N; u += NT) {
      const int i = u / N, n = u % N;
      float gc = 0.f, gb = 0.f;
      for (int j = 0; j < Q; ++j) {
        gc = fmaf(sE[i * LQ + j], sB[j * LN + n], gc);
        gb = fmaf(sE[j * LQ + i], sC[j * LN + n], gb);
      }
      gC[i * LN + n] += gc;
      gB[i * LN + n] += gb;
    }
    __syncthreads();   // before the boundary terms add to gC, gB
    // pairs with one end outside the chunk: per row t and term, the state
    // applied to the row's dy (U terms) or x (V terms), its product with the
    // row's C or B, and its share of dC or dB
    for (int u = tid; u < 4 * Q; u += NT) {
      const int term = u / Q, t = u % Q;
      const bool is_u = (term == 0 || term == 2);
      const float* a = is_u ? &sDY[t * LP] : &sX[t * LP];
      const float* vr = is_u ? &sC[t * LN] : &sB[t * LN];
      const float scale = term == 0 ? __expf(s_cs[t])
                        : term == 1 ? s_dt[t] * __expf(cs_last - s_cs[t])
                        : term == 2 ? __expf(cs_last - s_csx[t])
                                    : s_dt[t] * __expf(s_csx[t]);
      const float* st = sS[term];
      float part = 0.f;
      for (int n = 0; n < N; ++n) {
        float acc = 0.f;
        for (int p = 0; p < P; ++p) acc = fmaf(st[p * LN + n], a[p], acc);
        part = fmaf(acc, vr[n], part);
        atomicAdd(is_u ? &gC[t * LN + n] : &gB[t * LN + n], scale * acc);
      }
      const float v = scale * part;
      if (term == 0) atomicAdd(s_fw + t, v);                                        // U_f
      else if (term == 1) { atomicAdd(s_bw + t, v); atomicAdd(s_sub + t, v); }     // V_f
      else if (term == 2) atomicAdd(s_bw + t, v);                                   // U_b
      else { atomicAdd(s_fw + t, v); atomicAdd(s_sub + t, v); }                     // V_b
    }
    // both ends outside: K = e^{cs_last} (<hf1, hb2> + <hb1, hf2>)
    float k = 0.f;
    for (int u = tid; u < P * N; u += NT) {
      const int p = u / N, n = u % N;
      k = fmaf(sS[0][p * LN + n], sS[1][p * LN + n], k);
      k = fmaf(sS[2][p * LN + n], sS[3][p * LN + n], k);
    }
    atomicAdd(&s_k, k);
    __syncthreads();
    if (tid == 0) {
      const float kk = s_k * __expf(cs_last);
      // suffix sums of s_fw, prefix sums of s_bw, then R
      float suf = 0.f, pre = 0.f;
      for (int i = Q - 1; i >= 0; --i) { suf += s_fw[i]; s_fw[i] = suf; }
      for (int i = 0; i < Q; ++i) { pre += s_bw[i]; s_bw[i] = pre; }
      for (int i = 0; i < Q; ++i) R[(bl + s_tok[i]) * Hs + h] = s_fw[i] + s_bw[i] - s_sub[i] + kk;
    }
  }
  __syncthreads();
  for (int u = tid; u < Q * N; u += NT) {
    const int i = u / N, n = u % N;
    const int64_t row = ((bl + s_tok[i]) * G + g) * N + n;
    dC[row] = gC[i * LN + n];
    dB[row] = gB[i * LN + n];
  }
}

// Per token and head (head size 64), in canonical order (nothing here
// depends on the scan order or the chunks):
//   dx = dt yhat + 2 D dy,  ddt = x . yhat + A R,
// and the shares of dA = sum dt R and dD = 2 sum dy . x, with yhat =
// (M_f^T + M_b^T) dy / dt and R the crossing sums.  A workgroup takes
// kTokRows consecutive token rows and a slice of 32 heads: eight lanes share
// a head's 128-byte row (16 bytes each), so with 32 heads or more the
// workgroup reads 4 KiB of contiguous row per token.  A lane's head is
// fixed, so its dA, dD shares stay in registers until one atomic per head
// and workgroup.  kTokUnroll tokens' loads are issued before any is used.
// (fp32 storage: head size 32, eight lanes of four elements per head row.)
constexpr int kTokRows = 64, kTokUnroll = 4;
template <typename TS>
union Piece16 {
  uint4 u;
  TS e[16 / sizeof(TS)];
};
template <typename TS>
__global__ __launch_bounds__(256) void ma_bwd_token_kernel(
    const TS* __restrict__ x, const TS* __restrict__ dy, const float* __restrict__ dt,
    const float* __restrict__ A, const float* __restrict__ D, const TS* __restrict__ yh,
    const float* __restrict__ R, int64_t rows, int Hs, float* __restrict__ dx, float* __restrict__ ddt,
    float* __restrict__ dA, float* __restrict__ dD) {
  constexpr int V = 16 / int(sizeof(TS)), P = 8 * V, U = kTokUnroll;
  const int sub = threadIdx.x & 7;
  const int h = int(blockIdx.y) * 32 + int(threadIdx.x >> 3);
  const bool active = h < Hs;   // whole groups of eight lanes
  const int hc = active ? h : 0;
  const float two_d = 2.f * D[hc], a_h = A[hc];
  const int64_t r0 = int64_t(blockIdx.x) * kTokRows;
  const int nr = int(rows - r0 < kTokRows ? rows - r0 : kTokRows);
  float da = 0.f, dd = 0.f;
  for (int i0 = 0; i0 < nr; i0 += U) {
    int64_t rh[U];
    bool ok[U];
    float d[U], r[U];
    Piece16<TS> bx[U], bdy[U], bh[U];   // kept in the storage type until used
#pragma unroll
    for (int u = 0; u < U; ++u) {
      ok[u] = active && i0 + u < nr;
      rh[u] = (r0 + i0 + u) * Hs + hc;
      d[u] = r[u] = 0.f;
      bx[u].u = bdy[u].u = bh[u].u = uint4{0u, 0u, 0u, 0u};
      if (ok[u]) {
        d[u] = dt[rh[u]];
        r[u] = R[rh[u]];
        const int64_t off = rh[u] * P + sub * V;
        bx[u].u = *reinterpret_cast<const uint4*>(x + off);
        bdy[u].u = *reinterpret_cast<const uint4*>(dy + off);
        bh[u].u = *reinterpret_cast<const uint4*>(yh + off);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float gx[V], xyh = 0.f, dyx = 0.f;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float vx = to_f32(bx[u].e[e]), vdy = to_f32(bdy[u].e[e]), vh = to_f32(bh[u].e[e]);
        xyh = fmaf(vx, vh, xyh);
        dyx = fmaf(vdy, vx, dyx);
        gx[e] = fmaf(d[u], vh, two_d * vdy);
      }
      if (ok[u]) {
        float4* o = reinterpret_cast<float4*>(dx + rh[u] * P + sub * V);
#pragma unroll
        for (int q4 = 0; q4 < V / 4; ++q4) o[q4] = make_float4(gx[4 * q4], gx[4 * q4 + 1], gx[4 * q4 + 2], gx[4 * q4 + 3]);
      }
      xyh = sum8(xyh);
      dyx = sum8(dyx);
      if (ok[u] && sub == 0) {
        ddt[rh[u]] = xyh + a_h * r[u];
        da += d[u] * r[u];
        dd += 2.f * dyx;
      }
    }
  }
  if (active && sub == 0) {
    atomicAdd(dA + h, da);
    atomicAdd(dD + h, dd);
  }
}

// ---------------------------------------------------------------------------
// Review tokens.  The review state h_R (the state the pooled review tokens
// leave, scanned once from zero in canonical order, their outputs
// discarded) starts both directions, so the adjoint reaching it is the sum
// of the two directions' initial-state adjoints, dhR: the final carries of
// the adjoint state pass (the upward walk's carry is the reverse
// direction's, the downward walk's the forward direction's).  Walking the
// review scan backwards from dhR with no output adjoint gives, per head,
// with w_r = exp(A sum_{r' > r} dt_r') and K_r = <dhR, x_r B_r^T>:
//   dx_r  = w_r dt_r dhR B_r,        dB_r = w_r dt_r dhR^T x_r (over the group's heads),
//   ddt_r = w_r K_r + A sum_{r' < r} w_r' dt_r' K_r',
//   dA   += sum_r w_r dt_r K_r sum_{r' > r} dt_r'.
// Each pooled value is a block mean, so its gradient is then spread evenly
// over the tokens of its pooling block.
// ---------------------------------------------------------------------------

constexpr int kRevMaxP = 64, kRevMaxN = 128, kRevMaxR = 256;

// Zero n floats (grid-stride).
__global__ __launch_bounds__(kThreads) void zero_kernel(float* __restrict__ a, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < n; i += int64_t(gridDim.x) * kThreads) a[i] = 0.f;
}

// One workgroup per head.  h_last: fp32 [2][Hs][P][N]; rx [R][Hs][P], rdt
// [R][Hs], rb [R][G][N] (the pooled review tokens); gx, gdt like rx, rdt;
// gb like rb, zeroed by the caller (heads of a group add into it).
__global__ __launch_bounds__(kThreads) void review_bwd_kernel(const float* __restrict__ h_last,
                                                             const float* __restrict__ rx,
                                                             const float* __restrict__ rdt,
                                                             const float* __restrict__ rb,
                                                             const float* __restrict__ A, int R, int Hs, int P, int N,
                                                             int G, float* __restrict__ gx, float* __restrict__ gdt,
                                                             float* __restrict__ gb, float* __restrict__ dA) {
  // dhR rows padded by one float: the threads of the first product walk a
  // column (stride N + 1), those of the second a row.
  __shared__ float dh[kRevMaxP * (kRevMaxN + 1)];
  __shared__ float sx[kRevMaxP], sb[kRevMaxN], su[kRevMaxP];
  __shared__ float sw[kRevMaxR], sK[kRevMaxR];
  const int h = blockIdx.x, tid = threadIdx.x;
  const int grp = h / (Hs / G);
  const int64_t PN = int64_t(P) * N;
  for (int i = tid; i < P * N; i += kThreads)
    dh[(i / N) * (N + 1) + i % N] = h_last[int64_t(h) * PN + i] + h_last[(int64_t(Hs) + h) * PN + i];
  if (tid == 0) {
    float suf = 0.f;
    for (int r = R - 1; r >= 0; --r) {
      sw[r] = expf(A[h] * suf);
      suf += rdt[int64_t(r) * Hs + h];
    }
  }
  lds_barrier();
  for (int r = 0; r < R; ++r) {
    for (int p = tid; p < P; p += kThreads) sx[p] = rx[(int64_t(r) * Hs + h) * P + p];
    for (int n = tid; n < N; n += kThreads) sb[n] = rb[(int64_t(r) * G + grp) * N + n];
    lds_barrier();
    const float wd = sw[r] * rdt[int64_t(r) * Hs + h];
    for (int p = tid; p < P; p += kThreads) {
      float u = 0.f;
      for (int n = 0; n < N; ++n) u = fmaf(dh[p * (N + 1) + n], sb[n], u);
      su[p] = u;
      gx[(int64_t(r) * Hs + h) * P + p] = wd * u;
    }
    for (int n = tid; n < N; n += kThreads) {
      float v = 0.f;
      for (int p = 0; p < P; ++p) v = fmaf(dh[p * (N + 1) + n], sx[p], v);
      atomicAdd(&gb[(int64_t(r) * G + grp) * N + n], wd * v);
    }
    lds_barrier();
    if (tid < 64) {
      float k = 0.f;
      for (int p = tid; p < P; p += 64) k = fmaf(sx[p], su[p], k);
      k = sum64(k);
      if (tid == 0) sK[r] = k;
    }
    lds_barrier();
  }
  if (tid == 0) {
    float pre = 0.f;   // sum_{r' < r} w_r' dt_r' K_r'
    for (int r = 0; r < R; ++r) {
      const float d = rdt[int64_t(r) * Hs + h];
      gdt[int64_t(r) * Hs + h] = sw[r] * sK[r] + A[h] * pre;
      pre += sw[r] * d * sK[r];
    }
    float suf = 0.f, da = 0.f;   // suf = sum_{r' > r} dt_r'
    for (int r = R - 1; r >= 0; --r) {
      const float d = rdt[int64_t(r) * Hs + h];
      da += sw[r] * d * sK[r] * suf;
      suf += d;
    }
    atomicAdd(dA + h, da);
  }
}

// Review block geometry: pooling block, points per axis and the stride
// between sampled blocks (in blocks).
struct RevGeom {
  int pt, ph, pw, rt, rh, rw, st, sh, sw;
};

// Adds 1/|block| of review token r's gradients (gx, gdt, gb of batch
// element blockIdx.z) to every token of its pooling block.  Grid (R,
// tokens per block, batch); blocks are disjoint, so no two workgroups touch
// one token.
__global__ __launch_bounds__(kThreads) void review_scatter_kernel(const float* __restrict__ gx,
                                                                 const float* __restrict__ gdt,
                                                                 const float* __restrict__ gb, RevGeom g, int R,
                                                                 int T, int H, int W, int Hs, int P, int G, int N,
                                                                 float* __restrict__ dx, float* __restrict__ ddt,
                                                                 float* __restrict__ dB) {
  const int r = blockIdx.x, tl = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int i = r / (g.rh * g.rw), j = (r / g.rw) % g.rh, k = r % g.rw;
  const int a = tl / (g.ph * g.pw), bb = (tl / g.pw) % g.ph, c = tl % g.pw;
  const int64_t L = int64_t(T) * H * W;
  const int64_t tok = int64_t(b) * L +
                      ((int64_t(i * g.st * g.pt + a) * H + (j * g.sh * g.ph + bb)) * W + (k * g.sw * g.pw + c));
  const float inv = 1.f / float(g.pt * g.ph * g.pw);
  const int64_t rr = int64_t(b) * R + r;
  for (int e = tid; e < Hs * P; e += kThreads) dx[tok * Hs * P + e] += gx[rr * Hs * P + e] * inv;
  for (int e = tid; e < Hs; e += kThreads) ddt[tok * Hs + e] += gdt[rr * Hs + e] * inv;
  for (int e = tid; e < G * N; e += kThreads) dB[tok * G * N + e] += gb[rr * G * N + e] * inv;
}

// Byte offsets inside the caller's workspace.
struct BwdWs {
  size_t scan1, scan2, R, yh, hlast, gx, gdt, gb, total;
};

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// saved: the forward scan states come from the caller's saved buffer (no
// first scan workspace).
int bwd_layout(const lingen_mate_shape* s, BwdWs* w, bool saved = false) {
  const size_t rows = size_t(s->batch) * size_t(tokens(s));
  const size_t hs = size_t(s->ssd_heads), P = size_t(s->headdim);
  size_t ws_main = 0;
  if (int rc = lingen_mate_workspace_bytes(s, &ws_main)) return rc;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += align256(bytes); return o; };
  w->scan1 = take(saved ? 0 : ws_main);
  w->scan2 = take(ws_main);
  w->R = take(rows * hs * 4);
  w->yh = take(rows * hs * P * (s->dtype == LINGEN_BF16 ? 2 : 4));
  // review tokens: the adjoint states' final carries (one batch element at
  // a time) and the pooled tokens' gradients of every batch element
  const size_t nr = size_t(s->batch) * size_t(s->n_review);
  w->hlast = take(s->n_review ? 2 * hs * P * size_t(s->d_state) * 4 : 0);
  w->gx = take(nr * hs * P * 4);
  w->gdt = take(nr * hs * 4);
  w->gb = take(nr * size_t(s->ngroups) * size_t(s->d_state) * 4);
  w->total = off;
  return LINGEN_OK;
}

// The saved buffer of lingen_ma_fwd_saved: per batch element one forward
// workspace (ws_layout), which keeps that element's chunk states (and, with
// review tokens, the pooled review tokens) after the forward.
size_t saved_stride(const lingen_mate_shape* s) { return align256(ws_layout(s).total); }

// The crossing-sum kernels are compiled for the three scan families: bf16
// with P = 64 and N = Q = 64 or 128 (MFMA tiles), fp32 with P = 32 and
// N = Q = 16 (fp32 loops).
int check_bwd_shape(const lingen_mate_shape* s) {
  if (int rc = validate_shape(s)) return rc;
  if (s->dtype == LINGEN_BF16) {
    if (s->headdim != 64) return LINGEN_ERR_UNSUPPORTED;
    if (!((s->chunk == 64 && s->d_state == 64) || (s->chunk == 128 && s->d_state == 128))) return LINGEN_ERR_UNSUPPORTED;
    return LINGEN_OK;
  }
  if (s->headdim != 32 || s->chunk != 16 || s->d_state != 16) return LINGEN_ERR_UNSUPPORTED;
  return LINGEN_OK;
}


}  // namespace
}  // namespace lingen

using namespace lingen;

extern "C" int lingen_ma_bwd_workspace_bytes(const lingen_mate_shape* shape, size_t* bytes) {
  if (bytes == nullptr) return LINGEN_ERR_NULL;
  if (int rc = check_bwd_shape(shape)) return rc;
  BwdWs w{};
  if (int rc = bwd_layout(shape, &w)) return rc;
  *bytes = w.total;
  return LINGEN_OK;
}

namespace lingen {
namespace {
// The backward pass; saved (nullable) holds the forward scan states of every
// batch element as lingen_ma_fwd_saved left them, which replaces the first
// of the two chunk-state passes.
int ma_bwd_impl(const void* x, const float* dt, const float* A, const void* B, const void* C, const float* D,
                const void* dy, const void* saved, size_t saved_bytes, int32_t mode, const lingen_mate_shape* shape,
                float* dx, float* ddt, float* dA, float* dB, float* dC, float* dD, void* workspace,
                size_t workspace_bytes, hipStream_t stream) {
  if (int rc = check_bwd_shape(shape)) return rc;
  if (mode < 0 || mode > 3) return LINGEN_ERR_SHAPE;
  const void* ptrs[] = {x, dt, A, B, C, D, dy, dx, ddt, dA, dB, dC, dD, workspace};
  for (const void* p : ptrs)
    if (int rc = check_ptr(p)) return rc;
  if (saved != nullptr && saved_bytes < size_t(shape->batch) * saved_stride(shape)) return LINGEN_ERR_WORKSPACE;
  BwdWs w{};
  if (int rc = bwd_layout(shape, &w, saved != nullptr)) return rc;
  if (workspace_bytes < w.total) return LINGEN_ERR_WORKSPACE;

  char* ws = static_cast<char*>(workspace);
  auto at = [&](size_t off) { return static_cast<void*>(ws + off); };
  auto atf = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  const int L = int(tokens(shape)), Hs = shape->ssd_heads, P = shape->headdim, N = shape->d_state;
  const int G = shape->ngroups, Q = shape->chunk, nc = L / Q;
  const int64_t rows = int64_t(shape->batch) * L;
  const ScanOrder so{mode, shape->T, shape->H, shape->W};
  const __bf16* xb = static_cast<const __bf16*>(x);
  const __bf16* dyb = static_cast<const __bf16*>(dy);
  const bool f32 = shape->dtype == LINGEN_F32;
  int rc;
#define LINGEN_TRY(expr)                          \
  do {                                            \
    if ((rc = (expr)) != LINGEN_OK) return rc;    \
  } while (0)
#define LINGEN_LAUNCHED()                                             \
  do {                                                                \
    if (launch_status(__func__) != LINGEN_OK) return LINGEN_ERR_HIP;       \
  } while (0)

  // dA and dD accumulate from zero
  zero_floats_kernel<<<1, kThreads, 0, stream>>>(dA, dD, Hs);
  LINGEN_LAUNCHED();
  const int R = shape->n_review;
  lingen_mate_shape plain = *shape;   // the same scan without review tokens
  plain.n_review = 0;
  if (R) {
    const int64_t nb = int64_t(shape->batch) * R * G * N;   // the pooled B gradients add over heads
    zero_kernel<<<blocks_for(nb) < 1024 ? blocks_for(nb) : 1024, kThreads, 0, stream>>>(atf(w.gb), nb);
    LINGEN_LAUNCHED();
  }

  // crossing sums, then ddt, dx, dA, dD
  {
    const dim3 cgrid{unsigned(nc), unsigned(G), 1u};
    const WsLayout lay = ws_layout(shape);
    const int64_t per = int64_t(nc) * Hs * P * N;   // one direction's scan states
    const __bf16* st2 = reinterpret_cast<const __bf16*>(ws + w.scan2 + lay.states);
    const int64_t eb = f32 ? 4 : 2;
    for (int bi = 0; bi < shape->batch; ++bi) {
      // forward / reverse states of (x, B) and of (x', C) for this batch element, left in the two workspaces
      // (the first one saved by the forward, when given)
      const int64_t xo = int64_t(bi) * L * Hs * P * eb, bo = int64_t(bi) * L * G * N * eb;
      const char* scan1 = saved ? static_cast<const char*>(saved) + size_t(bi) * saved_stride(shape) : ws + w.scan1;
      const __bf16* st1 = reinterpret_cast<const __bf16*>(scan1 + lay.states);
      // with review tokens, this pass also pools them (into scan1's review
      // buffers) and starts both walks from their state
      if (!saved)
        LINGEN_TRY(scan_states_one(shape, mode, static_cast<const char*>(x) + xo, dt + int64_t(bi) * L * Hs, A,
                                   static_cast<const char*>(B) + bo, ws + w.scan1, stream, kWeightDt, nullptr));
      // the adjoint scan has no review state; its final carries are the
      // adjoints of the two directions' initial states
      LINGEN_TRY(scan_states_one(&plain, mode, static_cast<const char*>(dy) + xo, dt + int64_t(bi) * L * Hs, A,
                                 static_cast<const char*>(C) + bo, ws + w.scan2, stream, kWeightAdjoint,
                                 R ? atf(w.hlast) : nullptr));
      // the transposed outputs yhat = (M_f^T + M_b^T) dy / dt from the same adjoint states
      LINGEN_TRY(ma_transposed_one(&plain, mode, static_cast<const char*>(dy) + xo, dt + int64_t(bi) * L * Hs, A,
                                   static_cast<const char*>(B) + bo, static_cast<const char*>(C) + bo, ws + w.scan2,
                                   static_cast<char*>(at(w.yh)) + xo, stream));
      if (R) {
        const WsLayout rl = ws_layout(shape);
        const float* s1 = reinterpret_cast<const float*>(scan1);
        review_bwd_kernel<<<Hs, kThreads, 0, stream>>>(
            atf(w.hlast), s1 + rl.review_x / 4, s1 + rl.review_dt / 4, s1 + rl.review_b / 4, A, R, Hs, P, N, G,
            atf(w.gx) + int64_t(bi) * R * Hs * P, atf(w.gdt) + int64_t(bi) * R * Hs,
            atf(w.gb) + int64_t(bi) * R * G * N, dA);
        LINGEN_LAUNCHED();
      }
      if (f32)
        ma_bwd_cross_f32_kernel<16, 16, 32><<<cgrid, 256, 0, stream>>>(
            static_cast<const float*>(x), static_cast<const float*>(dy), dt, A, static_cast<const float*>(B),
            static_cast<const float*>(C), reinterpret_cast<const float*>(st1), reinterpret_cast<const float*>(st2),
            per, so, L, Hs, G, bi, atf(w.R), dB, dC);
      else if (Q == 128 && N == 128)
        ma_bwd_cross_kernel<128, 128><<<cgrid, kCrossThreads, 0, stream>>>(
            xb, dyb, dt, A, static_cast<const __bf16*>(B), static_cast<const __bf16*>(C), st1, st2, per, so, L, Hs,
            G, bi, static_cast<const __bf16*>(at(w.yh)), D, dx, ddt, dA, dD, dB, dC);
      else if (Q == 64 && N == 64)
        ma_bwd_cross_kernel<64, 64><<<cgrid, kCrossThreads, 0, stream>>>(
            xb, dyb, dt, A, static_cast<const __bf16*>(B), static_cast<const __bf16*>(C), st1, st2, per, so, L, Hs,
            G, bi, static_cast<const __bf16*>(at(w.yh)), D, dx, ddt, dA, dD, dB, dC);
      else
        return LINGEN_ERR_UNSUPPORTED;
      LINGEN_LAUNCHED();
    }
    // (the bf16 crossing-sum kernels form the per-token gradients themselves)
    if (f32) {
      const dim3 tgrid{unsigned((rows + kTokRows - 1) / kTokRows), unsigned((Hs + 31) / 32), 1u};
      ma_bwd_token_kernel<float><<<tgrid, 256, 0, stream>>>(static_cast<const float*>(x),
                                                            static_cast<const float*>(dy), dt, A, D,
                                                            static_cast<const float*>(at(w.yh)), atf(w.R), rows, Hs,
                                                            dx, ddt, dA, dD);
      LINGEN_LAUNCHED();
    }
    if (R) {
      RevGeom g;
      g.pt = shape->rpool_t; g.ph = shape->rpool_h; g.pw = shape->rpool_w;
      g.rt = shape->rgrid_t; g.rh = shape->rgrid_h; g.rw = shape->rgrid_w;
      g.st = (shape->T / g.pt) / g.rt; g.sh = (shape->H / g.ph) / g.rh; g.sw = (shape->W / g.pw) / g.rw;
      const dim3 sgrid{unsigned(R), unsigned(g.pt * g.ph * g.pw), unsigned(shape->batch)};
      review_scatter_kernel<<<sgrid, kThreads, 0, stream>>>(atf(w.gx), atf(w.gdt), atf(w.gb), g, R, shape->T,
                                                           shape->H, shape->W, Hs, P, G, N, dx, ddt, dB);
      LINGEN_LAUNCHED();
    }
  }
#undef LINGEN_TRY
#undef LINGEN_LAUNCHED
  return LINGEN_OK;
}
}  // namespace
}  // namespace lingen

extern "C" int lingen_ma_bwd(const void* x, const float* dt, const float* A, const void* B, const void* C,
                             const float* D, const void* dy, int32_t mode, const lingen_mate_shape* shape,
                             float* dx, float* ddt, float* dA, float* dB, float* dC, float* dD, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  return ma_bwd_impl(x, dt, A, B, C, D, dy, nullptr, 0, mode, shape, dx, ddt, dA, dB, dC, dD, workspace,
                     workspace_bytes, stream);
}

extern "C" int lingen_ma_saved_bytes(const lingen_mate_shape* shape, size_t* bytes) {
  if (bytes == nullptr) return LINGEN_ERR_NULL;
  if (int rc = check_bwd_shape(shape)) return rc;
  *bytes = size_t(shape->batch) * saved_stride(shape);
  return LINGEN_OK;
}

extern "C" int lingen_ma_fwd_saved(const void* x, const float* dt, const float* A, const void* B, const void* C,
                                   const float* D, int32_t mode, const lingen_mate_shape* shape, void* y_ma,
                                   void* saved, size_t saved_bytes, hipStream_t stream) {
  if (int rc = check_bwd_shape(shape)) return rc;
  if (mode < 0 || mode > 3) return LINGEN_ERR_SHAPE;
  const void* ptrs[] = {x, dt, A, B, C, D, y_ma, saved};
  for (const void* p : ptrs)
    if (int rc = check_ptr(p)) return rc;
  const size_t stride = saved_stride(shape);
  if (saved_bytes < size_t(shape->batch) * stride) return LINGEN_ERR_WORKSPACE;
  // one batch element at a time, each with its own slice of the saved
  // buffer as the forward's workspace
  lingen_mate_shape one = *shape;
  one.batch = 1;
  const int64_t L = tokens(shape), Hs = shape->ssd_heads, P = shape->headdim;
  const int64_t bn = int64_t(shape->ngroups) * shape->d_state;
  const int64_t eb = shape->dtype == LINGEN_F32 ? 4 : 2;
  for (int bi = 0; bi < shape->batch; ++bi) {
    const int64_t xo = bi * L * Hs * P * eb, bo = bi * L * bn * eb;
    if (int rc = lingen_ma_fwd(static_cast<const char*>(x) + xo, dt + bi * L * Hs, A,
                               static_cast<const char*>(B) + bo, static_cast<const char*>(C) + bo, D, mode, &one,
                               static_cast<char*>(y_ma) + xo, static_cast<char*>(saved) + size_t(bi) * stride,
                               stride, stream))
      return rc;
  }
  return LINGEN_OK;
}

extern "C" int lingen_ma_bwd_saved_workspace_bytes(const lingen_mate_shape* shape, size_t* bytes) {
  if (bytes == nullptr) return LINGEN_ERR_NULL;
  if (int rc = check_bwd_shape(shape)) return rc;
  BwdWs w{};
  if (int rc = bwd_layout(shape, &w, true)) return rc;
  *bytes = w.total;
  return LINGEN_OK;
}

extern "C" int lingen_ma_bwd_saved(const void* x, const float* dt, const float* A, const void* B, const void* C,
                                   const float* D, const void* dy, const void* saved, size_t saved_bytes,
                                   int32_t mode, const lingen_mate_shape* shape, float* dx, float* ddt, float* dA,
                                   float* dB, float* dC, float* dD, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  if (int rc = check_ptr(saved)) return rc;
  return ma_bwd_impl(x, dt, A, B, C, D, dy, saved, saved_bytes, mode, shape, dx, ddt, dA, dB, dC, dD, workspace,
                     workspace_bytes, stream);
}
