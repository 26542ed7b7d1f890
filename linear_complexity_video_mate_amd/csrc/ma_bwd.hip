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
// size 64): the crossing sums R_r behind ddt and dA, written to R [batch, L,
// Hs], and the gradients dB, dC of the chunk's tokens, written to [batch, L,
// G, N] fp32.  With cs the chunk-local inclusive cumulative sum of dt*A
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
    int G, int b, float* __restrict__ R, float* __restrict__ dB, float* __restrict__ dC) {
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
  __shared__ __attribute__((aligned(16))) __bf16 sU[U_ELEMS];   // E (Q x Q), then a state (P x N rows)
  __shared__ float s_cs[Q], s_csx[Q], s_dt[Q], s_fw[Q], s_bw[Q], s_sub[Q], red[NW];
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

#pragma unroll 1
  for (int hh = 0; hh < hpg; ++hh) {
    const int h = g * hpg + hh;
    const float a_h = A[h];
    lds_barrier();   // the previous head is done with every shared array
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
        f32x4 cb = {0.f, 0.f, 0.f, 0.f}, dx = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < N; k += 32) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(sC + (t0 + lr) * LDB + k + 8 * lg);
          const bf16x8 v = *reinterpret_cast<const bf16x8*>(sB + (s0 + lr) * LDB + k + 8 * lg);
          cb = mma(a, v, cb);
        }
#pragma unroll
        for (int k = 0; k < P; k += 32) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(sDY + (t0 + lr) * LDX + k + 8 * lg);
          const bf16x8 v = *reinterpret_cast<const bf16x8*>(sX + (s0 + lr) * LDX + k + 8 * lg);
          dx = mma(a, v, dx);
        }
        const int s2 = s0 + lr;
        const float ds = s_dt[s2], cs_s = s_cs[s2], csx_s = s_csx[s2];
        float cf = 0.f, cbk = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = t0 + 4 * lg + r;
          const float df = s2 <= t ? __expf(cs_t[r] - cs_s) : 0.f;
          const float db = s2 >= t ? __expf(csx_s - csx_t[r]) : 0.f;
          const float e = ds * dx[r];
          sE[t * LDE + s2] = static_cast<__bf16>(e * (df + db));
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
        const bf16x8 ea = perm_frag(sE + (r0 + lr) * LDE, kb, lane);     // E rows r0.., k = s
        const bf16x8 et = tr_frag(sE, LDE, kb, r0, lane);                  // E^T rows r0.., k = t
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
    auto do_term = [&](int term, const __bf16* sMt) {
      const bool is_u = (term == 0 || term == 2);          // U terms: dy, C, dC; V terms: x, B, dB
      const __bf16* sa = is_u ? sDY : sX;
      const __bf16* sv = is_u ? sC : sB;
      // rows of the term's operand (dy or x) as the MFMA's columns, k = p
      bf16x8 af[P / 32];
#pragma unroll
      for (int kk = 0; kk < P / 32; ++kk) af[kk] = perm_frag(sa + (r0 + lr) * LDX, 32 * kk, lane);
      // the row scale of this term for the lane's row t
      const int t = r0 + lr;
      const float scale = term == 0 ? __expf(s_cs[t])
                        : term == 1 ? s_dt[t] * __expf(cs_last - s_cs[t])
                        : term == 2 ? __expf(cs_last - s_csx[t])
                                    : s_dt[t] * __expf(s_csx[t]);
      const __bf16* svr = sv + t * LDB + 4 * lg;
      float part = 0.f;
#pragma unroll
      for (int nt = 0; nt < NTL; ++nt) {
        const int n0 = nt * 16;
        // (state^T a^T)[n][t] for n = n0 + 4 lg + r
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < P / 32; ++kk) acc = mma(tr_frag(sMt, LDB, 32 * kk, n0, lane), af[kk], acc);
        const bf16x4 v4 = *reinterpret_cast<const bf16x4*>(svr + n0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          part = fmaf(acc[r], static_cast<float>(v4[r]), part);
          if (is_u) gC[nt][r] = fmaf(scale, acc[r], gC[nt][r]);
          else gB[nt][r] = fmaf(scale, acc[r], gB[nt][r]);
        }
      }
      part = sum_rows(part);
      if (lg == 0) {
        const float v = scale * part;
        if (term == 0) s_fw[t] += v;                       // U_f
        else if (term == 1) { s_bw[t] += v; s_sub[t] += v; }  // V_f
        else if (term == 2) s_bw[t] += v;                  // U_b
        else { s_fw[t] += v; s_sub[t] += v; }              // V_b
      }
    };
#pragma unroll 1
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
      if (!owns_rows) continue;
      do_term(2 * round, sM0);
      do_term(2 * round + 1, sM1);
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
    if (tid < Q) R[(bl + s_tok[tid]) * Hs + h] = s_fw[tid] + s_bw[tid] - s_sub[tid] + k;
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
constexpr int kTokRows = 64, kTokUnroll = 4;
__global__ __launch_bounds__(256) void ma_bwd_token_kernel(
    const __bf16* __restrict__ x, const __bf16* __restrict__ dy, const float* __restrict__ dt,
    const float* __restrict__ A, const float* __restrict__ D, const __bf16* __restrict__ yh,
    const float* __restrict__ R, int64_t rows, int Hs, float* __restrict__ dx, float* __restrict__ ddt,
    float* __restrict__ dA, float* __restrict__ dD) {
  constexpr int P = 64, U = kTokUnroll;
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
    bf16x8 bx[U], bdy[U], bh[U];   // kept in bf16 until used
#pragma unroll
    for (int u = 0; u < U; ++u) {
      ok[u] = active && i0 + u < nr;
      rh[u] = (r0 + i0 + u) * Hs + hc;
      d[u] = r[u] = 0.f;
      bx[u] = bdy[u] = bh[u] = bf16x8{};
      if (ok[u]) {
        d[u] = dt[rh[u]];
        r[u] = R[rh[u]];
        const int64_t off = rh[u] * P + sub * 8;
        bx[u] = *reinterpret_cast<const bf16x8*>(x + off);
        bdy[u] = *reinterpret_cast<const bf16x8*>(dy + off);
        bh[u] = *reinterpret_cast<const bf16x8*>(yh + off);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float gx[8], xyh = 0.f, dyx = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float vx = static_cast<float>(bx[u][e]), vdy = static_cast<float>(bdy[u][e]),
                    vh = static_cast<float>(bh[u][e]);
        xyh = fmaf(vx, vh, xyh);
        dyx = fmaf(vdy, vx, dyx);
        gx[e] = fmaf(d[u], vh, two_d * vdy);
      }
      if (ok[u]) {
        float4* o = reinterpret_cast<float4*>(dx + rh[u] * P + sub * 8);
        o[0] = make_float4(gx[0], gx[1], gx[2], gx[3]);
        o[1] = make_float4(gx[4], gx[5], gx[6], gx[7]);
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

// Byte offsets inside the caller's workspace.
struct BwdWs {
  size_t scan1, scan2, R, yh, total;
};

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

int bwd_layout(const lingen_mate_shape* s, BwdWs* w) {
  const size_t rows = size_t(s->batch) * size_t(tokens(s));
  const size_t hs = size_t(s->ssd_heads), P = size_t(s->headdim);
  size_t ws_main = 0;
  if (int rc = lingen_mate_workspace_bytes(s, &ws_main)) return rc;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += align256(bytes); return o; };
  w->scan1 = take(ws_main);
  w->scan2 = take(ws_main);
  w->R = take(rows * hs * 4);
  w->yh = take(rows * hs * P * 2);
  w->total = off;
  return LINGEN_OK;
}

int check_bwd_shape(const lingen_mate_shape* s) {
  if (int rc = validate_shape(s)) return rc;
  if (s->n_review != 0) return LINGEN_ERR_UNSUPPORTED;
  // the crossing-sum kernel takes bf16 storage with head size 64
  if (s->dtype != LINGEN_BF16 || s->headdim != 64) return LINGEN_ERR_UNSUPPORTED;
  // the crossing-sum kernel is compiled for the two bf16 scan families with P = 64
  if (!((s->chunk == 64 && s->d_state == 64) || (s->chunk == 128 && s->d_state == 128))) return LINGEN_ERR_UNSUPPORTED;
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

extern "C" int lingen_ma_bwd(const void* x, const float* dt, const float* A, const void* B, const void* C,
                             const float* D, const void* dy, int32_t mode, const lingen_mate_shape* shape,
                             float* dx, float* ddt, float* dA, float* dB, float* dC, float* dD, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  if (int rc = check_bwd_shape(shape)) return rc;
  if (mode < 0 || mode > 3) return LINGEN_ERR_SHAPE;
  const void* ptrs[] = {x, dt, A, B, C, D, dy, dx, ddt, dA, dB, dC, dD, workspace};
  for (const void* p : ptrs)
    if (int rc = check_ptr(p)) return rc;
  BwdWs w{};
  if (int rc = bwd_layout(shape, &w)) return rc;
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
  int rc;
#define LINGEN_TRY(expr)                          \
  do {                                            \
    if ((rc = (expr)) != LINGEN_OK) return rc;    \
  } while (0)
#define LINGEN_LAUNCHED()                                             \
  do {                                                                \
    if (hipGetLastError() != hipSuccess) return LINGEN_ERR_HIP;       \
  } while (0)

  // dA and dD accumulate from zero
  zero_floats_kernel<<<1, kThreads, 0, stream>>>(dA, dD, Hs);
  LINGEN_LAUNCHED();

  // crossing sums, then ddt, dx, dA, dD
  {
    const dim3 cgrid{unsigned(nc), unsigned(G), 1u};
    const WsLayout lay = ws_layout(shape);
    const int64_t per = int64_t(nc) * Hs * P * N;   // one direction's scan states
    const __bf16* st1 = reinterpret_cast<const __bf16*>(ws + w.scan1 + lay.states);
    const __bf16* st2 = reinterpret_cast<const __bf16*>(ws + w.scan2 + lay.states);
    const int64_t eb = 2;
    for (int bi = 0; bi < shape->batch; ++bi) {
      // forward / reverse states of (x, B) and of (x', C) for this batch element, left in the two workspaces
      const int64_t xo = int64_t(bi) * L * Hs * P * eb, bo = int64_t(bi) * L * G * N * eb;
      LINGEN_TRY(scan_states_one(shape, mode, static_cast<const char*>(x) + xo, dt + int64_t(bi) * L * Hs, A,
                                 static_cast<const char*>(B) + bo, ws + w.scan1, stream, kWeightDt));
      LINGEN_TRY(scan_states_one(shape, mode, static_cast<const char*>(dy) + xo, dt + int64_t(bi) * L * Hs, A,
                                 static_cast<const char*>(C) + bo, ws + w.scan2, stream, kWeightAdjoint));
      // the transposed outputs yhat = (M_f^T + M_b^T) dy / dt from the same adjoint states
      LINGEN_TRY(ma_transposed_one(shape, mode, static_cast<const char*>(dy) + xo, dt + int64_t(bi) * L * Hs, A,
                                   static_cast<const char*>(B) + bo, static_cast<const char*>(C) + bo, ws + w.scan2,
                                   static_cast<char*>(at(w.yh)) + xo, stream));
      if (Q == 128 && N == 128)
        ma_bwd_cross_kernel<128, 128><<<cgrid, kCrossThreads, 0, stream>>>(
            xb, dyb, dt, A, static_cast<const __bf16*>(B), static_cast<const __bf16*>(C), st1, st2, per, so, L, Hs,
            G, bi, atf(w.R), dB, dC);
      else if (Q == 64 && N == 64)
        ma_bwd_cross_kernel<64, 64><<<cgrid, kCrossThreads, 0, stream>>>(
            xb, dyb, dt, A, static_cast<const __bf16*>(B), static_cast<const __bf16*>(C), st1, st2, per, so, L, Hs,
            G, bi, atf(w.R), dB, dC);
      else
        return LINGEN_ERR_UNSUPPORTED;
      LINGEN_LAUNCHED();
    }
    const dim3 tgrid{unsigned((rows + kTokRows - 1) / kTokRows), unsigned((Hs + 31) / 32), 1u};
    ma_bwd_token_kernel<<<tgrid, 256, 0, stream>>>(xb, dyb, dt, A, D, static_cast<const __bf16*>(at(w.yh)), atf(w.R),
                                                   rows, Hs, dx, ddt, dA, dD);
    LINGEN_LAUNCHED();
  }
#undef LINGEN_TRY
#undef LINGEN_LAUNCHED
  return LINGEN_OK;
}
