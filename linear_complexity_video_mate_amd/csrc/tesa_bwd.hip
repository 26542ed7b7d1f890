// Backward pass of TEmporal Swin Attention on gfx950: the gradients dq, dk,
// dv of the windowed softmax attention for an upstream gradient dO (page
// "LinGen：基于Mamba机制的线性复杂度高清长视频生成框架", section 关键算法创新 >
// TESA for the forward; the pages train the model, section 技术细节, which
// needs these gradients).  Per window and head, with P the softmax weights,
// s = 1/sqrt(d) and D_i = sum_d dO_i[d] o_i[d] = sum_j P_ij dP_ij:
//   dP = dO v^T,   dS = P * (dP - D),   dq = s dS k,   dk = s dS^T q,   dv = P^T dO.
//
// One workgroup of 8 waves per (window, head) item; the item's q, k, v and
// dO tiles (256 x 64 bf16 each) sit in LDS, filled by direct global-to-LDS
// loads.  Phase 1, each wave owning two 16-query tiles: an online-softmax
// sweep over 32-key blocks gives the row maximum and sum and the output o
// (fp32), hence log-sum-exp and D; a second sweep recomputes P, forms
// dP^T = V dO^T and dS^T, and accumulates dq^T = K^T dS^T.  Phase 2, each
// wave owning two 16-key tiles, sweeps 32-query blocks: P and dP from Q K^T
// and dO V^T with the stored per-query statistics, then dv^T = dO^T P and
// dk^T = Q^T dS.  The fragments a block reads from LDS serve both tiles.
// Every product is a 16x16x32 bf16 MFMA with fp32 accumulation; the
// k-permuted register operands and the transposing LDS reads are those of
// the forward window kernel.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "lingen_device.h"
#include "lingen_internal.h"
#include "lingen_window.h"

namespace lingen {

namespace {

constexpr int kBwdWin = 256, kBwdDim = 64;
constexpr int kBwdTiles = 2;   // 16-row tiles per wave

// 4-element pieces of the 16-wide d-tiles 2 r1 and 2 r1 + 1 exchanged between
// lane groups g and g ^ 1: the lane then holds d0 .. d0 + 7 of its row,
// d0 = 32 r1 + 16 (g & 1) + 8 (g >> 1), stored as one 16-byte piece.
__device__ __forceinline__ void store_rows16(__bf16* row, const f32x4 (&acc)[4], float scale, int grp) {
  __bf16* dst = row + 16 * (grp & 1) + 8 * (grp >> 1);
#pragma unroll
  for (int r1 = 0; r1 < 2; ++r1) {
    bf16x8 res;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[2 * r1][r]),
                                                       __float_as_uint(acc[2 * r1 + 1][r]), false, false);
      res[r] = static_cast<__bf16>(__uint_as_float(sw[0]) * scale);
      res[4 + r] = static_cast<__bf16>(__uint_as_float(sw[1]) * scale);
    }
    *reinterpret_cast<bf16x8*>(dst + 32 * r1) = res;
  }
}

}  // namespace

// QT row tiles of 16 per wave (16 / QT waves): the operand fragments read
// from LDS for a block are shared by the wave's QT tiles.
template <int QT>
__global__ __launch_bounds__(64 * 16 / QT) void tesa_bwd_kernel(const __bf16* __restrict__ q,
                                                                const __bf16* __restrict__ k,
                                                                const __bf16* __restrict__ v,
                                                                const __bf16* __restrict__ dO, WinGeom wg, int Ha,
                                                                __bf16* __restrict__ dq, __bf16* __restrict__ dk,
                                                                __bf16* __restrict__ dv) {
  constexpr int NWIN = kBwdWin, DH = kBwdDim, ET = DH / 16, NKS = DH / 32;
  constexpr int NW = 16 / QT, NTHR = NW * 64;
  static_assert(NWIN == 16 * QT * NW, "one 16-row tile per wave and QT");
  using KT = KvTile<__bf16, DH>;
  __shared__ __attribute__((aligned(16))) __bf16 sQ[NWIN * DH];
  __shared__ __attribute__((aligned(16))) __bf16 sK[NWIN * DH];
  __shared__ __attribute__((aligned(16))) __bf16 sV[NWIN * DH];
  __shared__ __attribute__((aligned(16))) __bf16 sG[NWIN * DH];   // dO
  __shared__ __attribute__((aligned(16))) int sTok[NWIN];
  __shared__ __attribute__((aligned(16))) int sCls[NWIN];
  __shared__ __attribute__((aligned(16))) float sLse[NWIN];   // log2-sum-exp of the scaled scores
  __shared__ __attribute__((aligned(16))) float sD[NWIN];     // sum_d dO . o

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, grp = lane >> 4;
  const int item = blockIdx.x;
  const int h = item % Ha, win = item / Ha;
  const int nwin_hw = wg.nwh * wg.nww;
  const int wi = win / nwin_hw, wj = (win / wg.nww) % wg.nwh, wk = win % wg.nww;
  const int64_t rowstride = int64_t(Ha) * DH;
  const int64_t hoff = int64_t(h) * DH;
  const float sc = kLog2e * rsqrtf(float(DH));   // scores in log2 units
  const float snat = rsqrtf(float(DH));          // 1/sqrt(d)

  for (int u = tid; u < NWIN; u += NTHR) {
    const int a = u / (wg.wh * wg.ww), b = (u / wg.ww) % wg.wh, c = u % wg.ww;
    int cl;
    sTok[u] = window_token(wg, wi, wj, wk, a, b, c, cl);
    sCls[u] = wg.masked ? cl : 0;
  }
  lds_barrier();
  // Direct loads of the four tiles: 16-byte chunk u of a tile is row u/8,
  // chunk (u%8) ^ (row%8) of that row (the KvTile permutation).
  constexpr int PER_WAVE = NWIN * 8 / (NW * 64);   // load instructions per wave and tile
#pragma unroll
  for (int d = 0; d < PER_WAVE; ++d) {
    const int base = (wave * PER_WAVE + d) * 64;
    const int u = base + lane, row = u / 8, ch = (u % 8) ^ (row & 7);
    const int64_t goff = int64_t(sTok[row]) * rowstride + hoff + ch * 8;
    lds_load16(q + goff, sQ + base * 8);
    lds_load16(k + goff, sK + base * 8);
    lds_load16(v + goff, sV + base * 8);
    lds_load16(dO + goff, sG + base * 8);
  }
  wait_vmem();
  lds_barrier();

  const bool wrapped = wg.masked && window_wrapped(wg, wi, wj, wk);
  // Per-lane LDS offsets: row fragments (A operand rows r16, or B operand
  // columns r16) and the transposing reads of a tile (as in the forward).
  int offk[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) offk[ks] = KT::at(r16, ks * 32 + grp * 8);
  int offv[ET];
#pragma unroll
  for (int et = 0; et < ET; ++et) offv[et] = KT::at(4 * grp + (r16 >> 2), et * 16 + 4 * (r16 & 3));
  auto rowfrag = [&](const __bf16* tile, int row0, int ks) {
    return *reinterpret_cast<const bf16x8*>(tile + offk[ks] + row0 * DH);
  };
  // Transposed A operand: rows e = et*16 + (lane's row), k = 32 rows from
  // row0 (lane group g brings rows 4g..4g+3 and 16+4g..16+4g+3).
  auto trfrag = [&](const __bf16* tile, int row0, int et) {
    lds_bf16* t = (lds_bf16*)(tile) + offv[et] + row0 * DH;
    const bf16x4 lo = lds_read_tr(t), hi = lds_read_tr(t + 16 * DH);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  // Pack the 4-row pieces of two 16-row score tiles as a B operand (k = the
  // tiles' rows in the order of trfrag).
  auto pack = [](const f32x4& a, const f32x4& b) {
    bf16x8 p;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = static_cast<__bf16>(a[r]);
      p[4 + r] = static_cast<__bf16>(b[r]);
    }
    return p;
  };
  auto mask = [&](f32x4& s, int j0, int c) {
    const int4 kc = *reinterpret_cast<const int4*>(&sCls[j0 + 4 * grp]);
    const int kcv[4] = {kc.x, kc.y, kc.z, kc.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] = kcv[r] != c ? -INFINITY : s[r];
  };

  // ---------------- Phase 1: the wave's query tiles -----------------------
  {
    int icls[QT];
    bf16x8 qf[QT][NKS], gf[QT][NKS];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int i0 = (wave * QT + qt) * 16;
      icls[qt] = sCls[i0 + r16];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        qf[qt][ks] = rowfrag(sQ, i0, ks);
        gf[qt][ks] = rowfrag(sG, i0, ks);
      }
    }
    // Sweep 1: online softmax statistics and the output o, 32 keys a step.
    float m[QT], l[QT];
    f32x4 o[QT][ET];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      m[qt] = -INFINITY;
      l[qt] = 0.f;
#pragma unroll
      for (int et = 0; et < ET; ++et) o[qt][et] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll 1
    for (int jb = 0; jb < NWIN; jb += 32) {
      bf16x8 kfr[2][NKS], vtr[ET];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) kfr[t][ks] = rowfrag(sK, jb + 16 * t, ks);
#pragma unroll
      for (int et = 0; et < ET; ++et) vtr[et] = trfrag(sV, jb, et);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        f32x4 s[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) s[t] = mma(kfr[t][ks], qf[qt][ks], s[t]);
          if (wrapped) mask(s[t], jb + 16 * t, icls[qt]);
        }
        float bm = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                         fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
        bm = max_rows(bm);
        const float mnew = fmaxf(m[qt], bm * sc);
        const float mref = mnew == -INFINITY ? 0.f : mnew;
        const float alpha = fast_exp2(m[qt] - mref);
        m[qt] = mnew;
        float ls = 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            s[t][r] = fast_exp2(fmaf(s[t][r], sc, -mref));
            ls += s[t][r];
          }
        l[qt] = fmaf(l[qt], alpha, ls);
        const bf16x8 pb = pack(s[0], s[1]);
#pragma unroll
        for (int et = 0; et < ET; ++et) {
#pragma unroll
          for (int r = 0; r < 4; ++r) o[qt][et][r] *= alpha;
          o[qt][et] = mma(vtr[et], pb, o[qt][et]);
        }
      }
    }
    float lse[QT], dsum[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int i0 = (wave * QT + qt) * 16;
      float lt = l[qt];
      lt = sum_rows(lt);
      const float inv = 1.f / lt;
      // D_i = sum_d dO_i[d] o_i[d]: the lane holds o for d = et*16 + 4g + r.
      float ds_ = 0.f;
#pragma unroll
      for (int et = 0; et < ET; ++et) {
        const bf16x4 g4 = *reinterpret_cast<const bf16x4*>(sG + KT::at(i0 + r16, et * 16 + 4 * grp));
#pragma unroll
        for (int r = 0; r < 4; ++r) ds_ = fmaf(static_cast<float>(g4[r]), o[qt][et][r] * inv, ds_);
      }
      ds_ = sum_rows(ds_);
      dsum[qt] = ds_;
      lse[qt] = m[qt] + log2f(lt);
      if (grp == 0) {
        sLse[i0 + r16] = lse[qt];
        sD[i0 + r16] = ds_;
      }
    }
    // Sweep 2: dS^T and dq^T = K^T dS^T, 32 keys a step.
    f32x4 gq[QT][ET];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int et = 0; et < ET; ++et) gq[qt][et] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int jb = 0; jb < NWIN; jb += 32) {
      bf16x8 kfr[2][NKS], vfr[2][NKS], ktr[ET];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          kfr[t][ks] = rowfrag(sK, jb + 16 * t, ks);
          vfr[t][ks] = rowfrag(sV, jb + 16 * t, ks);
        }
#pragma unroll
      for (int et = 0; et < ET; ++et) ktr[et] = trfrag(sK, jb, et);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        f32x4 ds[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f}, dp = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            s = mma(kfr[t][ks], qf[qt][ks], s);
            dp = mma(vfr[t][ks], gf[qt][ks], dp);
          }
          if (wrapped) mask(s, jb + 16 * t, icls[qt]);
#pragma unroll
          for (int r = 0; r < 4; ++r) ds[t][r] = fast_exp2(fmaf(s[r], sc, -lse[qt])) * (dp[r] - dsum[qt]);
        }
        const bf16x8 db = pack(ds[0], ds[1]);
#pragma unroll
        for (int et = 0; et < ET; ++et) gq[qt][et] = mma(ktr[et], db, gq[qt][et]);
      }
    }
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int i = (wave * QT + qt) * 16 + r16;
      store_rows16(dq + int64_t(sTok[i]) * rowstride + hoff, gq[qt], snat, grp);
    }
  }
  lds_barrier();   // every query's statistics are in LDS

  // ---------------- Phase 2: the wave's key tiles -------------------------
  {
    int jcls[QT];
    bf16x8 kf[QT][NKS], vf[QT][NKS];
#pragma unroll
    for (int kt = 0; kt < QT; ++kt) {
      const int j0 = (wave * QT + kt) * 16;
      jcls[kt] = sCls[j0 + r16];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        kf[kt][ks] = rowfrag(sK, j0, ks);
        vf[kt][ks] = rowfrag(sV, j0, ks);
      }
    }
    f32x4 gk[QT][ET], gv[QT][ET];
#pragma unroll
    for (int kt = 0; kt < QT; ++kt)
#pragma unroll
      for (int et = 0; et < ET; ++et) {
        gk[kt][et] = f32x4{0.f, 0.f, 0.f, 0.f};
        gv[kt][et] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll 1
    for (int ib = 0; ib < NWIN; ib += 32) {
      bf16x8 qfr[2][NKS], gfr[2][NKS];
      float lv[2][4], dv4[2][4];
      int qc[2][4];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int iq = ib + 16 * t;   // score rows iq + 4g + r
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          qfr[t][ks] = rowfrag(sQ, iq, ks);
          gfr[t][ks] = rowfrag(sG, iq, ks);
        }
        const float4 ls4 = *reinterpret_cast<const float4*>(&sLse[iq + 4 * grp]);
        const float4 dd = *reinterpret_cast<const float4*>(&sD[iq + 4 * grp]);
        lv[t][0] = ls4.x; lv[t][1] = ls4.y; lv[t][2] = ls4.z; lv[t][3] = ls4.w;
        dv4[t][0] = dd.x; dv4[t][1] = dd.y; dv4[t][2] = dd.z; dv4[t][3] = dd.w;
        const int4 c4 = *reinterpret_cast<const int4*>(&sCls[iq + 4 * grp]);
        qc[t][0] = c4.x; qc[t][1] = c4.y; qc[t][2] = c4.z; qc[t][3] = c4.w;
      }
#pragma unroll
      for (int kt = 0; kt < QT; ++kt) {
        f32x4 p[2], ds[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f}, dp = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            s = mma(qfr[t][ks], kf[kt][ks], s);
            dp = mma(gfr[t][ks], vf[kt][ks], dp);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float pv = (wrapped && qc[t][r] != jcls[kt]) ? 0.f : fast_exp2(fmaf(s[r], sc, -lv[t][r]));
            p[t][r] = pv;
            ds[t][r] = pv * (dp[r] - dv4[t][r]);
          }
        }
        const bf16x8 pb = pack(p[0], p[1]), db = pack(ds[0], ds[1]);
#pragma unroll
        for (int et = 0; et < ET; ++et) {
          gv[kt][et] = mma(trfrag(sG, ib, et), pb, gv[kt][et]);
          gk[kt][et] = mma(trfrag(sQ, ib, et), db, gk[kt][et]);
        }
      }
    }
#pragma unroll
    for (int kt = 0; kt < QT; ++kt) {
      const int j = (wave * QT + kt) * 16 + r16;
      const int64_t roff = int64_t(sTok[j]) * rowstride + hoff;
      store_rows16(dk + roff, gk[kt], snat, grp);
      store_rows16(dv + roff, gv[kt], 1.f, grp);
    }
  }
}


// Small windows (at most 32 slots: the 3x3x3 and 2x4x4 windows), any
// element type: one workgroup of 256 threads per (window, head) item.  The
// item's q, k, v and dO rows sit in LDS as fp32 (rows padded by one element,
// so that threads stepping along a row's neighbours hit distinct banks); the
// scores, the softmax weights P and dS = P * (dP - D) are dense NW x NW fp32
// tiles, and every product is a plain fp32 loop: an item is a few tens of
// thousands of multiply-adds, far below what an MFMA tiling would pay back.
// Masked pairs (slots of different wrap classes in a cut window) get P = 0.
template <typename TS, int DH, int NW>
__global__ __launch_bounds__(256) void tesa_bwd_small_kernel(const TS* __restrict__ q, const TS* __restrict__ k,
                                                             const TS* __restrict__ v, const TS* __restrict__ dO,
                                                             WinGeom wg, int Ha, TS* __restrict__ dq,
                                                             TS* __restrict__ dk, TS* __restrict__ dv) {
  static_assert(NW <= 32, "one thread per softmax row");
  constexpr int NTHR = 256, LD = DH + 1, LP = NW + 1;
  __shared__ float sQ[NW * LD], sK[NW * LD], sV[NW * LD], sG[NW * LD];
  __shared__ float sP[NW * LP], sD[NW * LP];
  __shared__ int sTok[NW], sCls[NW];
  const int tid = threadIdx.x;
  const int item = blockIdx.x, h = item % Ha, win = item / Ha;
  const int nwin_hw = wg.nwh * wg.nww;
  const int wi = win / nwin_hw, wj = (win / wg.nww) % wg.nwh, wk = win % wg.nww;
  const int64_t rowstride = int64_t(Ha) * DH, hoff = int64_t(h) * DH;
  const float scale = rsqrtf(float(DH));
  if (tid < NW) {
    int cl;
    sTok[tid] = window_token(wg, wi, wj, wk, tid / (wg.wh * wg.ww), (tid / wg.ww) % wg.wh, tid % wg.ww, cl);
    sCls[tid] = wg.masked ? cl : 0;
  }
  __syncthreads();
  for (int u = tid; u < NW * DH; u += NTHR) {
    const int i = u / DH, d = u % DH;
    const int64_t g = int64_t(sTok[i]) * rowstride + hoff + d;
    sQ[i * LD + d] = to_f32(q[g]);
    sK[i * LD + d] = to_f32(k[g]);
    sV[i * LD + d] = to_f32(v[g]);
    sG[i * LD + d] = to_f32(dO[g]);
  }
  __syncthreads();
  // scaled scores and dP = dO v^T
  for (int u = tid; u < NW * NW; u += NTHR) {
    const int i = u / NW, j = u % NW;
    float sc = 0.f, dp = 0.f;
#pragma unroll 8
    for (int d = 0; d < DH; ++d) {
      sc = fmaf(sQ[i * LD + d], sK[j * LD + d], sc);
      dp = fmaf(sG[i * LD + d], sV[j * LD + d], dp);
    }
    sP[i * LP + j] = sCls[i] == sCls[j] ? sc * scale : -INFINITY;
    sD[i * LP + j] = dp;
  }
  __syncthreads();
  // P = softmax of each row, D_i = sum_j P_ij dP_ij, dS = P (dP - D)
  if (tid < NW) {
    float* pr = &sP[tid * LP];
    float* dr = &sD[tid * LP];
    float m = -INFINITY;
    for (int j = 0; j < NW; ++j) m = fmaxf(m, pr[j]);   // the slot's own key is never masked
    float l = 0.f;
    for (int j = 0; j < NW; ++j) {
      const float e = expf(pr[j] - m);
      pr[j] = e;
      l += e;
    }
    const float inv = 1.f / l;
    float dsum = 0.f;
    for (int j = 0; j < NW; ++j) {
      pr[j] *= inv;
      dsum = fmaf(pr[j], dr[j], dsum);
    }
    for (int j = 0; j < NW; ++j) dr[j] = pr[j] * (dr[j] - dsum);
  }
  __syncthreads();
  // dq_i = scale sum_j dS_ij k_j;  dk_i = scale sum_j dS_ji q_j;  dv_i = sum_j P_ji dO_j
  for (int u = tid; u < NW * DH; u += NTHR) {
    const int i = u / DH, d = u % DH;
    float a = 0.f, b = 0.f, c = 0.f;
#pragma unroll 8
    for (int j = 0; j < NW; ++j) {
      a = fmaf(sD[i * LP + j], sK[j * LD + d], a);
      b = fmaf(sD[j * LP + i], sQ[j * LD + d], b);
      c = fmaf(sP[j * LP + i], sG[j * LD + d], c);
    }
    const int64_t g = int64_t(sTok[i]) * rowstride + hoff + d;
    dq[g] = from_f32<TS>(a * scale);
    dk[g] = from_f32<TS>(b * scale);
    dv[g] = from_f32<TS>(c);
  }
}

template <typename TS, int DH, int NW>
int launch_te_bwd_small(const lingen_mate_shape* s, const WinGeom& g, const void* q, const void* k, const void* v,
                        const void* d_out, void* dq, void* dk, void* dv, hipStream_t st) {
  const int64_t L = tokens(s);
  const int items = g.nwt * g.nwh * g.nww * s->attn_heads;
  const int64_t per = L * s->attn_heads * DH;
  for (int b = 0; b < s->batch; ++b) {
    const int64_t off = int64_t(b) * per;
    tesa_bwd_small_kernel<TS, DH, NW><<<items, 256, 0, st>>>(
        static_cast<const TS*>(q) + off, static_cast<const TS*>(k) + off, static_cast<const TS*>(v) + off,
        static_cast<const TS*>(d_out) + off, g, s->attn_heads, static_cast<TS*>(dq) + off,
        static_cast<TS*>(dk) + off, static_cast<TS*>(dv) + off);
    if (launch_status(__func__) != LINGEN_OK) return LINGEN_ERR_HIP;
  }
  return LINGEN_OK;
}

}  // namespace lingen

using namespace lingen;

extern "C" int lingen_te_bwd(const void* q, const void* k, const void* v, const void* d_out, int32_t shift_t,
                             int32_t shift_h, int32_t shift_w, int32_t masked, const lingen_mate_shape* shape,
                             void* dq, void* dk, void* dv, hipStream_t stream) {
  if (int rc = validate_shape(shape)) return rc;
  if (shift_t < 0 || shift_t >= shape->win_t || shift_h < 0 || shift_h >= shape->win_h || shift_w < 0 ||
      shift_w >= shape->win_w || (masked != 0 && masked != 1))
    return LINGEN_ERR_SHAPE;
  for (const void* p : {q, k, v, d_out, static_cast<const void*>(dq), static_cast<const void*>(dk),
                        static_cast<const void*>(dv)})
    if (int rc = check_ptr(p)) return rc;
  const int shift[3] = {shift_t, shift_h, shift_w};
  const WinGeom g = make_wingeom(shape, shift, masked);
  switch (attn_family(shape)) {
    case ATTN_BF16_D64_W256: break;
    case ATTN_BF16_D64_W27: return launch_te_bwd_small<__bf16, 64, 27>(shape, g, q, k, v, d_out, dq, dk, dv, stream);
    case ATTN_F32_D32_W32: return launch_te_bwd_small<float, 32, 32>(shape, g, q, k, v, d_out, dq, dk, dv, stream);
    default: return LINGEN_ERR_UNSUPPORTED;
  }
  const int64_t L = tokens(shape);
  const int items = g.nwt * g.nwh * g.nww * shape->attn_heads;
  const int64_t per = L * shape->attn_heads * kBwdDim;   // elements per batch element
  for (int b = 0; b < shape->batch; ++b) {
    const int64_t off = int64_t(b) * per;
    tesa_bwd_kernel<kBwdTiles><<<items, 64 * 16 / kBwdTiles, 0, stream>>>(
        static_cast<const __bf16*>(q) + off, static_cast<const __bf16*>(k) + off, static_cast<const __bf16*>(v) + off,
        static_cast<const __bf16*>(d_out) + off, g, shape->attn_heads, static_cast<__bf16*>(dq) + off,
        static_cast<__bf16*>(dk) + off, static_cast<__bf16*>(dv) + off);
    if (launch_status(__func__) != LINGEN_OK) return LINGEN_ERR_HIP;
  }
  return LINGEN_OK;
}
