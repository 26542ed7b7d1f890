// Backward pass of TEmporal Swin Attention on gfx950: the gradients dq, dk,
// dv of the windowed softmax attention for an upstream gradient dO (page
// "LinGen：基于Mamba机制的线性复杂度高清长视频生成框架", section 关键算法创新 >
// TESA for the forward; the pages train the model, section 技术细节, which
// needs these gradients).  Per window and head, with P the softmax weights,
// s = 1/sqrt(d) and D_i = sum_d dO_i[d] o_i[d] = sum_j P_ij dP_ij:
//   dP = dO v^T,   dS = P * (dP - D),   dq = s dS k,   dk = s dS^T q,   dv = P^T dO.
//
// One workgroup of 16 waves per (window, head) item; the item's q, k, v and
// dO tiles (256 x 64 bf16 each) sit in LDS, filled by direct global-to-LDS
// loads.  Phase 1, wave w owning queries 16w..16w+15: an online-softmax sweep
// over 64-key blocks gives the row maximum and sum and the output o (fp32),
// hence log-sum-exp and D; a second sweep recomputes P, forms dP^T = V dO^T
// and dS^T, and accumulates dq^T = K^T dS^T.  Phase 2, wave w owning keys
// 16w..16w+15, sweeps 32-query blocks: P and dP from Q K^T and dO V^T with
// the stored per-query statistics, then dv^T = dO^T P and dk^T = Q^T dS.
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

__global__ __launch_bounds__(1024) void tesa_bwd_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                                        const __bf16* __restrict__ v, const __bf16* __restrict__ dO,
                                                        WinGeom wg, int Ha, __bf16* __restrict__ dq,
                                                        __bf16* __restrict__ dk, __bf16* __restrict__ dv) {
  constexpr int NWIN = kBwdWin, DH = kBwdDim, ET = DH / 16, NKS = DH / 32;
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
  const float sc = kLog2e * rsqrtf(float(DH));   // scores in log2 units
  const float snat = rsqrtf(float(DH));          // 1/sqrt(d)

  {
    const int a = tid / (wg.wh * wg.ww), b = (tid / wg.ww) % wg.wh, c = tid % wg.ww;
    if (tid < NWIN) {
      int cl;
      sTok[tid] = window_token(wg, wi, wj, wk, a, b, c, cl);
      sCls[tid] = wg.masked ? cl : 0;
    }
  }
  lds_barrier();
  // Direct loads of the four tiles: 16-byte chunk u of a tile is row u/8,
  // chunk (u%8) ^ (row%8) of that row (the KvTile permutation).
  constexpr int PER_WAVE = NWIN * 8 / (16 * 64);   // load instructions per wave and tile
#pragma unroll
  for (int d = 0; d < PER_WAVE; ++d) {
    const int base = (wave * PER_WAVE + d) * 64;
    const int u = base + lane, row = u / 8, ch = (u % 8) ^ (row & 7);
    const int64_t goff = int64_t(sTok[row]) * rowstride + int64_t(h) * DH + ch * 8;
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

  // ---------------- Phase 1: queries i = 16 wave + r16 --------------------
  {
    const int i0 = wave * 16;
    const int icls = sCls[i0 + r16];
    bf16x8 qf[NKS], gf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      qf[ks] = rowfrag(sQ, i0, ks);
      gf[ks] = rowfrag(sG, i0, ks);
    }
    // S^T tile (16 keys from row j0) for the lane's query column, masked.
    auto scores = [&](int j0) {
      f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) s = mma(rowfrag(sK, j0, ks), qf[ks], s);
      if (wrapped) {
        const int4 kc = *reinterpret_cast<const int4*>(&sCls[j0 + 4 * grp]);
        const int kcv[4] = {kc.x, kc.y, kc.z, kc.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) s[r] = kcv[r] != icls ? -INFINITY : s[r];
      }
      return s;
    };
    // Sweep 1: online softmax statistics and the output o.
    float m = -INFINITY, l = 0.f;
    f32x4 o[ET];
#pragma unroll
    for (int et = 0; et < ET; ++et) o[et] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int jb = 0; jb < NWIN; jb += 64) {
      f32x4 s[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) s[t] = scores(jb + 16 * t);
      float bm = -INFINITY;
#pragma unroll
      for (int t = 0; t < 4; ++t) bm = fmaxf(bm, fmaxf(fmaxf(s[t][0], s[t][1]), fmaxf(s[t][2], s[t][3])));
      bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
      bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
      const float mnew = fmaxf(m, bm * sc);
      const float mref = mnew == -INFINITY ? 0.f : mnew;
      const float alpha = fast_exp2(m - mref);
      m = mnew;
      float ls = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          s[t][r] = fast_exp2(fmaf(s[t][r], sc, -mref));
          ls += s[t][r];
        }
      l = fmaf(l, alpha, ls);
#pragma unroll
      for (int et = 0; et < ET; ++et) {
#pragma unroll
        for (int r = 0; r < 4; ++r) o[et][r] *= alpha;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
          o[et] = mma(trfrag(sV, jb + 32 * sb, et), pack(s[2 * sb], s[2 * sb + 1]), o[et]);
      }
    }
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float inv = 1.f / l;
    // D_i = sum_d dO_i[d] o_i[d]: the lane holds o for d = et*16 + 4g + r.
    float dsum = 0.f;
#pragma unroll
    for (int et = 0; et < ET; ++et) {
      const bf16x4 g4 = *reinterpret_cast<const bf16x4*>(sG + KT::at(i0 + r16, et * 16 + 4 * grp));
#pragma unroll
      for (int r = 0; r < 4; ++r) dsum = fmaf(static_cast<float>(g4[r]), o[et][r] * inv, dsum);
    }
    dsum += __shfl_xor(dsum, 16, 64);
    dsum += __shfl_xor(dsum, 32, 64);
    const float lse = m + log2f(l);
    if (grp == 0) {
      sLse[i0 + r16] = lse;
      sD[i0 + r16] = dsum;
    }
    // Sweep 2: dS^T and dq^T = K^T dS^T.
    f32x4 gq[ET];
#pragma unroll
    for (int et = 0; et < ET; ++et) gq[et] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int jb = 0; jb < NWIN; jb += 64) {
      f32x4 ds[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int j0 = jb + 16 * t;
        const f32x4 s = scores(j0);
        f32x4 dp = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) dp = mma(rowfrag(sV, j0, ks), gf[ks], dp);
#pragma unroll
        for (int r = 0; r < 4; ++r) ds[t][r] = fast_exp2(fmaf(s[r], sc, -lse)) * (dp[r] - dsum);
      }
#pragma unroll
      for (int et = 0; et < ET; ++et)
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
          gq[et] = mma(trfrag(sK, jb + 32 * sb, et), pack(ds[2 * sb], ds[2 * sb + 1]), gq[et]);
    }
    store_rows16(dq + int64_t(sTok[i0 + r16]) * rowstride + int64_t(h) * DH, gq, snat, grp);
  }
  lds_barrier();   // every query's statistics are in LDS

  // ---------------- Phase 2: keys j = 16 wave + r16 -----------------------
  {
    const int j0 = wave * 16;
    const int jcls = sCls[j0 + r16];
    bf16x8 kf[NKS], vf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      kf[ks] = rowfrag(sK, j0, ks);
      vf[ks] = rowfrag(sV, j0, ks);
    }
    f32x4 gk[ET], gv[ET];
#pragma unroll
    for (int et = 0; et < ET; ++et) {
      gk[et] = f32x4{0.f, 0.f, 0.f, 0.f};
      gv[et] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll 1
    for (int ib = 0; ib < NWIN; ib += 32) {
      f32x4 p[2], ds[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int i0 = ib + 16 * t;   // lane holds rows i0 + 4g + r, column j0 + r16
        f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f}, dp = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          s = mma(rowfrag(sQ, i0, ks), kf[ks], s);
          dp = mma(rowfrag(sG, i0, ks), vf[ks], dp);
        }
        const float4 lse = *reinterpret_cast<const float4*>(&sLse[i0 + 4 * grp]);
        const float4 dd = *reinterpret_cast<const float4*>(&sD[i0 + 4 * grp]);
        const float lv[4] = {lse.x, lse.y, lse.z, lse.w}, dv4[4] = {dd.x, dd.y, dd.z, dd.w};
        int qc[4] = {0, 0, 0, 0};
        if (wrapped) {
          const int4 c4 = *reinterpret_cast<const int4*>(&sCls[i0 + 4 * grp]);
          qc[0] = c4.x; qc[1] = c4.y; qc[2] = c4.z; qc[3] = c4.w;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pv = (wrapped && qc[r] != jcls) ? 0.f : fast_exp2(fmaf(s[r], sc, -lv[r]));
          p[t][r] = pv;
          ds[t][r] = pv * (dp[r] - dv4[r]);
        }
      }
      const bf16x8 pb = pack(p[0], p[1]), db = pack(ds[0], ds[1]);
#pragma unroll
      for (int et = 0; et < ET; ++et) {
        gv[et] = mma(trfrag(sG, ib, et), pb, gv[et]);
        gk[et] = mma(trfrag(sQ, ib, et), db, gk[et]);
      }
    }
    const int64_t roff = int64_t(sTok[j0 + r16]) * rowstride + int64_t(h) * DH;
    store_rows16(dk + roff, gk, snat, grp);
    store_rows16(dv + roff, gv, 1.f, grp);
  }
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
  if (attn_family(shape) != ATTN_BF16_D64_W256) return LINGEN_ERR_UNSUPPORTED;
  const int shift[3] = {shift_t, shift_h, shift_w};
  const WinGeom g = make_wingeom(shape, shift, masked);
  const int64_t L = tokens(shape);
  const int items = g.nwt * g.nwh * g.nww * shape->attn_heads;
  const int64_t per = L * shape->attn_heads * kBwdDim;   // elements per batch element
  for (int b = 0; b < shape->batch; ++b) {
    const int64_t off = int64_t(b) * per;
    tesa_bwd_kernel<<<items, 1024, 0, stream>>>(
        static_cast<const __bf16*>(q) + off, static_cast<const __bf16*>(k) + off, static_cast<const __bf16*>(v) + off,
        static_cast<const __bf16*>(d_out) + off, g, shape->attn_heads, static_cast<__bf16*>(dq) + off,
        static_cast<__bf16*>(dk) + off, static_cast<__bf16*>(dv) + off);
    if (hipGetLastError() != hipSuccess) return LINGEN_ERR_HIP;
  }
  return LINGEN_OK;
}
