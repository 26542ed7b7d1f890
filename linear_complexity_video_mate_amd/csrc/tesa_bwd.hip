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
// loads in the order phase A needs them (Q and the first half of K and V
// before it starts, the rest waited for inside it).  Phase A, each wave owning 32 query rows: an online-softmax sweep
// over 32-key blocks gives each row's log-sum-exp and its output o (fp32),
// hence D; the reference maximum of a row moves only when a block exceeds it
// by more than 2^8 in weight, so most blocks skip the rescaling of o.  Phase
// B, each wave owning 32 key rows, sweeps 32-query blocks once: S and dP
// from Q K^T and dO V^T with the stored row statistics give P and dS, then
// dv^T += dO^T P and dk^T += Q^T dS accumulate in registers.  The same dS
// block, written key-major to LDS by all eight waves (in the space V no
// longer needs), gives the block's dq = s dS K: each wave forms one 16x16
// tile of it over all 256 keys, one block behind, beside the next block's
// score products; two buffers and one barrier per block keep the writes of
// a block clear of the reads of the one before.  Every product is a 16x16x32 bf16
// MFMA with fp32 accumulation; the k-permuted register operands and the
// transposing LDS reads are those of the forward window kernel.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "lingen_device.h"
#include "lingen_internal.h"
#include "lingen_window.h"

namespace lingen {

namespace {

constexpr int kBwdWin = 256, kBwdDim = 64, kBwdWaves = 8;
constexpr int kDsRow = 48;               // bf16 per key row of a dS block: 32 queries + padding
constexpr int kDsBuf = kBwdWin * kDsRow; // one 32-query dS block, key-major
constexpr float kLazy = 8.f;             // log2 of the largest weight before the row maximum moves

// s_waitcnt immediate: at most n vector-memory operations outstanding
// (vmcnt split over bits 3:0 and 15:14; expcnt and lgkmcnt not waited for).
constexpr int vmcnt_count(int n) { return 0x0f70 | (n & 15) | ((n >> 4) << 14); }

// Direct global-to-LDS load of 16 bytes per lane (lane i to lds_wave_base +
// 16 i), issued from inline asm.  The compiler does not see these loads, so
// it adds no wait of its own for them (it cannot tell which LDS array such a
// load writes, and would wait for all of them before any LDS read); the
// kernel waits for them itself with counted vmcnt waits, which also cover the
// compiler's own vector-memory operations, since those complete in order
// with these.  The instruction has no result register: its data goes to LDS.
__device__ __forceinline__ void lds_load16_counted(const void* src, void* lds_wave_base) {
  const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_bf16*)lds_wave_base));
  // (m0 is saved and restored around the load: the compiler reserves it)
  uint32_t keep;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(keep)
               : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// Barrier after waiting for this wave's direct global-to-LDS loads (vmcnt):
// the wave has no LDS stores of its own pending, so the release half of
// lds_barrier is not needed, and it would wait for every direct load still in
// flight (they count as the wave's LDS stores), not just the ones waited for.
__device__ __forceinline__ void dma_barrier() {
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Maxima of scores (finite or -inf, never NaN) in one instruction each,
// without the quieting of signalling NaNs that fmaxf adds to every operand.
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// maximum over the four rows (lanes l, l ^ 16, l ^ 32, l ^ 48)
__device__ __forceinline__ float vmax_rows(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

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

// The item's tiles and per-slot tables in LDS.
struct BwdLds {
  __bf16 *sQ, *sK, *sG, *sV;   // sV: V, then the two dS blocks of phase B
  int *sTok, *sCls;
  float *sLse, *sD;            // log2-sum-exp of the scaled scores; -sum_d dO . o
};

// Phases A and B of one item whose tiles are in LDS.  MASK: a window cut by
// the grid's border, whose slots of different wrap classes do not attend to
// each other; the two instantiations keep the loops free of branches.
// SAVED: the statistics come from the forward (its log2-sum-exp and its
// output o, from which D is formed before this function), so phase A is
// skipped.
template <bool MASK, bool SAVED>
__device__ __forceinline__ void bwd_phases(const BwdLds& S, int lane, int wave, int64_t rowstride, int64_t hoff,
                                           __bf16* __restrict__ dq, __bf16* __restrict__ dk,
                                           __bf16* __restrict__ dv) {
  constexpr int NWIN = kBwdWin, DH = kBwdDim, ET = DH / 16, NKS = DH / 32;
  using KT = KvTile<__bf16, DH>;
  const int r16 = lane & 15, grp = lane >> 4;
  const float sc = kLog2e * rsqrtf(float(DH));   // scores in log2 units
  const float snat = rsqrtf(float(DH));          // 1/sqrt(d)
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

  // ---------------- Phase A: statistics of the wave's query rows ----------
  if constexpr (!SAVED) {
    int icls[2] = {0, 0};
    bf16x8 qf[2][NKS];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const int i0 = (2 * wave + qt) * 16;
      if (MASK) icls[qt] = S.sCls[i0 + r16];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qf[qt][ks] = rowfrag(S.sQ, i0, ks);
    }
    // m: the reference maximum of the row's scaled scores (-inf until a
    // finite score), l: sum of the weights 2^(score - m) as rounded for the
    // products (a product with a ones operand: every entry holds the row's
    // sum), o: sum of the weights times v.
    float m[2];
    f32x4 l[2], o[2][ET];
    bf16x8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = static_cast<__bf16>(1.f);
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      m[qt] = -INFINITY;
      l[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int et = 0; et < ET; ++et) o[qt][et] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll 1
    for (int jb = 0; jb < NWIN; jb += 32) {
      if (jb == NWIN / 2) {
        // the last 128 rows of K and V (every wave's loads of them done)
        __builtin_amdgcn_s_waitcnt(vmcnt_count(4));
        dma_barrier();
      }
      bf16x8 kfr[2][NKS], vtr[ET];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) kfr[t][ks] = rowfrag(S.sK, jb + 16 * t, ks);
#pragma unroll
      for (int et = 0; et < ET; ++et) vtr[et] = trfrag(S.sV, jb, et);
      // S^T: the lane holds keys jb + 16 t + 4 g + r of query row r16
      f32x4 s[2][2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          s[qt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) s[qt][t] = mma(kfr[t][ks], qf[qt][ks], s[qt][t]);
        }
      if (MASK) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int4 kc = *reinterpret_cast<const int4*>(&S.sCls[jb + 16 * t + 4 * grp]);
          const int kcv[4] = {kc.x, kc.y, kc.z, kc.w};
#pragma unroll
          for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int r = 0; r < 4; ++r) s[qt][t][r] = kcv[r] != icls[qt] ? -INFINITY : s[qt][t][r];
        }
      }
      float bm[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const f32x4 a = s[qt][0], b = s[qt][1];
        bm[qt] = vmax_rows(vmax(vmax3(a[0], a[1], a[2]), vmax3(a[3], b[0], vmax3(b[1], b[2], b[3])))) * sc;
      }
      // Wave-uniform: move the reference maxima (and rescale) only when some
      // row's block maximum exceeds its reference by more than kLazy.
      if (__builtin_amdgcn_ballot_w64(bm[0] > m[0] + kLazy || bm[1] > m[1] + kLazy) != 0) {
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          const float mnew = fmaxf(m[qt], bm[qt]);
          const float alpha = m[qt] == -INFINITY ? 0.f : fast_exp2(m[qt] - mnew);
          m[qt] = mnew;
          l[qt][0] *= alpha;
#pragma unroll
          for (int et = 0; et < ET; ++et)
#pragma unroll
            for (int r = 0; r < 4; ++r) o[qt][et][r] *= alpha;
        }
      }
      bf16x8 pb[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        // all keys so far masked (a cut window): zero weights
        const float mref = m[qt] == -INFINITY ? 0.f : m[qt];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) s[qt][t][r] = fast_exp2(fmaf(s[qt][t][r], sc, -mref));
        pb[qt] = pack(s[qt][0], s[qt][1]);
      }
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        l[qt] = mma(ones, pb[qt], l[qt]);
#pragma unroll
        for (int et = 0; et < ET; ++et) o[qt][et] = mma(vtr[et], pb[qt], o[qt][et]);
      }
    }
    // dO (every wave's loads of it done)
    __builtin_amdgcn_s_waitcnt(vmcnt_count(0));
    dma_barrier();
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const int i0 = (2 * wave + qt) * 16;
      const float lt = l[qt][0];
      const float inv = 1.f / lt;
      // D_i = sum_d dO_i[d] o_i[d]: the lane holds o for d = et*16 + 4g + r.
      float ds_ = 0.f;
#pragma unroll
      for (int et = 0; et < ET; ++et) {
        const bf16x4 g4 = *reinterpret_cast<const bf16x4*>(S.sG + KT::at(i0 + r16, et * 16 + 4 * grp));
#pragma unroll
        for (int r = 0; r < 4; ++r) ds_ = fmaf(static_cast<float>(g4[r]), o[qt][et][r] * inv, ds_);
      }
      ds_ = sum_rows(ds_);
      if (grp == 0) {
        // the query's own key is never masked, so m is finite here
        S.sLse[i0 + r16] = m[qt] + log2f(lt);
        S.sD[i0 + r16] = -ds_;   // stored negated: it starts phase B's dP accumulators
      }
    }
  }
  lds_barrier();   // every query's statistics are in LDS

  // ---------------- Phase B: the wave's key rows ---------------------------
  {
    int jcls[2] = {0, 0};
    bf16x8 kf[2][NKS], vf[2][NKS];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int j0 = (2 * wave + kt) * 16;
      if (MASK) jcls[kt] = S.sCls[j0 + r16];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        kf[kt][ks] = rowfrag(S.sK, j0, ks);
        vf[kt][ks] = rowfrag(S.sV, j0, ks);
      }
    }
    f32x4 gk[2][ET], gv[2][ET];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int et = 0; et < ET; ++et) {
        gk[kt][et] = f32x4{0.f, 0.f, 0.f, 0.f};
        gv[kt][et] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    lds_barrier();   // every wave holds its rows of V: the dS blocks take that space
    // This wave's tile of each block's dq: d columns 16 eq .., queries 16 qh ..
    const int eq = wave & 3, qh = wave >> 2;
    // Offsets of the transposing reads of a dS block (key rows of kDsRow):
    // lane (r16, g) reads key row 4 g + r16 / 4, queries 16 qh + 4 (r16 % 4) ..
    const int offd = (4 * grp + (r16 >> 2)) * kDsRow + 16 * qh + 4 * (r16 & 3);

    f32x4 s[2][2], dp[2][2];   // [kt][t]
    float4 lv[2];
    f32x4 dd[2];   // -D of the block's rows
    // S and dP of block ib: the lane holds queries ib + 16 t + 4 g + r of key
    // row 32 wave + 16 kt + r16.
    auto scores = [&](int ib) {
      bf16x8 qfr[2][NKS], gfr[2][NKS];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int iq = ib + 16 * t;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          qfr[t][ks] = rowfrag(S.sQ, iq, ks);
          gfr[t][ks] = rowfrag(S.sG, iq, ks);
        }
        lv[t] = *reinterpret_cast<const float4*>(&S.sLse[iq + 4 * grp]);
        dd[t] = *reinterpret_cast<const f32x4*>(&S.sD[iq + 4 * grp]);
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          s[kt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
          dp[kt][t] = dd[t];   // dP - D: the products start from -D of the row
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            s[kt][t] = mma(qfr[t][ks], kf[kt][ks], s[kt][t]);
            dp[kt][t] = mma(gfr[t][ks], vf[kt][ks], dp[kt][t]);
          }
        }
    };
    // P and dS of block ib, dv^T += dO^T P and dk^T += Q^T dS, and dS into
    // the block's LDS buffer: key row 32 wave + 16 kt + r16, queries 16 t + 4 g ..
    auto grads = [&](int ib, __bf16* ds_blk) {
      bf16x8 trG[ET], trQ[ET];
#pragma unroll
      for (int et = 0; et < ET; ++et) {
        trG[et] = trfrag(S.sG, ib, et);
        trQ[et] = trfrag(S.sQ, ib, et);
      }
      bf16x8 pb[2], db[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f32x4 p[2], ds[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const float lvv[4] = {lv[t].x, lv[t].y, lv[t].z, lv[t].w};
          int qcv[4] = {0, 0, 0, 0};
          if (MASK) {
            const int4 c4 = *reinterpret_cast<const int4*>(&S.sCls[ib + 16 * t + 4 * grp]);
            qcv[0] = c4.x; qcv[1] = c4.y; qcv[2] = c4.z; qcv[3] = c4.w;
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float pv = fast_exp2(fmaf(s[kt][t][r], sc, -lvv[r]));
            if (MASK) pv = qcv[r] != jcls[kt] ? 0.f : pv;
            p[t][r] = pv;
            ds[t][r] = pv * dp[kt][t][r];
          }
        }
        pb[kt] = pack(p[0], p[1]);
        db[kt] = pack(ds[0], ds[1]);
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int et = 0; et < ET; ++et) {
          gv[kt][et] = mma(trG[et], pb[kt], gv[kt][et]);
          gk[kt][et] = mma(trQ[et], db[kt], gk[kt][et]);
        }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        __bf16* row = ds_blk + (32 * wave + 16 * kt + r16) * kDsRow + 4 * grp;
        *reinterpret_cast<bf16x4*>(row) = __builtin_shufflevector(db[kt], db[kt], 0, 1, 2, 3);
        *reinterpret_cast<bf16x4*>(row + 16) = __builtin_shufflevector(db[kt], db[kt], 4, 5, 6, 7);
      }
    };
    // dq of block ib once every wave's dS is in ds_blk: the wave's dq^T tile
    // = K^T dS^T over the 256 keys, both operands by transposing reads (keys
    // in the order 4 g .. 4 g + 3, 16 + 4 g ..); two accumulators halve the
    // dependent chain.
    bf16x8 kstrip[NWIN / 32];   // K^T rows of the wave's dq columns, all 256 keys
#pragma unroll
    for (int b = 0; b < NWIN / 32; ++b) kstrip[b] = trfrag(S.sK, 32 * b, eq);
    auto dq_block = [&](int ib, const __bf16* ds_blk) {
      f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int b = 0; b < NWIN / 32; ++b) {
        lds_bf16* t = (lds_bf16*)(ds_blk) + offd + 32 * b * kDsRow;
        const bf16x4 lo = lds_read_tr(t), hi = lds_read_tr(t + 16 * kDsRow);
        acc[b & 1] = mma(kstrip[b], __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7),
                         acc[b & 1]);
      }
      // the lane holds dq[query ib + 16 qh + r16][d = 16 eq + 4 g + r]
      bf16x4 out;
#pragma unroll
      for (int r = 0; r < 4; ++r) out[r] = static_cast<__bf16>((acc[0][r] + acc[1][r]) * snat);
      *reinterpret_cast<bf16x4*>(dq + int64_t(S.sTok[ib + 16 * qh + r16]) * rowstride + hoff + 16 * eq + 4 * grp) =
          out;
    };

    // Block n's dq is formed in iteration n + 1, beside block n + 1's score
    // products; one barrier per block publishes its dS and retires the reads
    // of the buffer the block writes next.
    scores(0);
    grads(0, S.sV);
#pragma unroll 1
    for (int n = 1; n < NWIN / 32; ++n) {
      lds_barrier();
      scores(32 * n);
      dq_block(32 * (n - 1), S.sV + ((n - 1) & 1) * kDsBuf);
      grads(32 * n, S.sV + (n & 1) * kDsBuf);
    }
    lds_barrier();
    dq_block(NWIN - 32, S.sV + ((NWIN / 32 - 1) & 1) * kDsBuf);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int j = (2 * wave + kt) * 16 + r16;
      const int64_t roff = int64_t(S.sTok[j]) * rowstride + hoff;
      store_rows16(dk + roff, gk[kt], snat, grp);
      store_rows16(dv + roff, gv[kt], 1.f, grp);
    }
  }
}

// SAVED: o (the forward's output, layout of q) and lse (its log2-sum-exp of
// the scaled scores per query and head, [L][Ha] fp32) replace phase A.
template <bool SAVED>
__global__ __launch_bounds__(64 * kBwdWaves) void tesa_bwd_kernel(const __bf16* __restrict__ q,
                                                                  const __bf16* __restrict__ k,
                                                                  const __bf16* __restrict__ v,
                                                                  const __bf16* __restrict__ dO, WinGeom wg, int Ha,
                                                                  __bf16* __restrict__ dq, __bf16* __restrict__ dk,
                                                                  __bf16* __restrict__ dv, const __bf16* __restrict__ o,
                                                                  const float* __restrict__ lse) {
  constexpr int NWIN = kBwdWin, DH = kBwdDim;
  constexpr int NW = kBwdWaves, NTHR = NW * 64;
  static_assert(NWIN == 32 * NW, "32 query rows and 32 key rows per wave");
  static_assert(2 * kDsBuf >= NWIN * DH, "the dS buffers fill the space of V");
  // One LDS array (the kernel's only one, so it starts at LDS address 0):
  // the four tiles filled by direct loads lie in its first 128 KiB, the
  // range those loads address, and V's 32 KiB, the last of them, take (with
  // the 16 KiB after them) the two dS blocks of phase B; the per-slot
  // tables follow.
  constexpr int TILE = NWIN * DH;
  __shared__ __attribute__((aligned(16))) unsigned char smem[(3 * TILE + 2 * kDsBuf) * 2 + 4 * NWIN * 4];
  static_assert(4 * TILE * 2 <= 128 * 1024, "direct-load targets below 128 KiB");
  __bf16* const tQ = reinterpret_cast<__bf16*>(smem);
  __bf16* const tK = tQ + TILE;
  __bf16* const tG = tQ + 2 * TILE;
  __bf16* const tV = tQ + 3 * TILE;
  int* const tTok = reinterpret_cast<int*>(tV + 2 * kDsBuf);
  int* const tCls = tTok + NWIN;
  float* const tLse = reinterpret_cast<float*>(tCls + NWIN);
  float* const tD = tLse + NWIN;
  BwdLds S{tQ, tK, tG, tV, tTok, tCls, tLse, tD};

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int item = blockIdx.x;
  const int h = item % Ha, win = item / Ha;
  const int nwin_hw = wg.nwh * wg.nww;
  const int wi = win / nwin_hw, wj = (win / wg.nww) % wg.nwh, wk = win % wg.nww;
  const int64_t rowstride = int64_t(Ha) * DH;
  const int64_t hoff = int64_t(h) * DH;

  for (int u = tid; u < NWIN; u += NTHR) {
    const int a = u / (wg.wh * wg.ww), b = (u / wg.ww) % wg.wh, c = u % wg.ww;
    int cl;
    S.sTok[u] = window_token(wg, wi, wj, wk, a, b, c, cl);
    S.sCls[u] = wg.masked ? cl : 0;
  }
  lds_barrier();
  // Direct loads of the four tiles in the order phase A needs them: Q, the
  // first 128 rows of K and V, their last 128 rows (waited for halfway
  // through phase A), then dO (waited for at its end).  16-byte chunk u of a
  // tile is row u/8, chunk (u%8) ^ (row%8) of that row (the KvTile
  // permutation); load d of a wave takes chunks (d * 8 + wave) * 64 .., so
  // loads 0 and 1 of every wave fill rows 0 .. 127.
  static_assert(NWIN * 8 == 4 * NW * 64, "four loads per wave and tile");
  auto issue = [&](const __bf16* src, __bf16* dst, int d) {
    const int base = (d * NW + wave) * 64;
    const int u = base + lane, row = u / 8, ch = (u % 8) ^ (row & 7);
    lds_load16_counted(src + int64_t(S.sTok[row]) * rowstride + hoff + ch * 8, dst + base * 8);
  };
#pragma unroll
  for (int d = 0; d < 4; ++d) issue(q, S.sQ, d);
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    issue(k, S.sK, d);
    issue(v, S.sV, d);
  }
#pragma unroll
  for (int d = 0; d < 4; ++d) issue(dO, S.sG, d);
  if constexpr (SAVED) {
    // D_i = sum_d dO_i[d] o_i[d] and the saved statistics of the wave's 32
    // query rows: lane group g takes d = 16 g .. 16 g + 15 of row r16
    using KT = KvTile<__bf16, DH>;
    const int r16 = lane & 15, grp = lane >> 4;
    bf16x8 ov[2][2];
    float lv[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const int tok = S.sTok[(2 * wave + qt) * 16 + r16];
      const __bf16* orow = o + int64_t(tok) * rowstride + hoff + 16 * grp;
      ov[qt][0] = *reinterpret_cast<const bf16x8*>(orow);
      ov[qt][1] = *reinterpret_cast<const bf16x8*>(orow + 8);
      lv[qt] = lse[int64_t(tok) * Ha + h];
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_count(0));   // every tile, o and the statistics
    dma_barrier();
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const int i = (2 * wave + qt) * 16 + r16;
      float ds_ = 0.f;
#pragma unroll
      for (int c8 = 0; c8 < 2; ++c8) {
        const bf16x8 g8 = *reinterpret_cast<const bf16x8*>(S.sG + KT::at(i, 16 * grp + 8 * c8));
#pragma unroll
        for (int e = 0; e < 8; ++e) ds_ = fmaf(static_cast<float>(g8[e]), static_cast<float>(ov[qt][c8][e]), ds_);
      }
      ds_ = sum_rows(ds_);
      if (grp == 0) {
        S.sLse[i] = lv[qt];
        S.sD[i] = -ds_;   // stored negated: it starts phase B's dP accumulators
      }
    }
  } else {
    __builtin_amdgcn_s_waitcnt(vmcnt_count(8));   // Q and the first halves of K and V
    dma_barrier();
  }

  if (wg.masked && window_wrapped(wg, wi, wj, wk))
    bwd_phases<true, SAVED>(S, lane, wave, rowstride, hoff, dq, dk, dv);
  else
    bwd_phases<false, SAVED>(S, lane, wave, rowstride, hoff, dq, dk, dv);
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

namespace lingen {
namespace {
// o, lse: null for the backward that forms the statistics itself
int te_bwd_impl(const void* q, const void* k, const void* v, const void* d_out, const void* o, const float* lse,
                int32_t shift_t, int32_t shift_h, int32_t shift_w, int32_t masked, const lingen_mate_shape* shape,
                void* dq, void* dk, void* dv, hipStream_t stream) {
  if (int rc = validate_shape(shape)) return rc;
  if (shift_t < 0 || shift_t >= shape->win_t || shift_h < 0 || shift_h >= shape->win_h || shift_w < 0 ||
      shift_w >= shape->win_w || (masked != 0 && masked != 1))
    return LINGEN_ERR_SHAPE;
  for (const void* p : {q, k, v, d_out, static_cast<const void*>(dq), static_cast<const void*>(dk),
                        static_cast<const void*>(dv)})
    if (int rc = check_ptr(p)) return rc;
  const bool saved = o != nullptr;
  if (saved) {
    if (attn_family(shape) != ATTN_BF16_D64_W256) return LINGEN_ERR_UNSUPPORTED;
    for (const void* p : {o, static_cast<const void*>(lse)})
      if (int rc = check_ptr(p)) return rc;
  }
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
    const __bf16* qb = static_cast<const __bf16*>(q) + off;
    const __bf16* kb = static_cast<const __bf16*>(k) + off;
    const __bf16* vb = static_cast<const __bf16*>(v) + off;
    const __bf16* gb = static_cast<const __bf16*>(d_out) + off;
    __bf16* dqb = static_cast<__bf16*>(dq) + off;
    __bf16* dkb = static_cast<__bf16*>(dk) + off;
    __bf16* dvb = static_cast<__bf16*>(dv) + off;
    if (saved)
      tesa_bwd_kernel<true><<<items, 64 * kBwdWaves, 0, stream>>>(
          qb, kb, vb, gb, g, shape->attn_heads, dqb, dkb, dvb, static_cast<const __bf16*>(o) + off,
          lse + int64_t(b) * L * shape->attn_heads);
    else
      tesa_bwd_kernel<false><<<items, 64 * kBwdWaves, 0, stream>>>(qb, kb, vb, gb, g, shape->attn_heads, dqb, dkb,
                                                                   dvb, nullptr, nullptr);
    if (launch_status(__func__) != LINGEN_OK) return LINGEN_ERR_HIP;
  }
  return LINGEN_OK;
}
}  // namespace
}  // namespace lingen

extern "C" int lingen_te_bwd(const void* q, const void* k, const void* v, const void* d_out, int32_t shift_t,
                             int32_t shift_h, int32_t shift_w, int32_t masked, const lingen_mate_shape* shape,
                             void* dq, void* dk, void* dv, hipStream_t stream) {
  return te_bwd_impl(q, k, v, d_out, nullptr, nullptr, shift_t, shift_h, shift_w, masked, shape, dq, dk, dv, stream);
}

extern "C" int lingen_te_bwd_saved(const void* q, const void* k, const void* v, const void* o, const void* d_out,
                                   const float* lse, int32_t shift_t, int32_t shift_h, int32_t shift_w,
                                   int32_t masked, const lingen_mate_shape* shape, void* dq, void* dk, void* dv,
                                   hipStream_t stream) {
  for (const void* p : {o, static_cast<const void*>(lse)})
    if (int rc = check_ptr(p)) return rc;
  return te_bwd_impl(q, k, v, d_out, o, lse, shift_t, shift_h, shift_w, masked, shape, dq, dk, dv, stream);
}
