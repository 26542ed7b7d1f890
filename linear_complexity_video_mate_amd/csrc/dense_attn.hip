// Dense (full) softmax attention over all tokens of a sequence, per head, on
// gfx950: the quadratic token mixer that MATE replaces.  It is not part of the
// MATE forward pass; it exists so that MATE's linear cost can be measured
// against the mixer it displaces at the same sequence length, heads and head
// size (page "Towards High-Resolution Minute-Length Text-to-Video Generation
// with Linear Computational Complexity", abstract: MATE against DiT's
// self-attention; page "视频生成模子太贵太慢如何办？", section 评估: latency and
// FLOP ratios against the attention model at equal size).
//
//   o_i = sum_j softmax_j(q_i . k_j / sqrt(d)) v_j,   j over all L tokens.
//
// One workgroup owns NW*QTW*16 queries of one head and streams every key and
// value of that head through LDS in blocks of 64, NS blocks in flight (direct
// global-to-LDS loads into a ring of separate LDS arrays).  Each wave keeps
// QTW query tiles of 16 in registers and computes, per block,
//   S^T = K Q^T           (MFMA, K fragments from LDS, Q fragments in registers)
//   P^T = 2^(S^T*sc - m)  (online softmax, running maximum per query)
//   O^T += V^T P^T        (MFMA, V^T fragments by transposing LDS reads, P^T
//                          straight from the S^T registers)
// and the K / V fragments of a block are shared by the wave's query tiles.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "lingen_device.h"
#include "lingen_internal.h"

namespace lingen {

template <int DH, int NW, int QTW>
struct DenseCfg {
  static constexpr int BK = 64;                 // keys per LDS block
  static constexpr int NS = 4;                  // blocks in flight
  static constexpr int QB = NW * QTW * 16;      // queries per workgroup
  static constexpr int VEC = 8;                 // bf16 per 16-byte chunk
  static constexpr int CPR = DH / VEC;          // chunks per row
  static constexpr int DMA = BK * CPR / (NW * 64);   // 16-byte loads per lane per tile
  static_assert(CPR == 8, "rows of 128 bytes");
  static_assert((BK * CPR) % (NW * 64) == 0 && DMA >= 1, "whole wave-wide LDS loads per tile");
};

template <int DH, int NW, int QTW>
__global__ __launch_bounds__(NW * 64, 2) void dense_attn_kernel(const __bf16* __restrict__ q,
                                                             const __bf16* __restrict__ k,
                                                             const __bf16* __restrict__ v, int L, int heads,
                                                             __bf16* __restrict__ o) {
  using Cfg = DenseCfg<DH, NW, QTW>;
  using KT = KvTile<__bf16, DH>;
  constexpr int BK = Cfg::BK, NS = Cfg::NS;
  constexpr int ET = DH / 16;      // output tiles along d
  constexpr int NKS = DH / 32;     // MFMA k-steps along d
  __shared__ __attribute__((aligned(16))) __bf16 sK0[BK * DH], sK1[BK * DH], sK2[BK * DH], sK3[BK * DH];
  __shared__ __attribute__((aligned(16))) __bf16 sV0[BK * DH], sV1[BK * DH], sV2[BK * DH], sV3[BK * DH];
  static_assert(NS == 4, "four LDS blocks in the ring");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, grp = lane >> 4;
  const int h = blockIdx.y;
  const int64_t rowstride = int64_t(heads) * DH;
  const int64_t boff = int64_t(blockIdx.z) * L * rowstride + int64_t(h) * DH;
  const __bf16* qb = q + boff;
  const __bf16* kb = k + boff;
  const __bf16* vb = v + boff;
  __bf16* ob = o + boff;
  const float sc = kLog2e * rsqrtf(float(DH));
  const int nblk = (L + BK - 1) / BK;

  // Direct loads of key block j into (dK, dV).  Rows past the end of the
  // sequence re-read the last token (their scores are masked below).
  auto issue = [&](int j, __bf16* dK, __bf16* dV) {
#pragma unroll
    for (int d = 0; d < Cfg::DMA; ++d) {
      const int base = (wave * Cfg::DMA + d) * 64;
      const int u = base + lane, row = u / Cfg::CPR, ch = (u % Cfg::CPR) ^ (row & 7);
      const int tok = min(j * BK + row, L - 1);
      const int64_t goff = int64_t(tok) * rowstride + ch * Cfg::VEC;
      lds_load16(kb + goff, dK + base * Cfg::VEC);
      lds_load16(vb + goff, dV + base * Cfg::VEC);
    }
  };

  // Query fragments (B operand of S^T = K Q^T): column r16 of query tile qt.
  const int q0 = blockIdx.x * Cfg::QB + wave * QTW * 16;
  bf16x8 qf[QTW][NKS];
#pragma unroll
  for (int qt = 0; qt < QTW; ++qt) {
    const int tok = min(q0 + qt * 16 + r16, L - 1);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[qt][ks] = Frag<__bf16>::load(qb + int64_t(tok) * rowstride + ks * 32, lane);
  }

  issue(0, sK0, sV0);
  if (nblk > 1) issue(1, sK1, sV1);
  if (nblk > 2) issue(2, sK2, sV2);

  int offk[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) offk[ks] = KT::at(r16, ks * 32 + grp * 8);
  int offv[ET];
#pragma unroll
  for (int et = 0; et < ET; ++et) offv[et] = KT::at(4 * grp + (r16 >> 2), et * 16 + 4 * (r16 & 3));

  // Running maximum (scaled units) and softmax denominator per query.  The
  // denominator is accumulated on the MFMA from the same bf16 weights as the
  // output: an all-ones A operand gives the column sums of P^T, so every lane
  // holds the sum of its query column.
  float m[QTW];
  f32x4 den[QTW];
  f32x4 acc[QTW][ET];
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = static_cast<__bf16>(1.f);
#pragma unroll
  for (int qt = 0; qt < QTW; ++qt) {
    m[qt] = -INFINITY;
    den[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int et = 0; et < ET; ++et) acc[qt][et] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Block j sits in (cK, cV); block j + 3 is loaded into (nK, nV), which
  // held block j - 1.
  auto step = [&](int j, const __bf16* cK, const __bf16* cV, __bf16* nK, __bf16* nV) __attribute__((always_inline)) {
    // Wait for this wave's loads of block j (two per lane and block; the
    // younger blocks j+1, j+2 may stay in flight), then for every wave's.
    if (j + 2 < nblk) __builtin_amdgcn_s_waitcnt(0x0f70 | (4 * Cfg::DMA));
    else wait_vmem();
    lds_barrier();
    if (j + 3 < nblk) issue(j + 3, nK, nV);

    // All K and V^T fragments of the block, shared by the wave's query tiles.
    bf16x8 kf[4][NKS], vf[2][ET];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) kf[kt][ks] = *reinterpret_cast<const bf16x8*>(cK + offk[ks] + kt * 16 * DH);
    lds_bf16* vl = (lds_bf16*)(cV);
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int et = 0; et < ET; ++et) {
        const bf16x4 lo = lds_read_tr(vl + offv[et] + (32 * sb) * DH);
        const bf16x4 hi = lds_read_tr(vl + offv[et] + (32 * sb + 16) * DH);
        vf[sb][et] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    const int kend = L - j * BK;   // valid keys in the block (all of them but in the last)

#pragma unroll
    for (int qt = 0; qt < QTW; ++qt) {
      f32x4 s[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) a = mma(kf[kt][ks], qf[qt][ks], a);
        s[kt] = a;
      }
      if (kend < BK) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (kt * 16 + 4 * grp + r >= kend) s[kt][r] = -INFINITY;
      }
      float bm = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) bm = fmaxf(bm, fmaxf(fmaxf(s[kt][0], s[kt][1]), fmaxf(s[kt][2], s[kt][3])));
      bm = max_rows(bm);
      const float mnew = fmaxf(m[qt], bm * sc);
      // Rescale the running output only when some query's maximum grew.
      if (__ballot(mnew > m[qt])) {
        const float alpha = fast_exp2(m[qt] - mnew);
#pragma unroll
        for (int r = 0; r < 4; ++r) den[qt][r] *= alpha;
#pragma unroll
        for (int et = 0; et < ET; ++et)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[qt][et][r] *= alpha;
        m[qt] = mnew;
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) s[kt][r] = fast_exp2(fmaf(s[kt][r], sc, -m[qt]));
      // P^T operand of a 32-key sub-block: lane group g brings keys
      // 4g..4g+3 of both 16-key tiles (the k order of the V^T reads).
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        bf16x8 pb;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pb[r] = static_cast<__bf16>(s[2 * sb][r]);
          pb[4 + r] = static_cast<__bf16>(s[2 * sb + 1][r]);
        }
#pragma unroll
        for (int et = 0; et < ET; ++et) acc[qt][et] = mma(vf[sb][et], pb, acc[qt][et]);
        den[qt] = mma(ones, pb, den[qt]);
      }
    }
  };

#pragma unroll 1
  for (int j = 0; j < nblk; j += NS) {
    step(j, sK0, sV0, sK3, sV3);
    if (j + 1 < nblk) step(j + 1, sK1, sV1, sK0, sV0);
    if (j + 2 < nblk) step(j + 2, sK2, sV2, sK1, sV1);
    if (j + 3 < nblk) step(j + 3, sK3, sV3, sK2, sV2);
  }

  // O^T[d][q]: lane holds d = et*16 + 4*grp + r of query column r16.
#pragma unroll
  for (int qt = 0; qt < QTW; ++qt) {
    const float inv = __builtin_amdgcn_rcpf(den[qt][0]);
    const int tok = q0 + qt * 16 + r16;
    if (tok < L) {
      __bf16* orow = ob + int64_t(tok) * rowstride;
#pragma unroll
      for (int et = 0; et < ET; ++et) {
        bf16x4 res;
#pragma unroll
        for (int r = 0; r < 4; ++r) res[r] = static_cast<__bf16>(acc[qt][et][r] * inv);
        *reinterpret_cast<bf16x4*>(orow + et * 16 + grp * 4) = res;
      }
    }
  }
}

namespace {

constexpr int kDenseWaves = 8, kDenseQTiles = 4;

}  // namespace
}  // namespace lingen

using namespace lingen;

extern "C" int lingen_dense_attn_fwd(const void* q, const void* k, const void* v, void* o, int32_t batch,
                                     int32_t L, int32_t heads, int32_t head_dim, int32_t dtype,
                                     hipStream_t stream) {
  if (dtype != LINGEN_F32 && dtype != LINGEN_BF16) return LINGEN_ERR_DTYPE;
  if (batch < 0 || L < 0 || heads < 0 || head_dim < 1) return LINGEN_ERR_SHAPE;
  if (int64_t(batch) * L * heads * head_dim > (int64_t(1) << 40)) return LINGEN_ERR_SHAPE;
  if (batch > 65535 || heads > 65535) return LINGEN_ERR_SHAPE;
  if (dtype != LINGEN_BF16 || head_dim != 64) return LINGEN_ERR_UNSUPPORTED;
  if (batch == 0 || L == 0 || heads == 0) return LINGEN_OK;
  for (const void* p : {q, k, v, static_cast<const void*>(o)})
    if (int rc = check_ptr(p)) return rc;
  using Cfg = DenseCfg<64, kDenseWaves, kDenseQTiles>;
  const int64_t qblocks = (int64_t(L) + Cfg::QB - 1) / Cfg::QB;
  const dim3 grid{unsigned(qblocks), unsigned(heads), unsigned(batch)};
  dense_attn_kernel<64, kDenseWaves, kDenseQTiles><<<grid, kDenseWaves * 64, 0, stream>>>(
      static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), static_cast<const __bf16*>(v), L, heads,
      static_cast<__bf16*>(o));
  return launch_status(__func__);
}
