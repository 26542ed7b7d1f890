// TEmporal Swin Attention over 256-token windows (4x8x8 at the workloads'
// shapes), bf16 storage, head size 64, on gfx950: softmax attention inside
// each (possibly shifted) 3D window, plus the fused branch sum y = y_MA + o
// (page "LinGen：基于Mamba机制的线性复杂度高清长视频生成框架", section 关键算法创新
// > TESA: fixed small windows, plain and shifted partitions alternating by
// layer; page "Towards High-Resolution Minute-Length Text-to-Video Generation
// with Linear Computational Complexity", abstract: MATE = MA branch + TE
// branch).
//
// A window holds only 256 keys, so a wave takes its 16 queries' scores in
// two halves of 128 keys, each half's scores in registers (8 MFMA result
// tiles, 32 VGPRs), and the exact maximum of a half before any exponential:
// one exp2 per score and a single rescale of the output per item (when the
// second half raises a query's maximum), instead of a running maximum per
// key block.  Per (window, head) item and wave, per half:
//   S^T[j][i] = K_j . Q_i        (MFMA; K from LDS, Q fragments in registers)
//   m_i = max(m_i, max_j S[i][j]) (masked scores are -inf)
//   P^T = 2^(S^T sc - m sc),  sc = log2(e)/sqrt(d), rounded to bf16
//   O^T += V^T P^T               (MFMA; V^T by transposing LDS reads)
//   l_i = sum_j P^T[j][i]        (MFMA against an all-ones operand, from the
//                                 same rounded weights as the output)
//   y_i = y_MA_i + O_i / l_i
// The kernel is persistent (one 16-wave workgroup per compute unit, one
// 16-query tile per wave).  With an even head count, an item is a window
// and two heads (tesa_win256_pair_kernel): the two heads' K and V rows,
// 256 contiguous bytes of each token row, arrive together by direct
// global-to-LDS loads into a ring of two window halves, each refilled with
// the next item's half as soon as both heads are done with it.  With an odd
// head count, an item is one window and head (tesa_win256_kernel): while it
// is computed, the next item's K and V stream into the second of two LDS
// buffer pairs and its Q fragments into registers.  The shift is index
// arithmetic: windows are enumerated on the offset grid, wrapping around each
// axis, and a wrap class per slot masks scores between tokens that the cut
// partition separates.
//
// Built without NaN semantics: scores are finite or -inf, and the maxima
// then take v_max3 without NaN-quieting instructions.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "lingen_device.h"
#include "lingen_internal.h"
#include "lingen_window.h"

namespace lingen {

namespace {

constexpr int kW256Waves = 16;  // one workgroup per compute unit, four waves per SIMD
constexpr int kW256QTiles = 1;  // 16-query tiles per wave
constexpr int kW256KBlocks = 2; // key blocks per item: 128 keys' scores per query tile live at a time

template <bool ACCUMULATE>
__global__ __launch_bounds__(kW256Waves * 64) void tesa_win256_kernel(const __bf16* __restrict__ q,
                                                                      const __bf16* __restrict__ k,
                                                                      const __bf16* __restrict__ v, WinGeom wg,
                                                                      int Ha, int n_items, int contiguous,
                                                                      __bf16* __restrict__ y) {
  constexpr int DH = 64, NWIN = 256, NWAVE = kW256Waves, QT = kW256QTiles, KB = kW256KBlocks;
  constexpr int BKEYS = NWIN / KB;                 // keys per block
  constexpr int NTHR = NWAVE * 64;
  constexpr int CPR = DH / 8;                      // 16-byte chunks per K / V row
  constexpr int DMA = NWIN * CPR / NTHR;           // direct loads per lane and tile
  static_assert(NWIN * CPR % NTHR == 0 && NWIN / 16 == NWAVE * QT, "query tiles cover the window");
  static_assert(NWIN <= NTHR, "one window slot per thread");
  using KT = KvTile<__bf16, DH>;
  __shared__ __attribute__((aligned(16))) __bf16 sK0[NWIN * DH];
  __shared__ __attribute__((aligned(16))) __bf16 sK1[NWIN * DH];
  __shared__ __attribute__((aligned(16))) __bf16 sV0[NWIN * DH];
  __shared__ __attribute__((aligned(16))) __bf16 sV1[NWIN * DH];
  __shared__ int sTok[2][NWIN];   // token of each window slot (item parity)
  __shared__ __attribute__((aligned(16))) int sCls[3][NWIN];   // wrap class of each slot (item mod 3)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, grp = lane >> 4;
  const int64_t rowstride = int64_t(Ha) * DH;
  const int nwin_hw = wg.nwh * wg.nww;
  const float sc = kLog2e * 0.125f;   // log2(e) / sqrt(64)

  // Items (window, head), item = window * Ha + head.  A workgroup walks
  // either every gridDim-th item (strided) or a contiguous range of items
  // (contiguous: the heads of one window one after another).
  int it_begin, it_end, it_step;
  if (contiguous) {
    it_begin = int(int64_t(blockIdx.x) * n_items / gridDim.x);
    it_end = int(int64_t(blockIdx.x + 1) * n_items / gridDim.x);
    it_step = 1;
  } else {
    it_begin = int(blockIdx.x);
    it_end = n_items;
    it_step = int(gridDim.x);
  }
  struct ItemPos { int item, h, wi, wj, wk; };
  auto decompose = [&](int it) {
    const int win = it / Ha;
    return ItemPos{it, it % Ha, win / nwin_hw, (win / wg.nww) % wg.nwh, win % wg.nww};
  };
  const ItemPos step_pos = decompose(it_step);
  auto advance = [&](ItemPos p) {   // p + it_step in mixed radix (head, wk, wj, wi)
    p.item += it_step;
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
  // This thread's window slot (tid < NWIN).
  const int slot_a = tid / (wg.wh * wg.ww), slot_b = (tid / wg.ww) % wg.wh, slot_c = tid % wg.ww;
  auto item_tokens = [&](const ItemPos& p, int* tok, int* cls) {
    if (tid < NWIN) {
      int cl;
      tok[tid] = window_token(wg, p.wi, p.wj, p.wk, slot_a, slot_b, slot_c, cl);
      cls[tid] = wg.masked ? cl : 0;
    }
  };
  // Direct global-to-LDS loads of an item's K and V tiles: 64 chunks (8
  // rows) per instruction, each lane fetching the chunk that lands in its
  // slot of the swizzled tile.
  auto issue_kv = [&](__bf16* dK, __bf16* dV, const int* tok, int h) {
#pragma unroll
    for (int d = 0; d < DMA; ++d) {
      const int base = (wave * DMA + d) * 64;
      const int u = base + lane, row = u / CPR, ch = (u % CPR) ^ (row & 7);
      const int64_t goff = int64_t(tok[row]) * rowstride + int64_t(h) * DH + ch * 8;
      lds_load16(k + goff, dK + base * 8);
      lds_load16(v + goff, dV + base * 8);
    }
  };
  // y is read and written in 16-byte pieces: after the exchange in the
  // epilogue a lane holds d0 .. d0 + 7 of the two 32-wide halves of its row.
  const int y16_off = 16 * (grp & 1) + 8 * (grp >> 1);
  // Per-lane registers of an item, loaded one item ahead: the wave's query
  // tiles (Q fragments, the B operand of S^T = K Q^T) and their tokens.
  struct QState {
    bf16x8 qf[QT][2];
    int tokq[QT];
  };
  auto load_q = [&](QState& qs, const int* tok, int h) {
#pragma unroll
    for (int qi = 0; qi < QT; ++qi) {
      qs.tokq[qi] = tok[(wave + qi * NWAVE) * 16 + r16];
      const __bf16* qrow = q + int64_t(qs.tokq[qi]) * rowstride + int64_t(h) * DH;
      qs.qf[qi][0] = Frag<__bf16>::load(qrow, lane);
      qs.qf[qi][1] = Frag<__bf16>::load(qrow + 32, lane);
    }
  };

  if (it_begin >= it_end) return;
  ItemPos pos = decompose(it_begin);
  item_tokens(pos, sTok[0], sCls[0]);
  lds_barrier();
  QState nxt;
  issue_kv(sK0, sV0, sTok[0], pos.h);
  load_q(nxt, sTok[0], pos.h);

  // Per-lane LDS offsets of the operand fragments in rows 0..15 of a tile;
  // a fragment 16 rows further down is 16*DH elements further on.
  const int offk0 = KT::at(r16, grp * 8), offk1 = KT::at(r16, 32 + grp * 8);
  int offv[4];
#pragma unroll
  for (int et = 0; et < 4; ++et) offv[et] = KT::at(4 * grp + (r16 >> 2), et * 16 + 4 * (r16 & 3));
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = static_cast<__bf16>(1.f);

  auto step = [&](int n, const __bf16* cK, const __bf16* cV, __bf16* nK, __bf16* nV) -> bool {
    const int h = pos.h;
    const ItemPos npos = advance(pos);
    const bool has_next = npos.item < it_end;
    if (has_next) item_tokens(npos, sTok[(n + 1) & 1], sCls[(n + 1) % 3]);
    wait_vmem();     // this wave's loads of the item (and its earlier stores) are done
    lds_barrier();   // ... and every wave's; the other buffer pair is free
    const QState cur = nxt;
    if (has_next) {
      issue_kv(nK, nV, sTok[(n + 1) & 1], npos.h);
      load_q(nxt, sTok[(n + 1) & 1], npos.h);
    }
    // The MA output this item adds to arrives while the products run.
    bf16x8 ya[QT][2];
    if constexpr (ACCUMULATE) {
#pragma unroll
      for (int qi = 0; qi < QT; ++qi) {
        const __bf16* yrow = y + int64_t(cur.tokq[qi]) * rowstride + int64_t(h) * DH + y16_off;
        ya[qi][0] = *reinterpret_cast<const bf16x8*>(yrow);
        ya[qi][1] = *reinterpret_cast<const bf16x8*>(yrow + 32);
      }
    }
    const bool wrapped = wg.masked && window_wrapped(wg, pos.wi, pos.wj, pos.wk);
    const int* cls = sCls[n % 3];
    int qcls[QT];
#pragma unroll
    for (int qi = 0; qi < QT; ++qi) qcls[qi] = cls[(wave + qi * NWAVE) * 16 + r16];

    // The keys in KB blocks: the scores of one block for the wave's query
    // tiles stay in registers (lane (grp, r16) holds keys
    // BKEYS hf + 16 kt + 4 grp + r of query r16 in s[qi][kt][r]), their
    // maximum is taken before any exponential, and the output so far is
    // rescaled when a later block raises a query's maximum.  Every K and V
    // fragment read from LDS serves all of the wave's query tiles.
    f32x4 o[QT][4], den[QT];
    float m[QT];
#pragma unroll
    for (int qi = 0; qi < QT; ++qi) {
      den[qi] = f32x4{0.f, 0.f, 0.f, 0.f};
      m[qi] = -INFINITY;   // running maximum, scaled units
#pragma unroll
      for (int et = 0; et < 4; ++et) o[qi][et] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    lds_bf16* vb = (lds_bf16*)(cV);
#pragma unroll
    for (int hf = 0; hf < KB; ++hf) {
      f32x4 s[QT][BKEYS / 16];
#pragma unroll
      for (int kt = 0; kt < BKEYS / 16; ++kt) {
        const int row = hf * BKEYS + kt * 16;
        const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(cK + offk0 + row * DH);
        const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(cK + offk1 + row * DH);
#pragma unroll
        for (int qi = 0; qi < QT; ++qi)
          s[qi][kt] = mma(k1, cur.qf[qi][1], mma(k0, cur.qf[qi][0], f32x4{0.f, 0.f, 0.f, 0.f}));
      }
      if (wrapped) {
#pragma unroll
        for (int kt = 0; kt < BKEYS / 16; ++kt) {
          const int4 kc = *reinterpret_cast<const int4*>(&cls[hf * BKEYS + kt * 16 + grp * 4]);
#pragma unroll
          for (int qi = 0; qi < QT; ++qi) {
            s[qi][kt][0] = kc.x != qcls[qi] ? -INFINITY : s[qi][kt][0];
            s[qi][kt][1] = kc.y != qcls[qi] ? -INFINITY : s[qi][kt][1];
            s[qi][kt][2] = kc.z != qcls[qi] ? -INFINITY : s[qi][kt][2];
            s[qi][kt][3] = kc.w != qcls[qi] ? -INFINITY : s[qi][kt][3];
          }
        }
      }
      float mref[QT];
#pragma unroll
      for (int qi = 0; qi < QT; ++qi) {
        float mx = fmaxf(fmaxf(s[qi][0][0], s[qi][0][1]), fmaxf(s[qi][0][2], s[qi][0][3]));
#pragma unroll
        for (int kt = 1; kt < BKEYS / 16; ++kt)
          mx = fmaxf(fmaxf(mx, fmaxf(s[qi][kt][0], s[qi][kt][1])), fmaxf(s[qi][kt][2], s[qi][kt][3]));
        const float mnew = fmaxf(m[qi], max_rows(mx) * sc);
        // A query whose keys so far are all masked (possible in the first
        // blocks of a cut window) keeps a zero output: its weights are
        // exp2(-inf - 0) = 0.  Its own key is always present, so the final
        // maximum is finite.
        mref[qi] = mnew == -INFINITY ? 0.f : mnew;
        if (hf) {
          const float alpha = fast_exp2(m[qi] - mref[qi]);
#pragma unroll
          for (int r = 0; r < 4; ++r) den[qi][r] *= alpha;
#pragma unroll
          for (int et = 0; et < 4; ++et)
#pragma unroll
            for (int r = 0; r < 4; ++r) o[qi][et][r] *= alpha;
        }
        m[qi] = mnew;
      }
#pragma unroll
      for (int sb = 0; sb < BKEYS / 32; ++sb) {
        const int row = hf * BKEYS + 32 * sb;
        // P^T operands of keys BKEYS hf + 32 sb .. + 31: lane group g brings
        // keys 4g .. 4g+3 of both 16-key tiles (the k order of the V^T reads).
        bf16x8 pb[QT];
#pragma unroll
        for (int qi = 0; qi < QT; ++qi) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            pb[qi][r] = static_cast<__bf16>(fast_exp2(fmaf(s[qi][2 * sb][r], sc, -mref[qi])));
            pb[qi][4 + r] = static_cast<__bf16>(fast_exp2(fmaf(s[qi][2 * sb + 1][r], sc, -mref[qi])));
          }
          den[qi] = mma(ones, pb[qi], den[qi]);
        }
#pragma unroll
        for (int et = 0; et < 4; ++et) {
          const bf16x4 lo = lds_read_tr(vb + offv[et] + row * DH);
          const bf16x4 hi = lds_read_tr(vb + offv[et] + (row + 16) * DH);
          const bf16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int qi = 0; qi < QT; ++qi) o[qi][et] = mma(vf, pb[qi], o[qi][et]);
        }
      }
    }

    // O^T[e][i]: the lane holds e = 16 et + 4 grp + r of query r16.  One
    // v_permlane16_swap per register pair exchanges the 4-element pieces of
    // d-tiles 2 r1 and 2 r1 + 1 between lane groups g and g ^ 1, so that the
    // lane holds 8 consecutive values and y moves in 16-byte pieces.
#pragma unroll
    for (int qi = 0; qi < QT; ++qi) {
      const float inv = __builtin_amdgcn_rcpf(den[qi][0]);
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
          res[e] = static_cast<__bf16>(ACCUMULATE ? static_cast<float>(ya[qi][r1][e]) + val : val);
        }
        __bf16* yrow = y + int64_t(cur.tokq[qi]) * rowstride + int64_t(h) * DH + y16_off;
        *reinterpret_cast<bf16x8*>(yrow + 32 * r1) = res;
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


// Two heads per item: item = (window, pair of heads h0 = 2 hp, h0 + 1).  A
// head's K or V row is 128 bytes of a 4 KiB token row; the two heads' rows
// are 256 contiguous bytes, and the direct loads fetch them together (four
// rows of 256 bytes per instruction instead of eight of 128), which the
// memory system serves faster.  The LDS holds the pair's keys in two slots
// of one window half each (keys 0..127, 128..255), K and V of both heads
// interleaved per key row ([row][head][64], 16-byte chunks permuted by
// row mod 8).  A wave takes its 16 queries through head h0 (half 0, half 1)
// and then head h1 (half 0, half 1); once every wave is done with h1's half
// in a slot, that slot is refilled with the next pair's half, which then has
// one half of compute to land.  Per half the arithmetic is the single-head
// kernel's: scores of 128 keys in registers, their exact maximum first, one
// rescale of the output if the second half raises it.
// s_waitcnt immediate: at most n vector-memory operations outstanding
// (vmcnt split over bits 3:0 and 15:14; expcnt and lgkmcnt not waited for).
constexpr int vmcnt_count(int n) { return 0x0f70 | (n & 15) | ((n >> 4) << 14); }

// SAVE_LSE: also write each query's log2-sum-exp of its scaled scores,
// lse[token][head] = m + log2(l) (m the row's maximum, l its sum of 2^(s - m),
// s = q.k log2(e) / sqrt(d)), which the backward pass reads instead of
// forming the row statistics again.
// The pair kernel's K and V rows are read once per launch: its direct loads
// are non-temporal.
__device__ __forceinline__ void lds_load16_nt(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, lds_wave_base, 16, 0, 2);
}

template <bool ACCUMULATE, bool SAVE_LSE = false>
__global__ __launch_bounds__(kW256Waves * 64) void tesa_win256_pair_kernel(const __bf16* __restrict__ q,
                                                                           const __bf16* __restrict__ k,
                                                                           const __bf16* __restrict__ v, WinGeom wg,
                                                                           int Ha, int n_items, int contiguous,
                                                                           __bf16* __restrict__ y,
                                                                           float* __restrict__ lse = nullptr) {
  constexpr int DH = 64, NWIN = 256, HALF = 128, NWAVE = kW256Waves;
  constexpr int NTHR = NWAVE * 64;
  constexpr int KT16 = HALF / 16;                  // 16-key tiles of a half
  constexpr int CPR = DH / 8;                      // 16-byte chunks per head row
  constexpr int DMA = HALF * 2 * CPR / NTHR;       // direct loads per lane, per tile and half
  static_assert(HALF * 2 * CPR % NTHR == 0 && NWIN / 16 == NWAVE, "one 16-query tile per wave");
  __shared__ __attribute__((aligned(16))) __bf16 sK0[HALF * 2 * DH];
  __shared__ __attribute__((aligned(16))) __bf16 sK1[HALF * 2 * DH];
  __shared__ __attribute__((aligned(16))) __bf16 sV0[HALF * 2 * DH];
  __shared__ __attribute__((aligned(16))) __bf16 sV1[HALF * 2 * DH];
  __shared__ int sTok[2][NWIN];
  __shared__ __attribute__((aligned(16))) int sCls[3][NWIN];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, grp = lane >> 4;
  const int64_t rowstride = int64_t(Ha) * DH;
  const int Hp = Ha / 2;
  const int nwin_hw = wg.nwh * wg.nww;
  const float sc = kLog2e * 0.125f;   // log2(e) / sqrt(64)

  int it_begin, it_end, it_step;
  if (contiguous) {
    it_begin = int(int64_t(blockIdx.x) * n_items / gridDim.x);
    it_end = int(int64_t(blockIdx.x + 1) * n_items / gridDim.x);
    it_step = 1;
  } else {
    it_begin = int(blockIdx.x);
    it_end = n_items;
    it_step = int(gridDim.x);
  }
  struct ItemPos { int item, hp, wi, wj, wk; };
  auto decompose = [&](int it) {
    const int win = it / Hp;
    return ItemPos{it, it % Hp, win / nwin_hw, (win / wg.nww) % wg.nwh, win % wg.nww};
  };
  const int slot_a = tid / (wg.wh * wg.ww), slot_b = (tid / wg.ww) % wg.wh, slot_c = tid % wg.ww;
  auto item_tokens = [&](const ItemPos& p, int* tok, int* cls) {
    if (tid < NWIN) {
      int cl;
      tok[tid] = window_token(wg, p.wi, p.wj, p.wk, slot_a, slot_b, slot_c, cl);
      cls[tid] = wg.masked ? cl : 0;
    }
  };
  // Direct loads of one half of the pair's K and V: unit u (16 bytes) of the
  // slot is key row u / 16, head (u / 8) mod 2, permuted chunk u mod 8.
  auto issue_half = [&](__bf16* dK, __bf16* dV, const int* tok, int hp, int half) {
#pragma unroll
    for (int d = 0; d < DMA; ++d) {
      const int base = (wave * DMA + d) * 64;
      const int u = base + lane, row = u / 16, e = (u / 8) & 1, ch = (u & 7) ^ (row & 7);
      const int64_t goff = int64_t(tok[half * HALF + row]) * rowstride + int64_t(2 * hp + e) * DH + ch * 8;
      lds_load16_nt(k + goff, dK + base * 8);
      lds_load16_nt(v + goff, dV + base * 8);
    }
  };
  const int y16_off = 16 * (grp & 1) + 8 * (grp >> 1);
  struct QState {
    bf16x8 qf[2];
    int tokq;
  };
  auto load_q = [&](QState& qs, const int* tok, int h) {
    qs.tokq = tok[wave * 16 + r16];
    const __bf16* qrow = q + int64_t(qs.tokq) * rowstride + int64_t(h) * DH;
    qs.qf[0] = Frag<__bf16>::load(qrow, lane);
    qs.qf[1] = Frag<__bf16>::load(qrow + 32, lane);
  };
  // Per-lane LDS offsets (elements) in a slot, for head e: K fragments of
  // key rows r16 (+16 per tile), V transposing reads of rows 4 grp + r16/4.
  auto k_off = [&](int e, int col) { return (2 * r16 + e) * DH + ((((col >> 3) ^ (r16 & 7)) << 3) | (col & 7)); };
  int offk[2][2], offv[2][4];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    offk[e][0] = k_off(e, grp * 8);
    offk[e][1] = k_off(e, 32 + grp * 8);
#pragma unroll
    for (int et = 0; et < 4; ++et) {
      const int row = 4 * grp + (r16 >> 2), col = et * 16 + 4 * (r16 & 3);
      offv[e][et] = (2 * row + e) * DH + ((((col >> 3) ^ (row & 7)) << 3) | (col & 7));
    }
  }
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = static_cast<__bf16>(1.f);

  if (it_begin >= it_end) return;
  ItemPos pos = decompose(it_begin);
  item_tokens(pos, sTok[0], sCls[0]);
  lds_barrier();
  QState nxt;
  issue_half(sK0, sV0, sTok[0], pos.hp, 0);
  load_q(nxt, sTok[0], 2 * pos.hp);
  issue_half(sK1, sV1, sTok[0], pos.hp, 1);
  wait_vmem();

  // One head of the pair over both halves, its output stored at the end;
  // after_half0 runs between the halves.  (SAVE_LSE: head h0's statistic
  // waits in lse0 and leaves with head h1's as one 8-byte store.)
  float lse0 = 0.f;
  auto head = [&](const QState& cur, int h, int e, const int* cls, bool wrapped, auto&& after_half0) {
    // The MA output this head adds to arrives while the products run.
    bf16x8 ya[2];
    if constexpr (ACCUMULATE) {
      const __bf16* yrow = y + int64_t(cur.tokq) * rowstride + int64_t(h) * DH + y16_off;
      ya[0] = *reinterpret_cast<const bf16x8*>(yrow);
      ya[1] = *reinterpret_cast<const bf16x8*>(yrow + 32);
    }
    const int qcls = cls[wave * 16 + r16];
    f32x4 o[4], den = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY;
#pragma unroll
    for (int et = 0; et < 4; ++et) o[et] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      if (hf == 1) after_half0();
      const __bf16* cK = hf ? sK1 : sK0;
      lds_bf16* vb = (lds_bf16*)(hf ? sV1 : sV0);
      f32x4 s[KT16];
#pragma unroll
      for (int kt = 0; kt < KT16; ++kt) {
        const int rb = kt * 16 * 2 * DH;
        const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(cK + offk[e][0] + rb);
        const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(cK + offk[e][1] + rb);
        s[kt] = mma(k1, cur.qf[1], mma(k0, cur.qf[0], f32x4{0.f, 0.f, 0.f, 0.f}));
      }
      if (wrapped) {
#pragma unroll
        for (int kt = 0; kt < KT16; ++kt) {
          const int4 kc = *reinterpret_cast<const int4*>(&cls[hf * HALF + kt * 16 + grp * 4]);
          s[kt][0] = kc.x != qcls ? -INFINITY : s[kt][0];
          s[kt][1] = kc.y != qcls ? -INFINITY : s[kt][1];
          s[kt][2] = kc.z != qcls ? -INFINITY : s[kt][2];
          s[kt][3] = kc.w != qcls ? -INFINITY : s[kt][3];
        }
      }
      float mx = fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3]));
#pragma unroll
      for (int kt = 1; kt < KT16; ++kt) mx = fmaxf(fmaxf(mx, fmaxf(s[kt][0], s[kt][1])), fmaxf(s[kt][2], s[kt][3]));
      const float mnew = fmaxf(m, max_rows(mx) * sc);
      // all keys of the first half masked (a cut window): zero weights until
      // the query's own key, which is always present
      const float mref = mnew == -INFINITY ? 0.f : mnew;
      if (hf) {
        const float alpha = fast_exp2(m - mref);
#pragma unroll
        for (int r = 0; r < 4; ++r) den[r] *= alpha;
#pragma unroll
        for (int et = 0; et < 4; ++et)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[et][r] *= alpha;
      }
      m = mnew;
#pragma unroll
      for (int sb = 0; sb < HALF / 32; ++sb) {
        const int rb = 32 * sb * 2 * DH;
        bf16x8 pb;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pb[r] = static_cast<__bf16>(fast_exp2(fmaf(s[2 * sb][r], sc, -mref)));
          pb[4 + r] = static_cast<__bf16>(fast_exp2(fmaf(s[2 * sb + 1][r], sc, -mref)));
        }
        den = mma(ones, pb, den);
#pragma unroll
        for (int et = 0; et < 4; ++et) {
          const bf16x4 lo = lds_read_tr(vb + offv[e][et] + rb);
          const bf16x4 hi = lds_read_tr(vb + offv[e][et] + rb + 16 * 2 * DH);
          o[et] = mma(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pb, o[et]);
        }
      }
    }
    const float inv = __builtin_amdgcn_rcpf(den[0]);
    if constexpr (SAVE_LSE) {
      // the query's own key is never masked, so m is finite here
      const float lv = m + log2f(den[0]);
      if (e == 0) lse0 = lv;
      else if (grp == 0) *reinterpret_cast<float2*>(lse + int64_t(cur.tokq) * Ha + h - 1) = make_float2(lse0, lv);
    }
#pragma unroll
    for (int r1 = 0; r1 < 2; ++r1) {
      float ov[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(o[2 * r1][r]), __float_as_uint(o[2 * r1 + 1][r]),
                                                         false, false);
        ov[r] = __uint_as_float(sw[0]);
        ov[4 + r] = __uint_as_float(sw[1]);
      }
      bf16x8 res;
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) {
        const float val = ov[e8] * inv;
        res[e8] = static_cast<__bf16>(ACCUMULATE ? static_cast<float>(ya[r1][e8]) + val : val);
      }
      __bf16* yrow = y + int64_t(cur.tokq) * rowstride + int64_t(h) * DH + y16_off;
      *reinterpret_cast<bf16x8*>(yrow + 32 * r1) = res;
    }
  };

#pragma unroll 1
  for (int n = 0;; ++n) {
    const int h0 = 2 * pos.hp;
    ItemPos npos = pos;
    npos.item += it_step;
    const bool has_next = npos.item < it_end;
    if (has_next) {
      npos = decompose(npos.item);
      item_tokens(npos, sTok[(n + 1) & 1], sCls[(n + 1) % 3]);
    }
    // This pair's half 0 (issued after the previous pair's h1 half 0) has
    // landed once at most the operations issued after it are pending: the
    // next q (2 loads), h1's output stores (2) and half 1 (2 DMA per lane).
    if (n == 0) wait_vmem();
    else __builtin_amdgcn_s_waitcnt(vmcnt_count(2 + 2 + 2 * DMA));
    lds_barrier();
    const QState cur0 = nxt;
    // (empty asm with a memory clobber: the counted groups of vector-memory
    // operations stay in program order)
    asm volatile("" ::: "memory");
    load_q(nxt, sTok[n & 1], h0 + 1);
    asm volatile("" ::: "memory");
    const bool wrapped = wg.masked && window_wrapped(wg, pos.wi, pos.wj, pos.wk);
    const int* cls = sCls[n % 3];
    // head h0; before its half 1, this pair's half 1 must have landed: the
    // operations after it are this head's MA-output loads (2) and the next
    // q loads (2).
    head(cur0, h0, 0, cls, wrapped, [&] {
      if (n > 0) {
        __builtin_amdgcn_s_waitcnt(vmcnt_count((ACCUMULATE ? 2 : 0) + 2));
        lds_barrier();
      }
    });
    const QState cur1 = nxt;
    head(cur1, h0 + 1, 1, cls, wrapped, [&] {
      // every wave is done with slot 0: refill it with the next pair's half 0
      lds_barrier();
      if (has_next) {
        asm volatile("" ::: "memory");
        issue_half(sK0, sV0, sTok[(n + 1) & 1], npos.hp, 0);
        asm volatile("" ::: "memory");
        load_q(nxt, sTok[(n + 1) & 1], 2 * npos.hp);
        asm volatile("" ::: "memory");
      }
    });
    if (!has_next) break;
    lds_barrier();   // every wave is done with slot 1
    asm volatile("" ::: "memory");
    issue_half(sK1, sV1, sTok[(n + 1) & 1], npos.hp, 1);
    asm volatile("" ::: "memory");
    pos = npos;
  }
}

}  // namespace

// The TE branch for the (bf16, d 64, 256-token window) family, one batch
// element after another; persistent grid of one workgroup per compute unit.
int launch_te_win256(const lingen_mate_shape* s, const int shift[3], int masked, const void* q, const void* k,
                     const void* v, void* y, int accumulate, hipStream_t st, float* lse) {
  const WinGeom g = make_wingeom(s, shift, masked);
  const int64_t L = tokens(s);
  const int nwin = g.nwt * g.nwh * g.nww;
  const int64_t per = L * s->attn_heads * 64 * 2;
  const int ncu = compute_units();
  if (ncu < 1) return LINGEN_ERR_HIP;
  for (int b = 0; b < s->batch; ++b) {
    const int64_t off = int64_t(b) * per;
    const __bf16* qb = reinterpret_cast<const __bf16*>(static_cast<const char*>(q) + off);
    const __bf16* kb = reinterpret_cast<const __bf16*>(static_cast<const char*>(k) + off);
    const __bf16* vb = reinterpret_cast<const __bf16*>(static_cast<const char*>(v) + off);
    __bf16* yb = reinterpret_cast<__bf16*>(static_cast<char*>(y) + off);
    const int items = nwin * s->attn_heads;
    if (lse != nullptr && s->attn_heads % 2) return LINGEN_ERR_UNSUPPORTED;
    if (s->attn_heads % 2 == 0) {
      // two heads per item; the item order as below, judged by head-items
      const int pairs = nwin * (s->attn_heads / 2);
      const int pgrid = pairs < ncu ? pairs : ncu;
      const int pcontig = items >= 128 * pgrid ? 1 : 0;
      if (lse != nullptr)
        tesa_win256_pair_kernel<false, true><<<pgrid, kW256Waves * 64, 0, st>>>(
            qb, kb, vb, g, s->attn_heads, pairs, pcontig, yb, lse + int64_t(b) * L * s->attn_heads);
      else if (accumulate)
        tesa_win256_pair_kernel<true><<<pgrid, kW256Waves * 64, 0, st>>>(qb, kb, vb, g, s->attn_heads, pairs, pcontig,
                                                                        yb);
      else
        tesa_win256_pair_kernel<false><<<pgrid, kW256Waves * 64, 0, st>>>(qb, kb, vb, g, s->attn_heads, pairs, pcontig,
                                                                         yb);
      if (launch_status(__func__) != LINGEN_OK) return LINGEN_ERR_HIP;
      continue;
    }
    const int grid = items < ncu ? items : ncu;
    // Item order: a contiguous range per workgroup (the heads of a window
    // one after another) once a workgroup has at least 128 items; measured
    // at 256 and 144 items per workgroup (the minute-length and 768p-like
    // workloads: 2.43 against 2.71 ms and 1.30 against 1.46 ms), while at 64
    // (the 512p-like workload) the strided order is 2% faster.
    const int contiguous = items >= 128 * grid ? 1 : 0;
    if (accumulate)
      tesa_win256_kernel<true><<<grid, kW256Waves * 64, 0, st>>>(qb, kb, vb, g, s->attn_heads, items, contiguous,
                                                                 yb);
    else
      tesa_win256_kernel<false><<<grid, kW256Waves * 64, 0, st>>>(qb, kb, vb, g, s->attn_heads, items, contiguous,
                                                                  yb);
    if (launch_status(__func__) != LINGEN_OK) return LINGEN_ERR_HIP;
  }
  return LINGEN_OK;
}

}  // namespace lingen

using namespace lingen;

extern "C" int lingen_te_fwd_saved(const void* q, const void* k, const void* v, int32_t shift_t, int32_t shift_h,
                                   int32_t shift_w, int32_t masked, const lingen_mate_shape* shape, void* y_te,
                                   float* lse, hipStream_t stream) {
  if (int rc = validate_shape(shape)) return rc;
  if (shift_t < 0 || shift_t >= shape->win_t || shift_h < 0 || shift_h >= shape->win_h || shift_w < 0 ||
      shift_w >= shape->win_w || (masked != 0 && masked != 1))
    return LINGEN_ERR_SHAPE;
  for (const void* p : {q, k, v, static_cast<const void*>(y_te), static_cast<const void*>(lse)})
    if (int rc = check_ptr(p)) return rc;
  if (attn_family(shape) != ATTN_BF16_D64_W256 || shape->attn_heads % 2) return LINGEN_ERR_UNSUPPORTED;
  const int shift[3] = {shift_t, shift_h, shift_w};
  return launch_te_win256(shape, shift, masked, q, k, v, y_te, 0, stream, lse);
}
