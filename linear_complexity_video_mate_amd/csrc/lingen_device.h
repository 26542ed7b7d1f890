// Device helpers shared by the HIP kernels of the library (gfx950 / CDNA4):
// vector types, the MFMA 16x16 tiles and their operand fragments, the
// swizzled 128-byte-row LDS tile with its transposing read, direct
// global-to-LDS loads, the LDS-only workgroup barrier and cross-lane
// reductions and scans.
#pragma once

#include <hip/hip_runtime.h>

namespace lingen {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// 2^x with the hardware instruction alone (no range reduction wrapper):
// exp2(-inf) = 0, and results below the normal range come out as zero or
// denormal, which is far below every tolerance the callers work to.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// v * sigmoid(v) with the hardware exp and reciprocal (about 1 ulp each): the
// activation after the scan-order convolution of the MA branch.  The
// standalone convolution and the one fused into the scan kernels share it, so
// the two paths round alike.
__device__ __forceinline__ float silu(float v) { return v * __builtin_amdgcn_rcpf(1.f + __expf(-v)); }

// softplus(a) = log(1 + e^a), written so that neither term overflows.
__device__ __forceinline__ float softplus(float a) { return fmaxf(a, 0.f) + log1pf(expf(-fabsf(a))); }

// Workgroup barrier for LDS traffic only.  The waves of a workgroup exchange
// data through LDS alone (never through global memory), so the barrier waits
// for this wave's LDS accesses but leaves its global loads and stores in
// flight: prefetches issued before a barrier keep streaming across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Cross-lane sums, maxima and scans without LDS traffic (every lane of the
// wave active).  DPP quad permutations swap neighbours and pairs inside each
// quad, the half-row mirror pairs the two quads of an 8-lane half-row and
// the row mirror the two halves of a 16-lane row; v_permlane16_swap and
// v_permlane32_swap exchange whole rows (lane l with l ^ 16, l ^ 32).
template <int CTRL>
__device__ __forceinline__ float dpp_plus(float v) {
  return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
// sum over each aligned group of 8 lanes, in every lane of the group
__device__ __forceinline__ float sum8(float v) {
  v = dpp_plus<0xB1>(v);       // quad_perm [1,0,3,2]
  v = dpp_plus<0x4E>(v);       // quad_perm [2,3,0,1]
  return dpp_plus<0x141>(v);   // row_half_mirror
}
// sum over each 16-lane row, in every lane of the row
__device__ __forceinline__ float sum16(float v) { return dpp_plus<0x140>(sum8(v)); /* row_mirror */ }
// sum and maximum over the four rows (lanes l, l ^ 16, l ^ 32, l ^ 48)
__device__ __forceinline__ float sum_rows(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float max_rows(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum64(float v) { return sum_rows(sum16(v)); }

// v + the value of the lane the DPP control names (0 where it names none,
// and in rows the row mask leaves out).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_shifted_plus(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}
// Inclusive prefix sum over the 64 lanes of the wave: row shifts by 1, 2, 4,
// 8 scan each 16-lane row, then the last lane of rows 0 and 2 is broadcast
// into the next row and the last lane of row 1 into rows 2 and 3.
__device__ __forceinline__ float wave_scan_incl(float v) {
  v = dpp_shifted_plus<0x111, 0xF>(v);   // row_shr:1
  v = dpp_shifted_plus<0x112, 0xF>(v);   // row_shr:2
  v = dpp_shifted_plus<0x114, 0xF>(v);   // row_shr:4
  v = dpp_shifted_plus<0x118, 0xF>(v);   // row_shr:8
  v = dpp_shifted_plus<0x142, 0xA>(v);   // row_bcast:15 into rows 1, 3
  return dpp_shifted_plus<0x143, 0xC>(v);   // row_bcast:31 into rows 2, 3
}

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(__bf16 v) { return static_cast<float>(v); }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float v) { return static_cast<__bf16>(v); }

// MFMA 16x16 tiles.  Output layout (both variants): lane l holds
// D[4*(l/16) + r][l%16] in element r.  Operand layout: lane l supplies row
// l%16 of A and column l%16 of B, for the k values of its lane group l/16.
__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Operand fragment of one MFMA from a k-contiguous row: 8 bf16 (k = 8*g ..
// 8*g+7) or one float (k = g), g = lane/16.
template <typename MT> struct Frag;
template <> struct Frag<__bf16> {
  using type = bf16x8;
  static constexpr int K = 32;
  __device__ static type load(const __bf16* row, int lane) {
    return *reinterpret_cast<const bf16x8*>(row + (lane >> 4) * 8);
  }
};
template <> struct Frag<float> {
  using type = float;
  static constexpr int K = 4;
  __device__ static type load(const float* row, int lane) { return row[lane >> 4]; }
};

// Row-major LDS tile of 128-byte rows (ROWLEN elements) with the 16-byte
// chunks of row r permuted as chunk ^ (r mod 8): row-contiguous 16-byte
// stores, 16-byte row reads and the transposing reads below all touch
// distinct banks.  Direct global-to-LDS loads fill it 64 chunks (8 rows) per
// instruction, each lane fetching the source chunk that lands in its slot.
template <typename TS, int ROWLEN>
struct KvTile {
  static constexpr int VEC = 16 / int(sizeof(TS));
  static_assert(ROWLEN / VEC == 8, "rows of eight 16-byte chunks");
  __device__ static __forceinline__ int at(int row, int col) {
    return row * ROWLEN + ((((col / VEC) ^ (row & 7)) * VEC) | (col % VEC));
  }
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) const __bf16 lds_bf16;
// Transposing LDS load (16-bit elements): within each group of 16 lanes,
// lane i receives element (i mod 4) of the 8-byte chunk read by lane
// 4r + i/4, in slot r.  Takes an LDS-space pointer so that constant parts
// of the address fold into the instruction's offset field.
__device__ __forceinline__ bf16x4 lds_read_tr(lds_bf16* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// 16-byte direct global-to-LDS load: lane l's chunk lands at lds_wave_base +
// 16*l (the base must be the same for all lanes of the wave).  Kept out of
// the kernel templates, whose host-side stubs are not emitted otherwise.
__device__ __forceinline__ void lds_load16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, lds_wave_base, 16, 0, 0);
}

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0f70); }   // vmcnt(0)

}  // namespace lingen
