// The whole MATE block around the mixer: the projections into and out of
// both branches (plain GEMMs, left to rocBLAS) with the library's own kernels
// between them.  Page "视频生成模子太贵太慢如何办？", section 要领：线性复杂度的
// MATE 模块: the block is an MA branch (a bidirectional Mamba2 block over the
// Rotary Major Scan) plus a TE branch (TEmporal Swin Attention).  Inside the
// MA branch the Mamba-2 block layout is followed ("Transformers are SSMs",
// Dao & Gu 2024, section 7): z, xBC and dt from the input projection; the
// scan-order convolution with SiLU and the dt softplus; the scan; the
// SiLU(z)-gated RMS norm; the output projection.  The TE branch projects q, k,
// v, attends inside the (shifted) windows and projects the result.  The two
// branch outputs are summed.

#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <cstdint>
#include <mutex>

#include "lingen_internal.h"

namespace lingen {
namespace {

constexpr int kMaxDevices = 64;
constexpr size_t kAlign = 256;

size_t align_up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

// Byte offsets of the block's buffers inside the caller's workspace.  Rows
// are batch*L tokens; "e" is the element size of the shape's dtype.
struct BlockWs {
  size_t z;        // [rows, Hs*P] e; reused for the attention output o
  size_t xbc;      // [rows, Hs*P + 2GN] e; reused for the normed scan output
  size_t dt_raw;   // [rows, Hs] fp32
  size_t xf, bf, cf, xb, bb, cb;   // convolved x, B, C per direction, e
  size_t dt;       // [rows, Hs] fp32
  size_t y;        // [rows, Hs*P] e: scan output
  size_t q, k, v;  // [rows, Ha*d] e
  size_t scan;     // the scan's workspace
  size_t total;
};

BlockWs block_layout(const lingen_mate_shape* s) {
  const size_t rows = size_t(s->batch) * size_t(tokens(s));
  const size_t e = s->dtype == LINGEN_BF16 ? 2 : 4;
  const size_t d = size_t(s->ssd_heads) * s->headdim, gn = size_t(s->ngroups) * s->d_state;
  const size_t da = size_t(s->attn_heads) * s->attn_headdim, hs = size_t(s->ssd_heads);
  BlockWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += align_up(bytes); return o; };
  w.z = take(rows * d * e);
  w.xbc = take(rows * (d + 2 * gn) * e);
  w.dt_raw = take(rows * hs * 4);
  w.xf = take(rows * d * e);
  w.bf = take(rows * gn * e);
  w.cf = take(rows * gn * e);
  w.xb = take(rows * d * e);
  w.bb = take(rows * gn * e);
  w.cb = take(rows * gn * e);
  w.dt = take(rows * hs * 4);
  w.y = take(rows * d * e);
  w.q = take(rows * da * e);
  w.k = take(rows * da * e);
  w.v = take(rows * da * e);
  size_t scan_bytes = 0;
  lingen_mate_workspace_bytes(s, &scan_bytes);
  w.scan = take(scan_bytes);
  w.total = off;
  return w;
}

// One rocBLAS handle per device, created on first use; the lock also
// serialises the handle's stream switch and the GEMM it precedes.
struct BlasState {
  std::mutex lock;
  rocblas_handle handle[kMaxDevices] = {};
};
BlasState& blas() {
  static BlasState s;
  return s;
}

// C[M, N] = A[M, K] * W[N, K]^T (+ beta * C), row-major; A and W in `in_t`,
// C in `out_t`, fp32 accumulation.  In rocBLAS's column-major terms this is
// C^T = W * A^T: op(W) transposed with ld K, A untransposed with ld K.
int gemm_rows(hipStream_t st, rocblas_datatype in_t, rocblas_datatype out_t, int64_t M, int N, int K, const void* A,
              const void* W, void* C, float beta) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LINGEN_ERR_HIP;
  BlasState& b = blas();
  std::lock_guard<std::mutex> g(b.lock);
  if (b.handle[dev] == nullptr && rocblas_create_handle(&b.handle[dev]) != rocblas_status_success) {
    b.handle[dev] = nullptr;
    return LINGEN_ERR_HIP;
  }
  rocblas_handle h = b.handle[dev];
  if (rocblas_set_stream(h, st) != rocblas_status_success) return LINGEN_ERR_HIP;
  const float alpha = 1.f;
  const rocblas_status rs =
      rocblas_gemm_ex(h, rocblas_operation_transpose, rocblas_operation_none, N, rocblas_int(M), K, &alpha, W, in_t,
                      K, A, in_t, K, &beta, C, out_t, N, C, out_t, N, rocblas_datatype_f32_r,
                      rocblas_gemm_algo_standard, 0, 0);
  return rs == rocblas_status_success ? LINGEN_OK : LINGEN_ERR_HIP;
}

int check_weights(const lingen_mate_block_weights* w) {
  if (w == nullptr) return LINGEN_ERR_NULL;
  const void* ptrs[] = {w->w_z,     w->w_xbc,  w->w_dt,   w->conv_w_f, w->conv_b_f, w->conv_w_b, w->conv_b_b,
                        w->dt_bias, w->A_f,    w->D_f,    w->A_b,      w->D_b,      w->norm_w,   w->w_out_ma,
                        w->w_q,     w->w_k,    w->w_v,    w->w_o};
  for (const void* p : ptrs)
    if (int rc = check_ptr(p)) return rc;
  return LINGEN_OK;
}

int check_block_shape(const lingen_mate_shape* s, int32_t d_model) {
  if (int rc = validate_shape(s)) return rc;
  if (d_model < 1 || d_model > 65536) return LINGEN_ERR_SHAPE;
  if (int64_t(s->batch) * tokens(s) > int64_t(0x7fffffff)) return LINGEN_ERR_SHAPE;   // GEMM row count
  return LINGEN_OK;
}

}  // namespace
}  // namespace lingen

using namespace lingen;

extern "C" int lingen_mate_block_workspace_bytes(const lingen_mate_shape* shape, int32_t d_model, size_t* bytes) {
  if (bytes == nullptr) return LINGEN_ERR_NULL;
  if (int rc = check_block_shape(shape, d_model)) return rc;
  *bytes = block_layout(shape).total;
  return LINGEN_OK;
}

extern "C" int lingen_mate_block_fwd(const void* u, const lingen_mate_block_weights* w, int32_t d_model,
                                     int32_t conv_k, float norm_eps, int32_t layer_idx,
                                     const lingen_mate_shape* shape, void* out, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  if (int rc = check_block_shape(shape, d_model)) return rc;
  if (layer_idx < 0 || conv_k < 1 || conv_k > 4 || !(norm_eps >= 0.f)) return LINGEN_ERR_SHAPE;
  const int d = shape->ssd_heads * shape->headdim, gn = shape->ngroups * shape->d_state;
  const int ev = shape->dtype == LINGEN_BF16 ? 8 : 4;
  if (d % ev || gn % ev || (d / shape->ngroups) % ev || d > 1024 * ev) return LINGEN_ERR_SHAPE;
  if (int rc = check_weights(w)) return rc;
  for (const void* p : {u, static_cast<const void*>(out), static_cast<const void*>(workspace)})
    if (int rc = check_ptr(p)) return rc;
  const BlockWs L = block_layout(shape);
  if (workspace_bytes < L.total) return LINGEN_ERR_WORKSPACE;

  char* ws = static_cast<char*>(workspace);
  const int64_t rows = int64_t(shape->batch) * tokens(shape);
  const int hs = shape->ssd_heads, da = shape->attn_heads * shape->attn_headdim, ch = d + 2 * gn;
  const rocblas_datatype et = shape->dtype == LINGEN_BF16 ? rocblas_datatype_bf16_r : rocblas_datatype_f32_r;
  const int mode = layer_idx % 4, shifted = layer_idx % 2;
  int rc;

  // MA branch: z, xBC, dt_raw = u W^T
  if ((rc = gemm_rows(stream, et, et, rows, d, d_model, u, w->w_z, ws + L.z, 0.f))) return rc;
  if ((rc = gemm_rows(stream, et, et, rows, ch, d_model, u, w->w_xbc, ws + L.xbc, 0.f))) return rc;
  if ((rc = gemm_rows(stream, et, rocblas_datatype_f32_r, rows, hs, d_model, u, w->w_dt, ws + L.dt_raw, 0.f)))
    return rc;
  // The convolution, SiLU and softplus as a pass of their own, then the
  // per-direction scan.  (lingen_ma_fwd_dirs_conv takes the three steps
  // inside the scan kernels with identical results, but on this GPU it is
  // the slower form: the convolution is formed again by both scan kernels of
  // each direction, and their vector-ALU time outgrows the pass it saves.)
  const float* dt_raw = reinterpret_cast<const float*>(ws + L.dt_raw);
  float* dt = reinterpret_cast<float*>(ws + L.dt);
  if ((rc = lingen_ma_prep(ws + L.xbc, dt_raw, w->conv_w_f, w->conv_b_f, w->conv_w_b, w->conv_b_b, w->dt_bias,
                           conv_k, mode, shape, ws + L.xf, ws + L.bf, ws + L.cf, ws + L.xb, ws + L.bb, ws + L.cb, dt,
                           stream)))
    return rc;
  if ((rc = lingen_ma_fwd_dirs(ws + L.xf, dt, w->A_f, ws + L.bf, ws + L.cf, w->D_f, ws + L.xb, dt, w->A_b, ws + L.bb,
                               ws + L.cb, w->D_b, mode, shape, ws + L.y, ws + L.scan, L.total - L.scan, stream)))
    return rc;
  // gated norm into the xBC buffer (no longer needed), one group per B/C group
  if ((rc = lingen_gated_rmsnorm(ws + L.y, ws + L.z, w->norm_w, norm_eps, rows, d, d / shape->ngroups,
                                 shape->dtype, ws + L.xbc, stream)))
    return rc;
  if ((rc = gemm_rows(stream, et, et, rows, d_model, d, ws + L.xbc, w->w_out_ma, out, 0.f))) return rc;

  // TE branch: q, k, v = u W^T; windowed attention into the z buffer; out += o W_o^T
  if ((rc = gemm_rows(stream, et, et, rows, da, d_model, u, w->w_q, ws + L.q, 0.f))) return rc;
  if ((rc = gemm_rows(stream, et, et, rows, da, d_model, u, w->w_k, ws + L.k, 0.f))) return rc;
  if ((rc = gemm_rows(stream, et, et, rows, da, d_model, u, w->w_v, ws + L.v, 0.f))) return rc;
  if ((rc = lingen_te_fwd(ws + L.q, ws + L.k, ws + L.v, shifted, shape, ws + L.z, stream))) return rc;
  return gemm_rows(stream, et, et, rows, d_model, da, ws + L.z, w->w_o, out, 1.f);
}
