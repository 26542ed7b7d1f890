// Host-side part of the MATE mixer library: argument validation, workspace
// planning, the host copy of the Rotary Major Scan index maps and the check
// after each kernel launch.  Nothing in this file launches a kernel, and the
// validation and planning functions touch no GPU, so they can be exercised
// without one.
#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "lingen_internal.h"

namespace lingen {

namespace {
constexpr int64_t kMaxTokens = (int64_t(1) << 31) - 1;
size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }
}  // namespace

int64_t tokens(const lingen_mate_shape* s) {
  return int64_t(s->T) * int64_t(s->H) * int64_t(s->W);
}

ScanFamily scan_family(const lingen_mate_shape* s) {
  if (s->dtype == LINGEN_F32 && s->headdim == 32 && s->d_state == 16 && s->chunk == 16)
    return SCAN_F32_P32_N16_Q16;
  if (s->dtype == LINGEN_BF16 && s->headdim == 64 && s->d_state == 64 && s->chunk == 64)
    return SCAN_BF16_P64_N64_Q64;
  if (s->dtype == LINGEN_BF16 && s->headdim == 64 && s->d_state == 128 && s->chunk == 128)
    return SCAN_BF16_P64_N128_Q128;
  return SCAN_NONE;
}

AttnFamily attn_family(const lingen_mate_shape* s) {
  const int64_t nw = int64_t(s->win_t) * s->win_h * s->win_w;
  if (s->dtype == LINGEN_F32 && s->attn_headdim == 32 && nw == 32) return ATTN_F32_D32_W32;
  if (s->dtype == LINGEN_BF16 && s->attn_headdim == 64 && nw == 256) return ATTN_BF16_D64_W256;
  if (s->dtype == LINGEN_BF16 && s->attn_headdim == 64 && nw == 27) return ATTN_BF16_D64_W27;
  return ATTN_NONE;
}

// Compute units of the current device, cached per device (the only state
// the library keeps; concurrent first calls store the same value).
int compute_units() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// LINGEN_DEBUG set to anything but "" or "0": after every kernel launch the
// library waits for the device and checks for errors, and reports a failure
// with the launching function's name on stderr.  Read once per process.
bool debug_sync() {
  static const bool on = [] {
    const char* v = std::getenv("LINGEN_DEBUG");
    return v != nullptr && v[0] != '\0' && std::strcmp(v, "0") != 0;
  }();
  return on;
}

int launch_status(const char* where) {
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && debug_sync()) e = hipDeviceSynchronize();
  if (e == hipSuccess) return LINGEN_OK;
  if (debug_sync()) std::fprintf(stderr, "lingen: kernel launched by %s failed: %s\n", where, hipGetErrorString(e));
  return LINGEN_ERR_HIP;
}

int check_ptr(const void* p) {
  if (p == nullptr) return LINGEN_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return LINGEN_ERR_ALIGN;
  return LINGEN_OK;
}

int validate_shape(const lingen_mate_shape* s) {
  if (s == nullptr) return LINGEN_ERR_NULL;
  if (s->dtype != LINGEN_F32 && s->dtype != LINGEN_BF16) return LINGEN_ERR_DTYPE;
  if (s->batch < 1 || s->T < 1 || s->H < 1 || s->W < 1) return LINGEN_ERR_SHAPE;
  const int64_t L = tokens(s);
  if (L > kMaxTokens) return LINGEN_ERR_SHAPE;
  if (s->ssd_heads < 1 || s->headdim < 1 || s->d_state < 1 || s->chunk < 1) return LINGEN_ERR_SHAPE;
  if (s->ngroups < 1 || s->ssd_heads % s->ngroups) return LINGEN_ERR_SHAPE;
  if (L % s->chunk != 0) return LINGEN_ERR_SHAPE;
  if (s->attn_heads < 1 || s->attn_headdim < 1) return LINGEN_ERR_SHAPE;
  if (int64_t(s->attn_heads) * s->attn_headdim != int64_t(s->ssd_heads) * s->headdim) return LINGEN_ERR_SHAPE;
  if (s->win_t < 1 || s->win_h < 1 || s->win_w < 1) return LINGEN_ERR_SHAPE;
  if (s->T % s->win_t || s->H % s->win_h || s->W % s->win_w) return LINGEN_ERR_SHAPE;
  // Every byte offset is formed in 64 bits; the per-batch row counts must
  // still fit the int32 token indices used on the device.
  if (int64_t(s->batch) * L > (int64_t(1) << 40)) return LINGEN_ERR_SHAPE;
  if (s->n_review < 0) return LINGEN_ERR_SHAPE;
  if (s->n_review > 0) {
    if (s->rpool_t < 1 || s->rpool_h < 1 || s->rpool_w < 1) return LINGEN_ERR_SHAPE;
    if (s->rgrid_t < 1 || s->rgrid_h < 1 || s->rgrid_w < 1) return LINGEN_ERR_SHAPE;
    if (s->T % s->rpool_t || s->H % s->rpool_h || s->W % s->rpool_w) return LINGEN_ERR_SHAPE;
    const int gt = s->T / s->rpool_t, gh = s->H / s->rpool_h, gw = s->W / s->rpool_w;
    if (gt % s->rgrid_t || gh % s->rgrid_h || gw % s->rgrid_w) return LINGEN_ERR_SHAPE;
    if (int64_t(s->rgrid_t) * s->rgrid_h * s->rgrid_w != s->n_review) return LINGEN_ERR_SHAPE;
    if (s->n_review > 256) return LINGEN_ERR_SHAPE;   // one workgroup holds all review weights
  }
  if (scan_family(s) == SCAN_NONE) return LINGEN_ERR_UNSUPPORTED;
  if (attn_family(s) == ATTN_NONE) return LINGEN_ERR_UNSUPPORTED;
  if (s->headdim != s->attn_headdim) return LINGEN_ERR_UNSUPPORTED;
  return LINGEN_OK;
}

WsLayout ws_layout(const lingen_mate_shape* s) {
  WsLayout w{};
  const size_t L = size_t(tokens(s));
  const size_t nc = L / size_t(s->chunk);
  const size_t hs = size_t(s->ssd_heads), P = size_t(s->headdim), N = size_t(s->d_state);
  const size_t R = size_t(s->n_review);
  size_t off = 0;
  w.states = off;
  // chunk states are kept in the element type of the inputs (fp32 or bf16)
  const size_t se = s->dtype == LINGEN_BF16 ? 2 : 4;
  off = align_up(off + 2 * nc * hs * P * N * se);
  w.decay = off;
  off = align_up(off + nc * hs * sizeof(float));
  w.review_h = off;
  off = align_up(off + (R ? hs * P * N * sizeof(float) : 0));
  w.review_x = off;
  off = align_up(off + R * hs * P * sizeof(float));
  w.review_dt = off;
  off = align_up(off + R * hs * sizeof(float));
  w.review_b = off;
  off = align_up(off + R * size_t(s->ngroups) * N * sizeof(float));
  w.total = off;
  return w;
}

}  // namespace lingen

extern "C" {

const char* lingen_status_str(int status) {
  switch (status) {
    case LINGEN_OK: return "ok";
    case LINGEN_ERR_NULL: return "null pointer";
    case LINGEN_ERR_SHAPE: return "invalid shape";
    case LINGEN_ERR_DTYPE: return "invalid dtype";
    case LINGEN_ERR_ALIGN: return "pointer not 16-byte aligned";
    case LINGEN_ERR_WORKSPACE: return "workspace too small";
    case LINGEN_ERR_HIP: return "HIP error";
    case LINGEN_ERR_UNSUPPORTED: return "no compiled kernel for this shape";
    case LINGEN_ERR_SCRATCH: return "shape needs more workspace than the no-allocation scratch array holds";
    default: return "unknown status";
  }
}

int lingen_mate_validate(const lingen_mate_shape* shape) { return lingen::validate_shape(shape); }

int lingen_mate_workspace_bytes(const lingen_mate_shape* shape, size_t* bytes) {
  if (bytes == nullptr) return LINGEN_ERR_NULL;
  const int st = lingen::validate_shape(shape);
  if (st != LINGEN_OK) return st;
  *bytes = lingen::ws_layout(shape).total;
  return LINGEN_OK;
}

int lingen_rms_index(int32_t mode, int32_t T, int32_t H, int32_t W, int32_t* perm_host, int32_t* inv_host) {
  if (mode < 0 || mode > 3) return LINGEN_ERR_SHAPE;
  if (T < 1 || H < 1 || W < 1) return LINGEN_ERR_SHAPE;
  const int64_t L = int64_t(T) * H * W;
  if (L > (int64_t(1) << 31) - 1) return LINGEN_ERR_SHAPE;
  // Walk the grid in scan order with three nested counters; the innermost
  // counter is the axis with the first unfolding priority.
  int64_t s = 0;
  auto emit = [&](int64_t t, int64_t h, int64_t w) {
    const int64_t c = (t * H + h) * W + w;
    if (perm_host) perm_host[s] = int32_t(c);
    if (inv_host) inv_host[c] = int32_t(s);
    ++s;
  };
  switch (mode) {
    case 0: for (int64_t t = 0; t < T; ++t) for (int64_t h = 0; h < H; ++h) for (int64_t w = 0; w < W; ++w) emit(t, h, w); break;
    case 1: for (int64_t t = 0; t < T; ++t) for (int64_t w = 0; w < W; ++w) for (int64_t h = 0; h < H; ++h) emit(t, h, w); break;
    case 2: for (int64_t h = 0; h < H; ++h) for (int64_t w = 0; w < W; ++w) for (int64_t t = 0; t < T; ++t) emit(t, h, w); break;
    default: for (int64_t w = 0; w < W; ++w) for (int64_t h = 0; h < H; ++h) for (int64_t t = 0; t < T; ++t) emit(t, h, w); break;
  }
  return LINGEN_OK;
}

}  // extern "C"
