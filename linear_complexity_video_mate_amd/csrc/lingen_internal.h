// Internal declarations shared by the host validation code and the kernel
// launchers of the MATE mixer library.  Not part of the public ABI.
#pragma once

#include <cstddef>
#include <cstdint>

#include "lingen_mate.h"

namespace lingen {

// Byte offsets of the sub-buffers inside the caller's workspace, for one
// batch element (batch elements are processed one after another and reuse
// the same workspace).
struct WsLayout {
  size_t states;   // [2][n_chunks][Hs][P][N] in the input dtype: chunk states, then scan states
  size_t decay;    // fp32 [n_chunks][Hs]: exp of the sum of dt*A over each chunk
  size_t review_h; // fp32 [Hs][P][N]: state left by the review tokens
  size_t review_x; // fp32 [R][Hs][P]: pooled review x
  size_t review_dt;// fp32 [R][Hs]
  size_t review_b; // fp32 [R][G][N]
  size_t total;
};

// Which compiled kernel families a shape uses.
enum ScanFamily { SCAN_F32_P32_N16_Q16 = 0, SCAN_BF16_P64_N64_Q64 = 1, SCAN_BF16_P64_N128_Q128 = 2, SCAN_NONE = -1 };
enum AttnFamily { ATTN_F32_D32_W32 = 0, ATTN_BF16_D64_W256 = 1, ATTN_BF16_D64_W27 = 2, ATTN_NONE = -1 };

int validate_shape(const lingen_mate_shape* s);   // lingen_status
int64_t tokens(const lingen_mate_shape* s);       // T*H*W
WsLayout ws_layout(const lingen_mate_shape* s);
ScanFamily scan_family(const lingen_mate_shape* s);
AttnFamily attn_family(const lingen_mate_shape* s);
int check_ptr(const void* p);                      // NULL / alignment check
// After a kernel launch: LINGEN_OK, or LINGEN_ERR_HIP if the launch failed.
// With the environment variable LINGEN_DEBUG set (not "0"), it also waits for
// the device and reports any error on stderr naming `where`: a sync-and-check
// mode for debugging (not for use under graph capture).
int launch_status(const char* where);
bool debug_sync();
int compute_units();                               // of the current device (cached per device), -1 on error
// How a token's input enters the chunked scan's states, with a = dt A its
// log decay:
//   kWeightDt       the SSD recurrence: token s contributes dt_s x_s (with B_s);
//   kWeightAdjoint  token s contributes e^{a_s} x_s, the recurrence of the
//                   input x e^{a} / dt (the adjoint states of the backward
//                   pass) without forming that input.
enum WeightMode { kWeightDt = 0, kWeightAdjoint = 2 };

// Chunk states and scan states of one batch element (x, dt, B of that
// element) into the workspace, at ws_layout(s).states in the storage dtype:
// [2][n_chunks][Hs][P][N], the state entering each chunk of the forward scan
// and then of the reverse scan.  With s->n_review > 0 the review tokens of
// (x, dt, B) are pooled and scanned first (into the workspace's review
// buffers) and their state starts both walks; pass a shape with n_review = 0
// for a scan without them.  wmode: kWeightDt or kWeightAdjoint.  h_last
// (optional, fp32 [2][Hs][P][N]): the state each walk carries out of its
// last chunk (the upward walk's first, then the downward walk's).
// lingen_status.
int scan_states_one(const lingen_mate_shape* s, int mode, const void* xb, const float* dtb, const float* A,
                    const void* Bb, void* workspace, hipStream_t stream, int wmode, float* h_last);
// The transposed bidirectional scan of one batch element, y = (M_f^T +
// M_b^T) u / dt, with M_f, M_b the matrices of the two directions of the
// shared-parameter SSD scan with dt, A, B, C (y_MA = (M_f + M_b) x + 2 D x;
// the division removes M's dt factor, so no dt enters y): the chunk states
// must be those that
// scan_states_one(s, mode, u, dt, A, C, workspace, ..., kWeightAdjoint) left
// in `workspace`.  bf16 families only; no review tokens.  Shapes and
// pointers are the caller's to validate.  lingen_status.
int ma_transposed_one(const lingen_mate_shape* s, int mode, const void* ub, const float* dtb, const float* A,
                      const void* Bb, const void* Cb, const void* workspace, void* yb, hipStream_t stream);

// The TE branch for the (bf16, d = 64, 256-token window) family
// (tesa_window.hip): y = o (accumulate = 0) or y += o (accumulate = 1), one
// batch element after another; lse (with accumulate = 0 and an even head
// count only): also each query's log2-sum-exp of its scaled scores,
// [batch, L, Ha] fp32.  Shapes and pointers are the caller's to validate.
// lingen_status.
int launch_te_win256(const lingen_mate_shape* s, const int shift[3], int masked, const void* q, const void* k,
                     const void* v, void* y, int accumulate, hipStream_t st, float* lse = nullptr);

}  // namespace lingen
