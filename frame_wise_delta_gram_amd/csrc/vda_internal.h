// Host-side plan and kernel launchers of the VDA library (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "vda.h"

namespace vda {

// Sizes derived from a validated descriptor, and the workspace carve-up.
// Workspace sections (fp32 but Sp, each 256-byte aligned):
//   A  [units][F + 1][d_k][d_k]   frame statistics, index 0 = text frame
//   B  [units][F + 1][d_v][d_k]
//   M  [units][F + 1][d_k][d_k]   transitions (I + A)^{-1}
//   Mc [units][n][d_k][d_k]       chunk transitions (forward order)
//   McT [units][n][d_k][d_k]      the same, transposed (rows = columns of Mc); with bf16
//                                 products, the frame-wise rule, no decay and d_k = d_v = 128
//                                 instead the forward scan's operand image of Mc (64 KB of
//                                 pre-split bf16 pieces per chunk, same size)
//   Jf [units][n][d_v][d_k]       chunk injections, forward
//   Jr [units][n][d_v][d_k]       chunk injections, reverse
//   ST [units][2][n + 1][d_v][d_k] boundary states: [0] = P (forward), [1] = R (reverse)
//   MrT [units][n][d_k][d_k]      reverse chunk transitions, transposed (decay only;
//                                 without decay the reverse transition is Mc^T); in the
//                                 case named under McT the reverse scan's operand image
//   Sp [units][n][69632 bytes]    bf16 features with d_k = d_v = 128: each chunk's gathered
//                                 state S~ split into bf16 hi + lo in the readout's LDS image
struct Plan {
  int units, F, U, T, dk, dv, C, r, n;
  float eps;
  int seed_mode, dtype;
  int anchors;    // 1: frames 0 and F - 1 are boundary anchors
  int rule;       // 0: frame-wise delta rule; 1, 2: batched comparison rules
  bool fp32_products;  // composition and scan on fp32 MFMA (always for fp32 features)
  int solver;     // 0: symmetric Gauss-Jordan sweep; 1: blocked Cholesky
  int qh;         // heads interleaved in q (1: the unit layout)
  float qeps;     // > 0: the readout L2-normalises each query row with this floor
  bool decay_ok;  // the decay path's launch grids fit too
  bool full_stats;  // store both triangles of every A_t (else the lower 32 x 32 blocks
                   // of latent frames only: all the frame-wise solve reads)
  size_t off[10];
  size_t total;
};

// Feature-map (prep) launch: batch x heads units of F frames of Hl x Wl tokens
struct PrepPlan {
  int batch, H, F, Hl, Wl, U, dk, dv, dtype, tiles_r, tiles_c;
  float eps;
};
hipError_t launch_prep(const PrepPlan& p, const void* q, const void* k, const void* v,
                       const float* wk_s, const float* wk_t, const float* wv_s, const float* wv_t,
                       void* qo, void* ko, void* vo, hipStream_t s);

// bf16 elements of one (unit, chunk) image in Sp: hi and lo, 128 rows of 136 each
constexpr size_t kSplitElems = 2 * 128 * 136;
// the bf16 readout with d_k = d_v = 128 (no decay) reads Sp
inline bool split_readout(int dtype, int dk, int dv) {
  return dtype == VDA_DTYPE_BF16 && dk == 128 && dv == 128;
}

struct WsPtrs {
  float *A, *B, *M, *Mc, *Jf, *Jr, *ST, *McT, *MrT;
  uint16_t* Sp;  // bf16 readout with d_k = d_v = 128: per (unit, chunk) the split S~ image
};

hipError_t launch_stats(const Plan& p, const void* k, const void* v, const float* beta,
                        const void* text_k, const void* text_v, const float* text_beta,
                        const WsPtrs& w, hipStream_t s);
// not_spd (device, nullable): set to VDA_ERR_NOT_SPD when a pivot is not positive
hipError_t launch_solve(const Plan& p, const WsPtrs& w, hipStream_t s, int* not_spd = nullptr);
// J [units][F + 1][d_v][d_k] = B_t M_t per frame (debug tap)
hipError_t launch_frame_injections(const Plan& p, const WsPtrs& w, float* J, hipStream_t s);
// alpha: decay gates [units][F][d_k] or nullptr (no decay)
hipError_t launch_compose(const Plan& p, const WsPtrs& w, const float* alpha,
                          hipStream_t s);  // Mc, McT, Jf, Jr (+ MrT with decay), seeds
hipError_t launch_scan(const Plan& p, const WsPtrs& w, bool decay, hipStream_t s);
// The readout's split images of S~ from ST when it reads them (split_readout):
// one per chunk in Sp, or with decay (alpha) one per frame in decay_images(w);
// else nothing
hipError_t launch_split(const Plan& p, const WsPtrs& w, const float* alpha, hipStream_t s);
// With decay the per-frame images (units x F x kSplitElems bf16) reuse the
// statistics' A and B regions, which are adjacent and dead once the scans have
// run: 2 x units x (F + 1) x 128 x 128 x 4 bytes >= units x F x kSplitElems x 2.
inline uint16_t* decay_images(const WsPtrs& w) { return reinterpret_cast<uint16_t*>(w.A); }
hipError_t launch_readout(const Plan& p, const void* q, const void* gate, const float* rms_weight,
                          void* out, const WsPtrs& w, const float* alpha, hipStream_t s);

}  // namespace vda
