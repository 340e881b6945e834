// Host-side plan and kernel launchers of the VDA library (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "vda.h"

namespace vda {

// Sizes derived from a validated descriptor, and the workspace carve-up.
// Workspace sections (all fp32, each 256-byte aligned):
//   A  [units][F + 1][d_k][d_k]   frame statistics, index 0 = text frame
//   B  [units][F + 1][d_v][d_k]
//   M  [units][F + 1][d_k][d_k]   transitions (I + A)^{-1}
//   Mc [units][n][d_k][d_k]       chunk transitions (forward order)
//   McT [units][n][d_k][d_k]      the same, transposed (rows = columns of Mc)
//   Jf [units][n][d_v][d_k]       chunk injections, forward
//   Jr [units][n][d_v][d_k]       chunk injections, reverse
//   ST [units][2][n + 1][d_v][d_k] boundary states: [0] = P (forward), [1] = R (reverse)
//   MrT [units][n][d_k][d_k]      reverse chunk transitions, transposed (decay only;
//                                 without decay the reverse transition is Mc^T)
struct Plan {
  int units, F, U, T, dk, dv, C, r, n;
  float eps;
  int seed_mode, dtype;
  int anchors;    // 1: frames 0 and F - 1 are boundary anchors
  int rule;       // 0: frame-wise delta rule; 1, 2: batched comparison rules
  bool decay_ok;  // the decay path's launch grids fit too
  bool full_stats;  // store both triangles of every A_t (else the lower 32 x 32 blocks
                   // of latent frames only: all the frame-wise solve reads)
  size_t off[9];
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

struct WsPtrs {
  float *A, *B, *M, *Mc, *Jf, *Jr, *ST, *McT, *MrT;
};

hipError_t launch_stats(const Plan& p, const void* k, const void* v, const float* beta,
                        const void* text_k, const void* text_v, const float* text_beta,
                        const WsPtrs& w, hipStream_t s);
hipError_t launch_solve(const Plan& p, const WsPtrs& w, hipStream_t s);
// alpha: decay gates [units][F][d_k] or nullptr (no decay)
hipError_t launch_compose(const Plan& p, const WsPtrs& w, const float* alpha,
                          hipStream_t s);  // Mc, McT, Jf, Jr (+ MrT with decay), seeds
hipError_t launch_scan(const Plan& p, const WsPtrs& w, bool decay, hipStream_t s);
hipError_t launch_readout(const Plan& p, const void* q, const void* gate, const float* rms_weight,
                          void* out, const WsPtrs& w, const float* alpha, hipStream_t s);

}  // namespace vda
