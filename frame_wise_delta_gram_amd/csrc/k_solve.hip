// Transition of the frame-wise delta rule ("Video DeltaNet", arXiv 2609.20744,
// Sec. 3.2 Eq. (5) and App. A.1 Eq. (A.1) with alpha = 1):
//   M_t = (I + A_t)^{-1}
// for every (unit, frame), the text frame included (its map seeds the scans;
// the chunk composition applies it).
//
// I + A_t is symmetric positive definite with every eigenvalue >= 1 (A_t is a
// Gram matrix), so a Cholesky factorisation without pivoting is stable and its
// diagonal is >= 1.  One workgroup (4 waves) per frame keeps the lower
// triangle of the d_k x d_k matrix in LDS as 32 x 32 blocks (fp32, row stride
// 33), in place, and works block by block:
//   1. blocked right-looking Cholesky  I + A = L L^T.  The 32-column diagonal
//      block is factored by one wave in registers (lane c holds column c;
//      pivots and columns move with readlane, no LDS round trips) and replaced
//      by the inverse of its factor, W_pp = L_pp^{-1}.  Panel (L_ip = G_ip
//      W_pp^T) and trailing (G_ij -= L_ip L_jp^T) updates are 32x32x32 fp32
//      MFMA block products spread over the 4 waves;
//   2. W = L^{-1} row block by row block: W_ij = -W_ii sum_{k=j}^{i-1} L_ik W_kj,
//      the blocks of one row in parallel; each sum is held in registers until
//      the whole row has read L, then parked in its own block for the W_ii
//      product, so no staging buffer is needed;
//   3. M = W^T W, the upper blocks by MFMA, mirrored on store.
// 42 KiB of LDS per workgroup lets three workgroups share a CU, so their serial
// diagonal work overlaps each other's MFMA work.  fp32 throughout.
#include "vda_device.h"
#include "vda_internal.h"

namespace vda {
namespace {

constexpr int SG = 33;   // row stride of a stored 32 x 32 block (odd: conflict-free column reads)
constexpr int kBlk = 32 * SG;  // floats per stored block
constexpr int kNBlk = 10;      // lower-triangle blocks of a 128 x 128 matrix

__device__ __forceinline__ float readlane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// Factor the 32x32 SPD block at G (stride SG) as L L^T and overwrite it with
// W = L^{-1} (lower triangular, zeros above the diagonal), by one wave.  The
// pivots of I + A and of its Schur complements are >= 1, so the hardware
// reciprocal square root (1 ulp) is safe.
__device__ void factor_invert_diag_block(float* G) {
  const int lane = lane_id();
  const int c = lane & 31;  // lanes 32..63 duplicate lanes 0..31 and do not store
  float col[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) col[k] = G[k * SG + c];  // column c (= row c)

  float rinv[32];  // 1 / L[j][j]
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const float d = readlane_f(col[j], j);
    const float inv = __builtin_amdgcn_rsqf(d);
    rinv[j] = inv;
    // lanes c > j: L[c][j] = D[c][j] / piv (own copy, the block is symmetric);
    // t = L[c][j] / piv so that D[k][c] -= L[k][j] L[c][j] = D[k][j] * t
    const float t = col[j] * (inv * inv);
#pragma unroll
    for (int k = j + 1; k < 32; ++k) {
      const float dkj = readlane_f(col[j], k);  // D[k][j] = D[j][k], held by lane k
      if (c > j) col[k] = fmaf(-dkj, t, col[k]);
    }
    if (c == j) {
      col[j] = d * inv;
#pragma unroll
      for (int k = j + 1; k < 32; ++k) col[k] *= inv;
    }
  }
  // col[k] = L[k][c] for k >= c.  Column c of W = L^{-1}: solve L x = e_c
  // right-looking, x[j] /= L[j][j] then x[i] -= L[i][j] x[j] for i > j (the
  // updates of one step are independent); L[i][j] sits in lane j.
  float x[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) x[k] = (k == c) ? 1.0f : 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    x[j] *= rinv[j];
#pragma unroll
    for (int i = j + 1; i < 32; ++i) x[i] = fmaf(-readlane_f(col[i], j), x[j], x[i]);
  }
  if (lane < 32) {
#pragma unroll
    for (int k = 0; k < 32; ++k) G[k * SG + c] = x[k];
  }
}

__global__ __launch_bounds__(256, 3) void solve_kernel(const float* __restrict__ A,
                                                      float* __restrict__ Mout, int dk, int Fp1) {
  __shared__ float Gs[kNBlk * kBlk];  // block (i, j), j <= i, at index i (i + 1) / 2 + j
  const int fi = blockIdx.x;
  const int u = blockIdx.y;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int Dk = pad32(dk);
  const int nb = Dk >> 5;
  auto G = [&](int i, int j) { return Gs + (i * (i + 1) / 2 + j) * kBlk; };

  {
    MatRegs m;
    mat_load(m, A + ((size_t)u * Fp1 + fi) * dk * dk, dk, dk, dk);
#pragma unroll
    for (int i = 0; i < 16; ++i) {  // keep the lower-triangle blocks, add the identity
      const int id = t + 256 * i;
      const int r = id >> 5;
      const int c = (id & 31) << 2;
      const int bi = r >> 5, bj = c >> 5;
      if (r < Dk && c < Dk && bj <= bi) {
        float* dst = G(bi, bj) + (r & 31) * SG + (c & 31);
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[e] = m.v[i][e] + (r == c + e ? 1.0f : 0.0f);
      }
    }
    __syncthreads();
  }

  // 1. blocked Cholesky; diagonal blocks end up holding W_pp = L_pp^{-1}
  for (int p = 0; p < nb; ++p) {
    if (w == 0) factor_invert_diag_block(G(p, p));
    __syncthreads();
    {  // panel: L_ip = G_ip L_pp^{-T} = G_ip W_pp^T
      const int i = p + 1 + w;
      if (i < nb) {
        const f32x16_t acc = blk_mm32<false, true>(zero16(), G(i, p), SG, G(p, p), SG);
        store_acc(G(i, p), SG, acc, 1.0f);
      }
    }
    __syncthreads();
    {  // trailing: G_ij -= L_ip L_jp^T, p < j <= i
      int q = 0;
      for (int i = p + 1; i < nb; ++i)
        for (int j = p + 1; j <= i; ++j, ++q) {
          if ((q & 3) != w) continue;
          const f32x16_t acc = blk_mm32<false, true>(zero16(), G(i, p), SG, G(j, p), SG);
          float* C = G(i, j);
#pragma unroll
          for (int r = 0; r < 16; ++r) C[acc_row(r, lane) * SG + (lane & 31)] -= acc[r];
        }
    }
    __syncthreads();
  }

  // 2. off-diagonal blocks of W = L^{-1}, row block by row block
  for (int i = 1; i < nb; ++i) {
    f32x16_t acc = zero16();
    if (w < i) {  // wave j = w: T_ij = sum_{k=j}^{i-1} L_ik W_kj
      const int j = w;
      for (int k = j; k < i; ++k) acc = blk_mm32<false, false>(acc, G(i, k), SG, G(k, j), SG);
    }
    __syncthreads();  // every L_ik of row i has been read
    if (w < i) {      // W_ij = -W_ii T_ij, T_ij parked in block (i, j)
      const int j = w;
      store_acc(G(i, j), SG, acc, 1.0f);
      wave_sync();
      const f32x16_t acc2 = blk_mm32<false, false>(zero16(), G(i, i), SG, G(i, j), SG);
      wave_sync();
      store_acc(G(i, j), SG, acc2, -1.0f);
    }
    __syncthreads();
  }

  // 3. M = W^T W: M_ab = sum_{k >= max(a,b)} W_ka^T W_kb, written to global
  float* Mg = Mout + ((size_t)u * Fp1 + fi) * dk * dk;
  {
    int q = 0;
    for (int b = 0; b < nb; ++b)
      for (int a = 0; a <= b; ++a, ++q) {
        if ((q & 3) != w) continue;
        f32x16_t acc = zero16();
        for (int k = b; k < nb; ++k) acc = blk_mm32<true, false>(acc, G(k, a), SG, G(k, b), SG);
        const int col = lane & 31;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int gi = 32 * a + acc_row(r, lane), gj = 32 * b + col;
          if (gi < dk && gj < dk) {
            Mg[(size_t)gi * dk + gj] = acc[r];
            if (a != b) Mg[(size_t)gj * dk + gi] = acc[r];
          }
        }
      }
  }
}

}  // namespace

hipError_t launch_solve(const Plan& p, const WsPtrs& w, hipStream_t s) {
  const dim3 grid(p.F + 1, p.units);
  hipLaunchKernelGGL(solve_kernel, grid, dim3(kThreads), 0, s, w.A, w.M, p.dk, p.F + 1);
  return hipGetLastError();
}

}  // namespace vda
