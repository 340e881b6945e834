// Transition of the frame-wise delta rule ("Video DeltaNet", arXiv 2609.20744,
// Sec. 3.2 Eq. (5) and App. A.1 Eq. (A.1) with alpha = 1):
//   M_t = (I + A_t)^{-1}
// for every (unit, frame), the text frame included (its map seeds the scans;
// the chunk composition applies it).
//
// I + A_t is symmetric positive definite with every eigenvalue >= 1 (A_t is a
// Gram matrix), so Gauss-Jordan elimination in the symmetric "sweep" form
// (Beaton 1964; Goodnight 1979, "A tutorial on the SWEEP operator") needs no
// pivoting: every pivot is a diagonal entry of a Schur complement of I + A_t,
// hence >= 1.  Sweeping index k of a symmetric matrix G with d = G_kk maps
//   G_ij -> G_ij - G_ik G_kj / d   (i, j != k),
//   G_ik -> G_ik / d,  G_kj -> G_kj / d,  G_kk -> -1 / d,
// and sweeping every index turns G into -G^{-1}.  Applied to 32 x 32 blocks
// (block P with S = G_PP^{-1}):
//   G_PP -> -S,  G_Pi -> S G_Pi,  G_iP -> G_iP S,  G_ij -> G_ij - G_iP S G_Pj.
// One workgroup (4 waves) per frame keeps the lower-triangle 32 x 32 blocks of
// G = I + A_t in LDS (fp32, row stride 33).  Per pivot block: one wave sweeps
// the block in its MFMA accumulators (below); each other wave forms one
// Y_i = S G_Pi and the updates G_ji -= G_jP Y_i with 32x32x2 fp32 MFMA, Y_i
// staying in registers as an MFMA operand.  At the end the blocks hold -M.
// 42 KiB of LDS per workgroup lets three workgroups share a CU.  fp32
// throughout.
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

// Sweep all 32 indices of the symmetric block T held in accumulator layout
// (register r of lane l = T[acc_row(r, l)][l % 32]), by one wave; T becomes
// -T^{-1}.  Row k sits in register rk = 4 (k / 8) + k % 4 of the lanes of half
// hk = (k / 4) % 2, so it feeds both operands of a rank-1 32x32x2 MFMA through
// the k-slot hk with no data movement.  The scaling of column k by 1/d is
// deferred: each lane keeps a factor g for its column (true T = stored T times
// g per column), which only column k's lanes change at step k, and the block is
// multiplied by it once at the end, so a step costs two lane reads, one
// reciprocal and a handful of vector ops besides the MFMA.  In stored terms, step
// k with d = S_kk g_k (the true pivot) is, for i, j != k,
//   S_ij -= (S_ki g_i) (S_kj / d)    (S_ki g_i = T_ki = T_ik by symmetry),
// then S_kj *= 1/d (j != k), S_kk *= -1/d, g_k *= 1/d; row and column k are left
// alone by the rank-1 update (its operands are zero at k).  The hardware
// reciprocal is within 1 ulp.
__device__ __forceinline__ void sweep_block(f32x16_t& T) {
  const int lane = lane_id();
  const int half = lane >> 5;
  const int c = lane & 31;
  float g = 1.0f;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const int rk = 4 * (k >> 3) + (k & 3);
    const int hk = (k >> 2) & 1;
    const float skk = readlane_f(T[rk], k + 32 * hk);
    const float gk = readlane_f(g, k);
    const float inv = __builtin_amdgcn_rcpf(skk * gk);
    const bool inrow = half == hk;
    const bool colk = c == k;
    const float s = (inrow && !colk) ? T[rk] : 0.0f;  // row k off the pivot (stored)
    const float xa = s * g;
    const float xb = s * inv;
    T[rk] *= inrow ? (colk ? -inv : inv) : 1.0f;
    g = colk ? g * inv : g;
    T = mfma_f32(-xa, xb, T);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) T[r] *= g;
}

// acc += op(A) Bm for 32 x 32 blocks, A in LDS (row stride sa, op = transpose
// when AT), Bm in accumulator layout (register r of lane l = Bm[acc_row(r, l)][l % 32]).
// The contraction index of k-step r, slot h is acc_row(r, 32 h) on both sides.
template <bool AT>
__device__ __forceinline__ f32x16_t blk_mm32_breg(f32x16_t acc, const float* A, int sa,
                                                  const f32x16_t& Bm) {
  const int lane = lane_id();
  const int m = lane & 31;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int k = acc_row(r, lane);
    const float a = AT ? A[k * sa + m] : A[m * sa + k];
    acc = mfma_f32(a, Bm[r], acc);
  }
  return acc;
}

__device__ __forceinline__ f32x16_t tile_from_lds(const float* G) {
  const int lane = lane_id();
  f32x16_t T;
#pragma unroll
  for (int r = 0; r < 16; ++r) T[r] = G[acc_row(r, lane) * SG + (lane & 31)];
  return T;
}

__device__ __forceinline__ void tile_to_lds_t(float* G, const f32x16_t& T) {
  const int lane = lane_id();
#pragma unroll
  for (int r = 0; r < 16; ++r) G[(lane & 31) * SG + acc_row(r, lane)] = T[r];
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

  {  // G = I + A (identity on the padding too), lower-triangle blocks only (the
     // statistics may leave the blocks above the diagonal unwritten)
    const float* Af = A + ((size_t)u * Fp1 + fi) * dk * dk;
    const f32x4_t z = {0.0f, 0.0f, 0.0f, 0.0f};
    f32x4_t m[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int id = t + 256 * i;
      const int r = id >> 5;
      const int c = (id & 31) << 2;
      const bool ok = r < dk && c < dk && (c >> 5) <= (r >> 5);
      m[i] = ok ? *reinterpret_cast<const f32x4_t*>(Af + (size_t)r * dk + c) : z;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int id = t + 256 * i;
      const int r = id >> 5;
      const int c = (id & 31) << 2;
      const int bi = r >> 5, bj = c >> 5;
      if (r < Dk && c < Dk && bj <= bi) {
        float* dst = G(bi, bj) + (r & 31) * SG + (c & 31);
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[e] = m[i][e] + (r == c + e ? 1.0f : 0.0f);
      }
    }
    __syncthreads();
  }

  for (int p = 0; p < nb; ++p) {
    if (w == 0) {  // G_PP -> -S
      f32x16_t T = tile_from_lds(G(p, p));
      sweep_block(T);
      store_acc(G(p, p), SG, T, 1.0f);
    }
    __syncthreads();
    const int i = w < p ? w : w + 1;  // this wave's non-pivot block
    const bool has = i < nb;
    f32x16_t Y;
    if (has) {
      // Y_i = S G_Pi = -(G_PP) G_Pi with G_Pi = G(p, i) (i < p) or G(i, p)^T
      Y = i < p ? blk_mm32<false, false>(zero16(), G(p, p), SG, G(p, i), SG)
                : blk_mm32<false, true>(zero16(), G(p, p), SG, G(i, p), SG);
#pragma unroll
      for (int r = 0; r < 16; ++r) Y[r] = -Y[r];
      // G_ji -= G_jP Y_i for the lower blocks (j >= i) of this column, G_jP still old
      for (int j = i; j < nb; ++j) {
        if (j == p) continue;
        const f32x16_t prod = j > p ? blk_mm32_breg<false>(zero16(), G(j, p), SG, Y)
                                    : blk_mm32_breg<true>(zero16(), G(p, j), SG, Y);
        float* C = G(j, i);
#pragma unroll
        for (int r = 0; r < 16; ++r) C[acc_row(r, lane) * SG + (lane & 31)] -= prod[r];
      }
    }
    __syncthreads();  // every old G_jP has been read
    if (has) {  // G_Pi -> Y_i, stored as block (p, i) or, transposed, (i, p)
      if (i < p)
        store_acc(G(p, i), SG, Y, 1.0f);
      else
        tile_to_lds_t(G(i, p), Y);
    }
    __syncthreads();
  }

  // M = -G, both triangles, row-major, one float4 of a row per store
  float* Mg = Mout + ((size_t)u * Fp1 + fi) * dk * dk;
#pragma unroll 4
  for (int i = 0; i < 16; ++i) {
    const int id = t + 256 * i;
    const int r = id >> 5;
    const int c = (id & 31) << 2;
    if (r >= dk || c >= dk) continue;
    const int bi = r >> 5, bj = c >> 5;
    f32x4_t v;
    if (bj <= bi) {
      const float* src = G(bi, bj) + (r & 31) * SG + (c & 31);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = -src[e];
    } else {
      const float* src = G(bj, bi) + (c & 31) * SG + (r & 31);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = -src[e * SG];
    }
    *reinterpret_cast<f32x4_t*>(Mg + (size_t)r * dk + c) = v;
  }
}

// Inherited-state factor of the batched comparison rules (SANA-WM's frozen-state
// update, Sec. 3.1 Eq. (3c)): M = I - s A, and with frame-size key scaling
// (App. A.2, rule 2) s = 1 / N and B <- B / sqrt(N), N the frame's token count
// (the text frame's own T); rule 1: s = 1.  One workgroup per (frame, unit),
// float4 element-wise.
__global__ __launch_bounds__(256) void batched_factor_kernel(const float* __restrict__ A,
                                                             float* __restrict__ M,
                                                             float* __restrict__ B, int dk,
                                                             int dv, int Fp1, int U, int T,
                                                             int rule) {
  const int fi = blockIdx.x;
  const int u = blockIdx.y;
  const size_t fr = (size_t)u * Fp1 + fi;
  const int N = fi == 0 ? T : U;
  const bool scale = rule == 2 && N > 0;
  const float s = scale ? 1.0f / (float)N : 1.0f;
  const f32x4_t* a = reinterpret_cast<const f32x4_t*>(A + fr * dk * dk);
  f32x4_t* m = reinterpret_cast<f32x4_t*>(M + fr * dk * dk);
  for (int i = threadIdx.x; i < dk * dk / 4; i += blockDim.x) {
    const int r = (4 * i) / dk;
    const int c = 4 * i - r * dk;
    f32x4_t x = a[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = (r == c + e ? 1.0f : 0.0f) - s * x[e];
    m[i] = x;
  }
  if (scale) {
    const float sb = 1.0f / sqrtf((float)N);
    f32x4_t* b = reinterpret_cast<f32x4_t*>(B + fr * dv * dk);
    for (int i = threadIdx.x; i < dv * dk / 4; i += blockDim.x) b[i] *= sb;
  }
}

}  // namespace

hipError_t launch_solve(const Plan& p, const WsPtrs& w, hipStream_t s) {
  const dim3 grid(p.F + 1, p.units);
  if (p.rule == 0)
    hipLaunchKernelGGL(solve_kernel, grid, dim3(kThreads), 0, s, w.A, w.M, p.dk, p.F + 1);
  else
    hipLaunchKernelGGL(batched_factor_kernel, grid, dim3(kThreads), 0, s, w.A, w.M, w.B, p.dk,
                       p.dv, p.F + 1, p.U, p.T, p.rule);
  return hipGetLastError();
}

}  // namespace vda
