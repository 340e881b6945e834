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
// G = I + A_t in LDS (fp32, row stride 33).  Per pivot block P: the waves form
// Y_i = S G_Pi for the other block columns and the updates G_ji -= G_jP Y_i
// with 32x32x2 fp32 MFMA, Y_i staying in registers as an MFMA operand; the
// next pivot block is swept (below, in one wave's MFMA accumulators) by the
// wave that forms its update, while the others finish pivot P's updates.  At
// the end the blocks hold -M.
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
// (register r of lane l = T[acc_row(r, l)][l % 32]), by one wave, two indices
// at a time; T becomes -T^{-1}.  Register q holds rows a = 8 (q / 4) + q % 4
// (lanes 0..31) and b = a + 4 (lanes 32..63), and those two rows are exactly
// the two k slots of a 32x32x2 MFMA operand, so sweeping the pair P = {a, b}
// is one rank-2 MFMA with no data movement beyond a half swap.  With the 2 x 2
// pivot block Pi = T_PP and S = Pi^{-1} (closed form, one reciprocal of its
// determinant), the block sweep is
//   T_ij -= T_iP S T_Pj   (i, j not in P),   T_Pj -> S T_Pj,   T_iP -> T_iP S,
//   T_PP -> -S,
// and the MFMA takes A[i][s] = -T_{i,P_s} (zero on the pivot rows, so they
// only take the values written here) and B[s][j] = (S T_Pj)_s off the pivot
// columns, (I - S)_{s,t} on pivot column P_t, which turns T_iP into T_iP S by
// the same update (the block stays symmetric throughout, so T_{i,P_s} is row
// P_s's entry in column i).  Sweeping a pair equals sweeping its two indices
// one after the other; 16 dependent steps instead of 32.  The hardware
// reciprocal is within 1 ulp.
// `bad` turns true when a 2 x 2 pivot block is not positive definite (or not a
// number): I + A_t was not numerically positive definite.
__device__ __forceinline__ void sweep_block(f32x16_t& T, bool& bad) {
  const int lane = lane_id();
  const int half = lane >> 5;
  const int c = lane & 31;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int a = 8 * (q >> 2) + (q & 3);
    const int b = a + 4;
    const float x = T[q];              // row P_half, column c
    const float y = lane_xor32(x);     // the other pivot row, column c
    const float taa = readlane_f(x, a);
    const float tab = readlane_f(x, b);
    const float tbb = readlane_f(x, 32 + b);
    const float det = taa * tbb - tab * tab;
    bad |= !(taa > 0.0f && det > 0.0f);
    const float inv = __builtin_amdgcn_rcpf(det);
    const float sown = (half ? taa : tbb) * inv;  // S[half][half]
    const float sab = -tab * inv;                 // S[0][1] = S[1][0]
    const float st = sown * x + sab * y;          // (S T_Pc)[half]
    const bool pa = c == a, pb = c == b;
    const float shc = (half == (int)pb) ? sown : sab;  // S[half][t] on pivot column P_t
    const float id = (half == (int)pb) ? 1.0f : 0.0f;
    const bool piv = pa || pb;
    const float bop = piv ? id - shc : st;
    const float aop = piv ? 0.0f : -x;
    T[q] = piv ? -shc : st;
    T = mfma_f32(aop, bop, T);
  }
}

// acc += op(A) Bm for 32 x 32 blocks, A in LDS (row stride sa, op = transpose
// when AT), Bm in accumulator layout (register r of lane l = Bm[acc_row(r, l)][l % 32]).
// The contraction index of k-step r, slot h is acc_row(r, 32 h) on both sides.
// The A operands are read before the first MFMA (16 dependent MFMAs back to
// back).
template <bool AT>
__device__ __forceinline__ f32x16_t blk_mm32_breg(f32x16_t acc, const float* A, int sa,
                                                  const f32x16_t& Bm) {
  const int lane = lane_id();
  const int m = lane & 31;
  float a[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int k = acc_row(r, lane);
    a[r] = AT ? A[k * sa + m] : A[m * sa + k];
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the MFMA chain
#pragma unroll
  for (int r = 0; r < 16; ++r) acc = mfma_f32(a[r], Bm[r], acc);
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

// not_spd (nullable): set to VDA_ERR_NOT_SPD when a pivot is not positive
__global__ __launch_bounds__(256, 3) void solve_kernel(const float* __restrict__ A,
                                                      float* __restrict__ Mout, int dk, int Fp1,
                                                      int* __restrict__ not_spd) {
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

  // Pivot block 0 is swept first; every later pivot block is swept as soon as
  // the previous pivot's update of it is formed (lookahead), by the wave that
  // owns its column, while the other waves finish that pivot's updates.
  if (w == 0) {  // G_00 -> -S
    f32x16_t T = tile_from_lds(G(0, 0));
    bool bad = false;
    sweep_block(T, bad);
    store_acc(G(0, 0), SG, T, 1.0f);
    if (not_spd && bad && lane == 0) *not_spd = VDA_ERR_NOT_SPD;
  }
  __syncthreads();
  for (int p = 0; p < nb; ++p) {
    // waves 0 .. 2 own the non-pivot block columns i (in order); wave 3 forms
    // Y for column n1 = p + 1 as well and updates that column below its
    // diagonal, so the owner of column n1 only updates and sweeps block (n1, n1)
    const int n1 = p + 1;
    const bool spare = w == 3;
    const int i = spare ? n1 : (w < p ? w : w + 1);
    const bool has = i < nb;
    const bool next_owner = !spare && i == n1;
    f32x16_t Y;
    if (has) {
      // Yn = -Y_i = -S G_Pi = (G_PP) G_Pi with G_Pi = G(p, i) (i < p) or G(i, p)^T
      Y = i < p ? blk_mm32<false, false>(zero16(), G(p, p), SG, G(p, i), SG)
                : blk_mm32<false, true>(zero16(), G(p, p), SG, G(i, p), SG);
      // G_ji -= G_jP Y_i for the lower blocks (j >= i, j != p) of this wave's
      // share of column i, G_jP still old: the MFMAs accumulate G_jP Yn onto G_ji
      const int jbeg = spare ? n1 + 1 : i;
      const int jend = next_owner ? n1 + 1 : nb;
      for (int j = jbeg; j < jend; ++j) {
        if (j == p) continue;
        float* C = G(j, i);
        const f32x16_t Cj = tile_from_lds(C);
        f32x16_t upd = j > p ? blk_mm32_breg<false>(Cj, G(j, p), SG, Y)
                             : blk_mm32_breg<true>(Cj, G(p, j), SG, Y);
        if (next_owner) {  // block (n1, n1) is final for pivot n1: G_{n1 n1} -> -S
          bool bad = false;
          sweep_block(upd, bad);
          if (not_spd && bad && lane == 0) *not_spd = VDA_ERR_NOT_SPD;
        }
        store_acc(C, SG, upd, 1.0f);
      }
    }
    __syncthreads();  // every old G_jP has been read
    if (has && !spare) {  // G_Pi -> Y_i = -Yn, stored as block (p, i) or, transposed, (i, p)
      if (i < p)
        store_acc(G(p, i), SG, Y, -1.0f);
      else
        tile_to_lds_t(G(i, p), -Y);
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

// ---------------------------------------------------------------------------
// The same transition through a blocked Cholesky factorisation (desc->solver
// = 1), the factor-and-solve route of a classical SPD inverse:
//   I + A_t = L L^T  (right-looking, 32 x 32 blocks: factor the diagonal block,
//                     its triangular inverse W_p, panel L_ip = G_ip W_p^T,
//                     trailing update G_ij -= L_ip L_jp^T),
//   Y = L^{-1}       (block column by block column: Y_jj = W_j,
//                     Y_ij = -W_i sum_{k=j}^{i-1} L_ik Y_kj),
//   M_t = Y^T Y.
// Every pivot of I + A_t is >= 1, so no pivoting.  One workgroup (4 waves)
// per frame: the lower blocks of G (then L, then Y) in LDS, the four W_p and a
// column of Y in progress next to them (72 KiB: two workgroups per CU); the
// diagonal blocks are factored and inverted by one wave each in its MFMA
// accumulators with rank-1 v_mfma_f32_32x32x2_f32 updates (32 dependent steps
// each, twice per block: 256 in all against the sweep's 128, the reason the
// sweep is the default).  fp32 throughout.

// Cholesky factor of the symmetric positive definite 32 x 32 block T (accumulator
// layout, both triangles), by one wave: T becomes L (lower, zeros above).  Step
// k: d = sqrt(T_kk); column k below the diagonal is scaled by 1 / d (lane k
// holds column k, and by symmetry the untouched T_ik = T_ki); the trailing
// block gets T_ij -= x_i x_j (x = row k / d beyond k) as a rank-1 MFMA through
// k-slot hk (row k sits in register rk of the lanes of half hk); row k beyond
// the diagonal is set to zero.
__device__ __forceinline__ void chol_block(f32x16_t& T, bool& bad) {
  const int lane = lane_id();
  const int half = lane >> 5;
  const int c = lane & 31;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const int rk = 4 * (k >> 3) + (k & 3);
    const int hk = (k >> 2) & 1;
    const float tkk = readlane_f(T[rk], k + 32 * hk);
    bad |= !(tkk > 0.0f);  // not positive definite (or not a number)
    const float d = __builtin_sqrtf(tkk);
    const float inv = 1.0f / d;
    const bool inrow = half == hk;
    const float x = (inrow && c > k) ? T[rk] * inv : 0.0f;  // L_ck for c > k
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = acc_row(r, lane);
      if (c == k) T[r] = i > k ? T[r] * inv : (i == k ? d : T[r]);
    }
    if (inrow && c > k) T[rk] = 0.0f;  // upper triangle
    T = mfma_f32(-x, x, T);
  }
}

// Inverse of the lower-triangular 32 x 32 block L (in LDS, row stride SG), by
// one wave: W = L^{-1} in accumulator layout.  Gauss-Jordan on the rows of
// W = I: step k divides row k by L_kk and subtracts L_ik (row k) from every row
// i > k, a rank-1 MFMA with L's column k (read from LDS) in k-slot hk.
__device__ __forceinline__ f32x16_t tri_inv_block(const float* L) {
  const int lane = lane_id();
  const int half = lane >> 5;
  const int c = lane & 31;
  f32x16_t W;
#pragma unroll
  for (int r = 0; r < 16; ++r) W[r] = acc_row(r, lane) == c ? 1.0f : 0.0f;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const int rk = 4 * (k >> 3) + (k & 3);
    const int hk = (k >> 2) & 1;
    const bool inrow = half == hk;
    const float lkk = L[k * SG + k];
    if (inrow) W[rk] *= 1.0f / lkk;
    const float a = (inrow && c > k) ? -L[c * SG + k] : 0.0f;  // -L_ck for rows c > k
    const float b = inrow ? W[rk] : 0.0f;                       // row k of W
    W = mfma_f32(a, b, W);
  }
  return W;
}

// q-th lower block (i, j), j <= i < n, in the order (0,0), (1,0), (1,1), (2,0), ...
__device__ __forceinline__ bool lower_pair(int q, int n, int& i, int& j) {
  i = 0;
  while (q > i && i < n) {
    q -= i + 1;
    ++i;
  }
  j = q;
  return i < n;
}

constexpr int kCholLds = (kNBlk + 4 + 3) * kBlk;  // L/Y blocks, the W_p, a column of Y

__global__ __launch_bounds__(256, 2) void solve_chol_kernel(const float* __restrict__ A,
                                                           float* __restrict__ Mout, int dk,
                                                           int Fp1, int* __restrict__ not_spd) {
  __shared__ float Gs[kCholLds];
  const int fi = blockIdx.x;
  const int u = blockIdx.y;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int Dk = pad32(dk);
  const int nb = Dk >> 5;
  auto G = [&](int i, int j) { return Gs + (i * (i + 1) / 2 + j) * kBlk; };
  auto Wb = [&](int i) { return Gs + (kNBlk + i) * kBlk; };
  auto Yc = [&](int i) { return Gs + (kNBlk + 4 + i) * kBlk; };  // column scratch, i = 0..2

  {  // G = I + A, lower-triangle blocks (identity on the padding)
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
  // the diagonal block of G is symmetric but only its lower triangle is stored
  // as read from A; complete it for the factorisation
  auto load_sym = [&](const float* Bk) {
    f32x16_t T;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = acc_row(r, lane), j = lane & 31;
      T[r] = i >= j ? Bk[i * SG + j] : Bk[j * SG + i];
    }
    return T;
  };

  for (int p = 0; p < nb; ++p) {
    if (w == 0) {
      f32x16_t T = load_sym(G(p, p));
      bool bad = false;
      chol_block(T, bad);
      store_acc(G(p, p), SG, T, 1.0f);
      if (not_spd && bad && lane == 0) *not_spd = VDA_ERR_NOT_SPD;
      wave_sync();
      const f32x16_t Wp = tri_inv_block(G(p, p));
      store_acc(Wb(p), SG, Wp, 1.0f);
    }
    __syncthreads();
    // panel: L_ip = G_ip W_p^T
    const int i = p + 1 + w;
    if (i < nb) {
      const f32x16_t L = blk_mm32<false, true>(zero16(), G(i, p), SG, Wb(p), SG);
      store_acc(G(i, p), SG, L, 1.0f);
    }
    __syncthreads();
    // trailing update G_ij -= L_ip L_jp^T, i >= j > p: the lower blocks of the
    // trailing matrix dealt over the waves
    for (int q = w;; q += 4) {
      int ii, jj;
      if (!lower_pair(q, nb - p - 1, ii, jj)) break;
      ii += p + 1;
      jj += p + 1;
      const f32x16_t prod = blk_mm32<false, true>(zero16(), G(ii, p), SG, G(jj, p), SG);
      float* C = G(ii, jj);
#pragma unroll
      for (int r = 0; r < 16; ++r) C[acc_row(r, lane) * SG + (lane & 31)] -= prod[r];
    }
    __syncthreads();
  }

  // Y = L^{-1}, block column j: Y_ij = -W_i sum_{k=j}^{i-1} L_ik Y_kj, i = j + 1 ..,
  // built in the scratch by wave 0 (each entry needs the previous ones), then
  // copied over L's column j (later columns read only L's columns > j)
  for (int j = 0; j + 1 < nb; ++j) {
    if (w == 0) {
      for (int i = j + 1; i < nb; ++i) {
        f32x16_t S = zero16();
        for (int k = j; k < i; ++k) {
          const float* Ykj = k == j ? Wb(j) : Yc(k - j - 1);
          S = blk_mm32<false, false>(S, G(i, k), SG, Ykj, SG);
        }
        store_acc(Yc(i - j - 1), SG, S, 1.0f);
        wave_sync();
        const f32x16_t Yij = blk_mm32<false, false>(zero16(), Wb(i), SG, Yc(i - j - 1), SG);
        wave_sync();
        store_acc(Yc(i - j - 1), SG, Yij, -1.0f);
        wave_sync();
      }
    }
    __syncthreads();
    for (int idx = t; idx < (nb - 1 - j) * 32 * 32; idx += 256) {
      const int b = idx >> 10, e = idx & 1023;
      const int r = e >> 5, c = e & 31;
      G(j + 1 + b, j)[r * SG + c] = Yc(b)[r * SG + c];
    }
    __syncthreads();
  }

  // M = Y^T Y: M_ij = sum_{k >= i} Y_ki^T Y_kj for the lower blocks (i >= j), at
  // most three per wave, held in registers until every wave has read Y, then
  // stored over the lower blocks (a diagonal block from its lower triangle, so
  // M is exactly symmetric) and written out row-major as in the sweep
  f32x16_t Mb[3];
#pragma unroll
  for (int s3 = 0; s3 < 3; ++s3) {
    Mb[s3] = zero16();
    int ii, jj;
    if (!lower_pair(w + 4 * s3, nb, ii, jj)) continue;
    for (int k = ii; k < nb; ++k) {
      const float* Yki = k == ii ? Wb(ii) : G(k, ii);
      const float* Ykj = k == jj ? Wb(jj) : G(k, jj);
      Mb[s3] = blk_mm32<true, false>(Mb[s3], Yki, SG, Ykj, SG);
    }
  }
  __syncthreads();
#pragma unroll
  for (int s3 = 0; s3 < 3; ++s3) {
    int ii, jj;
    if (!lower_pair(w + 4 * s3, nb, ii, jj)) continue;
    float* C = G(ii, jj);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = acc_row(r, lane), col = lane & 31;
      if (ii != jj || row >= col) C[row * SG + col] = Mb[s3][r];
      if (ii == jj && row > col) C[col * SG + row] = Mb[s3][r];
    }
  }
  __syncthreads();
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
      for (int e = 0; e < 4; ++e) v[e] = src[e];
    } else {
      const float* src = G(bj, bi) + (c & 31) * SG + (r & 31);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = src[e * SG];
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

// Per-frame injection J_t = B_t M_t (debug tap only; the forward pass folds it
// into the chunk composition): one workgroup per (unit, frame), each output a
// plain fp32 dot product over d_k.
__global__ __launch_bounds__(256) void frame_injection_kernel(const float* __restrict__ B,
                                                              const float* __restrict__ M,
                                                              float* __restrict__ J, int dk,
                                                              int dv, int Fp1) {
  const size_t fr = (size_t)blockIdx.y * Fp1 + blockIdx.x;
  const float* Bf = B + fr * dv * dk;
  const float* Mf = M + fr * dk * dk;
  float* Jf = J + fr * dv * dk;
  for (int idx = threadIdx.x; idx < dv * dk; idx += kThreads) {
    const int r = idx / dk;
    const int c = idx - r * dk;
    float acc = 0.0f;
    for (int k = 0; k < dk; ++k) acc = fmaf(Bf[(size_t)r * dk + k], Mf[(size_t)k * dk + c], acc);
    Jf[idx] = acc;
  }
}

hipError_t launch_frame_injections(const Plan& p, const WsPtrs& w, float* J, hipStream_t s) {
  hipLaunchKernelGGL(frame_injection_kernel, dim3(p.F + 1, p.units), dim3(kThreads), 0, s, w.B,
                     w.M, J, p.dk, p.dv, p.F + 1);
  return hipGetLastError();
}

hipError_t launch_solve(const Plan& p, const WsPtrs& w, hipStream_t s, int* not_spd) {
  const dim3 grid(p.F + 1, p.units);
  if (p.rule == 0 && p.solver == 1)
    hipLaunchKernelGGL(solve_chol_kernel, grid, dim3(kThreads), 0, s, w.A, w.M, p.dk, p.F + 1,
                       not_spd);
  else if (p.rule == 0)
    hipLaunchKernelGGL(solve_kernel, grid, dim3(kThreads), 0, s, w.A, w.M, p.dk, p.F + 1,
                       not_spd);
  else
    hipLaunchKernelGGL(batched_factor_kernel, grid, dim3(kThreads), 0, s, w.A, w.M, w.B, p.dk,
                       p.dv, p.F + 1, p.U, p.T, p.rule);
  return hipGetLastError();
}

}  // namespace vda
