// Chunk-wise scans of Video Delta Attention ("Video DeltaNet", arXiv
// 2609.20744, Sec. 5 "Chunk-wise scans", App. A.1 Eq. (A.1), App. A.3).
//
// Each frame acts on the state as the affine map S -> (S + B_t) M_t
// (= S M_t + J_t with J_t = B_t M_t, M_t = (I + A_t)^{-1}).  Attention reads
// memory only at chunk boundaries, so
//
//   compose: per (unit, chunk) and independently of every other chunk,
//     Mc = M_{f0} M_{f0+1} ... M_{f1-1}                 (forward transition)
//     Jf = (((B_{f0}) M_{f0} + B_{f0+1}) M_{f0+1} + ...) M_{f1-1}
//     Jr = (((B_{f1-1}) M_{f1-1} + B_{f1-2}) M_{f1-2} + ...) M_{f0}
//   The reverse transition is M_{f1-1} ... M_{f0} = Mc^T because every M_t is
//   symmetric (alpha = 1), so it is not stored.
//
//   scan: per (unit, direction, 32-row block of the state) -- the rows of S
//   evolve independently --
//     P[0] = seed, P[j+1] = P[j] Mc_j + Jf_j          (forward, chunks 0..n-1)
//     R[n] = seed, R[j]   = R[j+1] Mc_j^T + Jr_j      (reverse, chunks n-1..0)
//   Only these n + 1 boundary states per direction are ever written.
//
// The state and every map stay fp32 in memory ("the inverse and recurrent
// state updates remain in FP32", Sec. 5).  Products:
//   fp32 features: 32x32x2 fp32 MFMA block products (exact fp32 products);
//   bf16 features: split bf16 MFMA ("bf16x3"): each fp32 operand x is held
//     in LDS as x_hi = bf16(x), x_lo = bf16(x - x_hi) and x y is formed as
//     x_hi y_hi + x_hi y_lo + x_lo y_hi with fp32 accumulation (relative error
//     ~2^-16 per product, far inside the bf16 path's tolerance) at the bf16
//     MFMA rate.  Both operands are read as contiguous 16-byte rows: X is
//     row-major, and a transition is read by rows because M_t is symmetric
//     (the forward chunk map is stored transposed for the same reason).
#include "vda_device.h"
#include "vda_internal.h"

namespace vda {
namespace {

constexpr int SG = 129;

// acc-layout prefetch of a 32-row x 32-col tile (rows r0.., cols c0..) of a
// row-major fp32 matrix with `rows` x dk valid entries; zero outside
__device__ __forceinline__ void tile_prefetch(float (&dst)[16], const float* src, int dk, int rows,
                                              int r0, int c0) {
  const int lane = lane_id();
  const int col = c0 + (lane & 31);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = r0 + acc_row(r, lane);
    dst[r] = (row < rows && col < dk) ? src[(size_t)row * dk + col] : 0.0f;
  }
}

__global__ __launch_bounds__(256, 1) void compose_kernel(const float* __restrict__ Bw,
                                                        const float* __restrict__ Mw,
                                                        float* __restrict__ Mc,
                                                        float* __restrict__ McT,
                                                        float* __restrict__ Jf,
                                                        float* __restrict__ Jr, int dk, int dv,
                                                        int F, int C, int n) {
  __shared__ float Xs[128 * SG];
  __shared__ float Ms[128 * SG];
  const int c = blockIdx.x;
  const int u = blockIdx.y;
  const int chain = blockIdx.z;  // 0: Mc, 1: Jf, 2: Jr
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int f0 = c * C;
  const int f1 = min(f0 + C, F);
  const int nf = f1 - f0;
  const int rows = chain == 0 ? dk : dv;
  const int R32 = pad32(rows);
  const int nR = R32 >> 5;
  const int Dk = pad32(dk);
  const int nb = Dk >> 5;
  const size_t Fp1 = (size_t)F + 1;
  // workspace frame index f + 1 holds latent frame f (index 0 is the text frame)
  auto frame = [&](int s) { return chain == 2 ? f1 - 1 - s : f0 + s; };
  auto Mp = [&](int f) { return Mw + ((size_t)u * Fp1 + f + 1) * dk * dk; };
  auto Bp = [&](int f) { return Bw + ((size_t)u * Fp1 + f + 1) * dv * dk; };

  {
    MatRegs m;
    if (chain != 0) {
      mat_load(m, Bp(frame(0)), dk, dv, dk);
      mat_store_lds(m, Xs, SG, R32, Dk);
    } else {
      for (int idx = t; idx < R32 * Dk; idx += 256) {
        const int i = idx / Dk;
        const int j = idx - i * Dk;
        Xs[i * SG + j] = (i == j) ? 1.0f : 0.0f;
      }
    }
    mat_load(m, Mp(frame(0)), dk, dk, dk);
    mat_store_lds(m, Ms, SG, Dk, Dk);
  }
  __syncthreads();

  float* dst = chain == 0 ? Mc + ((size_t)u * n + c) * dk * dk
                          : (chain == 1 ? Jf : Jr) + ((size_t)u * n + c) * dv * dk;
  MatRegs mnext;
  float bnext[4][16];
  for (int s = 0; s < nf; ++s) {
    const bool last = s == nf - 1;
    if (!last) {  // next frame's transition (and write) fly while this step multiplies
      mat_load(mnext, Mp(frame(s + 1)), dk, dk, dk);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        if (chain != 0 && w < nR && ct < nb)
          tile_prefetch(bnext[ct], Bp(frame(s + 1)), dk, dv, 32 * w, 32 * ct);
        else
#pragma unroll
          for (int r = 0; r < 16; ++r) bnext[ct][r] = 0.0f;
      }
    }
    f32x16_t acc[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[ct] = zero16();
    if (w < nR) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        if (ct >= nb) continue;
        for (int kb = 0; kb < nb; ++kb)
          acc[ct] = blk_mm32<false, false>(acc[ct], Xs + 32 * w * SG + 32 * kb, SG,
                                           Ms + 32 * kb * SG + 32 * ct, SG);
      }
    }
    __syncthreads();
    if (w < nR) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        if (ct >= nb) continue;
        const int col = 32 * ct + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 32 * w + acc_row(r, lane);
          if (last) {
            if (row < rows && col < dk) {
              dst[(size_t)row * dk + col] = acc[ct][r];
              if (chain == 0) McT[((size_t)u * n + c) * dk * dk + (size_t)col * dk + row] = acc[ct][r];
            }
          } else {
            Xs[row * SG + col] = acc[ct][r] + bnext[ct][r];
          }
        }
      }
    }
    if (last) break;
    mat_store_lds(mnext, Ms, SG, Dk, Dk);
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void scan_kernel(const float* __restrict__ Mc,
                                                   const float* __restrict__ Jf,
                                                   const float* __restrict__ Jr,
                                                   float* __restrict__ ST, int dk, int dv, int n) {
  __shared__ float Xs[32 * SG];
  __shared__ float Ms[128 * SG];
  const int rb = blockIdx.x;  // rows [32 rb, 32 rb + 32) of the state
  const int u = blockIdx.y;
  const int dir = blockIdx.z;  // 0: forward (P), 1: reverse (R)
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int Dk = pad32(dk);
  const int nb = Dk >> 5;
  const size_t SS = (size_t)dv * dk;
  float* S = ST + (size_t)(u * 2 + dir) * (n + 1) * SS;
  const int r0 = 32 * rb;
  const int nrows = min(32, dv - r0);
  auto chunk = [&](int s) { return dir == 0 ? s : n - 1 - s; };
  const float* Jb = (dir == 0 ? Jf : Jr) + (size_t)u * n * SS;

  MatRegs m;
  mat_load(m, S + (size_t)(dir == 0 ? 0 : n) * SS + (size_t)r0 * dk, dk, nrows, dk);
  mat_store_lds(m, Xs, SG, 32, Dk);
  mat_load(m, Mc + ((size_t)u * n + chunk(0)) * dk * dk, dk, dk, dk);
  mat_store_lds(m, Ms, SG, Dk, Dk);
  float jreg[16];
  if (w < nb) tile_prefetch(jreg, Jb + (size_t)chunk(0) * SS + (size_t)r0 * dk, dk, nrows, 0, 32 * w);
  __syncthreads();
  for (int s = 0; s < n; ++s) {
    const int j = chunk(s);
    const bool last = s == n - 1;
    float jnext[16];
    if (!last) {
      mat_load(m, Mc + ((size_t)u * n + chunk(s + 1)) * dk * dk, dk, dk, dk);
      if (w < nb)
        tile_prefetch(jnext, Jb + (size_t)chunk(s + 1) * SS + (size_t)r0 * dk, dk, nrows, 0, 32 * w);
    }
    f32x16_t acc = zero16();
    if (w < nb) {
      for (int kb = 0; kb < nb; ++kb) {
        if (dir == 0)
          acc = blk_mm32<false, false>(acc, Xs + 32 * kb, SG, Ms + 32 * kb * SG + 32 * w, SG);
        else
          acc = blk_mm32<false, true>(acc, Xs + 32 * kb, SG, Ms + 32 * w * SG + 32 * kb, SG);
      }
    }
    __syncthreads();
    if (w < nb) {
      float* dst = S + (size_t)(dir == 0 ? j + 1 : j) * SS;
      const int col = 32 * w + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = acc_row(r, lane);
        const float x = (row < nrows && col < dk) ? acc[r] + jreg[r] : 0.0f;
        if (row < nrows && col < dk) dst[(size_t)(r0 + row) * dk + col] = x;
        Xs[row * SG + col] = x;
      }
    }
    if (last) break;
    mat_store_lds(m, Ms, SG, Dk, Dk);
#pragma unroll
    for (int r = 0; r < 16; ++r) jreg[r] = jnext[r];
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// bf16x3 versions (bf16 features).  LDS matrices are pairs of bf16 arrays
// (hi, lo) with a 136-element (272-byte) row stride: 16 consecutive rows read
// at one column offset land on 16 distinct 16-byte bank groups.
constexpr int SB = 136;

// hi/lo split of one fp32 value
__device__ __forceinline__ void split_bf16(float x, __bf16& h, __bf16& l) {
  h = (__bf16)x;
  l = (__bf16)(x - (float)h);
}

// MatRegs (row-major rows x cols, zero padded) -> (hi, lo) LDS, as stored
// (transpose = false) or transposed (true).
__device__ __forceinline__ void mat_store_split(const MatRegs& m, __bf16* hi, __bf16* lo, int R,
                                                int C, bool transpose) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int id = threadIdx.x + 256 * i;
    const int r = id >> 5;
    const int c = (id & 31) << 2;
    if (r < R && c < C) {
      __bf16 h[4], l[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) split_bf16(m.v[i][e], h[e], l[e]);
      if (!transpose) {
        bf16x2_t h01 = {h[0], h[1]}, h23 = {h[2], h[3]}, l01 = {l[0], l[1]}, l23 = {l[2], l[3]};
        u32x2_t hv = {__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23)};
        u32x2_t lv = {__builtin_bit_cast(uint32_t, l01), __builtin_bit_cast(uint32_t, l23)};
        *reinterpret_cast<u32x2_t*>(hi + r * SB + c) = hv;
        *reinterpret_cast<u32x2_t*>(lo + r * SB + c) = lv;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hi[(c + e) * SB + r] = h[e];
          lo[(c + e) * SB + r] = l[e];
        }
      }
    }
  }
}

// acc (+) = X_tile(rows xr.., all K) * B^T where B is given by rows (B[j][k]):
// 32 x 32 output tile at B rows jr.., K = Kp (multiple of 16) channels.
__device__ __forceinline__ f32x16_t split_mm(f32x16_t acc, const __bf16* xh, const __bf16* xl,
                                             int xr, const __bf16* bh, const __bf16* bl, int jr,
                                             int Kp) {
  const int lane = lane_id();
  const int il = lane & 31;
  const int g = lane >> 5;
  for (int k0 = 0; k0 < Kp; k0 += 16) {
    const int ka = (xr + il) * SB + k0 + 8 * g;
    const int kb = (jr + il) * SB + k0 + 8 * g;
    const u32x4_t ah = *reinterpret_cast<const u32x4_t*>(xh + ka);
    const u32x4_t al = *reinterpret_cast<const u32x4_t*>(xl + ka);
    const u32x4_t bh_ = *reinterpret_cast<const u32x4_t*>(bh + kb);
    const u32x4_t bl_ = *reinterpret_cast<const u32x4_t*>(bl + kb);
    acc = mfma_bf16(ah, bh_, acc);
    acc = mfma_bf16(ah, bl_, acc);
    acc = mfma_bf16(al, bh_, acc);
  }
  return acc;
}

// store one fp32 32x32 accumulator tile (rows r0.., cols c0..) into (hi, lo) LDS
__device__ __forceinline__ void acc_store_split(__bf16* hi, __bf16* lo, const f32x16_t& acc,
                                                const float (&add)[16], int r0, int c0) {
  const int lane = lane_id();
  const int col = c0 + (lane & 31);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = r0 + acc_row(r, lane);
    __bf16 h, l;
    split_bf16(acc[r] + add[r], h, l);
    hi[row * SB + col] = h;
    lo[row * SB + col] = l;
  }
}

__global__ __launch_bounds__(256, 1) void compose_split_kernel(const float* __restrict__ Bw,
                                                              const float* __restrict__ Mw,
                                                              float* __restrict__ Mc,
                                                              float* __restrict__ McT,
                                                              float* __restrict__ Jf,
                                                              float* __restrict__ Jr, int dk,
                                                              int dv, int F, int C, int n,
                                                              int units, unsigned per) {
  __shared__ __align__(16) __bf16 Xh[128 * SB];
  __shared__ __align__(16) __bf16 Xl[128 * SB];
  __shared__ __align__(16) __bf16 Mh[128 * SB];
  __shared__ __align__(16) __bf16 Ml[128 * SB];
  // work item = (unit, chunk, chain), chain fastest: the three chains of a chunk
  // read the same transitions and share an XCD
  const unsigned item = xcd_item(per);
  if (item >= (unsigned)units * n * 3) return;
  const int chain = item % 3;  // 0: Mc, 1: Jf, 2: Jr
  const int c = (item / 3) % n;
  const int u = item / (3 * n);
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int f0 = c * C;
  const int f1 = min(f0 + C, F);
  const int nf = f1 - f0;
  const int rows = chain == 0 ? dk : dv;
  const int nR = pad32(rows) >> 5;
  const int Dk = pad32(dk);
  const int nb = Dk >> 5;
  const int Kp = (dk + 15) & ~15;
  const size_t Fp1 = (size_t)F + 1;
  auto frame = [&](int s) { return chain == 2 ? f1 - 1 - s : f0 + s; };
  auto Mp = [&](int f) { return Mw + ((size_t)u * Fp1 + f + 1) * dk * dk; };
  auto Bp = [&](int f) { return Bw + ((size_t)u * Fp1 + f + 1) * dv * dk; };

  {
    MatRegs m;
    if (chain != 0) {
      mat_load(m, Bp(frame(0)), dk, dv, dk);
      mat_store_split(m, Xh, Xl, pad32(rows), Dk, false);
    } else {
      for (int idx = t; idx < Dk * Dk; idx += 256) {
        const int i = idx / Dk;
        const int j = idx - i * Dk;
        Xh[i * SB + j] = (__bf16)(i == j ? 1.0f : 0.0f);
        Xl[i * SB + j] = (__bf16)0.0f;
      }
    }
    mat_load(m, Mp(frame(0)), dk, dk, dk);
    mat_store_split(m, Mh, Ml, Dk, Dk, false);
  }
  __syncthreads();

  float* dst = chain == 0 ? Mc + ((size_t)u * n + c) * dk * dk
                          : (chain == 1 ? Jf : Jr) + ((size_t)u * n + c) * dv * dk;
  MatRegs mnext;
  float bnext[4][16];
  for (int s = 0; s < nf; ++s) {
    const bool last = s == nf - 1;
    if (!last) {  // next frame's transition (and write) fly while this step multiplies
      mat_load(mnext, Mp(frame(s + 1)), dk, dk, dk);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        if (chain != 0 && w < nR && ct < nb)
          tile_prefetch(bnext[ct], Bp(frame(s + 1)), dk, dv, 32 * w, 32 * ct);
        else
#pragma unroll
          for (int r = 0; r < 16; ++r) bnext[ct][r] = 0.0f;
      }
    }
    f32x16_t acc[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[ct] = zero16();
    if (w < nR) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        if (ct < nb) acc[ct] = split_mm(acc[ct], Xh, Xl, 32 * w, Mh, Ml, 32 * ct, Kp);
    }
    __syncthreads();
    if (w < nR) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        if (ct >= nb) continue;
        if (last) {
          const int col = 32 * ct + (lane & 31);
          float* dstT = McT + ((size_t)u * n + c) * dk * dk;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = 32 * w + acc_row(r, lane);
            if (row < rows && col < dk) {
              dst[(size_t)row * dk + col] = acc[ct][r];
              if (chain == 0) dstT[(size_t)col * dk + row] = acc[ct][r];
            }
          }
        } else {
          acc_store_split(Xh, Xl, acc[ct], bnext[ct], 32 * w, 32 * ct);
        }
      }
    }
    if (last) break;
    mat_store_split(mnext, Mh, Ml, Dk, Dk, false);
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void scan_split_kernel(const float* __restrict__ McR,
                                                         const float* __restrict__ McTr,
                                                         const float* __restrict__ Jf,
                                                         const float* __restrict__ Jr,
                                                         float* __restrict__ ST, int dk, int dv,
                                                         int n) {
  __shared__ __align__(16) __bf16 Xh[32 * SB];
  __shared__ __align__(16) __bf16 Xl[32 * SB];
  __shared__ __align__(16) __bf16 Mh[128 * SB];
  __shared__ __align__(16) __bf16 Ml[128 * SB];
  const int rb = blockIdx.x;  // rows [32 rb, 32 rb + 32) of the state
  const int u = blockIdx.y;
  const int dir = blockIdx.z;  // 0: forward (P), 1: reverse (R)
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int Dk = pad32(dk);
  const int nb = Dk >> 5;
  const int Kp = (dk + 15) & ~15;
  const size_t SS = (size_t)dv * dk;
  float* S = ST + (size_t)(u * 2 + dir) * (n + 1) * SS;
  const int r0 = 32 * rb;
  const int nrows = min(32, dv - r0);
  auto chunk = [&](int s) { return dir == 0 ? s : n - 1 - s; };
  const float* Jb = (dir == 0 ? Jf : Jr) + (size_t)u * n * SS;
  // the B operand is read by rows: forward S Mc needs the rows of Mc^T, reverse
  // S Mc^T the rows of Mc
  const float* Mc = dir == 0 ? McTr : McR;

  MatRegs m;
  mat_load(m, S + (size_t)(dir == 0 ? 0 : n) * SS + (size_t)r0 * dk, dk, nrows, dk);
  mat_store_split(m, Xh, Xl, 32, Dk, false);
  mat_load(m, Mc + ((size_t)u * n + chunk(0)) * dk * dk, dk, dk, dk);
  mat_store_split(m, Mh, Ml, Dk, Dk, false);
  float jreg[16];
  if (w < nb) tile_prefetch(jreg, Jb + (size_t)chunk(0) * SS + (size_t)r0 * dk, dk, nrows, 0, 32 * w);
  __syncthreads();
  const float zero[16] = {0.0f};
  for (int s = 0; s < n; ++s) {
    const int j = chunk(s);
    const bool last = s == n - 1;
    float jnext[16];
    if (!last) {
      mat_load(m, Mc + ((size_t)u * n + chunk(s + 1)) * dk * dk, dk, dk, dk);
      if (w < nb)
        tile_prefetch(jnext, Jb + (size_t)chunk(s + 1) * SS + (size_t)r0 * dk, dk, nrows, 0, 32 * w);
    }
    f32x16_t acc = zero16();
    if (w < nb) acc = split_mm(acc, Xh, Xl, 0, Mh, Ml, 32 * w, Kp);
    __syncthreads();
    if (w < nb) {
      float* dstp = S + (size_t)(dir == 0 ? j + 1 : j) * SS;
      const int col = 32 * w + (lane & 31);
      f32x16_t x;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = acc_row(r, lane);
        const bool ok = row < nrows && col < dk;
        x[r] = ok ? acc[r] + jreg[r] : 0.0f;
        if (ok) dstp[(size_t)(r0 + row) * dk + col] = x[r];
      }
      acc_store_split(Xh, Xl, x, zero, 0, 32 * w);
    }
    if (last) break;
    mat_store_split(m, Mh, Ml, Dk, Dk, false);
#pragma unroll
    for (int r = 0; r < 16; ++r) jreg[r] = jnext[r];
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_compose(const Plan& p, const WsPtrs& w, hipStream_t s) {
  if (p.dtype == VDA_DTYPE_BF16) {
    const unsigned per = xcd_per((unsigned)p.units * p.n * 3);
    hipLaunchKernelGGL(compose_split_kernel, dim3(kXcds * per), dim3(kThreads), 0, s, w.B, w.M,
                       w.Mc, w.McT, w.Jf, w.Jr, p.dk, p.dv, p.F, p.C, p.n, p.units, per);
  } else {
    hipLaunchKernelGGL(compose_kernel, dim3(p.n, p.units, 3), dim3(kThreads), 0, s, w.B, w.M, w.Mc,
                       w.McT, w.Jf, w.Jr, p.dk, p.dv, p.F, p.C, p.n);
  }
  return hipGetLastError();
}

hipError_t launch_scan(const Plan& p, const WsPtrs& w, hipStream_t s) {
  const dim3 grid(pad32(p.dv) >> 5, p.units, 2);
  if (p.dtype == VDA_DTYPE_BF16)
    hipLaunchKernelGGL(scan_split_kernel, grid, dim3(kThreads), 0, s, w.Mc, w.McT, w.Jf, w.Jr, w.ST,
                       p.dk, p.dv, p.n);
  else
    hipLaunchKernelGGL(scan_kernel, grid, dim3(kThreads), 0, s, w.Mc, w.Jf, w.Jr, w.ST, p.dk, p.dv,
                       p.n);
  return hipGetLastError();
}

}  // namespace vda
