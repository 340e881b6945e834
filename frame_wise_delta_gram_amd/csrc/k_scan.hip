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
//   With channel-wise decay (App. A.1 Eq. (A.1) with alpha_t in [0, 1]^{d_k})
//   a frame's map is S -> (S D_t + B_t) M_t, D_t = Diag(alpha_t), in both scan
//   directions: Mc = D_{f0} M_{f0} ... D_{f1-1} M_{f1-1}, each J picks up the
//   gate of every frame it enters, and the reverse transition
//   Mr = D_{f1-1} M_{f1-1} ... D_{f0} M_{f0} is a chain of its own, stored
//   transposed (MrT).
//
//   scan: per (unit, direction, 32-row block of the state) -- the rows of S
//   evolve independently --
//     P[0] = seed, P[j+1] = P[j] Mc_j + Jf_j          (forward, chunks 0..n-1)
//     R[n] = seed, R[j]   = R[j+1] Mc_j^T + Jr_j      (reverse, chunks n-1..0;
//                                                      Mr_j in place of Mc_j^T with decay)
//   Only these n + 1 boundary states per direction are ever written.
//
// The state and every map stay fp32 in memory (as the pages keep the inverse
// and the recurrent state updates in fp32, Sec. 5).  Products:
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
                                                        const float* __restrict__ alpha,
                                                        float* __restrict__ Mc,
                                                        float* __restrict__ McT,
                                                        float* __restrict__ MrT,
                                                        float* __restrict__ Jf,
                                                        float* __restrict__ Jr,
                                                        float* __restrict__ ST, int dk, int dv,
                                                        int F, int C, int n, float seed_scale,
                                                        int anchors, int batched) {
  __shared__ float Xs[128 * SG];
  __shared__ float Ms[128 * SG];
  const int c = blockIdx.x;
  const int u = blockIdx.y;
  // 0: Mc, 1: Jf, 2: Jr, 3: text seed (one per unit), 4: reverse transition (decay only)
  const int chain = blockIdx.z;
  if (chain == 3 && c != 0) return;
  const bool mchain = chain == 0 || chain == 4;    // transition chains
  const bool reverse = chain == 2 || chain == 4;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  // the seed is the text frame's map applied once: (0 + s B_T) M_T
  const int f0 = chain == 3 ? -1 : c * C;
  const int f1 = chain == 3 ? 0 : min(f0 + C, F);
  const int nf = f1 - f0;
  const int rows = mchain ? dk : dv;
  const int R32 = pad32(rows);
  const int nR = R32 >> 5;
  const int Dk = pad32(dk);
  const int nb = Dk >> 5;
  const size_t Fp1 = (size_t)F + 1;
  // workspace frame index f + 1 holds latent frame f (index 0 is the text frame)
  auto frame = [&](int s) { return reverse ? f1 - 1 - s : f0 + s; };
  auto Mp = [&](int f) { return Mw + ((size_t)u * Fp1 + f + 1) * dk * dk; };
  auto Bp = [&](int f) { return Bw + ((size_t)u * Fp1 + f + 1) * dv * dk; };
  // decay gate of latent frame f, key channel j (1 without decay and for the
  // boundary anchors, which leave the states alone)
  auto gate = [&](int f, int j) {
    const bool anchor = anchors && (f == 0 || f == F - 1);
    return alpha && j < dk && !anchor ? alpha[((size_t)u * F + f) * dk + j] : 1.0f;
  };
  // batched comparison rule: a write chain (and the seed) starts at X = B of its
  // first frame and steps X <- X M_g + B_g over the others
  const int sh = batched && !mchain ? 1 : 0;
  const int nsteps = nf - sh;
  const size_t SS = (size_t)dv * dk;
  float* dst = chain == 0 ? Mc + ((size_t)u * n + c) * dk * dk
               : chain == 3 ? ST + (size_t)u * 2 * (n + 1) * SS                  // P[0]
               : chain == 4 ? nullptr                                            // MrT only
                            : (chain == 1 ? Jf : Jr) + ((size_t)u * n + c) * SS;
  float* dst2 = ST + ((size_t)(u * 2 + 1) * (n + 1) + n) * SS;                 // R[n]
  if (batched && nsteps == 0) {  // the chain is its first frame's write
    const float scale = chain == 3 ? seed_scale : 1.0f;
    const float* src = Bp(frame(0));
    for (size_t i = t; i < SS; i += 256) {
      dst[i] = src[i] * scale;
      if (chain == 3) dst2[i] = src[i] * scale;
    }
    return;
  }

  {
    MatRegs m;
    if (!mchain) {
      mat_load(m, Bp(frame(0)), dk, dv, dk);
      if (chain == 3)
#pragma unroll
        for (int i = 0; i < 16; ++i) m.v[i] *= seed_scale;
      mat_store_lds(m, Xs, SG, R32, Dk);
    } else {  // the decayed identity Diag(alpha) of the first frame
      for (int idx = t; idx < R32 * Dk; idx += 256) {
        const int i = idx / Dk;
        const int j = idx - i * Dk;
        Xs[i * SG + j] = (i == j) ? gate(frame(0), i) : 0.0f;
      }
    }
    mat_load(m, Mp(frame(sh)), dk, dk, dk);
    mat_store_lds(m, Ms, SG, Dk, Dk);
  }
  __syncthreads();

  MatRegs mnext;
  float bnext[4][16];
  for (int s = 0; s < nsteps; ++s) {
    const bool last = s == nsteps - 1;
    if (!last || sh) {  // next frame's transition (and write) fly while this step multiplies
      if (!last) mat_load(mnext, Mp(frame(s + 1 + sh)), dk, dk, dk);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        if (!mchain && w < nR && ct < nb)
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
        // entering the next frame: the state is decayed by its gate, then written
        const float a = last ? 1.0f : gate(frame(s + 1), col);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 32 * w + acc_row(r, lane);
          if (last) {
            if (row < rows && col < dk) {
              const size_t tix = ((size_t)u * n + c) * dk * dk + (size_t)col * dk + row;
              const float val = acc[ct][r] + (sh ? bnext[ct][r] : 0.0f);
              if (chain == 4) {
                MrT[tix] = val;
              } else {
                dst[(size_t)row * dk + col] = val;
                if (chain == 0) McT[tix] = val;
                if (chain == 3) dst2[(size_t)row * dk + col] = val;
              }
            }
          } else {
            Xs[row * SG + col] = acc[ct][r] * a + bnext[ct][r];
          }
        }
      }
    }
    if (last) break;
    mat_store_lds(mnext, Ms, SG, Dk, Dk);
    __syncthreads();
  }
}

// Mrt: the transposed reverse transition, Mc itself without decay
__global__ __launch_bounds__(256) void scan_kernel(const float* __restrict__ Mc,
                                                   const float* __restrict__ Mrt,
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
  const float* Mb = dir == 0 ? Mc : Mrt;

  MatRegs m;
  mat_load(m, S + (size_t)(dir == 0 ? 0 : n) * SS + (size_t)r0 * dk, dk, nrows, dk);
  mat_store_lds(m, Xs, SG, 32, Dk);
  mat_load(m, Mb + ((size_t)u * n + chunk(0)) * dk * dk, dk, dk, dk);
  mat_store_lds(m, Ms, SG, Dk, Dk);
  float jreg[16];
  if (w < nb) tile_prefetch(jreg, Jb + (size_t)chunk(0) * SS + (size_t)r0 * dk, dk, nrows, 0, 32 * w);
  __syncthreads();
  for (int s = 0; s < n; ++s) {
    const int j = chunk(s);
    const bool last = s == n - 1;
    float jnext[16];
    if (!last) {
      mat_load(m, Mb + ((size_t)u * n + chunk(s + 1)) * dk * dk, dk, dk, dk);
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
// bf16x3 versions (bf16 features).  X (the composed map or state) and the
// current transition live in LDS as pairs of bf16 arrays (hi, lo) with a
// 136-element (272-byte) row stride.  The product is formed transposed,
//   T = M[jr .. jr + 31, :] X^T = ((X M)[:, jr .. jr + 31])^T   (M symmetric),
// so a wave's transition operand is 32 rows of M (loaded from memory as whole
// contiguous rows, split, staged in LDS, read back as 16-byte operand rows), X
// is the B operand (16-byte LDS rows), and each accumulator lane ends up
// holding 4 consecutive columns of one row of X M, which are stored as one
// 8-byte LDS write per half or one 16-byte global store.
constexpr int SB = 136;

// fp32 -> (hi, lo) bf16 operand pairs: hi = bf16(x), lo = bf16(x - hi)
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t& h, uint32_t& l) {
  h = pack_bf16(x0, x1);
  l = pack_bf16(x0 - bf16_lo(h), x1 - bf16_hi(h));
}

// A wave's share of the rows jr .. jr + 31 of a d_k x d_k fp32 matrix, loaded
// contiguously: NL 16-byte pieces per lane, piece i = row jr + (64 i + l) / W,
// channels c0 + 4 ((64 i + l) % W) .. + 3 with W = (channels per row) / 4 lanes
// per row (W = 32: whole 512-byte rows, two per instruction; W = 16: 256-byte
// half rows, four per instruction).  Addresses are clamped into the matrix;
// rows_split zeroes what lies outside.
template <int NL>
struct RowsF32 {
  f32x4_t v[NL];
};

template <int NL, int W>
__device__ __forceinline__ void rows_load(RowsF32<NL>& t, const float* M, int dk, int jr, int c0) {
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int e = 64 * i + lane;
    const int row = min(jr + e / W, dk - 1);
    const int col = min(c0 + 4 * (e % W), dk - 4);
    t.v[i] = *reinterpret_cast<const f32x4_t*>(M + (size_t)row * dk + col);
  }
}

// ... split into (hi, lo) LDS rows (row stride SB, row `row - rbase` of the
// region at mh / ml), zero outside the d_k x d_k matrix
template <int NL, int W>
__device__ __forceinline__ void rows_split(__bf16* mh, __bf16* ml, int rbase, const RowsF32<NL>& t,
                                           int dk, int jr, int c0) {
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int e = 64 * i + lane;
    const int row = jr + e / W;
    const int col = c0 + 4 * (e % W);
    const bool ok = row < dk && col < dk;
    uint32_t h0, l0, h1, l1;
    split_pair(ok ? t.v[i][0] : 0.0f, ok ? t.v[i][1] : 0.0f, h0, l0);
    split_pair(ok ? t.v[i][2] : 0.0f, ok ? t.v[i][3] : 0.0f, h1, l1);
    const int off = (row - rbase) * SB + col;
    *reinterpret_cast<u32x2_t*>(mh + off) = u32x2_t{h0, h1};
    *reinterpret_cast<u32x2_t*>(ml + off) = u32x2_t{l0, l1};
  }
}

// split_mm_t with the transition operand read from (hi, lo) LDS rows jr ..
template <int NX>
__device__ __forceinline__ void split_mm_t_lds(f32x16_t (&acc)[NX], const __bf16* mh,
                                               const __bf16* ml, int jr, const __bf16* xh,
                                               const __bf16* xl, int xr0, int nk) {
  const int lane = lane_id();
  const int mbase = (jr + (lane & 31)) * SB + 8 * (lane >> 5);
  const int base = (xr0 + (lane & 31)) * SB + 8 * (lane >> 5);
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    if (kk < nk) {
      const u32x4_t ah = *reinterpret_cast<const u32x4_t*>(mh + mbase + 16 * kk);
      const u32x4_t al = *reinterpret_cast<const u32x4_t*>(ml + mbase + 16 * kk);
#pragma unroll
      for (int x = 0; x < NX; ++x) {
        const int off = base + 32 * x * SB + 16 * kk;
        const u32x4_t bh = *reinterpret_cast<const u32x4_t*>(xh + off);
        const u32x4_t bl = *reinterpret_cast<const u32x4_t*>(xl + off);
        acc[x] = mfma_bf16(ah, bh, acc[x]);
        acc[x] = mfma_bf16(al, bh, acc[x]);
        acc[x] = mfma_bf16(ah, bl, acc[x]);
      }
    }
  }
}

// The accumulator's share of a row-major rows x d_k fp32 matrix in the
// transposed layout: b[x][q] = row xr0 + 32 x + l % 32, columns
// jr + 8 q + 4 (l / 32) .. + 3 (clamped; out_mask() says what is real).
template <int NX>
__device__ __forceinline__ void rows_prefetch_t(f32x4_t (&b)[NX][4], const float* src, int rows,
                                                int dk, int xr0, int jr) {
  const int lane = lane_id();
#pragma unroll
  for (int x = 0; x < NX; ++x) {
    const int row = min(xr0 + 32 * x + (lane & 31), rows - 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int col = min(jr + 8 * q + 4 * (lane >> 5), dk - 4);
      b[x][q] = *reinterpret_cast<const f32x4_t*>(src + (size_t)row * dk + col);
    }
  }
}

__device__ __forceinline__ bool out_ok(int rows, int dk, int xr0, int x, int jr, int q) {
  const int lane = lane_id();
  return xr0 + 32 * x + (lane & 31) < rows && jr + 8 * q + 4 * (lane >> 5) < dk;
}

// the 4 values of accumulator x, group q (+ b when given and real)
template <int NX>
__device__ __forceinline__ f32x4_t out_quad(const f32x16_t (&acc)[NX], int x, int q) {
  return f32x4_t{acc[x][4 * q], acc[x][4 * q + 1], acc[x][4 * q + 2], acc[x][4 * q + 3]};
}

__device__ __forceinline__ void x_store_quad(__bf16* xh, __bf16* xl, int row, int col, f32x4_t v) {
  uint32_t h0, l0, h1, l1;
  split_pair(v[0], v[1], h0, l0);
  split_pair(v[2], v[3], h1, l1);
  *reinterpret_cast<u32x2_t*>(xh + row * SB + col) = u32x2_t{h0, h1};
  *reinterpret_cast<u32x2_t*>(xl + row * SB + col) = u32x2_t{l0, l1};
}

// Row-major rows x d_k fp32 matrix (times scale) -> (hi, lo) LDS rows
// [0, pad32(rows)), zero padded; rows == 0 gives the identity (d_k x d_k), or
// Diag(diag) when diag is given.  By the first 256 threads of the workgroup.
__device__ __forceinline__ void x_fill(__bf16* xh, __bf16* xl, const float* src, int rows, int dk,
                                       float scale, const float* diag = nullptr) {
  const int t = threadIdx.x;
  if (t >= 256) return;
  const int R = pad32(rows == 0 ? dk : rows);
  MatRegs m;
  if (rows > 0) {
    mat_load(m, src, dk, rows, dk);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int id = t + 256 * i;
      const int r = id >> 5;
      const int c = (id & 31) << 2;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        m.v[i][e] = (r == c + e && r < dk) ? (diag ? diag[r] : 1.0f) : 0.0f;
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int id = t + 256 * i;
    const int r = id >> 5;
    const int c = (id & 31) << 2;
    if (r < R) x_store_quad(xh, xl, r, c, scale * m.v[i]);
  }
}

// The scan's transition operands, pre-split (bf16 features, d_k = 128).  A scan
// step multiplies a 32-row block of the state by a chunk transition T (the
// forward step by Mc, the reverse step by Mc^T), as the product T'[a][i] =
// sum_k op[a][k] X[i][k] with op = Mc^T (forward) or Mc (reverse).  Wave w of
// the scan owns rows a = 32 w .. + 31 of op and takes them as the A operand of
// v_mfma_f32_32x32x16_bf16: in k step kk lane l needs
// op[32 w + l % 32][16 kk + 8 (l / 32) .. + 7], hi and lo.  An image holds
// exactly these 16-byte pieces in that order, piece ((w * 8 + kk) * 2 + h) * 64
// + l (h = 0: hi, 1: lo), 64 KB per chunk, so each of the scan's loads reads 1 KB
// contiguously straight into the operand registers and no scan step splits
// anything.  Both images are written from split(Mc) in LDS (row stride SB):
// the reverse pieces are row pieces of Mc, the forward pieces column pieces.
constexpr int kImgPieces = 4096;  // 16-byte pieces per image

__device__ __forceinline__ void op_images(const __bf16* Xh, const __bf16* Xl,
                                          u32x4_t* __restrict__ imgF, u32x4_t* __restrict__ imgR) {
  static_assert(kImgPieces % 512 == 0, "512-thread workgroups");
#pragma unroll
  for (int p = threadIdx.x; p < kImgPieces; p += 512) {
    const int l = p & 63;
    const uint16_t* X = reinterpret_cast<const uint16_t*>(((p >> 6) & 1) ? Xl : Xh);
    const int a = 32 * (p >> 10) + (l & 31);
    const int k0 = 16 * ((p >> 7) & 7) + 8 * (l >> 5);
    imgR[p] = *reinterpret_cast<const u32x4_t*>(X + a * SB + k0);
    u32x4_t f;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      f[e] = (uint32_t)X[(k0 + 2 * e) * SB + a] | ((uint32_t)X[(k0 + 2 * e + 1) * SB + a] << 16);
    imgF[p] = f;
  }
}

// Forward transition chain and reverse injection of one chunk in one pass over
// its frames (bf16 features, alpha = 1, frame-wise rule, d_k = d_v = 128).
// Every M_t is symmetric, so the reverse injection
//   Jr = sum_t B_t M_t M_{t-1} ... M_{f0} = sum_t B_t X_t^T,
//   X_t = M_{f0} M_{f0+1} ... M_t   (the forward transition chain's prefix),
// and both come from one sweep over the chunk's frames in forward order, the
// order in which the chunk's Jf workgroup reads the same transitions (the two
// run side by side on one XCD, so the second read of each transition hits L2).
// Frame f0: X = M_{f0}, Jr = B_{f0} X^T.  Frame t > f0: X_t = X_{t-1} M_t (M_t
// in LDS as the A operand, X_{t-1} as B), then B_t is staged where M_t was and
// Jr += B_t X_t^T (X_t as the A operand, B_t as B; the product helper returns
// the tile in the layout of Jr's rows).  The next frame's transition and write
// are in flight while the current one is multiplied.  Writes Mc = X_{f1-1},
// Jr and the scan's two operand images of Mc (see op_images).
__device__ __forceinline__ void compose_mc_jr(__bf16* Xh, __bf16* Xl, __bf16* Mh, __bf16* Ml,
                                              const float* __restrict__ Mw,
                                              const float* __restrict__ Bw, float* __restrict__ Mc,
                                              u32x4_t* __restrict__ imgF,
                                              u32x4_t* __restrict__ imgR, float* __restrict__ Jr,
                                              int u, int c, int F, int C, int n) {
  constexpr int dk = 128;
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int jr = 32 * (w & 3);
  const int kh = w >> 2;
  const int xr0 = 64 * kh;
  const int f0 = c * C;
  const int f1 = min(f0 + C, F);
  const size_t Fp1 = (size_t)F + 1;
  auto Mp = [&](int f) { return Mw + ((size_t)u * Fp1 + f + 1) * dk * dk; };
  auto Bp = [&](int f) { return Bw + ((size_t)u * Fp1 + f + 1) * dk * dk; };
  const size_t tile = ((size_t)u * n + c) * dk * dk;
  RowsF32<8> mf, bf;  // this wave's share (rows jr .., columns 64 kh ..) of a transition, a write
  f32x16_t accj[2] = {zero16(), zero16()};
  f32x16_t accx[2] = {zero16(), zero16()};

  rows_load<8, 16>(bf, Bp(f0), dk, jr, 64 * kh);
  if (f0 + 1 < f1) rows_load<8, 16>(mf, Mp(f0 + 1), dk, jr, 64 * kh);
  x_fill(Xh, Xl, Mp(f0), dk, dk, 1.0f);  // X = M_{f0}
  rows_split<8, 16>(Mh, Ml, 0, bf, dk, jr, 64 * kh);
  __syncthreads();
  if (f0 + 1 < f1) rows_load<8, 16>(bf, Bp(f0 + 1), dk, jr, 64 * kh);
  split_mm_t_lds<2>(accj, Xh, Xl, jr, Mh, Ml, xr0, 8);  // Jr = B_{f0} X^T
  __syncthreads();
  for (int t = f0 + 1; t < f1; ++t) {
    const bool last = t == f1 - 1;
    rows_split<8, 16>(Mh, Ml, 0, mf, dk, jr, 64 * kh);  // M_t
    __syncthreads();
    if (!last) rows_load<8, 16>(mf, Mp(t + 1), dk, jr, 64 * kh);
    accx[0] = zero16();
    accx[1] = zero16();
    split_mm_t_lds<2>(accx, Mh, Ml, jr, Xh, Xl, xr0, 8);  // X_t = X_{t-1} M_t
    __syncthreads();  // every wave has read X_{t-1} and M_t
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        x_store_quad(Xh, Xl, xr0 + 32 * x + (lane & 31), jr + 8 * q + 4 * (lane >> 5),
                     out_quad(accx, x, q));
    rows_split<8, 16>(Mh, Ml, 0, bf, dk, jr, 64 * kh);  // B_t
    __syncthreads();
    if (!last) rows_load<8, 16>(bf, Bp(t + 1), dk, jr, 64 * kh);
    split_mm_t_lds<2>(accj, Xh, Xl, jr, Mh, Ml, xr0, 8);  // Jr += B_t X_t^T
    __syncthreads();  // every wave has read B_t
  }
  // Mc = X_{f1-1} (a one-frame chunk: M_{f0})
  if (f1 - f0 == 1) {
    const f32x4_t* src = reinterpret_cast<const f32x4_t*>(Mp(f0));
    for (int i = threadIdx.x; i < dk * dk / 4; i += blockDim.x)
      reinterpret_cast<f32x4_t*>(Mc + tile)[i] = src[i];
  }
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = xr0 + 32 * x + (lane & 31);
      const int col = jr + 8 * q + 4 * (lane >> 5);
      *reinterpret_cast<f32x4_t*>(Jr + tile + (size_t)row * dk + col) = out_quad(accj, x, q);
      if (f1 - f0 > 1)
        *reinterpret_cast<f32x4_t*>(Mc + tile + (size_t)row * dk + col) = out_quad(accx, x, q);
    }
  // the split X in LDS is split(Mc) (the last step stored it, every wave has
  // passed the loop's final barrier since)
  op_images(Xh, Xl, imgF + ((size_t)u * n + c) * kImgPieces, imgR + ((size_t)u * n + c) * kImgPieces);
}

// compose (bf16): one workgroup of 8 waves per work item; wave w owns output
// columns jr = 32 (w % 4) .. + 31 for X rows 64 (w / 4) .. + 63.  The two waves
// of a column block load one half each (contiguous 256-byte half rows) of the
// transition rows they share and stage them, split, in LDS.  Work items:
// (unit, chunk, chain) with the chain fastest (the chains of a chunk read the
// same transitions and share an XCD), then one text-seed item per unit.
// Chains: 0 Mc, 1 Jf, 2 Jr and, with decay (DECAY), 3 the reverse transition
// Mr = D_{f1-1} M_{f1-1} ... D_{f0} M_{f0}, which no longer equals Mc^T.  With
// decay each step enters the next frame as X <- (X M) Diag(alpha_next) + B_next
// and a transition chain starts from Diag(alpha) of its first frame.
// BATCHED (the frozen-state comparison rule, S -> S M + B with M = I - A):
// a write chain starts at X = B of its first frame and steps X <- X M_g + B_g
// over the others (the transition index runs one frame ahead of the write's);
// the seed and one-frame chunks are plain copies of B.
// MCJR (frame-wise rule, no decay, d_k = d_v = 128): two items per chunk, the
// forward transition chain with the reverse injection (compose_mc_jr, which
// also writes the scan's operand images of Mc into the McT and MrT regions)
// and Jf.
template <bool FULL, bool DECAY, bool BATCHED, bool MCJR = false>
__global__ __launch_bounds__(512, 1) void compose_split_kernel(
    const float* __restrict__ Bw, const float* __restrict__ Mw, const float* __restrict__ alpha,
    float* __restrict__ Mc, float* __restrict__ McT, float* __restrict__ MrT,
    float* __restrict__ Jf, float* __restrict__ Jr, float* __restrict__ ST, int dk, int dv, int F,
    int C, int n, int units, unsigned per, float seed_scale, int anchors) {
  __shared__ __align__(16) __bf16 Xh[128 * SB];
  __shared__ __align__(16) __bf16 Xl[128 * SB];
  __shared__ __align__(16) __bf16 Mh[128 * SB];
  __shared__ __align__(16) __bf16 Ml[128 * SB];
  constexpr unsigned nch = MCJR ? 2 : (DECAY ? 4 : 3);
  const unsigned item = xcd_item(per);
  const unsigned chain_items = (unsigned)units * n * nch;
  if (item >= chain_items + units) return;
  const bool seed = item >= chain_items;
  const int chain = seed ? 1 : item % nch;  // the seed runs as a forward B chain
  const int c = seed ? 0 : (item / nch) % n;
  const int u = seed ? item - chain_items : item / (nch * n);
  if (MCJR && chain == 0) {
    compose_mc_jr(Xh, Xl, Mh, Ml, Mw, Bw, Mc, reinterpret_cast<u32x4_t*>(McT),
                  reinterpret_cast<u32x4_t*>(MrT), Jr, u, c, F, C, n);
    return;
  }
  const bool mchain = !seed && (chain == 0 || chain == 3);
  const bool reverse = !seed && (chain == 2 || chain == 3);
  const int w = threadIdx.x >> 6;
  const int jr = 32 * (w & 3);
  const int kh = w >> 2;
  const int xr0 = 64 * kh;
  const int nk = FULL ? 8 : dk >> 4;
  // the seed is the text frame's map applied once: (0 + s B_T) M_T
  const int f0 = seed ? -1 : c * C;
  const int f1 = seed ? 0 : min(f0 + C, F);
  const int nf = f1 - f0;
  const int rows = mchain ? dk : dv;
  const size_t Fp1 = (size_t)F + 1;
  const size_t SS = (size_t)dv * dk;
  // workspace frame index f + 1 holds latent frame f (index 0 is the text frame)
  auto frame = [&](int s) { return reverse ? f1 - 1 - s : f0 + s; };
  auto Mp = [&](int f) { return Mw + ((size_t)u * Fp1 + f + 1) * dk * dk; };
  auto Bp = [&](int f) { return Bw + ((size_t)u * Fp1 + f + 1) * SS; };
  auto Ap = [&](int f) { return alpha + ((size_t)u * F + f) * dk; };
  // boundary anchors carry no gate (the identity)
  auto anchor = [&](int f) { return anchors && (f == 0 || f == F - 1); };
  const bool active = jr < dk && xr0 < rows;
  const int sh = BATCHED && !mchain ? 1 : 0;  // transition index offset of a write chain
  const int nsteps = nf - sh;

  const size_t tile = ((size_t)u * n + c) * dk * dk;
  float* dst = chain == 0 && !seed ? Mc + tile
               : seed              ? ST + (size_t)u * 2 * (n + 1) * SS  // P[0]
               : chain == 3        ? nullptr                            // MrT only
                                   : (chain == 1 ? Jf : Jr) + ((size_t)u * n + c) * SS;
  float* dst2 = seed ? ST + ((size_t)(u * 2 + 1) * (n + 1) + n) * SS  // R[n]
                     : (chain == 3 ? MrT : McT) + tile;
  if (BATCHED && nsteps == 0) {  // the chain is its first frame's write
    const float scale = seed ? seed_scale : 1.0f;
    const f32x4_t* src = reinterpret_cast<const f32x4_t*>(Bp(frame(0)));
    for (int i = threadIdx.x; i < (int)(SS / 4); i += blockDim.x) {
      const f32x4_t v = src[i] * scale;
      reinterpret_cast<f32x4_t*>(dst)[i] = v;
      if (seed) reinterpret_cast<f32x4_t*>(dst2)[i] = v;
    }
    return;
  }

  RowsF32<8> mf;
  rows_load<8, 16>(mf, Mp(frame(sh)), dk, jr, 64 * kh);
  x_fill(Xh, Xl, mchain ? nullptr : Bp(frame(0)), mchain ? 0 : dv, dk, seed ? seed_scale : 1.0f,
         DECAY && mchain && !anchor(frame(0)) ? Ap(frame(0)) : nullptr);
  rows_split<8, 16>(Mh, Ml, 0, mf, dk, jr, 64 * kh);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  f32x4_t bq[2][4];
  f32x4_t aq[4];
  for (int s = 0; s < nsteps; ++s) {
    const bool last = s == nsteps - 1;
    if (BATCHED && last && !mchain) rows_prefetch_t<2>(bq, Bp(frame(s + 1)), dv, dk, xr0, jr);
    if (!last) {  // the next frame's transition and write fly while this step multiplies
      rows_load<8, 16>(mf, Mp(frame(s + 1 + sh)), dk, jr, 64 * kh);
      if (!mchain) rows_prefetch_t<2>(bq, Bp(frame(s + 1)), dv, dk, xr0, jr);
      if (DECAY) {
        const bool one = anchor(frame(s + 1));
#pragma unroll
        for (int q = 0; q < 4; ++q)
          aq[q] = one ? f32x4_t{1.0f, 1.0f, 1.0f, 1.0f}
                      : *reinterpret_cast<const f32x4_t*>(
                            Ap(frame(s + 1)) + min(jr + 8 * q + 4 * (lane >> 5), dk - 4));
      }
    }
    f32x16_t acc[2] = {zero16(), zero16()};
    if (active) split_mm_t_lds<2>(acc, Mh, Ml, jr, Xh, Xl, xr0, nk);
    __syncthreads();  // every wave has read X and M
    if (last) {
      if (active) {
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (!out_ok(rows, dk, xr0, x, jr, q)) continue;
            const int row = xr0 + 32 * x + (lane & 31);
            const int col = jr + 8 * q + 4 * (lane >> 5);
            f32x4_t v = out_quad(acc, x, q);
            if (BATCHED && !mchain) v += bq[x][q];
            if (!DECAY || chain != 3 || seed)
              *reinterpret_cast<f32x4_t*>(dst + (size_t)row * dk + col) = v;
            if (seed) {
              *reinterpret_cast<f32x4_t*>(dst2 + (size_t)row * dk + col) = v;
            } else if (mchain) {  // Mc^T, or Mr^T
#pragma unroll
              for (int e = 0; e < 4; ++e) dst2[(size_t)(col + e) * dk + row] = v[e];
            }
          }
      }
      break;
    }
    if (active) {
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f32x4_t v = out_quad(acc, x, q);
          if (DECAY) v *= aq[q];
          if (!mchain && out_ok(rows, dk, xr0, x, jr, q)) v += bq[x][q];
          x_store_quad(Xh, Xl, xr0 + 32 * x + (lane & 31), jr + 8 * q + 4 * (lane >> 5), v);
        }
    }
    rows_split<8, 16>(Mh, Ml, 0, mf, dk, jr, 64 * kh);
    __syncthreads();
  }
}

// scan (bf16): one workgroup per (32-row block of the state, unit, direction);
// wave w owns state columns 32 w .. + 31, i.e. transition rows 32 w .. + 31,
// which it loads contiguously (whole 512-byte rows) one chunk ahead and stages,
// split, in its own LDS region.  The transition operand of the forward step
// S Mc is read from the rows of Mc^T, that of the reverse step S Mc^T from the
// rows of Mc.  The next chunk's loads are unconditional (the last step
// refetches its own chunk) and the injections alternate between two register
// sets, so that no wait for a load also waits for the state stores issued
// after it.  FULL: d_k = 128 and d_v a multiple of 32 (no masking anywhere).
template <bool FULL>
__global__ __launch_bounds__(256) void scan_split_kernel(const float* __restrict__ McR,
                                                         const float* __restrict__ McTr,
                                                         const float* __restrict__ Jf,
                                                         const float* __restrict__ Jr,
                                                         float* __restrict__ ST, int dk, int dv,
                                                         int n, int units, unsigned per) {
  __shared__ __align__(16) __bf16 Xh[32 * SB];
  __shared__ __align__(16) __bf16 Xl[32 * SB];
  __shared__ __align__(16) __bf16 Mh[128 * SB];
  __shared__ __align__(16) __bf16 Ml[128 * SB];
  // work item (unit, direction, row block), row block fastest: the row blocks of
  // one chain read the same transitions every step and share an XCD (its L2)
  const int nrb = (dv + 31) >> 5;
  const unsigned item = xcd_item(per);
  if (item >= (unsigned)units * 2 * nrb) return;
  const int rb = item % nrb;  // rows [32 rb, 32 rb + 32) of the state
  const int u = (item / nrb) % units;
  const int dir = item / (nrb * units);  // 0: forward (P), 1: reverse (R)
  const int lane = threadIdx.x & 63;
  const int jr = 32 * (threadIdx.x >> 6);
  const int nk = FULL ? 8 : dk >> 4;
  const size_t SS = (size_t)dv * dk;
  float* S = ST + (size_t)(u * 2 + dir) * (n + 1) * SS;
  const int r0 = 32 * rb;
  const int nrows = FULL ? 32 : min(32, dv - r0);
  auto chunk = [&](int s) { return dir == 0 ? s : n - 1 - s; };
  const float* Jb = (dir == 0 ? Jf : Jr) + (size_t)u * n * SS + (size_t)r0 * dk;
  const float* Mb = (dir == 0 ? McTr : McR) + (size_t)u * n * dk * dk;
  const bool active = FULL || jr < dk;

  RowsF32<16> mf;
  f32x4_t ja[1][4], jb[1][4];
  rows_load<16, 32>(mf, Mb + (size_t)chunk(0) * dk * dk, dk, jr, 0);
  rows_prefetch_t<1>(ja, Jb + (size_t)chunk(0) * SS, nrows, dk, 0, jr);
  x_fill(Xh, Xl, S + (size_t)(dir == 0 ? 0 : n) * SS + (size_t)r0 * dk, nrows, dk, 1.0f);
  rows_split<16, 32>(Mh, Ml, 0, mf, dk, jr, 0);
  __syncthreads();

  // one chunk: X <- X Mc_j + J_j using jcur, fetching chunk s + 1 into jnext
  auto step = [&](int s, f32x4_t (&jcur)[1][4], f32x4_t (&jnext)[1][4]) {
    const int j = chunk(s);
    const int sn = min(s + 1, n - 1);
    rows_load<16, 32>(mf, Mb + (size_t)chunk(sn) * dk * dk, dk, jr, 0);
    rows_prefetch_t<1>(jnext, Jb + (size_t)chunk(sn) * SS, nrows, dk, 0, jr);
    f32x16_t acc[1] = {zero16()};
    if (active) split_mm_t_lds<1>(acc, Mh, Ml, jr, Xh, Xl, 0, nk);
    __syncthreads();  // every wave has read X
    if (active) {
      float* dstp = S + (size_t)(dir == 0 ? j + 1 : j) * SS + (size_t)r0 * dk;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = lane & 31;
        const int col = jr + 8 * q + 4 * (lane >> 5);
        const bool ok = FULL || out_ok(nrows, dk, 0, 0, jr, q);
        f32x4_t v = out_quad(acc, 0, q);
        if (ok) v += jcur[0][q];
        if (FULL || ok) *reinterpret_cast<f32x4_t*>(dstp + (size_t)row * dk + col) = v;
        x_store_quad(Xh, Xl, row, col, v);
      }
    }
    // this wave's transition rows: its own MFMA reads of them are done
    rows_split<16, 32>(Mh, Ml, 0, mf, dk, jr, 0);
    __syncthreads();
  };
  int s = 0;
  for (; s + 1 < n; s += 2) {
    step(s, ja, jb);
    step(s + 1, jb, ja);
  }
  if (s < n) step(s, ja, jb);
}

// scan (bf16, d_k = 128, d_v a multiple of 32) on the composition's operand
// images: one workgroup per (32-row block of the state, unit, direction), row
// blocks of one chain consecutive on one XCD as above.  Wave w owns state
// columns 32 w .. + 31; its A operands for a chunk are 16 registers of 16 bytes
// loaded from the image (1 KB contiguous per instruction), NS - 1 chunks ahead
// in a ring of NS register sets, the injections likewise; the state block is
// the B operand, split in LDS.  A step: 24 MFMAs, a barrier, the new state
// (injection added) stored and split into LDS, a barrier.  The products and
// their order are those of scan_split_kernel, so the states are bitwise the same.
template <int NS>
__global__ __launch_bounds__(256) void scan_img_kernel(const u32x4_t* __restrict__ imgF,
                                                       const u32x4_t* __restrict__ imgR,
                                                       const float* __restrict__ Jf,
                                                       const float* __restrict__ Jr,
                                                       float* __restrict__ ST, int dv, int n,
                                                       int units, unsigned per) {
  constexpr int dk = 128;
  __shared__ __align__(16) __bf16 Xh[32 * SB];
  __shared__ __align__(16) __bf16 Xl[32 * SB];
  const int nrb = dv >> 5;
  const unsigned item = xcd_item(per);
  if (item >= (unsigned)units * 2 * nrb) return;
  const int rb = item % nrb;
  const int u = (item / nrb) % units;
  const int dir = item / (nrb * units);  // 0: forward (P), 1: reverse (R)
  const int lane = threadIdx.x & 63;
  const int jr = 32 * (threadIdx.x >> 6);
  const size_t SS = (size_t)dv * dk;
  float* S = ST + (size_t)(u * 2 + dir) * (n + 1) * SS;
  const int r0 = 32 * rb;
  auto chunk = [&](int s) { return dir == 0 ? s : n - 1 - s; };
  const float* Jb = (dir == 0 ? Jf : Jr) + (size_t)u * n * SS + (size_t)r0 * dk;
  const u32x4_t* Ib = (dir == 0 ? imgF : imgR) + (size_t)u * n * kImgPieces +
                      16 * (threadIdx.x & ~63) + lane;
  auto load = [&](u32x4_t (&a)[16], f32x4_t (&j)[1][4], int s) {
    const u32x4_t* src = Ib + (size_t)chunk(s) * kImgPieces;
#pragma unroll
    for (int i = 0; i < 16; ++i) a[i] = src[64 * i];
    rows_prefetch_t<1>(j, Jb + (size_t)chunk(s) * SS, 32, dk, 0, jr);
  };

  u32x4_t A[NS][16];
  f32x4_t J[NS][1][4];
#pragma unroll
  for (int i = 0; i + 1 < NS; ++i) load(A[i], J[i], min(i, n - 1));
  x_fill(Xh, Xl, S + (size_t)(dir == 0 ? 0 : n) * SS + (size_t)r0 * dk, 32, dk, 1.0f);
  __syncthreads();

  const int xb = (lane & 31) * SB + 8 * (lane >> 5);
  for (int s0 = 0; s0 < n; s0 += NS) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int s = s0 + i;
      if (s >= n) break;
      // chunk s + NS - 1 (clamped: the last steps refetch the last chunk)
      load(A[(i + NS - 1) % NS], J[(i + NS - 1) % NS], min(s + NS - 1, n - 1));
      // every B operand is read before the MFMA chain, so the 24 dependent
      // MFMAs issue back to back instead of each waiting for its LDS read
      u32x4_t bh[8], bl[8];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        bh[kk] = *reinterpret_cast<const u32x4_t*>(Xh + xb + 16 * kk);
        bl[kk] = *reinterpret_cast<const u32x4_t*>(Xl + xb + 16 * kk);
      }
      __builtin_amdgcn_sched_barrier(0);
      f32x16_t acc = zero16();
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        acc = mfma_bf16(A[i][2 * kk], bh[kk], acc);
        acc = mfma_bf16(A[i][2 * kk + 1], bh[kk], acc);
        acc = mfma_bf16(A[i][2 * kk], bl[kk], acc);
      }
      __syncthreads();  // every wave has read X
      float* dstp = S + (size_t)(dir == 0 ? chunk(s) + 1 : chunk(s)) * SS + (size_t)r0 * dk;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = lane & 31;
        const int col = jr + 8 * q + 4 * (lane >> 5);
        const f32x4_t v = f32x4_t{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]} +
                          J[i][0][q];
        *reinterpret_cast<f32x4_t*>(dstp + (size_t)row * dk + col) = v;
        x_store_quad(Xh, Xl, row, col, v);
      }
      __syncthreads();
    }
  }
}

}  // namespace

// bf16 products, frame-wise rule, no decay, d_k = d_v = 128: the composition
// runs as compose_mc_jr items plus Jf items and leaves the scan's operand
// images (op_images) in the McT (forward) and MrT (reverse) regions, which the
// scan reads with scan_img_kernel
static bool mcjr_path(const Plan& p, bool decay) {
  return !p.fp32_products && p.rule == 0 && !decay && p.dk == 128 && p.dv == 128;
}
constexpr int kScanRing = 3;  // register sets of the image scan (loads kScanRing - 1 chunks ahead)

template <bool FULL, bool DECAY, bool BATCHED = false, bool MCJR = false>
void launch_compose_split(const Plan& p, const WsPtrs& w, const float* alpha, float seed_scale,
                          hipStream_t s) {
  const unsigned per = xcd_per((unsigned)p.units * (p.n * (MCJR ? 2 : DECAY ? 4 : 3) + 1));
  hipLaunchKernelGGL((compose_split_kernel<FULL, DECAY, BATCHED, MCJR>), dim3(kXcds * per), dim3(512),
                     0, s, w.B,
                     w.M, alpha, w.Mc, w.McT, w.MrT, w.Jf, w.Jr, w.ST, p.dk, p.dv, p.F, p.C, p.n,
                     p.units, per, seed_scale, p.anchors);
}

hipError_t launch_compose(const Plan& p, const WsPtrs& w, const float* alpha, hipStream_t s) {
  const float seed_scale = p.seed_mode == 1 ? 1.0f : 0.5f;
  if (!p.fp32_products) {
    if (p.rule != 0)  // the batched comparison rules (no decay)
      p.dk == 128 ? launch_compose_split<true, false, true>(p, w, nullptr, seed_scale, s)
                  : launch_compose_split<false, false, true>(p, w, nullptr, seed_scale, s);
    else if (mcjr_path(p, alpha != nullptr))
      launch_compose_split<true, false, false, true>(p, w, alpha, seed_scale, s);
    else if (p.dk == 128)
      alpha ? launch_compose_split<true, true>(p, w, alpha, seed_scale, s)
            : launch_compose_split<true, false>(p, w, alpha, seed_scale, s);
    else
      alpha ? launch_compose_split<false, true>(p, w, alpha, seed_scale, s)
            : launch_compose_split<false, false>(p, w, alpha, seed_scale, s);
  } else {
    hipLaunchKernelGGL(compose_kernel, dim3(p.n, p.units, alpha ? 5 : 4), dim3(kThreads), 0, s,
                       w.B, w.M, alpha, w.Mc, w.McT, w.MrT, w.Jf, w.Jr, w.ST, p.dk, p.dv, p.F, p.C,
                       p.n, seed_scale, p.anchors, p.rule != 0 ? 1 : 0);
  }
  return hipGetLastError();
}

// The reverse step reads the rows of the reverse transition's transpose: Mc
// itself without decay (Mr = Mc^T), the stored Mr^T with it.
hipError_t launch_scan(const Plan& p, const WsPtrs& w, bool decay, hipStream_t s) {
  const dim3 grid(pad32(p.dv) >> 5, p.units, 2);
  const float* rev = decay ? w.MrT : w.Mc;
  if (mcjr_path(p, decay)) {  // the composition left the operand images in McT and MrT
    const unsigned per = xcd_per((unsigned)(p.dv >> 5) * p.units * 2);
    hipLaunchKernelGGL(scan_img_kernel<kScanRing>, dim3(kXcds * per), dim3(kThreads), 0, s,
                       reinterpret_cast<const u32x4_t*>(w.McT), reinterpret_cast<const u32x4_t*>(w.MrT),
                       w.Jf, w.Jr, w.ST, p.dv, p.n, p.units, per);
  } else if (!p.fp32_products) {
    const unsigned per = xcd_per((unsigned)(pad32(p.dv) >> 5) * p.units * 2);
    if (p.dk == 128 && p.dv % 32 == 0)
      hipLaunchKernelGGL(scan_split_kernel<true>, dim3(kXcds * per), dim3(kThreads), 0, s, rev,
                         w.McT, w.Jf, w.Jr, w.ST, p.dk, p.dv, p.n, p.units, per);
    else
      hipLaunchKernelGGL(scan_split_kernel<false>, dim3(kXcds * per), dim3(kThreads), 0, s, rev,
                         w.McT, w.Jf, w.Jr, w.ST, p.dk, p.dv, p.n, p.units, per);
  } else {
    hipLaunchKernelGGL(scan_kernel, grid, dim3(kThreads), 0, s, w.Mc, rev, w.Jf, w.Jr, w.ST, p.dk,
                       p.dv, p.n);
  }
  return hipGetLastError();
}

}  // namespace vda
