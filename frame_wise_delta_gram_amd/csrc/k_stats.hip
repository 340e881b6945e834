// Frame statistics of Video Delta Attention ("Video DeltaNet", arXiv 2609.20744,
// Sec. 3.1 Eq. (3b)):
//   A_t = K_t^T Diag(beta_t) K_t,   B_t = V_t^T Diag(beta_t) K_t
// for every (unit, frame), with the text tokens as a leading virtual frame
// (Sec. 5, "Chunk-wise scans").  Both statistics come from ONE contraction
// over the frame's tokens,
//   [A_t ; B_t] = [X_t | Y_t]^T X_t,   X_t = Diag(sqrt(beta_t)) K_t,
//                                      Y_t = Diag(sqrt(beta_t)) V_t,
// so every K/V byte is read from HBM once ("in one pass, sharing input reads
// and reduction work", Sec. 5).  Splitting beta as sqrt(beta) * sqrt(beta)
// makes the computed A = X^T X positive semidefinite by construction even
// after X is rounded to bf16, so I + A stays SPD with every eigenvalue >= 1
// and ||(I + A)^{-1}||_2 <= 1 (Prop. 1) holds for the computed transition too.
//
// bf16 path: one workgroup (8 waves) per (unit, frame); wave w owns output
// row tile w of [A; B].  Tokens stream in tiles of 128.  Each thread loads a
// 4-token x 8-channel block of K and of V (16-byte coalesced loads: one wave
// instruction covers four whole 256-byte rows), scales it by sqrt(beta) in fp32, rounds to bf16 and packs it in
// channel-major order (the transposition happens in the packing), and writes
// the two channel-major tiles to LDS with an XOR swizzle that keeps both the
// 8-byte staging writes and the 16-byte MFMA operand reads free of bank
// conflicts.  X serves as both MFMA operands of the A block.  The contraction runs on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulators held for the whole frame.
// Per tile there is one barrier: the next tile is staged into the other LDS
// stage channel by channel between the k-steps of the current tile's
// products (vector ALU work overlapping the MFMAs), and the global loads of
// the tile after that are in flight meanwhile (two register sets).
//
// fp32 path: the same contraction in fp32 on the vector ALUs (exact fp32
// products, fp32 accumulation) for fp32 features.
#include "vda_device.h"
#include "vda_internal.h"

namespace vda {
namespace {

constexpr int kTok = 128;                 // tokens per tile
constexpr int kStatsThreads = 512;        // 8 waves
constexpr int kRowBytes = kTok * 2;       // one LDS row: 128 bf16 tokens of one channel
constexpr int kXRows = 256;               // sqrt(beta) K channels in rows [0,128), sqrt(beta) V in [128,256)
constexpr int kStageBytes = kXRows * kRowBytes;  // 32 KiB

// Swizzle of a channel row: XOR (< 16) applied to the 16-byte chunk index (a
// row is 256 bytes = 16 chunks, so rows alias in banks).  Rows r..r+15 (r a
// multiple of 16) get 16 distinct values: the 16 lanes of an MFMA operand read
// that the LDS serves together hit 16 different chunks.  Rows 8c+x for 16
// consecutive c get 16 distinct values: the 32 lanes of a staging write (two
// 8-byte slots per chunk) hit 32 different slots.  Any 8 consecutive rows also
// get distinct low 3 bits, so the pattern stays conflict-free when the LDS
// serves 8 lanes of 16 bytes or 16 lanes of 8 bytes per pass.
__device__ __forceinline__ uint32_t swz(uint32_t row) { return (row & 15) ^ ((row >> 3) & 15); }
// byte offset of the 8-byte slot `slot` (tokens 4*slot..4*slot+3) of `row`
__device__ __forceinline__ uint32_t off8(uint32_t row, uint32_t slot) {
  return row * kRowBytes + ((slot ^ (swz(row) << 1)) << 3);
}
// byte offset of the 16-byte chunk `j` (tokens 8*j..8*j+7) of `row`
__device__ __forceinline__ uint32_t off16(uint32_t row, uint32_t j) {
  return row * kRowBytes + ((j ^ swz(row)) << 4);
}

// DK, DV > 0: compile-time d_k and d_v (the common 128 case); 0: runtime.
template <int DK, int DV>
__global__ __launch_bounds__(512, 1) void stats_bf16_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const float* __restrict__ beta,
    const uint16_t* __restrict__ tk, const uint16_t* __restrict__ tv,
    const float* __restrict__ tb, float* __restrict__ Aout, float* __restrict__ Bout, int F, int U,
    int T, int dk_rt, int dv_rt, float text_scale) {
  const int dk = DK > 0 ? DK : dk_rt;
  const int dv = DV > 0 ? DV : dv_rt;
  __shared__ __align__(16) unsigned char smem[2 * kStageBytes];

  const int fi = blockIdx.x;  // 0 = text frame, f + 1 = latent frame f
  const int u = blockIdx.y;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;

  const uint16_t* sk;
  const uint16_t* sv;
  const float* sb;
  int ntok;
  float bscale;
  if (fi == 0) {
    sk = tk + (size_t)u * T * dk;
    sv = tv + (size_t)u * T * dv;
    sb = tb + (size_t)u * T;
    ntok = T;
    bscale = text_scale;
  } else {
    const size_t fr = (size_t)u * F + (fi - 1);
    sk = k + fr * U * dk;
    sv = v + fr * U * dv;
    sb = beta + fr * U;
    ntok = U;
    bscale = 1.0f;
  }

  // staging role: token group tg (4 tokens) x channel group cg (8 channels)
  const int tg = (t & 1) | ((t >> 5) << 1);
  const int cg = (t >> 1) & 15;
  const bool kact = cg * 8 < dk;
  const bool vact = cg * 8 < dv;

  // one tile's worth of this thread's raw inputs (16-byte bf16 vectors).  The
  // loads are unconditional from always valid addresses and nothing uses their
  // values until the tile is staged: vmcnt retires in issue order, so a tile's
  // loads stay in flight behind later work.  Tokens past the frame's end get
  // write strength 0 when staged.
  struct TileRegs {
    u32x4_t k[4], v[4];
    float b[4];  // beta of the 4 tokens
  };
  const int kcg = kact ? cg : 0;
  const int vcg = vact ? cg : 0;
  const int last_tok = ntok > 0 ? ntok - 1 : 0;
  // element offsets of the thread's 4 tokens within a tile (full tiles)
  const uint32_t koff = (uint32_t)(4 * tg) * dk + 8 * kcg;
  const uint32_t voff = (uint32_t)(4 * tg) * dv + 8 * vcg;

  // a tile that lies wholly inside the frame: uniform base, per-thread offsets
  auto load_full = [&](TileRegs& r, int tile) {
    const int tok0 = tile * kTok;
    const uint16_t* bk = sk + (size_t)tok0 * dk + koff;
    const uint16_t* bv = sv + (size_t)tok0 * dv + voff;
    const float* bb = sb + tok0 + 4 * tg;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      r.k[s] = ld_stream(bk + s * dk);
      r.v[s] = ld_stream(bv + s * dv);
      r.b[s] = bb[s];
    }
  };
  // any tile: token indices clamped to the frame's last token
  auto load = [&](TileRegs& r, int tile) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int tok = min(tile * kTok + 4 * tg + s, last_tok);
      r.k[s] = ld_stream(sk + (size_t)tok * dk + 8 * kcg);
      r.v[s] = ld_stream(sv + (size_t)tok * dv + 8 * vcg);
      r.b[s] = sb[tok];
    }
  };

  // sqrt(beta) of the thread's 4 tokens of tile `tile` (0 past the end)
  auto sqrt_beta = [&](const TileRegs& r, int tile, float (&sb4)[4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      sb4[s] = tile * kTok + 4 * tg + s < ntok ? __builtin_amdgcn_sqrtf(r.b[s] * bscale) : 0.0f;
  };

  // channel c of the thread's 8-channel group, tokens 0..3: scale, round, pack
  auto scaled_pair = [&](const u32x4_t* x4, const float* b, int c) {
    const int p = c >> 1;
    const bool hi = (c & 1) != 0;
    float x[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) x[s] = (hi ? bf16_hi(x4[s][p]) : bf16_lo(x4[s][p])) * b[s];
    // b[s] is 0 for tokens past the end; their registers hold a copy of the
    // frame's last token, so the product is exactly 0 (a non-finite input there
    // would already make the frame's statistics non-finite)
    u32x2_t e;
    e[0] = pack_bf16(x[0], x[1]);
    e[1] = pack_bf16(x[2], x[3]);
    return e;
  };

  // staging write offsets: channel row 8 cg + c, slot tg.  With
  // Q = swz(8 cg + c) ^ c = (8 (cg & 1)) ^ cg (independent of c),
  // off8(8 cg + c, tg) = ((2048 cg) | (8 tg ^ 16 Q)) ^ (16 c) + 256 c; V rows
  // 128 + 8 cg + c have the same swizzle, 32 KiB further.
  const uint32_t wbase = (uint32_t)(2048 * cg) | ((8u * tg) ^ (16u * ((8u * (cg & 1)) ^ cg)));
  auto write_channel = [&](const TileRegs& r, const float (&sb4)[4], int stage, int c) {
    unsigned char* X = smem + stage * kStageBytes + 256 * c;
    const uint32_t o = wbase ^ (16u * c);
    if (kact) *reinterpret_cast<u32x2_t*>(X + o) = scaled_pair(r.k, sb4, c);
    if (vact) *reinterpret_cast<u32x2_t*>(X + o + 128 * kRowBytes) = scaled_pair(r.v, sb4, c);
  };
  auto write_all = [&](const TileRegs& r, int tile, int stage) {
    float sb4[4];
    sqrt_beta(r, tile, sb4);
#pragma unroll
    for (int c = 0; c < 8; ++c) write_channel(r, sb4, stage, c);
  };

  // contraction role: wave w owns output row tile w of [A; B]
  const int nK = pad32(dk) >> 5;
  const int nV = pad32(dv) >> 5;
  const int nR = nK + nV;
  const bool ract = w < nR;
  const int rbase = w < nK ? 32 * w : 128 + 32 * (w - nK);
  f32x16_t acc[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) acc[ct] = zero16();

  // operand offsets: off16(row, j) with j = 2 kk + kh equals
  // (row * 256 + ((16 kh) ^ (swz(row) << 4))) ^ (32 kk)
  const int il = lane & 31;
  const int kh = lane >> 5;
  auto opbase = [&](int row) {
    return (uint32_t)row * kRowBytes + ((16u * kh) ^ (swz(row) << 4));
  };
  const uint32_t abase = opbase(rbase + il);
  uint32_t bbase[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) bbase[ct] = opbase(32 * ct + il);

  // Multiply the tile in `cstage` (8 k-steps of 16 tokens, operands fetched
  // one k-step ahead) and, interleaved with it, stage channel c = kk of the
  // register set `r` (tile `wtile`) into `wstage`.
  auto compute_write = [&](int cstage, bool do_write, const TileRegs& r, int wtile, int wstage) {
    const unsigned char* X = smem + cstage * kStageBytes;
    float sb4[4];
    if (do_write) sqrt_beta(r, wtile, sb4);
    u32x4_t a0, b0[4];
    auto fetch = [&](int kk, u32x4_t& a, u32x4_t (&b)[4]) {
      a = *reinterpret_cast<const u32x4_t*>(X + (abase ^ (32u * kk)));
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        if (ct < nK) b[ct] = *reinterpret_cast<const u32x4_t*>(X + (bbase[ct] ^ (32u * kk)));
    };
    if (ract) fetch(0, a0, b0);
#pragma unroll
    for (int kk = 0; kk < kTok / 16; ++kk) {
      u32x4_t a1, b1[4];
      if (ract && kk + 1 < kTok / 16) fetch(kk + 1, a1, b1);
      if (ract) {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
          if (ct < nK) acc[ct] = mfma_bf16(a0, b0[ct], acc[ct]);
      }
      if (do_write) write_channel(r, sb4, wstage, kk);
      a0 = a1;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) b0[ct] = b1[ct];
    }
  };

  // Stage (it & 1) holds tile it.  Each tile: one barrier, then tile it + 2's
  // loads are issued into the register set tile it came from, and tile it is
  // multiplied while tile it + 1 (loaded one tile earlier) is staged into the
  // other stage.  The steady-state loop only meets full tiles and always
  // stages, so every register set's loads are consumed on every path (no
  // conservative waits before reloading a set); the generic loop finishes the
  // frame.
  const int ntiles = (ntok + kTok - 1) / kTok;
  TileRegs ra, rb;
  if (ntiles > 0) load(ra, 0);
  if (ntiles > 1) load(rb, 1);
  if (ntiles > 0) write_all(ra, 0, 0);
  int it = 0;
  for (; (it + 4) * kTok <= ntok; it += 2) {  // tiles it + 2, it + 3 are full
    __syncthreads();
    load_full(ra, it + 2);
    compute_write(0, true, rb, it + 1, 1);
    __syncthreads();
    load_full(rb, it + 3);
    compute_write(1, true, ra, it + 2, 0);
  }
  for (; it < ntiles; it += 2) {
    __syncthreads();
    if (it + 2 < ntiles) load(ra, it + 2);
    compute_write(0, it + 1 < ntiles, rb, it + 1, 1);
    if (it + 1 >= ntiles) break;
    __syncthreads();
    if (it + 3 < ntiles) load(rb, it + 3);
    compute_write(1, it + 2 < ntiles, ra, it + 2, 0);
  }

  // results: rows of A (K tiles) or B (V tiles), columns are key channels
  if (ract) {
    const size_t fr = (size_t)u * (F + 1) + fi;
    const bool isA = w < nK;
    const int ch0 = isA ? 32 * w : 32 * (w - nK);
    const int nrows = isA ? dk : dv;
    float* dst = isA ? Aout + fr * dk * dk : Bout + fr * dv * dk;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      if (ct >= nK) continue;
      const int col = 32 * ct + (lane & 31);
      if (col >= dk) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = ch0 + acc_row(r, lane);
        if (row < nrows) dst[(size_t)row * dk + col] = acc[ct][r];
      }
    }
  }
}

// fp32 features: the same contraction, [sqrt(b) K | sqrt(b) V]^T (sqrt(b) K), on
// the vector ALUs.
constexpr int kTokF = 32;
constexpr int kXS = 257;  // LDS row stride (floats) of the token tile [K | V]
constexpr int kBS = 129;

__global__ __launch_bounds__(256) void stats_f32_kernel(
    const float* __restrict__ k, const float* __restrict__ v, const float* __restrict__ beta,
    const float* __restrict__ tk, const float* __restrict__ tv, const float* __restrict__ tb,
    float* __restrict__ Aout, float* __restrict__ Bout, int F, int U, int T, int dk, int dv,
    float text_scale) {
  __shared__ float Xs[kTokF * kXS];
  __shared__ float Bs[kTokF * kBS];

  const int fi = blockIdx.x;
  const int u = blockIdx.y;
  const int t = threadIdx.x;
  const float* sk;
  const float* sv;
  const float* sb;
  int ntok;
  float bscale;
  if (fi == 0) {
    sk = tk + (size_t)u * T * dk;
    sv = tv + (size_t)u * T * dv;
    sb = tb + (size_t)u * T;
    ntok = T;
    bscale = text_scale;
  } else {
    const size_t fr = (size_t)u * F + (fi - 1);
    sk = k + fr * U * dk;
    sv = v + fr * U * dv;
    sb = beta + fr * U;
    ntok = U;
    bscale = 1.0f;
  }
  // thread t accumulates rows 16*(t/16) .. +15 of [K | V] channels x key columns 8*(t%16) .. +7
  const int rb = t >> 4;
  const int cb = t & 15;
  float acc[16][8];
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;

  for (int base = 0; base < ntok; base += kTokF) {
    for (int idx = t; idx < kTokF * 128; idx += 256) {
      const int s = idx >> 7;
      const int ch = idx & 127;
      const int tok = base + s;
      const bool ok = tok < ntok;
      const float rb_ = ok ? sqrtf(sb[tok] * bscale) : 0.0f;
      const float kv = (ok && ch < dk) ? sk[(size_t)tok * dk + ch] * rb_ : 0.0f;
      const float vv = (ok && ch < dv) ? sv[(size_t)tok * dv + ch] * rb_ : 0.0f;
      Xs[s * kXS + ch] = kv;
      Xs[s * kXS + 128 + ch] = vv;
      Bs[s * kBS + ch] = kv;
    }
    __syncthreads();
    for (int s = 0; s < kTokF; ++s) {
      float xv[16], bv[8];
#pragma unroll
      for (int i = 0; i < 16; ++i) xv[i] = Xs[s * kXS + 16 * rb + i];
#pragma unroll
      for (int j = 0; j < 8; ++j) bv[j] = Bs[s * kBS + 8 * cb + j];
#pragma unroll
      for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(xv[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
  const size_t fr = (size_t)u * (F + 1) + fi;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = 16 * rb + i;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int col = 8 * cb + j;
      if (col >= dk) continue;
      if (row < 128) {
        if (row < dk) Aout[fr * dk * dk + (size_t)row * dk + col] = acc[i][j];
      } else if (row - 128 < dv) {
        Bout[fr * dv * dk + (size_t)(row - 128) * dk + col] = acc[i][j];
      }
    }
  }
}

}  // namespace

hipError_t launch_stats(const Plan& p, const void* k, const void* v, const float* beta,
                        const void* text_k, const void* text_v, const float* text_beta,
                        const WsPtrs& w, hipStream_t s) {
  const dim3 grid(p.F + 1, p.units);
  const float ts = p.seed_mode == 1 ? 0.5f : 1.0f;
  if (p.dtype == VDA_DTYPE_BF16) {
    auto kern = (p.dk == 128 && p.dv == 128) ? stats_bf16_kernel<128, 128> : stats_bf16_kernel<0, 0>;
    hipLaunchKernelGGL(kern, grid, dim3(kStatsThreads), 0, s,
                       static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), beta,
                       static_cast<const uint16_t*>(text_k), static_cast<const uint16_t*>(text_v),
                       text_beta, w.A, w.B, p.F, p.U, p.T, p.dk, p.dv, ts);
  } else {
    hipLaunchKernelGGL(stats_f32_kernel, grid, dim3(kThreads), 0, s,
                       static_cast<const float*>(k), static_cast<const float*>(v), beta,
                       static_cast<const float*>(text_k), static_cast<const float*>(text_v),
                       text_beta, w.A, w.B, p.F, p.U, p.T, p.dk, p.dv, ts);
  }
  return hipGetLastError();
}

}  // namespace vda
