// Frame statistics of Video Delta Attention ("Video DeltaNet", arXiv 2609.20744,
// Sec. 3.1 Eq. (3b)):
//   A_t = K_t^T Diag(beta_t) K_t,   B_t = V_t^T Diag(beta_t) K_t
// for every (unit, frame), with the text tokens as one more frame placed before
// the first latent frame
// (Sec. 5, "Chunk-wise scans").  Both statistics come from ONE contraction
// over the frame's tokens,
//   [A_t ; B_t] = [X_t | Y_t]^T X_t,   X_t = Diag(sqrt(beta_t)) K_t,
//                                      Y_t = Diag(sqrt(beta_t)) V_t,
// so every K/V byte is read from HBM once and A_t and B_t come out of the same
// token reduction (the fused statistics kernel of Sec. 5).  Splitting beta as sqrt(beta) * sqrt(beta)
// makes the computed A = X^T X positive semidefinite by construction even
// after X is rounded to bf16, so I + A stays SPD with every eigenvalue >= 1
// and ||(I + A)^{-1}||_2 <= 1 (Prop. 1) holds for the computed transition too.
//
// bf16 path, latent frames: a persistent kernel (below); wave w owns output
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
// bf16 path, text frame: fp32 products on v_mfma_f32_32x32x2_f32 with
// sqrt(beta) x formed in fp32 (text_tile).  The text state seeds both scans
// and, unlike a latent frame's thousands of tokens, a handful of text tokens
// does not average out the bf16 rounding of sqrt(beta) k: the seed is
// low-rank, its rounding errors are not, and a query mostly orthogonal to the
// text keys reads the errors almost alone.  The text frame is a small share of
// the work (T tokens per unit against F U): at d_k = d_v = 128 its tiles are
// extra work items of the persistent kernel's workgroups that have one frame
// fewer than the others (no launch of its own), else a kernel of its own.
//
// fp32 path: the same contraction in fp32 on the vector ALUs (exact fp32
// products, fp32 accumulation) for fp32 features.
#include "vda_device.h"
#include "vda_internal.h"

#include <algorithm>

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

// Text frame, bf16 features: tile `tile` (32 x 32, rows of [A; B], columns of
// key channels) of unit u's [sqrt(b) K | sqrt(b) V]^T (sqrt(b) K), sqrt(b) x
// formed in fp32 (never rounded to bf16) and multiplied on
// v_mfma_f32_32x32x2_f32 (fp32 products and sums) by the NW waves of the
// calling workgroup.  The waves split the text tokens, two per instruction
// (the k slots: lane l reads token 2 p + l / 32, channel l % 32 of the tile's
// row and column channels, 64 contiguous bytes per half-wave), loading one
// batch of PAIRS token pairs ahead; their partial tiles are summed in a fixed
// order through Ps ((NW - 1) x 4 KiB of LDS).  Every thread of the workgroup
// calls it (it holds a barrier).
template <int NW, int PAIRS>
__device__ __forceinline__ void text_tile(const uint16_t* __restrict__ tk,
                                          const uint16_t* __restrict__ tv,
                                          const float* __restrict__ tb, float* __restrict__ Aout,
                                          float* __restrict__ Bout, int F, int T, int dk, int dv,
                                          float text_scale, int u, int tile, float* Ps) {
  const int nK = pad32(dk) >> 5;
  const int rt = tile / nK;
  const int ct = tile - rt * nK;
  const bool isA = rt < nK;
  const int rch0 = 32 * (isA ? rt : rt - nK);
  const int nrows = isA ? dk : dv;
  const int cch0 = 32 * ct;
  const uint16_t* K = tk + (size_t)u * T * dk;
  const uint16_t* R = isA ? K : tv + (size_t)u * T * dv;  // source of the row channels
  const int ldr = isA ? dk : dv;
  const float* Bt = tb + (size_t)u * T;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int ks = lane >> 5;
  // channels clamped into the row (padding lanes read a valid channel, zeroed below)
  const int rch = min(rch0 + (lane & 31), nrows - 1);
  const int cch = min(cch0 + (lane & 31), dk - 1);
  const bool rok = rch0 + (lane & 31) < nrows;
  const bool cok = cch0 + (lane & 31) < dk;
  const int npairs = (T + 1) >> 1;
  const int per = (npairs + NW - 1) / NW;
  const int p0 = min(w * per, npairs);
  const int p1 = min(p0 + per, npairs);

  struct Batch {
    uint16_t a[PAIRS], b[PAIRS];
    float beta[PAIRS];
  };
  auto load = [&](Batch& g, int p) {
#pragma unroll
    for (int e = 0; e < PAIRS; ++e) {
      const int tok = 2 * (p + e) + ks;
      const bool ok = tok < T && p + e < p1;
      const int tc = ok ? tok : 0;  // T > 0 whenever a batch is loaded
      g.a[e] = R[(size_t)tc * ldr + rch];
      g.b[e] = K[(size_t)tc * dk + cch];
      g.beta[e] = ok ? Bt[tc] : 0.0f;
    }
  };
  auto bf = [](uint16_t x) { return __uint_as_float((uint32_t)x << 16); };
  f32x16_t acc0 = zero16(), acc1 = zero16();
  auto mul = [&](const Batch& g) {
#pragma unroll
    for (int e = 0; e < PAIRS; e += 2) {
      const float s0 = __builtin_amdgcn_sqrtf(g.beta[e] * text_scale);
      const float s1 = __builtin_amdgcn_sqrtf(g.beta[e + 1] * text_scale);
      acc0 = mfma_f32(rok ? s0 * bf(g.a[e]) : 0.0f, cok ? s0 * bf(g.b[e]) : 0.0f, acc0);
      acc1 = mfma_f32(rok ? s1 * bf(g.a[e + 1]) : 0.0f, cok ? s1 * bf(g.b[e + 1]) : 0.0f, acc1);
    }
  };
  Batch ga, gb;
  int p = p0;
  if (p < p1) load(ga, p);
  while (p < p1) {
    if (p + PAIRS < p1) load(gb, p + PAIRS);
    mul(ga);
    p += PAIRS;
    if (p >= p1) break;
    if (p + PAIRS < p1) load(ga, p + PAIRS);
    mul(gb);
    p += PAIRS;
  }
  f32x16_t acc = acc0 + acc1;
  if (w > 0 && w < NW) {
#pragma unroll
    for (int r = 0; r < 16; ++r) Ps[((w - 1) * 16 + r) * 64 + lane] = acc[r];
  }
  __syncthreads();
  if (w == 0) {
#pragma unroll 1
    for (int q = 0; q < NW - 1; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] += Ps[(q * 16 + r) * 64 + lane];
    float* dst = isA ? Aout + (size_t)u * (F + 1) * dk * dk : Bout + (size_t)u * (F + 1) * dv * dk;
    const int col = cch0 + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = rch0 + acc_row(r, lane);
      if (row < nrows && col < dk) dst[(size_t)row * dk + col] = acc[r];
    }
  }
  __syncthreads();  // Ps is free again
}

constexpr int kWavesT = 8;  // waves of the text-frame kernel

// The text frame as a kernel of its own: one workgroup per (tile, unit).
__global__ __launch_bounds__(64 * kWavesT) void stats_text_kernel(
    const uint16_t* __restrict__ tk, const uint16_t* __restrict__ tv, const float* __restrict__ tb,
    float* __restrict__ Aout, float* __restrict__ Bout, int F, int T, int dk, int dv,
    float text_scale) {
  __shared__ float Ps[(kWavesT - 1) * 16 * 64];
  text_tile<kWavesT, 16>(tk, tv, tb, Aout, Bout, F, T, dk, dv, text_scale, blockIdx.y, blockIdx.x,
                         Ps);
}

// Persistent: one workgroup per CU (the 128 KiB of LDS allow no more) walks
// the frames b, b + P, b + 2P, ... of the flattened (unit, latent frame) list,
// g = u F + f (stored at workspace frame u (F + 1) + f + 1), as ONE continuous
// tile stream: the first tiles of the next frame are in flight while the last tile
// of the current one is multiplied and its results are stored.

// DK, DV > 0: compile-time d_k and d_v (the common 128 case); 0: runtime.
// NT: tokens each thread stages per tile: 4 with 512 threads (wave w owns
// output row tile w and all four column tiles), 2 with 1024 threads (wave w
// owns row tile w % 8 and column tiles 2 (w / 8), + 1: four waves per SIMD).
template <int DK, int DV, int NT>
__global__ __launch_bounds__(512 * (4 / NT), 1) void stats_bf16_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const float* __restrict__ beta,
    float* __restrict__ Aout, float* __restrict__ Bout, int F, int U, int dk_rt, int dv_rt,
    int nframes, int anchors, const uint16_t* __restrict__ tk, const uint16_t* __restrict__ tv,
    const float* __restrict__ tb, int T, float text_scale, int text_items, int upper) {
  const int dk = DK > 0 ? DK : dk_rt;
  const int dv = DV > 0 ? DV : dv_rt;
  __shared__ __align__(16) unsigned char smem[2 * kStageBytes];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int P = gridDim.x;
  const int b0 = blockIdx.x;

  struct FrameSrc {
    const uint16_t* k;
    const uint16_t* v;
    const float* b;
    int ntok;
  };
  // boundary anchors (frames 0 and F - 1) write nothing: read as empty frames
  auto frame_src = [&](int g) {
    const int f = g % F;
    const bool anchor = anchors && (f == 0 || f == F - 1);
    return FrameSrc{k + (size_t)g * U * dk, v + (size_t)g * U * dv, beta + (size_t)g * U,
                    anchor ? 0 : U};
  };
  auto ntiles_of = [&](int ntok) { return ntok > 0 ? (ntok + kTok - 1) / kTok : 1; };
  // tile cursor: frame g (>= nframes past this workgroup's last frame), tile i
  struct Cur {
    int g, i;
  };
  auto next = [&](Cur c) {
    if (c.g < nframes && c.i + 1 < ntiles_of(frame_src(c.g).ntok)) return Cur{c.g, c.i + 1};
    return Cur{c.g + P, 0};
  };

  constexpr int NCT = NT == 4 ? 4 : 2;  // column tiles per wave
  // staging role: token group tg (NT tokens) x channel group cg (8 channels)
  const int tg = (t & 1) | ((t >> 5) << 1);
  const int cg = (t >> 1) & 15;
  const bool kact = cg * 8 < dk;
  const bool vact = cg * 8 < dv;

  // one tile's worth of this thread's raw inputs (16-byte bf16 vectors).
  // Buffer loads through a per-tile descriptor whose range ends at the frame's
  // last token: tokens past the end (and every token of an empty frame) read
  // as exact zeros without touching memory, and the addresses are per-thread
  // constants (no address arithmetic per load).  Nothing uses the values until
  // the tile is staged: vmcnt retires in issue order, so a tile's loads stay
  // in flight behind later work.
  struct TileRegs {
    u32x4_t k[NT], v[NT];
    float b[NT];  // beta of the NT tokens
  };
  const int kcg = kact ? cg : 0;
  const int vcg = vact ? cg : 0;
  // byte offsets of the thread's NT tokens within a tile
  const int koff = ((NT * tg) * dk + 8 * kcg) * 2;
  const int voff = ((NT * tg) * dv + 8 * vcg) * 2;
  const int boff = 4 * NT * tg;

  auto load = [&](TileRegs& r, Cur c) {
    const bool past = c.g >= nframes;  // past this workgroup's last frame: zeros, never used
    const FrameSrc f = frame_src(past ? b0 : c.g);
    const int tok0 = c.i * kTok;
    const int rem = past ? 0 : max(f.ntok - tok0, 0);
    const size_t t0 = past ? 0 : (size_t)tok0;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(f.k + t0 * dk, rem * dk * 2);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(f.v + t0 * dv, rem * dv * 2);
    const __amdgpu_buffer_rsrc_t rbb = make_rsrc(f.b + t0, rem * 4);
#pragma unroll
    for (int s = 0; s < NT; ++s) {
      r.k[s] = buf_load16_nt(rk, koff + s * dk * 2);
      r.v[s] = buf_load16_nt(rv, voff + s * dv * 2);
      r.b[s] = buf_load4(rbb, boff + 4 * s);
    }
  };

  // sqrt(beta) of the thread's NT tokens of a tile (beta reads 0 past the end)
  auto sqrt_beta = [&](const TileRegs& r, Cur, float (&sb4)[NT]) {
#pragma unroll
    for (int s = 0; s < NT; ++s) sb4[s] = __builtin_amdgcn_sqrtf(r.b[s]);
  };

  // channel c of the thread's 8-channel group, its NT tokens: scale, round, pack
  auto scaled = [&](const u32x4_t* x4, const float* bq, int c, uint32_t (&e)[NT / 2]) {
    const int p = c >> 1;
    const bool hi = (c & 1) != 0;
    float x[NT];
#pragma unroll
    for (int s = 0; s < NT; ++s) x[s] = (hi ? bf16_hi(x4[s][p]) : bf16_lo(x4[s][p])) * bq[s];
#pragma unroll
    for (int s = 0; s < NT / 2; ++s) e[s] = pack_bf16(x[2 * s], x[2 * s + 1]);
  };

  // staging write offsets: channel row 8 cg + c, token slot tg (NT tokens,
  // 2 NT bytes; 8 / NT slots per 16-byte chunk).  With
  // Q = swz(8 cg + c) ^ c = (8 (cg & 1)) ^ cg (independent of c), the byte
  // offset is ((2048 cg) | (((tg / (8 / NT)) ^ Q) << 4) | (2 NT (tg % (8 / NT))))
  // ^ (16 c), + 256 c; V rows 128 + 8 cg + c have the same swizzle, 32 KiB further.
  constexpr int kSlots = 8 / NT;
  const uint32_t Q = (8u * (cg & 1)) ^ cg;
  const uint32_t wbase = (uint32_t)(2048 * cg) | ((((uint32_t)tg / kSlots) ^ Q) << 4) |
                         (2u * NT * ((uint32_t)tg % kSlots));
  auto write_channel = [&](const TileRegs& r, const float (&sb4)[NT], int stage, int c) {
    unsigned char* X = smem + stage * kStageBytes + 256 * c;
    const uint32_t o = wbase ^ (16u * c);
    uint32_t e[NT / 2];
    if (kact) {
      scaled(r.k, sb4, c, e);
      if constexpr (NT == 4) *reinterpret_cast<u32x2_t*>(X + o) = u32x2_t{e[0], e[NT / 2 - 1]};
      else *reinterpret_cast<uint32_t*>(X + o) = e[0];
    }
    if (vact) {
      scaled(r.v, sb4, c, e);
      if constexpr (NT == 4) *reinterpret_cast<u32x2_t*>(X + o + 128 * kRowBytes) = u32x2_t{e[0], e[NT / 2 - 1]};
      else *reinterpret_cast<uint32_t*>(X + o + 128 * kRowBytes) = e[0];
    }
  };
  // contraction role: wave w owns output row tile rt of [A; B] and column
  // tiles ct0 .. ct0 + NCT - 1
  const int nK = pad32(dk) >> 5;
  const int nV = pad32(dv) >> 5;
  const int nR = nK + nV;
  const int rt = NT == 4 ? w : (w & 7);
  const int ct0 = NT == 4 ? 0 : 2 * (w >> 3);
  const bool ract = rt < nR;
  const int rbase = rt < nK ? 32 * rt : 128 + 32 * (rt - nK);
  f32x16_t acc[NCT];
#pragma unroll
  for (int j = 0; j < NCT; ++j) acc[j] = zero16();

  // operand offsets: off16(row, j) with j = 2 kk + kh equals
  // (row * 256 + ((16 kh) ^ (swz(row) << 4))) ^ (32 kk)
  const int il = lane & 31;
  const int kh = lane >> 5;
  auto opbase = [&](int row) {
    return (uint32_t)row * kRowBytes + ((16u * kh) ^ (swz(row) << 4));
  };
  const uint32_t abase = opbase(rbase + il);
  uint32_t bbase[NCT];
#pragma unroll
  for (int j = 0; j < NCT; ++j) bbase[j] = opbase(32 * (ct0 + j) + il);

  // Multiply the tile in `cstage` (8 k-steps of 16 tokens) and, interleaved
  // with it, stage channel c = kk of the
  // register set `r` (tile cw) into `wstage`.
  auto compute_write = [&](int cstage, const TileRegs& r, Cur cw, int wstage) {
    const unsigned char* X = smem + cstage * kStageBytes;
    float sb4[NT];
    sqrt_beta(r, cw, sb4);
#pragma unroll
    for (int kk = 0; kk < kTok / 16; ++kk) {
      if (ract) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(X + (abase ^ (32u * kk)));
#pragma unroll
        for (int j = 0; j < NCT; ++j) {
          if (ct0 + j < nK) {
            const u32x4_t bq = *reinterpret_cast<const u32x4_t*>(X + (bbase[j] ^ (32u * kk)));
            acc[j] = mfma_bf16(a, bq, acc[j]);
          }
        }
      }
      write_channel(r, sb4, wstage, kk);
    }
  };

  // results of frame g: rows of A (K tiles) or B (V tiles), columns are key
  // channels; the accumulators restart at zero.  A is symmetric and the
  // frame-wise solve reads only its lower 32 x 32 blocks, so unless `upper` is
  // set (the batched rules read all of A, the statistics tap returns it) the
  // blocks above the diagonal are not stored.  Non-temporal stores: in the
  // k / v read stream, plain stores of the 128 KB per frame measured about 25%
  // slower on MI355X (a stats-shaped read probe: 0.425 ms without stores,
  // 0.540 ms with plain ones, 0.481 ms with non-temporal ones)
  auto store_frame = [&](int g) {
    if (ract) {
      const bool isA = rt < nK;
      const int ch0 = isA ? 32 * rt : 32 * (rt - nK);
      const int nrows = isA ? dk : dv;
      const size_t slot = (size_t)g + g / F + 1;  // after the unit's text frame
      float* dst = isA ? Aout + slot * dk * dk : Bout + slot * dv * dk;
#pragma unroll
      for (int j = 0; j < NCT; ++j) {
        if (ct0 + j >= nK) continue;
        if (isA && !upper && ct0 + j > rt) continue;  // A's upper blocks: not read
        const int col = 32 * (ct0 + j) + (lane & 31);
        if (col >= dk) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = ch0 + acc_row(r, lane);
          if (row < nrows) __builtin_nontemporal_store(acc[j][r], dst + (size_t)row * dk + col);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NCT; ++j) acc[j] = zero16();
  };
  auto last_tile = [&](Cur c) { return c.i + 1 == ntiles_of(frame_src(c.g).ntok); };

  // Stage 0 / 1 alternate.  Each tile: one barrier, then the loads of the
  // tile two ahead go into the register set the current tile came from, and
  // the current tile is multiplied while the next one (loaded one tile
  // earlier) is staged into the other stage.  Every register set is staged on
  // every path, so no wait before reloading a set is needed.
  Cur c0{b0, 0};
  Cur c1 = next(c0);
  Cur c2 = next(c1);
  TileRegs ra, rb;
  load(ra, c0);
  load(rb, c1);
  {
    float sb4[NT];
    sqrt_beta(ra, c0, sb4);
#pragma unroll
    for (int c = 0; c < 8; ++c) write_channel(ra, sb4, 0, c);
  }
  while (true) {
    __syncthreads();
    load(ra, c2);
    compute_write(0, rb, c1, 1);
    if (last_tile(c0)) store_frame(c0.g);
    c0 = c1;
    c1 = c2;
    c2 = next(c2);
    if (c0.g >= nframes) break;
    __syncthreads();
    load(rb, c2);
    compute_write(1, ra, c1, 0);
    if (last_tile(c0)) store_frame(c0.g);
    c0 = c1;
    c1 = c2;
    c2 = next(c2);
    if (c0.g >= nframes) break;
  }

  // text-frame tiles (text_items > 0 only with 16 waves at d_k = d_v = 128):
  // taken round robin by the workgroups with one frame fewer than the others
  // when there are enough of them for at most 8 tiles each, else by all
  if (NT == 2 && text_items > 0) {
    __syncthreads();  // the stages are free
    const int rem = nframes % P;
    const bool slack = rem != 0 && (P - rem) * 8 >= text_items;
    const int slot = slack ? b0 - rem : b0;
    const int nslots = slack ? P - rem : P;
    const int tiles = text_items / (nframes / F);  // per unit
    if (slot >= 0)
      for (int j = slot; j < text_items; j += nslots)
        text_tile<16, 4>(tk, tv, tb, Aout, Bout, F, T, dk, dv, text_scale, j / tiles, j % tiles,
                         reinterpret_cast<float*>(smem));
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
    float text_scale, int anchors) {
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
    ntok = anchors && (fi == 1 || fi == F) ? 0 : U;  // boundary anchors write nothing
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

// compute units of the current device (cached per device)
int compute_units() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

}  // namespace

hipError_t launch_stats(const Plan& p, const void* k, const void* v, const float* beta,
                        const void* text_k, const void* text_v, const float* text_beta,
                        const WsPtrs& w, hipStream_t s) {
  const dim3 grid(p.F + 1, p.units);
  const float ts = p.seed_mode == 1 ? 0.5f : 1.0f;
  if (p.dtype == VDA_DTYPE_BF16) {
    const int nK = pad32(p.dk) >> 5;
    const int tiles = (nK + (pad32(p.dv) >> 5)) * nK;  // text-frame tiles per unit
    const int nframes = p.units * p.F;                 // latent frames
    const int P = std::min(nframes, compute_units());
    const int upper = p.rule != 0 || p.full_stats ? 1 : 0;
    const uint16_t* tk = static_cast<const uint16_t*>(text_k);
    const uint16_t* tv = static_cast<const uint16_t*>(text_v);
    if (p.dk == 128 && p.dv == 128) {  // the text tiles ride in the persistent kernel
      hipLaunchKernelGGL((stats_bf16_kernel<128, 128, 2>), dim3(P), dim3(2 * kStatsThreads), 0, s,
                         static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), beta,
                         w.A, w.B, p.F, p.U, p.dk, p.dv, nframes, p.anchors, tk, tv, text_beta,
                         p.T, ts, p.units * tiles, upper);
    } else {
      hipLaunchKernelGGL(stats_text_kernel, dim3(tiles, p.units), dim3(64 * kWavesT), 0, s, tk, tv,
                         text_beta, w.A, w.B, p.F, p.T, p.dk, p.dv, ts);
      hipLaunchKernelGGL((stats_bf16_kernel<0, 0, 4>), dim3(P), dim3(kStatsThreads), 0, s,
                         static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), beta,
                         w.A, w.B, p.F, p.U, p.dk, p.dv, nframes, p.anchors, tk, tv, text_beta,
                         p.T, ts, 0, upper);
    }
  } else {
    hipLaunchKernelGGL(stats_f32_kernel, grid, dim3(kThreads), 0, s,
                       static_cast<const float*>(k), static_cast<const float*>(v), beta,
                       static_cast<const float*>(text_k), static_cast<const float*>(text_v),
                       text_beta, w.A, w.B, p.F, p.U, p.T, p.dk, p.dv, ts, p.anchors);
  }
  return hipGetLastError();
}

}  // namespace vda
