// Feature map of the linear branch ("Video DeltaNet", arXiv 2609.20744,
// Sec. 2.3; fused with the layout conversion as Sec. 5 "Fused VDA kernels"
// describes):
//   K' = L2(SiLU(conv(K))),   V' = SiLU(conv(V)),   Q' = L2(Q)
// conv: depthwise (one filter per head and channel) separable short
// convolution, a 5 x 5 spatial and a five-tap temporal filter, applied as the
// centred 3-D correlation with kernel w_t[tau] w_s[a][b] and zero padding at
// the clip's and the frame's borders.  L2(x) = x / max(||x||_2, eps) over the d
// channels of one (token, head).  Input layout: the projection output
// [batch][F][H_l][W_l][heads][d]; output: [batch * heads][F][H_l * W_l][d].
//
// Two convolution kernels share the tiling below: bf16 features run the
// spatial filter on the matrix cores (prep_mfma_kernel, described with it);
// fp32 features take the vector-ALU kernel described here.
//
// conv kernel: one workgroup (16 waves, four per SIMD to hide LDS latency) per
// (unit, 8 x 8 spatial tile), sweeping all frames.  Per input frame the
// 12 x 12 halo tile of the unit's channels is staged in LDS as fp32 (converted
// once) while the next frame's tile is in flight in registers.  Wave w owns
// output row w % 8, columns 4 (w / 8) .. + 3 of the tile, lane l the channel
// pair 2l, 2l + 1: its 4 outputs x 2 channels are a 5 x 8 window product (read
// once per window row, 8-byte conflict-free LDS reads); the
// spatial taps of the unit's channels sit in LDS (one 8-byte read per tap
// serves the lane's 8 outputs), its five temporal taps in registers.  The temporal filter runs
// in scatter form: input frame t adds w_t[tau] times its spatial result to the
// pending outputs t + 2 - tau, kept in a ring of five register sets (the frame
// loop is unrolled by five so every ring index is static); output frame t - 2
// is then complete: SiLU, the channel sum of squares across the wave's 64
// lanes, scaling, one 256-byte row per position.  The kernel does about 30
// fp32 FMA per output element against 4 bytes (bf16 in + out) of HBM traffic,
// so it is bound by the vector ALUs rather than by HBM.
//
// One launch does all three tensors: the K sweeps and the V sweeps (each XCD
// takes a range of K sweeps, then the same range of V) and, as its last
// workgroups, the bandwidth-bound Q pass, which fills the CUs that the sweeps'
// last round leaves idle.
#include <type_traits>

#include "vda_device.h"
#include "vda_internal.h"

namespace vda {
namespace {

constexpr int kTR = 8;            // output tile rows
constexpr int kTC = 8;            // output tile columns
constexpr int kHR = kTR + 4;      // halo tile rows
constexpr int kHC = kTC + 4;      // halo tile columns
constexpr int kPrepThreads = 1024;
constexpr int kCols = 4;          // output columns per wave
constexpr unsigned kQBlocks = 1024;  // workgroups of the Q pass (16 waves each)

// 16-byte pieces of a tensor element type: 8 bf16 or 4 fp32 channels
template <typename T>
struct Piece;
template <>
struct Piece<uint16_t> {
  static constexpr int kElems = 8;
  __device__ static void to_f32(const u32x4_t& v, float* out) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      out[2 * e] = bf16_lo(v[e]);
      out[2 * e + 1] = bf16_hi(v[e]);
    }
  }
};
template <>
struct Piece<float> {
  static constexpr int kElems = 4;
  __device__ static void to_f32(const u32x4_t& v, float* out) {
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = __uint_as_float(v[e]);
  }
};

__device__ __forceinline__ void store2(uint16_t* p, float a, float b) {
  *reinterpret_cast<uint32_t*>(p) = pack_bf16(a, b);
}
__device__ __forceinline__ void store2(float* p, float a, float b) {
  *reinterpret_cast<float2*>(p) = make_float2(a, b);
}

__device__ __forceinline__ float silu(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

// Value of lane ^ 16, by gfx950's row-swap permute (a VALU instruction, no
// LDS round trip; lane ^ 32 is lane_xor32): permlane16_swap(x, x) returns
// {rows [x0, x0, x2, x2], rows [x1, x1, x3, x3]} (rows of 16 lanes).
__device__ __forceinline__ float lane_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float((lane_id() & 16) ? r[0] : r[1]);
}
// x plus the value of a lane in the other half of its quad, 8-lane or 16-lane
// group (DPP: quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror,
// row_mirror); four steps leave the 16-lane sum in every lane of a row.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sums over the wave's 64 lanes of 4 values per lane at once, as a halving
// butterfly: after the exchanges across lane bits 5 and 4 each lane holds one
// partial sum, of value (lane >> 4) & 3, which the four in-row steps complete.
// 6 lane exchanges instead of 24, all on the vector ALUs.  Returns the sum of
// value (lane >> 4) & 3.
__device__ __forceinline__ float wave_sum4(const float (&v)[4]) {
  const int lane = lane_id();
  const bool h5 = lane & 32, h4 = lane & 16;
  float a[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float keep = h5 ? v[i + 2] : v[i];
    const float send = h5 ? v[i] : v[i + 2];
    a[i] = keep + lane_xor32(send);
  }
  float c = (h4 ? a[1] : a[0]) + lane_xor16(h4 ? a[0] : a[1]);
  c = dpp_add<0xB1>(c);
  c = dpp_add<0x4E>(c);
  c = dpp_add<0x141>(c);
  c = dpp_add<0x140>(c);
  return c;
}

// Q' = L2(Q) with the layout conversion: G = d / EPP lanes per (token, head)
// row, rows taken in input order (contiguous reads), each written as one
// contiguous row of its unit.  Wave `wave` of `nwaves` takes every nwaves-th
// group of 64 / G rows.
template <typename T>
__device__ __forceinline__ void q_rows(const T* __restrict__ x, T* __restrict__ y, long rows, int F,
                                       int U, int H, int d, float eps, long wave, long nwaves) {
  constexpr int EPP = Piece<T>::kElems;
  constexpr int G = 128 / EPP;  // lanes per row (some idle when d < 128)
  const int lane = threadIdx.x & 63;
  const int sub = lane % G;
  const int rows_per_wave = 64 / G;
  const bool act = sub * EPP < d;
  for (long r0 = wave * rows_per_wave; r0 < rows; r0 += nwaves * rows_per_wave) {
    const long r = r0 + lane / G;  // (b, t, p, h) row in input order
    const bool ok = r < rows && act;
    u32x4_t raw = ok ? *reinterpret_cast<const u32x4_t*>(x + r * d + sub * EPP)
                     : u32x4_t{0u, 0u, 0u, 0u};
    float v[EPP];
    Piece<T>::to_f32(raw, v);
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < EPP; ++e) ss = fmaf(v[e], v[e], ss);
#pragma unroll
    for (int m = G / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
    const float inv = 1.0f / fmaxf(sqrtf(ss), eps);
    if (!ok) continue;
    const long h = r % H;
    const long tp = r / H;  // (b F + t) U + p
    const long p = tp % U;
    const long bt = tp / U;  // b F + t
    const long t = bt % F;
    const long b = bt / F;
    T* dst = y + ((((b * H + h) * F + t) * U + p) * d + sub * EPP);
#pragma unroll
    for (int e = 0; e < EPP; e += 2) store2(dst + e, v[e] * inv, v[e + 1] * inv);
  }
}

// One tensor of the convolution: input, spatial taps [head][channel][25],
// temporal taps [head][channel][5], output, channel count.
template <typename T>
struct ConvSide {
  const T* x;
  const float* ws;
  const float* wt;
  T* y;
  int d;
};

// K (L2 normalised) and V in one launch, so that the last, partial round of
// (unit, tile) sweeps is shared by the two tensors.  XCD x takes the sweeps
// x * per .. x * per + per - 1 of K, then the same sweeps of V (workgroup L
// runs on XCD L % 8 as the L / 8-th of its queue), so the sweeps running side
// by side on an XCD are neighbouring tiles of one tensor at the same pace and
// share their halo reads in its L2.
// The Q rows follow as the last qblocks workgroups of the launch: they are
// dispatched once every convolution sweep has started, onto the CUs that the
// sweeps' last, partial round leaves free, so the bandwidth-bound Q pass runs
// beside the ALU-bound tail of the convolution instead of after it.
template <typename T>
__global__ __launch_bounds__(kPrepThreads, 1) void prep_conv_kernel(
    ConvSide<T> ks, ConvSide<T> vs, int F, int Hl, int Wl, int H, int tiles_r, int tiles_c,
    int units, unsigned per, float eps, const T* __restrict__ qx, T* __restrict__ qy, long qrows,
    int dq, unsigned qblocks) {
  __shared__ __align__(16) float Xs[kHR * kHC * 128];  // one frame's halo tile, [pos][channel]
  __shared__ __align__(16) float Ws[25 * 128];          // spatial taps, [tap][channel]
  constexpr int EPP = Piece<T>::kElems;
  constexpr int kIter = (kHR * kHC * (128 / EPP) + kPrepThreads - 1) / kPrepThreads;
  constexpr int kWaves = kPrepThreads / 64;
  if (blockIdx.x >= 2 * kXcds * per) {
    const unsigned qb = blockIdx.x - 2 * kXcds * per;
    q_rows(qx, qy, qrows, F, Hl * Wl, H, dq, eps, (long)qb * kWaves + (threadIdx.x >> 6),
           (long)qblocks * kWaves);
    return;
  }
  const unsigned ntiles = (unsigned)tiles_r * tiles_c;
  const unsigned j = blockIdx.x / kXcds;  // position in the XCD's queue
  const bool norm = j < per;              // K first, then V
  const unsigned item = (blockIdx.x % kXcds) * per + (norm ? j : j - per);
  if (j >= 2 * per || item >= (unsigned)units * ntiles) return;
  const ConvSide<T> side = norm ? ks : vs;
  const T* __restrict__ x = side.x;
  const float* __restrict__ ws = side.ws;
  const float* __restrict__ wt = side.wt;
  T* __restrict__ y = side.y;
  const int d = side.d;
  const int unit = item / ntiles;
  const int tile = item - unit * ntiles;
  const int b = unit / H;
  const int h = unit - b * H;
  const int r0 = (tile / tiles_c) * kTR;
  const int c0 = (tile % tiles_c) * kTC;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int orow = w & 7;            // output row of the tile
  const int oc0 = kCols * (w >> 3);  // first output column
  const int ch = 2 * lane;
  const bool cact = ch < d;
  const int U = Hl * Wl;

  // filters of head h: spatial taps to LDS (zero for channels past d, which
  // only idle lanes read), this lane's temporal taps (channels ch, ch + 1)
  for (int i = t; i < 25 * 128; i += kPrepThreads) {
    const int tap = i >> 7;
    const int c = i & 127;
    Ws[i] = c < d ? ws[((size_t)h * d + c) * 25 + tap] : 0.0f;
  }
  float ft[2][5];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const size_t c = (size_t)h * d + (cact ? ch + e : 0);
#pragma unroll
    for (int i = 0; i < 5; ++i) ft[e][i] = cact ? wt[c * 5 + i] : 0.0f;
  }

  // staging: 16-byte pieces of the halo tile's positions, loaded through a
  // per-frame buffer descriptor: a piece outside the frame (or past the tile)
  // gets an offset past the descriptor's range and reads as zero
  const int gpp = d / EPP;  // pieces per position
  const int npieces = kHR * kHC * gpp;
  const int frame_bytes = U * H * d * (int)sizeof(T);
  int poff[kIter];
#pragma unroll
  for (int i = 0; i < kIter; ++i) {
    const int p = t + kPrepThreads * i;
    const int pos = p / gpp;
    const int cg = p - pos * gpp;
    const int gi = r0 - 2 + pos / kHC;
    const int gj = c0 - 2 + pos % kHC;
    const bool ok = p < npieces && gi >= 0 && gi < Hl && gj >= 0 && gj < Wl;
    poff[i] = ok ? (((gi * Wl + gj) * H + h) * d + cg * EPP) * (int)sizeof(T) : frame_bytes;
  }
  u32x4_t pre[kIter];
  auto load_frame = [&](int tin) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(x + ((size_t)b * F + tin) * U * H * d, frame_bytes);
#pragma unroll
    for (int i = 0; i < kIter; ++i) pre[i] = buf_load16(rs, poff[i]);
  };
  auto store_frame = [&]() {
#pragma unroll
    for (int i = 0; i < kIter; ++i) {
      const int p = t + kPrepThreads * i;
      if (p >= npieces) continue;
      const int pos = p / gpp;
      const int cg = p - pos * gpp;
      float v[EPP];
      Piece<T>::to_f32(pre[i], v);
      float* dst = Xs + pos * 128 + cg * EPP;
#pragma unroll
      for (int e = 0; e < EPP; e += 4)
        *reinterpret_cast<f32x4_t*>(dst + e) = f32x4_t{v[e], v[e + 1], v[e + 2], v[e + 3]};
    }
  };

  float acc[5][2][kCols];
#pragma unroll
  for (int s = 0; s < 5; ++s)
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int o = 0; o < kCols; ++o) acc[s][e][o] = 0.0f;

  const int gi_out = r0 + orow;
  T* ybase = y + ((size_t)unit * F * U + (size_t)gi_out * Wl + c0 + oc0) * d + ch;
  // one input frame tin (k = tin mod 5): spatial product of the staged tile,
  // scatter into the ring, then output frame tin - 2 is complete
  auto step = [&](int tin, auto kc) {
    constexpr int k = decltype(kc)::value;
    if (tin < F) store_frame();
    if (tin + 1 < F) load_frame(tin + 1);  // in flight during the products below
    __syncthreads();
    if (tin < F) {
      float s[2][kCols];
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int o = 0; o < kCols; ++o) s[e][o] = 0.0f;
#pragma unroll
      for (int a = 0; a < 5; ++a) {
        float xr[2][kCols + 4];
        const float* row = Xs + ((orow + a) * kHC + oc0) * 128 + ch;
#pragma unroll
        for (int c = 0; c < kCols + 4; ++c) {
          const float2 v = *reinterpret_cast<const float2*>(row + c * 128);
          xr[0][c] = v.x;
          xr[1][c] = v.y;
        }
#pragma unroll
        for (int bb = 0; bb < 5; ++bb) {
          const float2 f = *reinterpret_cast<const float2*>(Ws + (a * 5 + bb) * 128 + ch);
#pragma unroll
          for (int o = 0; o < kCols; ++o) {
            s[0][o] = fmaf(f.x, xr[0][o + bb], s[0][o]);
            s[1][o] = fmaf(f.y, xr[1][o + bb], s[1][o]);
          }
        }
      }
      // input frame tin feeds output frame t_out = tin + 2 - tau with w_t[tau];
      // ring slot t_out mod 5 = (k + 2 - tau) mod 5
#pragma unroll
      for (int sl = 0; sl < 5; ++sl) {
        const int tau = (k + 2 - sl + 10) % 5;
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int o = 0; o < kCols; ++o) acc[sl][e][o] = fmaf(ft[e][tau], s[e][o], acc[sl][e][o]);
      }
    }
    // output frame tin - 2 (ring slot (k + 3) mod 5) is complete
    constexpr int fin = (k + 3) % 5;
    const int t_out = tin - 2;
    if (t_out >= 0) {
      float v[2][kCols];
#pragma unroll
      for (int o = 0; o < kCols; ++o) {
        v[0][o] = silu(acc[fin][0][o]);
        v[1][o] = silu(acc[fin][1][o]);
      }
      if (norm) {  // sum of squares over the position's d channels (all 64 lanes)
        float sq[kCols];
#pragma unroll
        for (int o = 0; o < kCols; ++o) sq[o] = cact ? v[0][o] * v[0][o] + v[1][o] * v[1][o] : 0.0f;
        const float inv_l = 1.0f / fmaxf(sqrtf(wave_sum4(sq)), eps);  // of output (lane >> 4) & 3
#pragma unroll
        for (int o = 0; o < kCols; ++o) {
          const float inv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(inv_l), 16 * o));
          v[0][o] *= inv;
          v[1][o] *= inv;
        }
      }
#pragma unroll
      for (int o = 0; o < kCols; ++o) {
        const int gj = c0 + oc0 + o;
        if (cact && gi_out < Hl && gj < Wl)
          store2(ybase + ((size_t)t_out * U + o) * d, v[0][o], v[1][o]);
      }
    }
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int o = 0; o < kCols; ++o) acc[fin][e][o] = 0.0f;
    __syncthreads();  // every wave is done with the staged tile
  };

  if (F > 0) load_frame(0);
  for (int tb = 0; tb < F + 2; tb += 5) {
    step(tb, std::integral_constant<int, 0>{});
    if (tb + 1 < F + 2) step(tb + 1, std::integral_constant<int, 1>{});
    if (tb + 2 < F + 2) step(tb + 2, std::integral_constant<int, 2>{});
    if (tb + 3 < F + 2) step(tb + 3, std::integral_constant<int, 3>{});
    if (tb + 4 < F + 2) step(tb + 4, std::integral_constant<int, 4>{});
  }
}


// ---------------------------------------------------------------------------
// bf16 convolution on the matrix cores.  The 5 x 5 spatial filter of one
// channel, along one halo row, is a banded Toeplitz product: outputs
// x0 .. x0 + 3 of that row are T_a (4 x 8) times halo columns x0 .. x0 + 7,
// T_a[m][k] = w_s[a][k - m] for 0 <= k - m <= 4.  v_mfma_f32_4x4x4_16b_bf16
// runs 16 independent 4 x 4 x 4 products, one per channel: block b = lane / 4
// is channel 16 g + b of the wave's channel group g, the A operand of lane
// (b, m = lane % 4) is row m of T_a (a k step of 4 columns), the B operand of
// lane (b, n = lane % 4) is 4 consecutive halo columns of row 4 hh + n + a,
// and the accumulator of lane (b, n) ends holding outputs x0 .. x0 + 3 of
// output row 4 hh + n.  The taps are split into bf16 hi + lo (hi = bf16(w),
// lo = bf16(w - hi)); the inputs are bf16 already, so every product is exact
// and only the fp32 accumulation rounds, as on the vector path.  Per frame a
// wave forms two such 4 x 4 position blocks (columns 0 .. 3 and 4 .. 7 of four
// output rows) for its 16 channels: 5 rows x 2 k steps x 2 (hi, lo) x 2
// blocks = 40 MFMAs from 15 + 20 eight-byte LDS reads (inputs, taps).
//
// Temporal filter in scatter form on the accumulators, with four ring slots:
// input frame tin adds w_t[tau] times its spatial result to pending output
// tin + 2 - tau; output tin - 2 is finished by its last term and leaves the
// slot that output tin + 2 then starts in (slot = output frame mod 4).
//
// Staged tile: channel-major bf16, 40 eight-byte slots per channel (slot
// 3 hr + q = halo row hr, columns 4 q .. 4 q + 3), channel pitch 88 words,
// slot index XORed with (c / 4) mod 8.  Both access patterns then touch 32
// distinct banks per 16 lanes: the MFMA operand reads (4 channels x 4 rows:
// channel pitch 24 mod 32 words, rows 3 slots apart, the XOR constant over the
// 4 channels) and the staging writes (16 channel pairs of one slot: the XOR
// spreads them).  Staging: lane l loads channels 2 l, 2 l + 1 (4 bytes) of the
// slot's four positions, so one wave instruction reads one position's row of
// channels and the lane holds both slot rows after two byte permutes each.
//
// Output: each lane applies SiLU to its own 8 outputs; for K the sum of
// squares over the wave's 16 channels of each position comes from a halving
// butterfly across lane bits 5 .. 2, the 8 channel groups' partial sums meet in
// LDS, and the scaled values are stored one frame step later, while the next
// frame's products run (two barriers per frame step).
constexpr int kXPitch = 88;   // words (bf16 pairs) per channel of the staged tile
constexpr int kXSlots = 40;   // 8-byte slots per channel (36 used, the XOR reaches 39)
static_assert(kXPitch >= 2 * kXSlots && kXPitch % 32 == 24, "staged tile pitch");
// taps: 8 bytes per (channel, row a, k step s, hi / lo, A row m), channel pitch
// 168 words (8 mod 32: a read's 16 lanes, 4 channels x 4 rows m, hit 32
// distinct banks)
constexpr int kWPitch = 168;
static_assert(kWPitch >= 2 * 5 * 2 * 2 * 4 && kWPitch % 32 == 8, "tap table pitch");

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma4(u32x2_t a, u32x2_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(bf16x4_t, a),
                                                __builtin_bit_cast(bf16x4_t, b), c, 0, 0, 0);
}

// word offset of slot (halo row hr, column quad q) of channel c
__device__ __forceinline__ int xs_word(int c, int hr, int q) {
  return kXPitch * c + 2 * ((3 * hr + q) ^ ((c >> 2) & 7));
}
// word offset of the A operand (row a, k step s, hi / lo part hl, A row m) of channel c
__device__ __forceinline__ int wt_word(int c, int a, int s, int hl, int m) {
  return kWPitch * c + 2 * (4 * (2 * (2 * a + s) + hl) + m);
}

// Sum over the 32 lanes of a half wave (every lane gets it).
__device__ __forceinline__ float half_wave_sum(float x) {
  x = dpp_add<0xB1>(x);
  x = dpp_add<0x4E>(x);
  x = dpp_add<0x141>(x);
  x = dpp_add<0x140>(x);
  return x + lane_xor16(x);
}

__global__ __launch_bounds__(kPrepThreads, 1) void prep_mfma_kernel(
    ConvSide<uint16_t> ks, ConvSide<uint16_t> vs, int F, int Hl, int Wl, int H, int tiles_r,
    int tiles_c, int units, unsigned per, float eps, const uint16_t* __restrict__ qx,
    uint16_t* __restrict__ qy, long qrows, int dq, unsigned qblocks) {
  __shared__ __align__(16) uint32_t Xs[128 * kXPitch];  // staged halo tile (bf16 pairs)
  __shared__ __align__(16) uint32_t Wt[128 * kWPitch];  // spatial taps as A operands
  __shared__ float Rs[8 * 64];                           // K: partial sums of squares [group][pos]
  __shared__ __align__(16) float Is[64];                 // K: inverse norms of the positions
  __shared__ float Ft[5 * 128];                          // temporal taps [tau][channel]
  constexpr int kWaves = kPrepThreads / 64;
  if (blockIdx.x >= 2 * kXcds * per) {
    const unsigned qb = blockIdx.x - 2 * kXcds * per;
    q_rows(qx, qy, qrows, F, Hl * Wl, H, dq, eps, (long)qb * kWaves + (threadIdx.x >> 6),
           (long)qblocks * kWaves);
    return;
  }
  const unsigned ntiles = (unsigned)tiles_r * tiles_c;
  const unsigned jq = blockIdx.x / kXcds;  // position in the XCD's queue
  bool norm = jq < per;                    // K first, then V
  unsigned item = (blockIdx.x % kXcds) * per + (norm ? jq : jq - per);
  if (jq >= 2 * per || item >= (unsigned)units * ntiles) return;
  // With a last tile column at most 4 wide (half tiles: one column block of
  // outputs) the XCD's queue runs its full tiles first (K, then V) and its half
  // tiles last (K, then V), so the cheaper half sweeps fill the last round.
  // Item g is a half tile when g % tiles_c == tiles_c - 1 (the last tile of
  // each tile row; the rows of all units follow each other).
  if (Wl % kTC != 0 && Wl % kTC <= 4 && tiles_c > 1) {
    const unsigned tc = tiles_c;
    const unsigned a = (blockIdx.x % kXcds) * per;
    const unsigned bnd = min(a + per, (unsigned)units * ntiles);
    // the XCD's valid queue positions [0, m) (K) and [per, per + m) (V), compacted
    const unsigned jc = jq < per ? jq : jq - per + (bnd - a);
    auto nfull = [&](unsigned g) { return g - g / tc; };  // full items in [0, g)
    const unsigned f0 = nfull(a), nF = nfull(bnd) - f0;
    const unsigned r0q = a / tc, nR = bnd / tc - r0q;   // half items: g = r tc + tc - 1
    auto full_at = [&](unsigned f) { return (f / (tc - 1)) * tc + f % (tc - 1); };
    if (jc < 2 * nF) {
      norm = jc < nF;
      item = full_at(f0 + (norm ? jc : jc - nF));
    } else {
      const unsigned r = jc - 2 * nF;
      norm = r < nR;
      item = (r0q + (norm ? r : r - nR)) * tc + tc - 1;
    }
  }
  // K (NORM: L2-normalised) and V sweeps as two compiled bodies
  auto sweep = [&](auto nc, auto hc) {
    constexpr bool NORM = decltype(nc)::value;
    constexpr bool half = decltype(hc)::value;
    const ConvSide<uint16_t> side = NORM ? ks : vs;
    const uint16_t* __restrict__ x = side.x;
    const float* __restrict__ ws = side.ws;
    const float* __restrict__ wt = side.wt;
    uint16_t* __restrict__ y = side.y;
    const int d = side.d;
    const int unit = item / ntiles;
    const int tile = item - unit * ntiles;
    const int b = unit / H;
    const int h = unit - b * H;
    const int r0 = (tile / tiles_c) * kTR;
    const int c0 = (tile % tiles_c) * kTC;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = t >> 6;
    const int U = Hl * Wl;

    // this wave's compute role: channel group g (16 channels), output rows
    // 4 hh .. 4 hh + 3 (lane (blk, n): row 4 hh + n), both column blocks
    const int g = w & 7;
    const int hh = w >> 3;
    const bool gact = 16 * g < d;
    const int blk = lane >> 2;
    const int n = lane & 3;
    const int ch = 16 * g + blk;  // this lane's channel (operands and accumulators)

    // tap table: each active lane writes its own A operands (row n of T_a, per
    // row a and k step, hi and lo); temporal taps to LDS as well
    {
      const float* wsc = ws + ((size_t)h * d + (gact ? ch : 0)) * 25;
      if (gact) {
  #pragma unroll
        for (int a = 0; a < 5; ++a)
  #pragma unroll
          for (int s = 0; s < 2; ++s) {
            float v[4];
  #pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
              const int dx = 4 * s + kk - n;
              v[kk] = (dx >= 0 && dx <= 4) ? wsc[a * 5 + max(0, min(dx, 4))] : 0.0f;
            }
            const uint32_t h0 = pack_bf16(v[0], v[1]), h1 = pack_bf16(v[2], v[3]);
            *reinterpret_cast<u32x2_t*>(Wt + wt_word(ch, a, s, 0, n)) = u32x2_t{h0, h1};
            *reinterpret_cast<u32x2_t*>(Wt + wt_word(ch, a, s, 1, n)) =
                u32x2_t{pack_bf16(v[0] - bf16_lo(h0), v[1] - bf16_hi(h0)),
                        pack_bf16(v[2] - bf16_lo(h1), v[3] - bf16_hi(h1))};
          }
      }
      if (n == 0) {  // zero for channels past d (their accumulators stay zero)
        const float* wtc = wt + ((size_t)h * d + (gact ? ch : 0)) * 5;
  #pragma unroll
        for (int i = 0; i < 5; ++i) Ft[i * 128 + ch] = gact ? wtc[i] : 0.0f;
      }
    }

    // staging: wave w takes the halo slots w, w + 16, w + 32 (those below 36;
    // slot 3 hr + q = row hr, columns 4 q .. 4 q + 3), lane l the channel pair
    // 2 l, 2 l + 1: one 4-byte load per column (a wave instruction reads one
    // position's whole row of channels), so a lane ends holding its two channels
    // at the slot's four columns, which two byte permutes per channel turn into
    // the slot's two 8-byte rows.  Positions are wave-uniform: the scalar offset
    // of a position outside the frame lies past the descriptor's range and reads
    // as zero.
    constexpr int kSlots = kHR * (kHC / 4);
    constexpr int kSlotIter = (kSlots + kWaves - 1) / kWaves;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const bool pact = 2 * lane < d;
    const int frame_bytes = U * H * d * (int)sizeof(uint16_t);
    uint32_t pre[kSlotIter][4];
    auto load_frame = [&](int tin) {
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(x + ((size_t)b * F + tin) * U * H * d, frame_bytes);
  #pragma unroll
      for (int j = 0; j < kSlotIter; ++j) {
        const int sl = wu + kWaves * j;
        if (sl >= kSlots) break;
        if (half && sl % 3 == 2) continue;
        const int gi = r0 - 2 + sl / 3;
  #pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int gj = c0 - 2 + 4 * (sl % 3) + k;
          const bool ok = gi >= 0 && gi < Hl && gj >= 0 && gj < Wl;
          const int soff = ok ? ((gi * Wl + gj) * H + h) * d * (int)sizeof(uint16_t) : frame_bytes;
          pre[j][k] = __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * lane, soff, 0);
        }
      }
    };
    auto store_frame = [&]() {
      if (!pact) return;
  #pragma unroll
      for (int j = 0; j < kSlotIter; ++j) {
        const int sl = wu + kWaves * j;
        if (sl >= kSlots) break;
        if (half && sl % 3 == 2) continue;
        const uint32_t* v = pre[j];  // v[k] = channels 2 l, 2 l + 1 at column 4 q + k
        const u32x2_t lo = u32x2_t{__builtin_amdgcn_perm(v[1], v[0], 0x05040100u),
                                   __builtin_amdgcn_perm(v[3], v[2], 0x05040100u)};
        const u32x2_t hi = u32x2_t{__builtin_amdgcn_perm(v[1], v[0], 0x07060302u),
                                   __builtin_amdgcn_perm(v[3], v[2], 0x07060302u)};
        // channel 2 l + 1 sits one channel pitch after 2 l: (2 l + 1) / 4 = 2 l / 4
        const int wd = xs_word(2 * lane, sl / 3, sl % 3);
        *reinterpret_cast<u32x2_t*>(Xs + wd) = lo;
        *reinterpret_cast<u32x2_t*>(Xs + wd + kXPitch) = hi;
      }
    };

    f32x4_t ring[4][2];
  #pragma unroll
    for (int sl = 0; sl < 4; ++sl) ring[sl][0] = ring[sl][1] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // SiLU of the last finished output frame, stored one step later (block 1 stays
    // zero in a half tile)
    f32x4_t pend[2] = {f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}};

    const int orow = 4 * hh + n;  // this lane's output row in the tile
    const int gi_out = r0 + orow;
    const int ylane = (gi_out * Wl + c0) * d + ch;  // in-frame offset (the frame is < 2^31 bytes)
    // the finished output frame t_out from pend: scale (K: by the inverse norms of
    // its 8 positions, from invs) and store it, a channel pair per 4-byte store
    auto finish = [&](int t_out) {
      if (!gact || gi_out >= Hl) return;
      f32x4_t sc[2] = {f32x4_t{1.0f, 1.0f, 1.0f, 1.0f}, f32x4_t{1.0f, 1.0f, 1.0f, 1.0f}};
      if (NORM) {
        sc[0] = *reinterpret_cast<const f32x4_t*>(Is + orow * 8);
        sc[1] = *reinterpret_cast<const f32x4_t*>(Is + orow * 8 + 4);
      }
      // lanes l and l ^ 4 hold channels 2 j and 2 j + 1 of the same row: the even
      // one stores both channels of columns 0 .. 3, the odd one of columns 4 .. 7,
      // one 4-byte store per column (DPP row rotations by 4 and 12 reach l ^ 4)
      const bool odd = (lane >> 2) & 1;
      float v[8];
  #pragma unroll
      for (int xb = 0; xb < 2; ++xb)
  #pragma unroll
        for (int m = 0; m < 4; ++m) v[4 * xb + m] = pend[xb][m] * sc[xb][m];
      uint32_t* const yt = reinterpret_cast<uint32_t*>(y + ((size_t)unit * F + t_out) * U * d +
                                                        ylane - (odd ? 1 : 0));
  #pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int send = __float_as_int(odd ? v[i] : v[4 + i]);
        // even 4-lane banks (odd = 0) take lane + 4 (row_ror:12), odd banks lane - 4
        // (row_ror:4); each DPP writes only its banks and leaves the others as they were
        const int t12 = __builtin_amdgcn_update_dpp(send, send, 0x12C, 0xF, 0x5, false);
        const float got = __int_as_float(__builtin_amdgcn_update_dpp(t12, send, 0x124, 0xF, 0xA, false));
        const int col = (odd ? 4 : 0) + i;
        const uint32_t wv = pack_bf16(odd ? got : v[i], odd ? v[4 + i] : got);
        if (c0 + col < Wl) yt[(size_t)col * (d >> 1)] = wv;
      }
    };

    auto step = [&](int tin, auto kc) {
      constexpr int k = decltype(kc)::value;  // tin mod 4
      constexpr int fin = (k + 2) % 4;        // slot of output tin - 2, then of tin + 2
      __syncthreads();                        // staged tile tin and the inverse norms of tin - 3
      f32x4_t acc[2] = {f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}};
      if (half && gact && tin < F) {
  #pragma unroll
        for (int a = 0; a < 5; ++a) {
          const int hr = orow + a;
          const u32x2_t x0 = *reinterpret_cast<const u32x2_t*>(Xs + xs_word(ch, hr, 0));
          const u32x2_t x1 = *reinterpret_cast<const u32x2_t*>(Xs + xs_word(ch, hr, 1));
          const u32x2_t h0 = *reinterpret_cast<const u32x2_t*>(Wt + wt_word(ch, a, 0, 0, n));
          const u32x2_t l0 = *reinterpret_cast<const u32x2_t*>(Wt + wt_word(ch, a, 0, 1, n));
          const u32x2_t h1 = *reinterpret_cast<const u32x2_t*>(Wt + wt_word(ch, a, 1, 0, n));
          const u32x2_t l1 = *reinterpret_cast<const u32x2_t*>(Wt + wt_word(ch, a, 1, 1, n));
          acc[0] = mfma4(h0, x0, acc[0]);
          acc[0] = mfma4(l0, x0, acc[0]);
          acc[0] = mfma4(h1, x1, acc[0]);
          acc[0] = mfma4(l1, x1, acc[0]);
        }
      } else if (!half && gact && tin < F) {
  #pragma unroll
        for (int a = 0; a < 5; ++a) {
          const int hr = orow + a;
          const u32x2_t x0 = *reinterpret_cast<const u32x2_t*>(Xs + xs_word(ch, hr, 0));
          const u32x2_t x1 = *reinterpret_cast<const u32x2_t*>(Xs + xs_word(ch, hr, 1));
          const u32x2_t x2 = *reinterpret_cast<const u32x2_t*>(Xs + xs_word(ch, hr, 2));
          const u32x2_t h0 = *reinterpret_cast<const u32x2_t*>(Wt + wt_word(ch, a, 0, 0, n));
          const u32x2_t l0 = *reinterpret_cast<const u32x2_t*>(Wt + wt_word(ch, a, 0, 1, n));
          const u32x2_t h1 = *reinterpret_cast<const u32x2_t*>(Wt + wt_word(ch, a, 1, 0, n));
          const u32x2_t l1 = *reinterpret_cast<const u32x2_t*>(Wt + wt_word(ch, a, 1, 1, n));
          acc[0] = mfma4(h0, x0, acc[0]);
          acc[1] = mfma4(h0, x1, acc[1]);
          acc[0] = mfma4(l0, x0, acc[0]);
          acc[1] = mfma4(l0, x1, acc[1]);
          acc[0] = mfma4(h1, x1, acc[0]);
          acc[1] = mfma4(h1, x2, acc[1]);
          acc[0] = mfma4(l1, x1, acc[0]);
          acc[1] = mfma4(l1, x2, acc[1]);
        }
      }
      // output tin - 3 (finished last step) leaves while the products run
      if (tin >= 3) finish(tin - 3);
      // input frame tin feeds output frame tin + 2 - tau with w_t[tau]
      float ft[5];
  #pragma unroll
      for (int i = 0; i < 5; ++i) ft[i] = Ft[i * 128 + ch];
      f32x4_t out[2];
      out[1] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  #pragma unroll
      for (int xb = 0; xb < 2; ++xb) {
        if (xb == 1 && half) break;
        out[xb] = ring[fin][xb] + ft[4] * acc[xb];  // output tin - 2 is complete
        ring[fin][xb] = ft[0] * acc[xb];            // output tin + 2 starts
        ring[(k + 3) % 4][xb] += ft[3] * acc[xb];   // tin - 1
        ring[k][xb] += ft[2] * acc[xb];             // tin
        ring[(k + 1) % 4][xb] += ft[1] * acc[xb];   // tin + 1
      }
      const bool emit = tin >= 2;  // output tin - 2 exists
      if (emit) {
  #pragma unroll
        for (int xb = 0; xb < 2; ++xb) {
          if (xb == 1 && half) break;
  #pragma unroll
          for (int m = 0; m < 4; ++m) pend[xb][m] = silu(out[xb][m]);
        }
        if (NORM && gact) {
          // sum of squares over the wave's 16 channels (lane bits 2 .. 5) of each
          // of the lane's 8 positions, halving butterfly: the lane ends holding
          // position column e = 4 bit5 + 2 bit4 + bit3 of its row
          const bool h5 = lane & 32, h4 = lane & 16, h3 = lane & 8;
          float a4[4];
  #pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v0 = pend[0][i] * pend[0][i], v1 = pend[1][i] * pend[1][i];
            a4[i] = (h5 ? v1 : v0) + lane_xor32(h5 ? v0 : v1);
          }
          float a2[2];
  #pragma unroll
          for (int i = 0; i < 2; ++i)
            a2[i] = (h4 ? a4[i + 2] : a4[i]) + lane_xor16(h4 ? a4[i] : a4[i + 2]);
          const float keep = h3 ? a2[1] : a2[0];
          const float send = h3 ? a2[0] : a2[1];
          float s1 = keep + __int_as_float(__builtin_amdgcn_update_dpp(
                                0, __float_as_int(send), 0x128, 0xF, 0xF, false));  // lane ^ 8
          s1 += __shfl_xor(s1, 4);
          if (!(lane & 4)) Rs[g * 64 + orow * 8 + (h5 ? 4 : 0) + (h4 ? 2 : 0) + (h3 ? 1 : 0)] = s1;
        }
      }
      __syncthreads();  // every wave is done with the staged tile; partial sums complete
      if (emit && NORM && t < 64) {
        float ss = 0.0f;
        for (int gg = 0; gg < (d >> 4); ++gg) ss += Rs[gg * 64 + t];
        Is[t] = 1.0f / fmaxf(sqrtf(ss), eps);
      }
      if (tin + 1 < F) store_frame();
      if (tin + 2 < F) load_frame(tin + 2);  // in flight during the next frame's products
    };

    if (F > 0) {
      load_frame(0);
      store_frame();
      if (F > 1) load_frame(1);
    }
    for (int tb = 0; tb < F + 2; tb += 4) {
      step(tb, std::integral_constant<int, 0>{});
      if (tb + 1 < F + 2) step(tb + 1, std::integral_constant<int, 1>{});
      if (tb + 2 < F + 2) step(tb + 2, std::integral_constant<int, 2>{});
      if (tb + 3 < F + 2) step(tb + 3, std::integral_constant<int, 3>{});
    }
    if (F > 0) {
      __syncthreads();  // the inverse norms of the last output frame
      finish(F - 1);
    }
  };
  // a half tile (at most 4 columns left in the frame): only output column block
  // 0 exists, so halo column slot 2, column block 1's products and its temporal
  // filter and SiLU are left out (a body of its own)
  const bool half = (int)((item % ntiles) % tiles_c) * kTC + 4 >= Wl;
  if (norm) {
    if (half)
      sweep(std::true_type{}, std::true_type{});
    else
      sweep(std::true_type{}, std::false_type{});
  } else {
    if (half)
      sweep(std::false_type{}, std::true_type{});
    else
      sweep(std::false_type{}, std::false_type{});
  }
}

template <typename T>
hipError_t launch_prep_typed(const PrepPlan& p, const void* q, const void* k, const void* v,
                             const float* wk_s, const float* wk_t, const float* wv_s,
                             const float* wv_t, void* qo, void* ko, void* vo, hipStream_t s) {
  const long rows = (long)p.batch * p.F * p.U * p.H;
  if (rows > 0) {
    const unsigned per = xcd_per((unsigned)(p.batch * p.H) * p.tiles_r * p.tiles_c);
    const ConvSide<T> ks{static_cast<const T*>(k), wk_s, wk_t, static_cast<T*>(ko), p.dk};
    const ConvSide<T> vs{static_cast<const T*>(v), wv_s, wv_t, static_cast<T*>(vo), p.dv};
    const unsigned qblocks = q ? kQBlocks : 0;  // no query pass without q
    if constexpr (std::is_same<T, uint16_t>::value)
      hipLaunchKernelGGL(prep_mfma_kernel, dim3(2 * kXcds * per + qblocks), dim3(kPrepThreads), 0,
                         s, ks, vs, p.F, p.Hl, p.Wl, p.H, p.tiles_r, p.tiles_c, p.batch * p.H, per,
                         p.eps, static_cast<const T*>(q), static_cast<T*>(qo), rows, p.dk, qblocks);
    else
      hipLaunchKernelGGL(prep_conv_kernel<T>, dim3(2 * kXcds * per + qblocks), dim3(kPrepThreads),
                         0, s, ks, vs, p.F, p.Hl, p.Wl, p.H, p.tiles_r, p.tiles_c, p.batch * p.H,
                         per, p.eps, static_cast<const T*>(q), static_cast<T*>(qo), rows, p.dk,
                         qblocks);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prep(const PrepPlan& p, const void* q, const void* k, const void* v,
                       const float* wk_s, const float* wk_t, const float* wv_s, const float* wv_t,
                       void* qo, void* ko, void* vo, hipStream_t s) {
  if (p.dtype == VDA_DTYPE_BF16)
    return launch_prep_typed<uint16_t>(p, q, k, v, wk_s, wk_t, wv_s, wv_t, qo, ko, vo, s);
  return launch_prep_typed<float>(p, q, k, v, wk_s, wk_t, wv_s, wv_t, qo, ko, vo, s);
}

}  // namespace vda
