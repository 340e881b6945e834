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

// Value of lane ^ 32 and of lane ^ 16, by gfx950's row-swap permutes (VALU
// instructions, no LDS round trip).  permlane32_swap(x, x) returns
// {[x_lo, x_lo], [x_hi, x_hi]} (halves of 32 lanes), permlane16_swap(x, x)
// returns {rows [x0, x0, x2, x2], rows [x1, x1, x3, x3]} (rows of 16 lanes).
__device__ __forceinline__ float lane_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(lane_id() < 32 ? r[1] : r[0]);
}
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


template <typename T>
hipError_t launch_prep_typed(const PrepPlan& p, const void* q, const void* k, const void* v,
                             const float* wk_s, const float* wk_t, const float* wv_s,
                             const float* wv_t, void* qo, void* ko, void* vo, hipStream_t s) {
  const long rows = (long)p.batch * p.F * p.U * p.H;
  if (rows > 0) {
    const unsigned per = xcd_per((unsigned)(p.batch * p.H) * p.tiles_r * p.tiles_c);
    const ConvSide<T> ks{static_cast<const T*>(k), wk_s, wk_t, static_cast<T*>(ko), p.dk};
    const ConvSide<T> vs{static_cast<const T*>(v), wv_s, wv_t, static_cast<T*>(vo), p.dv};
    const unsigned qblocks = kQBlocks;
    hipLaunchKernelGGL(prep_conv_kernel<T>, dim3(2 * kXcds * per + qblocks), dim3(kPrepThreads), 0,
                       s, ks, vs, p.F, p.Hl, p.Wl, p.H, p.tiles_r, p.tiles_c, p.batch * p.H, per,
                       p.eps, static_cast<const T*>(q), static_cast<T*>(qo), rows, p.dk, qblocks);
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
