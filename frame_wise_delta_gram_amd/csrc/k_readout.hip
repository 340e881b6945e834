// Readout of the bidirectional linear memory ("Video DeltaNet", arXiv
// 2609.20744, Sec. 2.2 Eq. (1a), App. A.3 Eq. (A.4) with alpha = 1, Sec. 2.3
// Eq. (1c)), fused with the gather and the epilogue:
//
//   gather:  a query of chunk c reads S~ = P[max(c - r, 0)] + R[min(c + r + 1, n)]
//            (forward state of the chunks before the window, reverse state of
//            those after it; the two regions are disjoint)
//   readout: o = S~ q                              (d_v outputs per token)
//   epilogue: out = sigmoid(g) * w * o / sqrt(mean(o^2) + eps)
//
// bf16 path.  One workgroup per (unit, chunk, row block); all frames of a
// chunk share S~.  A chunk's rows are cut into 128-row pieces dealt round-robin
// to its nblk workgroups (workgroup b takes pieces b, b + nblk, b + 2 nblk,
// b + 3 nblk), so the workgroups of a chunk sweep its rows side by side (on
// MI355X about 2% faster than contiguous 1024-row blocks per workgroup).  S~ is formed in fp32, split into a bf16 high
// part and a bf16 residual (S~ = hi + lo to ~2^-17 relative) and kept in LDS,
// so the readout is two bf16 MFMAs with fp32 accumulation and the HBM-bound
// stream of q, gate and out never waits on a conversion.  The transposed
// product O^T = S~ Q^T runs on v_mfma_f32_16x16x32_bf16 with q as the B
// operand, loaded straight from HBM: lane l serves token l % 16, and the four
// lanes of a token read four consecutive 16-byte pieces of its row, so one
// load instruction covers 16 rows x 64 contiguous bytes (measured on MI355X as
// fast as fully contiguous streaming, where 32 rows x 16 bytes per instruction
// lose about a quarter of the bandwidth).  S~'s rows are stored permuted so
// that accumulator register r of tile T in lane group h = l / 16 holds output
// channel 32 (T / 2) + 8 h + 4 (T % 2) + r: each lane ends with four
// 8-channel groups of its token (channels 32 m + 8 h .. + 7), gate loads and output stores are
// 16-byte vectors in the same 16-rows x 64-bytes pattern, and the RMSNorm
// reduction is a lane-local sum plus two cross-lane adds.  Math in the
// epilogue is fp32; the output is rounded to bf16 (nearest even).
//
// With channel-wise decay (App. A.3 Eq. (A.4) with alpha_t in [0, 1]^{d_k}) the
// gathered state depends on the frame: frame f of chunk c reads
//   S~_f = P[max(c - r, 0)] Diag(prod_{s=l}^{f} alpha_s)
//        + R[min(c + r + 1, n)] Diag(prod_{s=f}^{h} alpha_s),
// [l, h] = the window's frames C max(c - r, 0) .. min(C (c + r + 1), F) - 1.
// The work is then split by frame instead of by chunk (a segment is one frame),
// the two channel-wise products are formed in LDS by the workgroup before the
// gather, and the gather scales P's and R's columns by them.
//
// Boundary anchors (Sec. 2.1, App. A.3, Algorithm 1 step 7): frames 0 and F - 1
// wrote nothing into the states (they are identity frames there, so the
// chunk-indexed states and the window clipped to the interior frames agree),
// carry no gate in the bridge products, and their rows are written as zeros,
// as are all rows of a segment whose window spans the whole clip (bypass).
//
// fp32 path: the same computation on the vector ALUs in fp32.
#include "vda_device.h"
#include "vda_internal.h"

namespace vda {
namespace {

constexpr int kThreadsR = 512;            // 8 waves; two workgroups per CU
constexpr int kGroups = 4;                // 16-row groups per wave (one per 128-row piece)
constexpr int kRows = 8 * 16 * kGroups;   // token rows per workgroup

// Channel-wise decay products of the bridge for frame f of chunk c, by threads
// 0 .. 255 of the workgroup: D[k] = prod_{s=l}^{f} alpha_s[k] (applied to P's
// column k), D[128 + k] = prod_{s=f}^{h} alpha_s[k] (R's); zero past d_k.  The
// gates are read eight frames at a time (independent loads).
__device__ __forceinline__ void bridge_products(float* D, const float* alpha, int u, int f, int c,
                                                int F, int C, int radius, int dk, int anchors) {
  const int t = threadIdx.x;
  if (t >= 256) return;
  const int k = t & 127;
  const bool rev = t >= 128;
  const long l = (long)C * max(c - radius, 0);
  const long hw = (long)C * (c + radius + 1);
  const int s0 = rev ? f : (int)l;
  const int s1 = rev ? (int)(hw < F ? hw : F) - 1 : f;
  float d = 1.0f;
  if (k < dk) {
    const float* a = alpha + (size_t)u * F * dk + k;
    for (int s = s0; s <= s1; s += 8) {
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int g = s + i;
        const bool one = g > s1 || (anchors && (g == 0 || g == F - 1));
        x[i] = one ? 1.0f : a[(size_t)g * dk];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) d *= x[i];
    }
  }
  D[t] = k < dk ? d : 0.0f;
}

// Rows of a segment (frames f0 .. f1-1 of chunk c, U rows each) that get linear
// output: [zlo, zhi).  Without anchors, all of them.  With anchors, none when
// the window (chunks c - radius .. c + radius) spans the whole clip, else all
// but the rows of frames 0 and F - 1.
__device__ __forceinline__ void live_rows(int anchors, int f0, int f1, int c, int F, int U, int C,
                                          int radius, long rows_total, long& zlo, long& zhi) {
  zlo = 0;
  zhi = rows_total;
  if (!anchors) return;
  if (c - radius <= 0 && (long)C * (c + radius + 1) >= F) {
    zhi = 0;
    return;
  }
  if (f0 == 0) zlo = U;
  if (f1 == F) zhi = (long)(F - 1 - f0) * U;
}

// DK, DV > 0: compile-time d_k and d_v (the common 128 case); 0: runtime.
// DECAY: one segment per frame, bridged gather (see header); else one segment
// per chunk.
template <int DK, int DV, bool DECAY>
__global__ __launch_bounds__(512, 4) void readout_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ gate,
    const float* __restrict__ wrms, uint16_t* __restrict__ out, const float* __restrict__ ST,
    const float* __restrict__ alpha, int dk_rt, int dv_rt, int F, int U, int C, int radius, int n,
    float eps, int units, int nseg, int nblk, unsigned per, int anchors, int qh, float rqeps) {
  const int dk = DK > 0 ? DK : dk_rt;
  const int dv = DV > 0 ? DV : dv_rt;
  __shared__ __align__(16) uint16_t Shi[128 * 136];
  __shared__ __align__(16) uint16_t Slo[128 * 136];
  __shared__ __align__(16) float Ws[128];  // RMSNorm weight (LDS: its reads use lgkmcnt, not vmcnt)
  __shared__ __align__(16) float Dbr[DECAY ? 256 : 1];  // bridge products (P: 0.., R: 128..)

  // work item = (unit, segment, row block), row block fastest: the blocks of
  // one segment (which all read the same two states) share an XCD; with q in
  // the projection layout unit u reads head u % qh of entry u / qh
  const unsigned item = xcd_item(per);
  if (item >= (unsigned)units * nseg * nblk) return;
  const int blk = item % nblk;
  const int seg = (item / nblk) % nseg;
  const int u = item / (nblk * nseg);
  const int hq = u % qh;
  const int c = DECAY ? seg / C : seg;
  const int f0 = DECAY ? seg : c * C;
  const int f1 = DECAY ? seg + 1 : min(f0 + C, F);
  const long rows_total = (long)(f1 - f0) * U;
  const long row0 = (long)blk * 128;  // first of the workgroup's 128-row pieces
  if (row0 >= rows_total) return;
  long zlo, zhi;  // rows [zlo, zhi) of the segment get linear output
  live_rows(anchors, f0, f1, c, F, U, C, radius, rows_total, zlo, zhi);

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int Dvp = pad32(dv);   // output channels incl. padding (pairs of 16-channel tiles)
  const int NT = Dvp >> 4;     // 16-channel output tiles (even)
  const int Dkp = pad32(dk);   // contraction incl. padding
  const int NKS = Dkp >> 5;    // k-steps of 32 channels
  const int SROW = 136;        // LDS row stride (bf16 elements): 17 x 16 bytes

  if (t < 128) Ws[t] = t < dv ? wrms[t] : 0.0f;
  if (DECAY) {
    bridge_products(Dbr, alpha, u, f0, c, F, C, radius, dk, anchors);
    __syncthreads();
  }
  // gather S~ and split it into bf16 hi + lo, rows permuted (see header);
  // padding rows and columns are zero
  {
    const size_t SS = (size_t)dv * dk;
    const int pi = max(c - radius, 0);
    const int ri = min(c + radius + 1, n);
    const float* P = ST + ((size_t)(u * 2 + 0) * (n + 1) + pi) * SS;
    const float* R = ST + ((size_t)(u * 2 + 1) * (n + 1) + ri) * SS;
    const int k8n = Dkp >> 3;
    const int items = Dvp * k8n;  // <= 2048 = 4 per thread, in two rounds of 2
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      f32x4_t pv[2][2], rv[2][2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {  // issue the round's loads first
        const int it = t + kThreadsR * (2 * half + i);
        const int ch = it / k8n;
        const int k8 = it - ch * k8n;
        const f32x4_t z = {0.0f, 0.0f, 0.0f, 0.0f};
        const bool ok = it < items && ch < dv && 8 * k8 < dk;
        const f32x4_t* pp = reinterpret_cast<const f32x4_t*>(P + (size_t)(ok ? ch : 0) * dk + (ok ? 8 * k8 : 0));
        const f32x4_t* rp = reinterpret_cast<const f32x4_t*>(R + (size_t)(ok ? ch : 0) * dk + (ok ? 8 * k8 : 0));
        pv[i][0] = ok ? pp[0] : z;
        pv[i][1] = ok ? pp[1] : z;
        rv[i][0] = ok ? rp[0] : z;
        rv[i][1] = ok ? rp[1] : z;
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int it = t + kThreadsR * (2 * half + i);
        if (it >= items) continue;
        const int ch = it / k8n;
        const int k8 = it - ch * k8n;
        // channel ch = 32 m + 8 h + 4 (T % 2) + r  ->  LDS row 16 T + 4 h + r
        const int T = 2 * (ch >> 5) + ((ch >> 2) & 1);
        const int lrow = 16 * T + 4 * ((ch >> 3) & 3) + (ch & 3);
        float x[8];
        if (DECAY) {
          f32x4_t df[2], dr[2];
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            df[j] = *reinterpret_cast<const f32x4_t*>(Dbr + 8 * k8 + 4 * j);
            dr[j] = *reinterpret_cast<const f32x4_t*>(Dbr + 128 + 8 * k8 + 4 * j);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[e] = pv[i][0][e] * df[0][e] + rv[i][0][e] * dr[0][e];
            x[4 + e] = pv[i][1][e] * df[1][e] + rv[i][1][e] * dr[1][e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[e] = pv[i][0][e] + rv[i][0][e];
            x[4 + e] = pv[i][1][e] + rv[i][1][e];
          }
        }
        u32x4_t hi, lo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t hp = pack_bf16(x[2 * e], x[2 * e + 1]);
          hi[e] = hp;
          lo[e] = pack_bf16(x[2 * e] - bf16_lo(hp), x[2 * e + 1] - bf16_hi(hp));
        }
        *reinterpret_cast<u32x4_t*>(Shi + lrow * SROW + 8 * k8) = hi;
        *reinterpret_cast<u32x4_t*>(Slo + lrow * SROW + 8 * k8) = lo;
      }
    }
  }
  __syncthreads();

  const int h = lane >> 4;      // lane group: k slots of the operands, output channel group
  const int jl = lane & 15;     // token within a 16-row group
  const size_t chunk_row0 = ((size_t)u * F + f0) * U;
  const float inv_dv = 1.0f / (float)dv;
  const u32x4_t z4 = {0u, 0u, 0u, 0u};
  const bool kpad = (dk & 31) != 0;  // last k-step partly past d_k

  // Loads are unconditional from clamped, valid addresses (rows past the chunk's
  // end reread its last row, channel groups past d_k / d_v reread the last valid
  // one); such rows are never stored, padded S~ columns are zero (and the
  // partly padded k-step is masked), padded output channels are never stored.
  // One 16-row group: 4 k-steps of q (fetched one group ahead) and 4 channel
  // groups of gate (fetched when the group starts: first used after its MFMAs).
  auto grow_of = [&](long rg) { return chunk_row0 + (size_t)min(rg + jl, rows_total - 1); };
  // the segment's first query row (row stride qh x d_k)
  const uint16_t* qbase = q + ((((size_t)(u / qh) * F + f0) * U) * qh + hq) * dk;
  auto load_q = [&](u32x4_t (&qr)[4], long rg) {
    const uint16_t* qp = qbase + (size_t)min(rg + jl, rows_total - 1) * qh * dk;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qr[s] = *reinterpret_cast<const u32x4_t*>(qp + min(32 * s + 8 * h, dk - 8));
  };
  auto load_g = [&](u32x4_t (&gr)[4], long rg) {
    const uint16_t* gp = gate + grow_of(rg) * dv;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      gr[m] = *reinterpret_cast<const u32x4_t*>(gp + min(32 * m + 8 * h, dv - 8));
  };

  // one 16-row group: MFMAs on qr, then the RMSNorm/gate epilogue and the stores
  auto process = [&](const u32x4_t (&qr)[4], const u32x4_t (&gr)[4], long rg) {
    f32x4_t acc[8];
#pragma unroll
    for (int T = 0; T < 8; ++T) acc[T] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    float qq = 0.0f;  // the token's ||q||^2 (query map only)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s >= NKS) continue;
      u32x4_t b0 = qr[s];
      if (kpad && 32 * s + 8 * h >= dk) b0 = z4;
      if (rqeps > 0.0f)
#pragma unroll
        for (int d = 0; d < 4; ++d) qq = dot2_bf16(b0[d], b0[d], qq);
#pragma unroll
      for (int T = 0; T < 8; ++T) {
        if (T >= NT) continue;
        const int off = (16 * T + jl) * SROW + 32 * s + 8 * h;
        const u32x4_t ah = *reinterpret_cast<const u32x4_t*>(Shi + off);
        const u32x4_t al = *reinterpret_cast<const u32x4_t*>(Slo + off);
        acc[T] = mfma16_bf16(ah, b0, acc[T]);
        acc[T] = mfma16_bf16(al, b0, acc[T]);
      }
    }
    // RMSNorm over the token's d_v outputs: 4 lanes x 32 channels each
    float ss = 0.0f;
#pragma unroll
    for (int T = 0; T < 8; ++T)
#pragma unroll
      for (int r = 0; r < 4; ++r) ss = fmaf(acc[T][r], acc[T][r], ss);
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    // RMSNorm of o' = rn o, rn = 1 / max(||q||, q_l2_eps) with the query map, else 1
    float rn = 1.0f;
    if (rqeps > 0.0f) {
      qq += __shfl_xor(qq, 16);
      qq += __shfl_xor(qq, 32);
      rn = fminf(rsqrtf(qq), rqeps);
    }
    const float inv = rn * rsqrtf(ss * (rn * rn) * inv_dv + eps);
    const long myrow = rg + jl;
    const bool live = myrow >= zlo && myrow < zhi;
    if (myrow < rows_total) {
      const size_t grow = chunk_row0 + (size_t)myrow;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int ch = 32 * m + 8 * h;
        if (ch >= dv) continue;
        const f32x4_t w0 = *reinterpret_cast<const f32x4_t*>(Ws + ch);
        const f32x4_t w1 = *reinterpret_cast<const f32x4_t*>(Ws + ch + 4);
        const u32x4_t gv = gr[m];
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float o = acc[2 * m + (e >> 2)][e & 3];
          const float gl = (e & 1) ? bf16_hi(gv[e >> 1]) : bf16_lo(gv[e >> 1]);
          const float ww = e < 4 ? w0[e] : w1[e - 4];
          const float sig = __builtin_amdgcn_rcpf(1.0f + __expf(-gl));
          y[e] = live ? o * inv * ww * sig : 0.0f;
        }
        u32x4_t ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = pack_bf16(y[2 * e], y[2 * e + 1]);
        *reinterpret_cast<u32x4_t*>(out + grow * dv + ch) = ov;
      }
    }
  };

  // wave w takes rows 16 w .. 16 w + 15 of each of the workgroup's pieces; q
  // ping-pongs between two register sets, unrolled by two (no register copies
  // between groups)
  u32x4_t q0[4], q1[4], gr[4];
  auto grp_row = [&](int it) { return ((long)it * nblk + blk) * 128 + (long)w * 16; };
  load_q(q0, grp_row(0));
  for (int it = 0; it < kGroups; it += 2) {
    if (grp_row(it) >= rows_total) break;
    load_g(gr, grp_row(it));
    if (it + 1 < kGroups) load_q(q1, grp_row(it + 1));
    process(q0, gr, grp_row(it));
    if (it + 1 >= kGroups || grp_row(it + 1) >= rows_total) break;
    load_g(gr, grp_row(it + 1));
    if (it + 2 < kGroups) load_q(q0, grp_row(it + 2));
    process(q1, gr, grp_row(it + 1));
  }
}

// ---------------------------------------------------------------------------
// bf16 with d_k = d_v = 128, no decay: the same readout in two kernels.
//
// (1) split_states_kernel: for every (unit, chunk) S~ = P[max(c - r, 0)] +
//     R[min(c + r + 1, n)] in fp32, split into bf16 hi + lo and written in the
//     readout's LDS image (hi rows, then lo rows, 136 bf16 per row, rows
//     permuted as below): 69632 bytes per chunk.
// (2) readout_c128_kernel: one workgroup (8 waves) per (unit, chunk, 256-row
//     block) copies its chunk's image into LDS with global_load_lds (68 x 1 KB,
//     no registers), then each wave runs two 16-row groups.
//
// Access pattern.  Every q / gate load and out store instruction covers 8
// rows x 128 contiguous bytes (eight full cache lines; the bytes are streamed,
// so the loads and stores are non-temporal): in the four instructions i =
// (i1, i0) of a 16-row group, lane l takes row 8 i1 + (l & 7) and 16-byte chunk
// 8 i0 + (l >> 3) of that row.  The MFMA operand wants token = l & 15, so one
// exchange of register bit i1 with lane bit 3 (DPP row_ror:8, which is lane
// xor 8 inside each row of 16 lanes, and a select) gives register s = (c0, c3)
// at lane (h = l >> 4, token l & 15) the chunk 8 (s & 1) + 2 h + (s >> 1) of
// its token.  That is the B operand of k-step s (the k order inside a step is
// a fixed permutation; S~'s columns are read in the same order), and, applied
// to gate, the epilogue's operand.  S~'s rows (output channels) are permuted
// so that the accumulators of output register s are the 8 channels of the
// same chunk, so the outputs go back through the same exchange and leave as
// 8 rows x 128 B stores.
constexpr int kSRow = 136;                      // bf16 per LDS row of S~ (17 x 16 bytes)
constexpr int kSplitBytes = 2 * 128 * kSRow * 2;  // hi + lo image of one chunk's S~
static_assert(kSplitBytes == 2 * kSplitElems, "split image size");

// chunk of 8 channels held in output register s by lane group h
__device__ __forceinline__ int c128_chunk(int s, int h) { return 8 * (s & 1) + 2 * h + (s >> 1); }
// LDS row of S~'s output channel ch: tile T = 2 s + (e >> 2), row 4 h + (e & 3)
__device__ __forceinline__ int c128_row(int ch) {
  const int chunk = ch >> 3, e = ch & 7;
  const int s = 2 * (chunk & 1) + (chunk >> 3);
  const int h = (chunk >> 1) & 3;
  return 16 * (2 * s + (e >> 2)) + 4 * h + (e & 3);
}

// Work item (unit, segment) on a 1-D grid, segment fastest: the segments of a
// unit that read the same two states run side by side on one XCD (its L2).
// DECAY: one image per frame (segment = frame f of chunk c = f / C), S~_f =
// P Diag(bridge of P) + R Diag(bridge of R) with the window's gate products.
template <bool DECAY>
__global__ __launch_bounds__(256) void split_states_kernel(const float* __restrict__ ST,
                                                           const float* __restrict__ alpha,
                                                           uint16_t* __restrict__ Sp, int n,
                                                           int radius, int F, int C, int anchors,
                                                           int units, unsigned per) {
  __shared__ __align__(16) float Dbr[DECAY ? 256 : 1];  // bridge products (P: 0.., R: 128..)
  const int nseg = DECAY ? F : n;
  const unsigned item = xcd_item(per);
  if (item >= (unsigned)units * nseg) return;
  const int seg = item % nseg;
  const int u = item / nseg;
  const int c = DECAY ? seg / C : seg;
  if (DECAY) {
    bridge_products(Dbr, alpha, u, seg, c, F, C, radius, 128, anchors);
    __syncthreads();
  }
  const size_t SS = 128 * 128;
  const float* P = ST + ((size_t)(u * 2 + 0) * (n + 1) + max(c - radius, 0)) * SS;
  const float* R = ST + ((size_t)(u * 2 + 1) * (n + 1) + min(c + radius + 1, n)) * SS;
  uint16_t* dst = Sp + ((size_t)u * nseg + seg) * (kSplitBytes / 2);
  for (int it = threadIdx.x; it < 128 * 17; it += kThreads) {
    const int ch = it / 17, k8 = it - 17 * (it / 17);
    u32x4_t hi = {0u, 0u, 0u, 0u}, lo = {0u, 0u, 0u, 0u};
    if (k8 < 16) {  // column group 16 is the row's padding
      const f32x4_t* pp = reinterpret_cast<const f32x4_t*>(P + (size_t)ch * 128 + 8 * k8);
      const f32x4_t* rp = reinterpret_cast<const f32x4_t*>(R + (size_t)ch * 128 + 8 * k8);
      const f32x4_t p0 = pp[0], p1 = pp[1], r0 = rp[0], r1 = rp[1];
      float x[8];
      if (DECAY) {
        const f32x4_t df0 = *reinterpret_cast<const f32x4_t*>(Dbr + 8 * k8);
        const f32x4_t df1 = *reinterpret_cast<const f32x4_t*>(Dbr + 8 * k8 + 4);
        const f32x4_t dr0 = *reinterpret_cast<const f32x4_t*>(Dbr + 128 + 8 * k8);
        const f32x4_t dr1 = *reinterpret_cast<const f32x4_t*>(Dbr + 128 + 8 * k8 + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = p0[e] * df0[e] + r0[e] * dr0[e];
          x[4 + e] = p1[e] * df1[e] + r1[e] * dr1[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = p0[e] + r0[e];
          x[4 + e] = p1[e] + r1[e];
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t hp = pack_bf16(x[2 * e], x[2 * e + 1]);
        hi[e] = hp;
        lo[e] = pack_bf16(x[2 * e] - bf16_lo(hp), x[2 * e + 1] - bf16_hi(hp));
      }
    }
    const int lr = c128_row(ch);
    *reinterpret_cast<u32x4_t*>(dst + lr * kSRow + 8 * k8) = hi;
    *reinterpret_cast<u32x4_t*>(dst + 128 * kSRow + lr * kSRow + 8 * k8) = lo;
  }
}

__device__ __forceinline__ uint32_t lane_xor8(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128 /* row_ror:8 */, 0xF, 0xF, false);
}
// exchange register bit 1 with lane bit 3 (b3) across X[0..3]; every lane runs it
// (the DPP reads other lanes), so both rotated values are formed before selecting
__device__ __forceinline__ void c128_exchange(u32x4_t (&X)[4], bool b3) {
#pragma unroll
  for (int lo = 0; lo < 2; ++lo) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t a = X[lo][d], b = X[lo + 2][d];
      const uint32_t ra = lane_xor8(a), rb = lane_xor8(b);
      X[lo][d] = b3 ? rb : a;
      X[lo + 2][d] = b3 ? b : ra;
    }
  }
}

constexpr int kGroupsC = 2;                       // 16-row groups per wave
constexpr int kRowsC = 8 * 16 * kGroupsC;         // token rows per workgroup

// QN: the query map (each query row L2-normalised in the epilogue, rqeps =
// 1 / q_l2_eps); without it the kernel is the plain readout
template <bool QN>
__global__ __launch_bounds__(512, 4) void readout_c128_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ gate,
    const float* __restrict__ wrms, uint16_t* __restrict__ out, const uint16_t* __restrict__ Sp,
    int F, int U, int C, int radius, int n, float eps, int units, int nblk, unsigned per,
    int anchors, int per_frame, int qh, float rqeps) {
  __shared__ __align__(16) uint16_t S[kSplitBytes / 2];  // hi rows 0..127, lo rows 128..255
  __shared__ __align__(16) float Ws[128];
  // segments: chunks, or frames (per_frame: with decay each frame has its own S~)
  const int nseg = per_frame ? F : n;
  const unsigned item = xcd_item(per);
  if (item >= (unsigned)units * nseg * nblk) return;
  // work item (unit, segment, block), block fastest: the blocks of one segment
  // read the same image and share an XCD (its L2).  With q in the projection
  // layout (qh > 1) unit u reads head u % qh of entry u / qh; this order
  // measured faster than running the heads of one token block side by side
  const int blk = item % nblk;
  const int seg = (item / nblk) % nseg;
  const int u = item / (nblk * nseg);
  const int hq = u % qh;
  const int c = per_frame ? seg / C : seg;
  const int f0 = per_frame ? seg : c * C;
  const int f1 = per_frame ? seg + 1 : min(f0 + C, F);
  const long rows_total = (long)(f1 - f0) * U;
  if ((long)blk * 128 >= rows_total) return;
  long zlo, zhi;
  live_rows(anchors, f0, f1, c, F, U, C, radius, rows_total, zlo, zhi);

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int h = lane >> 4;
  const int jl = lane & 15;
  const bool b3 = (lane >> 3) & 1;
  const size_t chunk_row0 = ((size_t)u * F + f0) * U;
  const uint16_t* Shi = S;
  const uint16_t* Slo = S + 128 * kSRow;
  // the segment's first row of gate / out, and of q (row stride qh x 128)
  const uint16_t* gbase = gate + chunk_row0 * 128;
  const uint16_t* qbase = q + ((((size_t)(u / qh) * F + f0) * U) * qh + hq) * 128;
  const size_t qstride = (size_t)qh * 128;
  // lane's row (within a 16-row group) and 16-byte chunk in load / store instruction i
  auto row_in = [&](int i) { return 8 * (i >> 1) + (lane & 7); };
  auto chunk_in = [&](int i) { return 8 * (i & 1) + (lane >> 3); };
  auto load16 = [&](u32x4_t (&X)[4], const uint16_t* base, size_t stride, long rg) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const long r = min(rg + row_in(i), rows_total - 1);  // clamped: never stored
      X[i] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(base + (size_t)r * stride + 8 * chunk_in(i)));
    }
  };
  auto grp_row = [&](int it) { return ((long)it * nblk + blk) * 128 + (long)w * 16; };

  // S~ image -> LDS by DMA, then the first group's q and gate
  {
    const char* src = reinterpret_cast<const char*>(Sp + ((size_t)u * nseg + seg) * (kSplitBytes / 2));
    char* dst = reinterpret_cast<char*>(S);
    for (int j = w; j < kSplitBytes / 1024; j += 8)
      __builtin_amdgcn_global_load_lds(
          static_cast<const void*>(src + (size_t)j * 1024 + lane * 16),
          (void __attribute__((address_space(3)))*)(dst + j * 1024), 16, 0, 0);
  }
  if (t < 128) Ws[t] = wrms[t];
  u32x4_t q0[4], q1[4], gr[4], g1[4];
  load16(q0, qbase, qstride, grp_row(0));
  load16(gr, gbase, 128, grp_row(0));
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the DMA into LDS has landed
  __syncthreads();

  auto process = [&](u32x4_t (&qr)[4], u32x4_t (&g)[4], long rg) {
    c128_exchange(qr, b3);
    // with the query map: rn = 1 / max(||q||, q_l2_eps) of this lane's token
    // (its 128 channels: 32 per lane of the four lane groups)
    float rn = 1.0f;
    if (QN) {
      float qq = 0.0f;
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int d = 0; d < 4; ++d) qq = dot2_bf16(qr[s][d], qr[s][d], qq);
      qq += __shfl_xor(qq, 16);
      qq += __shfl_xor(qq, 32);
      rn = fminf(rsqrtf(qq), rqeps);
    }
    f32x4_t acc[8];
#pragma unroll
    for (int T = 0; T < 8; ++T) acc[T] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int col = 8 * c128_chunk(s, h);
#pragma unroll
      for (int T = 0; T < 8; ++T) {
        const int off = (16 * T + jl) * kSRow + col;
        const u32x4_t ah = *reinterpret_cast<const u32x4_t*>(Shi + off);
        const u32x4_t al = *reinterpret_cast<const u32x4_t*>(Slo + off);
        acc[T] = mfma16_bf16(ah, qr[s], acc[T]);
        acc[T] = mfma16_bf16(al, qr[s], acc[T]);
      }
    }
    c128_exchange(g, b3);
    float ss = 0.0f;
#pragma unroll
    for (int T = 0; T < 8; ++T)
#pragma unroll
      for (int r = 0; r < 4; ++r) ss = fmaf(acc[T][r], acc[T][r], ss);
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    // RMSNorm of o' = rn o (rn = 1 without the query map)
    const float inv = rn * rsqrtf(ss * (rn * rn) * (1.0f / 128.0f) + eps);
    const long myrow = rg + jl;
    const bool live = myrow >= zlo && myrow < zhi;
    u32x4_t ov[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int ch = 8 * c128_chunk(m, h);
      const f32x4_t w0 = *reinterpret_cast<const f32x4_t*>(Ws + ch);
      const f32x4_t w1 = *reinterpret_cast<const f32x4_t*>(Ws + ch + 4);
      const u32x4_t gv = g[m];
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float o = acc[2 * m + (e >> 2)][e & 3];
        const float gl = (e & 1) ? bf16_hi(gv[e >> 1]) : bf16_lo(gv[e >> 1]);
        const float ww = e < 4 ? w0[e] : w1[e - 4];
        const float sig = __builtin_amdgcn_rcpf(1.0f + __expf(-gl));
        y[e] = live ? o * inv * ww * sig : 0.0f;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) ov[m][e] = pack_bf16(y[2 * e], y[2 * e + 1]);
    }
    c128_exchange(ov, b3);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const long r = rg + row_in(i);
      if (r < rows_total)
        __builtin_nontemporal_store(ov[i], reinterpret_cast<u32x4_t*>(
            out + (chunk_row0 + (size_t)r) * 128 + 8 * chunk_in(i)));
    }
  };

  // two groups per wave: q and gate of the second are fetched before the first
  // is processed
  if (grp_row(0) >= rows_total) return;
  load16(q1, qbase, qstride, grp_row(1));
  load16(g1, gbase, 128, grp_row(1));
  process(q0, gr, grp_row(0));
  if (grp_row(1) >= rows_total) return;
  process(q1, g1, grp_row(1));
}

// fp32 features: 64 token rows per workgroup, S~ and the rows' queries in LDS.
// Work item (unit, segment, row block) on a 1-D grid, segments as in the bf16
// path (a frame with decay, given by alpha != nullptr; else a chunk).
constexpr int SG = 129;
constexpr int kRowsF = 64;

__global__ __launch_bounds__(256) void readout_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ gate, const float* __restrict__ wrms,
    float* __restrict__ out, const float* __restrict__ ST, const float* __restrict__ alpha, int dk,
    int dv, int F, int U, int C, int radius, int n, float eps, int nseg, int nblk, int anchors,
    int qh, float rqeps) {
  __shared__ float Ss[128 * SG];
  __shared__ float Qs[kRowsF * SG];
  __shared__ float Dbr[256];
  const bool decay = alpha != nullptr;
  // work item (unit, segment, row block); with q in the projection layout unit
  // u reads head u % qh of entry u / qh
  const unsigned item = blockIdx.x;
  const int blk = item % nblk;
  const int seg = (item / nblk) % nseg;
  const int u = item / (nblk * nseg);
  const int hq = u % qh;
  const int c = decay ? seg / C : seg;
  const int f0 = decay ? seg : c * C;
  const int f1 = decay ? seg + 1 : min(f0 + C, F);
  const long rows_total = (long)(f1 - f0) * U;
  const long row0 = (long)blk * kRowsF;
  if (row0 >= rows_total) return;
  long zlo, zhi;
  live_rows(anchors, f0, f1, c, F, U, C, radius, rows_total, zlo, zhi);
  const int t = threadIdx.x;
  const size_t SS = (size_t)dv * dk;
  const int pi = max(c - radius, 0);
  const int ri = min(c + radius + 1, n);
  const float* P = ST + ((size_t)(u * 2 + 0) * (n + 1) + pi) * SS;
  const float* R = ST + ((size_t)(u * 2 + 1) * (n + 1) + ri) * SS;
  if (decay) {
    bridge_products(Dbr, alpha, u, f0, c, F, C, radius, dk, anchors);
    __syncthreads();
  }
  for (int idx = t; idx < dv * dk; idx += 256) {
    const int i = idx / dk;
    const int j = idx - i * dk;
    Ss[i * SG + j] = decay ? P[idx] * Dbr[j] + R[idx] * Dbr[128 + j] : P[idx] + R[idx];
  }
  const size_t chunk_row0 = ((size_t)u * F + f0) * U;
  const float* qbase = q + ((((size_t)(u / qh) * F + f0) * U) * qh + hq) * dk;
  for (int idx = t; idx < kRowsF * dk; idx += 256) {
    const int i = idx / dk;
    const int j = idx - i * dk;
    const long row = row0 + i;
    Qs[i * SG + j] = row < rows_total ? qbase[(size_t)row * qh * dk + j] : 0.0f;
  }
  __syncthreads();
  const int lr = t >> 2;
  const int part = t & 3;
  const long myrow = row0 + lr;
  float o[32];
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const int ch = part + 4 * j;
    float a = 0.0f;
    if (ch < dv)
      for (int kx = 0; kx < dk; ++kx) a = fmaf(Ss[ch * SG + kx], Qs[lr * SG + kx], a);
    o[j] = a;
    ss = fmaf(a, a, ss);
  }
  ss += __shfl_xor(ss, 1);
  ss += __shfl_xor(ss, 2);
  // RMSNorm of o' = rn o, rn = 1 / max(||q||, q_l2_eps) with the query map, else 1
  float rn = 1.0f;
  if (rqeps > 0.0f) {
    float qq = 0.0f;
    for (int kx = part; kx < dk; kx += 4) qq = fmaf(Qs[lr * SG + kx], Qs[lr * SG + kx], qq);
    qq += __shfl_xor(qq, 1);
    qq += __shfl_xor(qq, 2);
    rn = fminf(1.0f / sqrtf(qq), rqeps);
  }
  const float inv = rn / sqrtf(ss * (rn * rn) / (float)dv + eps);
  if (myrow < rows_total) {
    const size_t grow = chunk_row0 + (size_t)myrow;
    const bool live = myrow >= zlo && myrow < zhi;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const int ch = part + 4 * j;
      if (ch < dv) {
        const float gl = gate[grow * dv + ch];
        out[grow * dv + ch] = live ? wrms[ch] * o[j] * inv / (1.0f + expf(-gl)) : 0.0f;
      }
    }
  }
}

}  // namespace

// 1 / q_l2_eps with the query map (q_l2_eps >= FLT_MIN, so finite), else 0
static float query_map_rcp(const Plan& p) { return p.qeps > 0.0f ? 1.0f / p.qeps : 0.0f; }

template <int DK, int DV, bool DECAY>
void launch_readout_bf16(const Plan& p, const void* q, const void* gate, const float* rms_weight,
                         void* out, const WsPtrs& w, const float* alpha, int nseg, int nblk,
                         hipStream_t s) {
  const unsigned per = xcd_per((unsigned)p.units * nseg * nblk);
  hipLaunchKernelGGL((readout_bf16_kernel<DK, DV, DECAY>), dim3(kXcds * per), dim3(kThreadsR), 0,
                     s, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(gate),
                     rms_weight, static_cast<uint16_t*>(out), w.ST, alpha, p.dk, p.dv, p.F, p.U,
                     p.C, p.r, p.n, p.eps, p.units, nseg, nblk, per, p.anchors, p.qh,
                     query_map_rcp(p));
}

hipError_t launch_split(const Plan& p, const WsPtrs& w, const float* alpha, hipStream_t s) {
  if (!split_readout(p.dtype, p.dk, p.dv) || p.units == 0 || p.n == 0 || p.U == 0)
    return hipSuccess;
  const unsigned per = xcd_per((unsigned)p.units * (alpha ? p.F : p.n));
  if (alpha)
    hipLaunchKernelGGL(split_states_kernel<true>, dim3(kXcds * per), dim3(kThreads), 0, s, w.ST,
                       alpha, decay_images(w), p.n, p.r, p.F, p.C, p.anchors, p.units, per);
  else
    hipLaunchKernelGGL(split_states_kernel<false>, dim3(kXcds * per), dim3(kThreads), 0, s, w.ST,
                       alpha, w.Sp, p.n, p.r, p.F, p.C, p.anchors, p.units, per);
  return hipGetLastError();
}

hipError_t launch_readout(const Plan& p, const void* q, const void* gate, const float* rms_weight,
                          void* out, const WsPtrs& w, const float* alpha, hipStream_t s) {
  // segments: frames with decay (each frame reads its own bridged state), else chunks
  const long max_rows = alpha ? (long)p.U : (long)p.C * p.U;
  const int nseg = alpha ? p.F : p.n;
  if (max_rows == 0 || nseg == 0 || p.units == 0) return hipSuccess;
  if (p.dtype == VDA_DTYPE_BF16) {
    const int nblk = (int)((max_rows + kRows - 1) / kRows);
    const bool d128 = p.dk == 128 && p.dv == 128;
    if (d128) {  // the split images were written by launch_split after the scans
      const int nb = (int)((max_rows + kRowsC - 1) / kRowsC);
      const unsigned per = xcd_per((unsigned)p.units * nseg * nb);
      hipLaunchKernelGGL(p.qeps > 0.0f ? readout_c128_kernel<true> : readout_c128_kernel<false>,
                         dim3(kXcds * per), dim3(kThreadsR), 0, s,
                         static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(gate),
                         rms_weight, static_cast<uint16_t*>(out), alpha ? decay_images(w) : w.Sp,
                         p.F, p.U, p.C, p.r, p.n, p.eps, p.units, nb, per, p.anchors,
                         alpha ? 1 : 0, p.qh, query_map_rcp(p));
    } else if (alpha)
      launch_readout_bf16<0, 0, true>(p, q, gate, rms_weight, out, w, alpha, nseg, nblk, s);
    else
      launch_readout_bf16<0, 0, false>(p, q, gate, rms_weight, out, w, alpha, nseg, nblk, s);
  } else {
    const int nblk = (int)((max_rows + kRowsF - 1) / kRowsF);
    const unsigned items = (unsigned)p.units * nseg * nblk;
    hipLaunchKernelGGL(readout_f32_kernel, dim3(items), dim3(kThreads), 0, s,
                       static_cast<const float*>(q), static_cast<const float*>(gate), rms_weight,
                       static_cast<float*>(out), w.ST, alpha, p.dk, p.dv, p.F, p.U, p.C, p.r, p.n,
                       p.eps, nseg, nblk, p.anchors, p.qh, query_map_rcp(p));
  }
  return hipGetLastError();
}

}  // namespace vda
