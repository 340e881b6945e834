// Device-side helpers shared by the VDA kernels (gfx950 / CDNA4).
//
// MFMA conventions used throughout (wave64):
//   v_mfma_f32_32x32x16_bf16  C[32x32] += A[32x16] B[16x32]
//     A operand: lane l holds A[i = l % 32][k = 8 (l / 32) .. + 7]   (8 bf16)
//     B operand: lane l holds B[k = 8 (l / 32) .. + 7][j = l % 32]   (8 bf16)
//   v_mfma_f32_32x32x2_f32    C[32x32] += A[32x2] B[2x32]
//     A operand: lane l holds A[i = l % 32][k = l / 32]
//     B operand: lane l holds B[k = l / 32][j = l % 32]
//   accumulator (both): register r of lane l holds C[acc_row(r, l)][l % 32]
//     with acc_row(r, l) = 8 (r / 4) + 4 (l / 32) + r % 4.
// Which contraction index sits in which k slot is free as long as the A and B
// operands of one instruction agree; the kernels use that freedom to keep
// every operand a contiguous 16-byte load.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vda {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;  // every kernel: 4 waves of 64

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

__device__ __forceinline__ int acc_row(int r, int lane) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

__device__ __forceinline__ f32x16_t mfma_bf16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// v_mfma_f32_16x16x32_bf16: A lane l = A[l % 16][8 (l / 16) .. + 7],
// B lane l = B[8 (l / 16) .. + 7][l % 16], accumulator register r of lane l
// = C[4 (l / 16) + r][l % 16].
__device__ __forceinline__ f32x4_t mfma16_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t mfma_f32(float a, float b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

// Streaming 16-byte accesses for data touched exactly once (q, gate, k, v,
// out): non-temporal, so they do not evict reused data from the caches.
__device__ __forceinline__ u32x4_t ld_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
__device__ __forceinline__ void st_stream(void* p, u32x4_t v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}

// bf16 <-> fp32.  A bf16 is the top half of an fp32, so widening is a shift.
__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2_t r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

// c + a.lo b.lo + a.hi b.hi for two packed bf16 pairs (v_dot2c_f32_bf16; the
// bf16 products are exact in fp32)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Make this wave's earlier LDS writes visible to its other lanes (LDS
// operations of one wave execute in order; this stops the compiler from
// moving memory accesses across the point).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__host__ __device__ __forceinline__ int pad32(int d) { return (d + 31) & ~31; }

// Workgroups of a launch are dispatched round-robin over the 8 XCDs (each with
// its own L2).  For a 1-D grid of 8 * per workgroups, give XCD x the
// contiguous work items [x * per, (x + 1) * per), so items that share inputs
// (neighbouring items) are served by one L2.  Returns the work item of this
// workgroup (may be >= the real item count: the caller skips those).
// Raw buffer access (gfx9 descriptor: stride 0, range in bytes, dword 3 =
// 0x00020000): loads at or past `bytes` return 0 without a memory access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
// 16 bytes, non-temporal (cache policy bit 1)
__device__ __forceinline__ u32x4_t buf_load16_nt(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}
// 16 bytes, default cache policy
__device__ __forceinline__ u32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ float buf_load4(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// Value of lane ^ 32, by gfx950's half swap (a VALU permute, no LDS round
// trip): permlane32_swap(x, x) returns {[x_lo, x_lo], [x_hi, x_hi]} (halves of
// 32 lanes).
__device__ __forceinline__ float lane_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(lane_id() < 32 ? r[1] : r[0]);
}

constexpr int kXcds = 8;
__device__ __forceinline__ unsigned xcd_item(unsigned per) {
  const unsigned L = blockIdx.x;
  return (L % kXcds) * per + L / kXcds;
}
__host__ __forceinline__ unsigned xcd_per(unsigned items) { return (items + kXcds - 1) / kXcds; }

// ---------------------------------------------------------------------------
// 32x32x32 fp32 block product on MFMA, operands in LDS (row-major with the
// given strides, in floats).  acc += op(A) op(B), op = transpose when the
// template flag is set.  Strides should be odd (e.g. 129) so that the 32
// lanes reading one column of a row-major block hit 32 distinct banks.
// Every operand is read before the first MFMA, so the 16 dependent MFMAs
// issue back to back instead of each waiting for its own LDS round trip.
template <bool AT, bool BT>
__device__ __forceinline__ f32x16_t blk_mm32(f32x16_t acc, const float* A, int sa, const float* B,
                                             int sb) {
  const int lane = lane_id();
  const int i = lane & 31;
  const int kh = lane >> 5;
  float a[16], b[16];
#pragma unroll
  for (int kk = 0; kk < 16; ++kk) {
    const int k = 2 * kk + kh;
    a[kk] = AT ? A[k * sa + i] : A[i * sa + k];
    b[kk] = BT ? B[i * sb + k] : B[k * sb + i];
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the MFMA chain
#pragma unroll
  for (int kk = 0; kk < 16; ++kk) acc = mfma_f32(a[kk], b[kk], acc);
  return acc;
}

// Store a 32x32 accumulator tile into LDS/global (row-major, stride sc) scaled.
__device__ __forceinline__ void store_acc(float* C, int sc, const f32x16_t& acc, float scale) {
  const int lane = lane_id();
#pragma unroll
  for (int r = 0; r < 16; ++r) C[acc_row(r, lane) * sc + (lane & 31)] = scale * acc[r];
}

}  // namespace vda

namespace vda {

// Register half of an LDS fill: a thread's share (16 float4) of a row-major
// fp32 matrix with `rows` x `cols` valid entries (leading dimension ld, cols
// a multiple of 4, both <= 128), optionally plus a second matrix of the same
// shape.  All loads are issued before any value is used, so one memory
// latency covers the whole matrix; entries outside the valid range are 0.
struct MatRegs {
  f32x4_t v[16];
};

__device__ __forceinline__ void mat_load(MatRegs& m, const float* src, int ld, int rows, int cols,
                                         const float* add = nullptr) {
  const f32x4_t z = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int id = threadIdx.x + 256 * i;
    const int r = id >> 5;
    const int c = (id & 31) << 2;
    const bool ok = r < rows && c < cols;
    m.v[i] = ok ? *reinterpret_cast<const f32x4_t*>(src + (size_t)r * ld + c) : z;
  }
  if (add) {
    f32x4_t a[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int id = threadIdx.x + 256 * i;
      const int r = id >> 5;
      const int c = (id & 31) << 2;
      const bool ok = r < rows && c < cols;
      a[i] = ok ? *reinterpret_cast<const f32x4_t*>(add + (size_t)r * ld + c) : z;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) m.v[i] += a[i];
  }
}

// LDS half: write the registers into an R x C region (row stride sdst) of LDS.
__device__ __forceinline__ void mat_store_lds(const MatRegs& m, float* dst, int sdst, int R,
                                              int C) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int id = threadIdx.x + 256 * i;
    const int r = id >> 5;
    const int c = (id & 31) << 2;
    if (r < R && c < C) {
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[r * sdst + c + e] = m.v[i][e];
    }
  }
}

}  // namespace vda
