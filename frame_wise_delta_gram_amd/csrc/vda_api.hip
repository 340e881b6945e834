// C ABI of the VDA forward library: argument checks, workspace carve-up and
// the launch sequence on the caller's stream (statistics, solve, composition,
// scan, readout; a separate text-frame statistics launch except at bf16 with
// d_k = d_v = 128).  See include/vda.h for the
// contract of every entry point.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "vda_internal.h"

namespace vda {
namespace {

constexpr int64_t kMaxGridYZ = 65535;
constexpr int64_t kMaxFrames = INT64_C(1) << 20;  // the solve grid's x extent is frames + 1

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

int make_plan(const vda_desc_t* d, Plan* p) {
  if (!d) return VDA_ERR_INVALID_ARG;
  if (d->in_dtype != VDA_DTYPE_F32 && d->in_dtype != VDA_DTYPE_BF16) return VDA_ERR_BAD_DTYPE;
  if (d->out_dtype != d->in_dtype) return VDA_ERR_BAD_DTYPE;
  if (d->units < 0 || d->frames < 0 || d->tokens < 0 || d->text_tokens < 0)
    return VDA_ERR_INVALID_ARG;
  if (d->d_k < 16 || d->d_k > 128 || d->d_k % 16) return VDA_ERR_INVALID_ARG;
  if (d->d_v < 16 || d->d_v > 128 || d->d_v % 16) return VDA_ERR_INVALID_ARG;
  if (d->chunk < 1 || d->radius < 0) return VDA_ERR_INVALID_ARG;
  if (!(d->rms_eps >= 0.0f) || !isfinite(d->rms_eps)) return VDA_ERR_INVALID_ARG;
  if (d->seed_mode != 0 && d->seed_mode != 1) return VDA_ERR_INVALID_ARG;
  if (d->anchors != 0 && d->anchors != 1) return VDA_ERR_INVALID_ARG;
  if (d->rule < 0 || d->rule > 2) return VDA_ERR_INVALID_ARG;
  if (d->fp32_products != 0 && d->fp32_products != 1) return VDA_ERR_INVALID_ARG;
  if (d->solver != 0 && d->solver != 1) return VDA_ERR_INVALID_ARG;
  if (d->solver == 1 && d->rule != 0) return VDA_ERR_INVALID_ARG;  // a factor of I + A_t only
  if (d->q_heads < 0 || d->q_heads > kMaxGridYZ) return VDA_ERR_INVALID_ARG;
  if (d->q_heads > 1 && d->units % d->q_heads != 0) return VDA_ERR_INVALID_ARG;
  // 0, or a normal float (its reciprocal is finite)
  if (!isfinite(d->q_l2_eps) || (d->q_l2_eps != 0.0f && !(d->q_l2_eps >= 1.17549435e-38f)))
    return VDA_ERR_INVALID_ARG;
  if (d->units > kMaxGridYZ) return VDA_ERR_INVALID_ARG;
  const int64_t n = d->frames > 0 ? (d->frames + (int64_t)d->chunk - 1) / d->chunk : 0;
  if (n > kMaxGridYZ) return VDA_ERR_INVALID_ARG;
  // every element count must fit in int64 (and the kernels' size_t arithmetic)
  int64_t rows, elems, x;
  if (!mul_ok(d->units, d->frames, &rows) || !mul_ok(rows, d->tokens, &rows)) return VDA_ERR_INVALID_ARG;
  if (!mul_ok(rows, 128, &elems)) return VDA_ERR_INVALID_ARG;
  if (!mul_ok((int64_t)d->chunk, d->tokens, &x)) return VDA_ERR_INVALID_ARG;
  if (!mul_ok(d->units, d->text_tokens, &x) || !mul_ok(x, 128, &x)) return VDA_ERR_INVALID_ARG;
  // one frame's tokens are addressed with 32-bit byte offsets; the frame list
  // (units x (frames + 1)) is indexed with int
  if ((int64_t)d->tokens * 512 > INT32_MAX || (int64_t)d->text_tokens * 512 > INT32_MAX)
    return VDA_ERR_INVALID_ARG;
  if ((int64_t)d->units * ((int64_t)d->frames + 1) > (INT64_C(1) << 30)) return VDA_ERR_INVALID_ARG;
  if (d->frames > kMaxFrames) return VDA_ERR_INVALID_ARG;
  // A launch holds fewer than 2^32 work-items along x: at most 2^22 workgroups
  // on the 512-thread 1-D grids (readout, bf16 composition), fewer than 2^24 on
  // the 256-thread fp32 readout grid.  Readout work items: units x segments x
  // row blocks (512 rows bf16, 64 rows fp32); segments are chunks, or frames
  // with decay (checked by the decay entry points).
  const int64_t rows_per_chunk = (int64_t)d->chunk * d->tokens;
  const bool bf16 = d->in_dtype == VDA_DTYPE_BF16;
  auto grid_ok = [&](int64_t segs, int64_t seg_rows, int64_t comp_items) {
    int64_t items;
    if (!mul_ok((int64_t)d->units * segs, (seg_rows + (bf16 ? 511 : 63)) / (bf16 ? 512 : 64),
                &items))
      return false;
    return items < (bf16 ? (INT64_C(1) << 22) : (INT64_C(1) << 24)) &&
           (int64_t)d->units * comp_items <= (INT64_C(1) << 22);
  };
  if (!grid_ok(n, rows_per_chunk, 3 * n + 1)) return VDA_ERR_INVALID_ARG;
  p->decay_ok = grid_ok(d->frames, d->tokens, 4 * n + 1);
  p->full_stats = false;

  p->units = d->units;
  p->F = d->frames;
  p->U = d->tokens;
  p->T = d->text_tokens;
  p->dk = d->d_k;
  p->dv = d->d_v;
  p->C = d->chunk;
  p->r = d->radius;
  p->n = (int)n;
  p->eps = d->rms_eps;
  p->seed_mode = d->seed_mode;
  p->anchors = d->anchors;
  p->rule = d->rule;
  p->fp32_products = d->fp32_products != 0 || d->in_dtype == VDA_DTYPE_F32;
  p->solver = d->solver;
  p->dtype = d->in_dtype;
  p->qh = d->q_heads > 1 ? d->q_heads : 1;
  p->qeps = d->q_l2_eps;

  const size_t U_ = (size_t)p->units, Fp1 = (size_t)p->F + 1, N = (size_t)p->n;
  const size_t kk = (size_t)p->dk * p->dk * 4, vk = (size_t)p->dv * p->dk * 4;
  size_t sz[10];
  sz[0] = U_ * Fp1 * kk;          // A
  sz[1] = U_ * Fp1 * vk;          // B
  sz[2] = U_ * Fp1 * kk;          // M
  sz[3] = U_ * N * kk;            // Mc
  sz[4] = U_ * N * vk;            // Jf
  sz[5] = U_ * N * vk;            // Jr
  sz[6] = U_ * 2 * (N + 1) * vk;  // ST
  sz[7] = U_ * N * kk;            // McT
  sz[8] = U_ * N * kk;            // MrT
  sz[9] = split_readout(p->dtype, p->dk, p->dv) ? U_ * N * kSplitElems * 2 : 0;  // Sp
  if (p->units == 0 || p->F == 0)
    for (size_t& s : sz) s = 0;
  size_t off = 0;
  for (int i = 0; i < 10; ++i) {
    p->off[i] = off;
    off += align256(sz[i]);
  }
  p->total = off;
  return VDA_OK;
}

WsPtrs carve(const Plan& p, void* ws) {
  char* b = static_cast<char*>(ws);
  WsPtrs w;
  w.A = reinterpret_cast<float*>(b + p.off[0]);
  w.B = reinterpret_cast<float*>(b + p.off[1]);
  w.M = reinterpret_cast<float*>(b + p.off[2]);
  w.Mc = reinterpret_cast<float*>(b + p.off[3]);
  w.Jf = reinterpret_cast<float*>(b + p.off[4]);
  w.Jr = reinterpret_cast<float*>(b + p.off[5]);
  w.ST = reinterpret_cast<float*>(b + p.off[6]);
  w.McT = reinterpret_cast<float*>(b + p.off[7]);
  w.MrT = reinterpret_cast<float*>(b + p.off[8]);
  w.Sp = reinterpret_cast<uint16_t*>(b + p.off[9]);
  return w;
}

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

// Input checks shared by every entry point that runs the state pipeline
// (alpha: optional decay gates); the workspace is checked separately.
int check_state_tensors(const Plan& p, const void* k, const void* v, const float* beta,
                        const void* tk, const void* tv, const float* tb,
                        const float* alpha = nullptr) {
  const bool video = (size_t)p.units * p.F * p.U > 0;
  const bool text = (size_t)p.units * p.T > 0 && p.F > 0;
  if (video && (!k || !v || !beta)) return VDA_ERR_INVALID_ARG;
  if (text && (!tk || !tv || !tb)) return VDA_ERR_INVALID_ARG;
  if (video && (!aligned(k, 16) || !aligned(v, 16) || !aligned(beta, 4))) return VDA_ERR_MISALIGNED;
  if (text && (!aligned(tk, 16) || !aligned(tv, 16) || !aligned(tb, 4))) return VDA_ERR_MISALIGNED;
  if (alpha && !aligned(alpha, 16)) return VDA_ERR_MISALIGNED;
  return VDA_OK;
}

int check_workspace(const Plan& p, const void* ws, size_t ws_bytes) {
  if (p.total > 0 && !ws) return VDA_ERR_INVALID_ARG;
  if (ws_bytes < p.total) return VDA_ERR_WORKSPACE_TOO_SMALL;
  if (ws && !aligned(ws, 256)) return VDA_ERR_MISALIGNED;
  return VDA_OK;
}

int check_state_inputs(const Plan& p, const void* k, const void* v, const float* beta,
                       const void* tk, const void* tv, const float* tb, const void* ws,
                       size_t ws_bytes, const float* alpha = nullptr) {
  const int st = check_state_tensors(p, k, v, beta, tk, tv, tb, alpha);
  return st != VDA_OK ? st : check_workspace(p, ws, ws_bytes);
}

// The readout's tensors (the forward entry points).
int check_readout_tensors(const Plan& p, const void* q, const void* gate, const float* rms_weight,
                          const void* out) {
  const bool video = (size_t)p.units * p.F * p.U > 0;
  if (video && (!q || !gate || !out || !rms_weight)) return VDA_ERR_INVALID_ARG;
  if (video && (!aligned(q, 16) || !aligned(gate, 16) || !aligned(out, 16) ||
                !aligned(rms_weight, 16)))
    return VDA_ERR_MISALIGNED;
  return VDA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? VDA_OK : VDA_ERR_HIP; }

// stages: 1 stats, 2 solve, 3 compose, 4 scan (and the readout's split
// states).  alpha (optional): decay gates.  events (optional): recorded before
// each launched stage.
int run_states(const Plan& p, const void* k, const void* v, const float* beta, const void* tk,
               const void* tv, const float* tb, const WsPtrs& w, hipStream_t s, int upto,
               const float* alpha = nullptr, hipEvent_t const* ev = nullptr) {
  auto rec = [&](int i) { return ev && ev[i] ? hipEventRecord(ev[i], s) : hipSuccess; };
  if (p.units == 0 || p.F == 0) {  // nothing to launch; keep the event sequence complete
    for (int i = 0; i < upto; ++i)
      if (rec(i) != hipSuccess) return VDA_ERR_HIP;
    return VDA_OK;
  }
  if (upto >= 1 && (rec(0) != hipSuccess || launch_stats(p, k, v, beta, tk, tv, tb, w, s) != hipSuccess))
    return VDA_ERR_HIP;
  if (upto >= 2 && (rec(1) != hipSuccess || launch_solve(p, w, s) != hipSuccess)) return VDA_ERR_HIP;
  if (upto >= 3 && (rec(2) != hipSuccess || launch_compose(p, w, alpha, s) != hipSuccess))
    return VDA_ERR_HIP;
  if (upto >= 4 && (rec(3) != hipSuccess || launch_scan(p, w, alpha != nullptr, s) != hipSuccess ||
                    launch_split(p, w, alpha, s) != hipSuccess))
    return VDA_ERR_HIP;
  return VDA_OK;
}

// The forward pass on a checked plan and workspace.
int launch_forward(const Plan& p, const void* q, const void* k, const void* v, const float* beta,
                   const float* alpha, const void* gate, const void* text_k, const void* text_v,
                   const float* text_beta, const float* rms_weight, void* out, void* workspace,
                   vda_stream_t stream, hipEvent_t const* ev) {
  const bool video = (size_t)p.units * p.F * p.U > 0;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const WsPtrs w = carve(p, workspace);
  int st = run_states(p, k, v, beta, text_k, text_v, text_beta, w, s, 4, alpha, ev);
  if (st != VDA_OK) return st;
  if (ev && ev[4] && hipEventRecord(ev[4], s) != hipSuccess) return VDA_ERR_HIP;
  if (video && launch_readout(p, q, gate, rms_weight, out, w, alpha, s) != hipSuccess)
    return VDA_ERR_HIP;
  if (ev && ev[5] && hipEventRecord(ev[5], s) != hipSuccess) return VDA_ERR_HIP;
  return VDA_OK;
}

int forward_impl(const vda_desc_t* desc, const void* q, const void* k, const void* v,
                 const float* beta, const float* alpha, const void* gate, const void* text_k,
                 const void* text_v, const float* text_beta, const float* rms_weight, void* out,
                 void* workspace, size_t workspace_bytes, vda_stream_t stream,
                 hipEvent_t const* ev) {
  Plan p;
  int st = make_plan(desc, &p);
  if (st != VDA_OK) return st;
  st = check_state_inputs(p, k, v, beta, text_k, text_v, text_beta, workspace, workspace_bytes,
                          alpha);
  if (st != VDA_OK) return st;
  st = check_readout_tensors(p, q, gate, rms_weight, out);
  if (st != VDA_OK) return st;
  return launch_forward(p, q, k, v, beta, alpha, gate, text_k, text_v, text_beta, rms_weight, out,
                        workspace, stream, ev);
}

// Extra checks of the decay entry points: the gates are required whenever a
// frame exists, and the per-frame readout grid must fit.
int check_decay(const vda_desc_t* desc, const float* alpha) {
  Plan p;
  const int st = make_plan(desc, &p);
  if (st != VDA_OK) return st;
  if (!p.decay_ok) return VDA_ERR_INVALID_ARG;
  if (p.rule != 0) return VDA_ERR_INVALID_ARG;  // the batched comparison rules run without decay
  if (p.units > 0 && p.F > 0 && !alpha) return VDA_ERR_INVALID_ARG;
  return VDA_OK;
}

// Debug tap bodies shared by the plain and decay variants.
// want_mr: the caller asked for the reverse maps (Mr_t_out must then be non-NULL)
int chunks_impl(const vda_desc_t* desc, const void* k, const void* v, const float* beta,
                const float* alpha, const void* text_k, const void* text_v,
                const float* text_beta, float* Mc_out, float* Mr_t_out, bool want_mr,
                float* Jf_out, float* Jr_out, void* workspace, size_t workspace_bytes,
                vda_stream_t stream) {
  Plan p;
  int st = make_plan(desc, &p);
  if (st != VDA_OK) return st;
  st = check_state_inputs(p, k, v, beta, text_k, text_v, text_beta, workspace, workspace_bytes,
                          alpha);
  if (st != VDA_OK) return st;
  if (p.units == 0 || p.F == 0) return VDA_OK;
  if (!Mc_out || !Jf_out || !Jr_out || (want_mr && !Mr_t_out)) return VDA_ERR_INVALID_ARG;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const WsPtrs w = carve(p, workspace);
  st = run_states(p, k, v, beta, text_k, text_v, text_beta, w, s, 3, alpha);
  if (st != VDA_OK) return st;
  const size_t nc = (size_t)p.units * p.n;
  const size_t mb = nc * p.dk * p.dk * 4;
  if (hipMemcpyAsync(Mc_out, w.Mc, mb, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return VDA_ERR_HIP;
  // without decay the reverse transition is Mc^T, whose transpose is Mc
  if (Mr_t_out && hipMemcpyAsync(Mr_t_out, alpha ? w.MrT : w.Mc, mb, hipMemcpyDeviceToDevice, s) !=
                      hipSuccess)
    return VDA_ERR_HIP;
  if (hipMemcpyAsync(Jf_out, w.Jf, nc * p.dv * p.dk * 4, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return VDA_ERR_HIP;
  return hip_status(hipMemcpyAsync(Jr_out, w.Jr, nc * p.dv * p.dk * 4, hipMemcpyDeviceToDevice, s));
}

int states_impl(const vda_desc_t* desc, const void* k, const void* v, const float* beta,
                const float* alpha, const void* text_k, const void* text_v,
                const float* text_beta, float* P_out, float* R_out, void* workspace,
                size_t workspace_bytes, vda_stream_t stream) {
  Plan p;
  int st = make_plan(desc, &p);
  if (st != VDA_OK) return st;
  st = check_state_inputs(p, k, v, beta, text_k, text_v, text_beta, workspace, workspace_bytes,
                          alpha);
  if (st != VDA_OK) return st;
  if (p.units == 0 || p.F == 0) return VDA_OK;
  if (!P_out || !R_out) return VDA_ERR_INVALID_ARG;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const WsPtrs w = carve(p, workspace);
  st = run_states(p, k, v, beta, text_k, text_v, text_beta, w, s, 4, alpha);
  if (st != VDA_OK) return st;
  const size_t dirb = (size_t)(p.n + 1) * p.dv * p.dk * 4;
  if (hipMemcpy2DAsync(P_out, dirb, w.ST, 2 * dirb, dirb, p.units, hipMemcpyDeviceToDevice, s) !=
      hipSuccess)
    return VDA_ERR_HIP;
  return hip_status(hipMemcpy2DAsync(R_out, dirb, reinterpret_cast<char*>(w.ST) + dirb, 2 * dirb,
                                     dirb, p.units, hipMemcpyDeviceToDevice, s));
}

}  // namespace
}  // namespace vda

namespace vda {
namespace {

int make_prep_plan(const vda_prep_desc_t* d, PrepPlan* p) {
  if (!d) return VDA_ERR_INVALID_ARG;
  if (d->dtype != VDA_DTYPE_F32 && d->dtype != VDA_DTYPE_BF16) return VDA_ERR_BAD_DTYPE;
  if (d->batch < 0 || d->heads < 0 || d->frames < 0 || d->height < 0 || d->width < 0)
    return VDA_ERR_INVALID_ARG;
  if ((int64_t)d->batch * d->heads > kMaxGridYZ) return VDA_ERR_INVALID_ARG;
  if (d->frames > kMaxFrames) return VDA_ERR_INVALID_ARG;
  if ((int64_t)d->height * d->width > 4194303) return VDA_ERR_INVALID_ARG;
  // each side alone too (an empty frame with one side at INT32_MAX would overflow the tiling)
  if (d->height > 4194303 || d->width > 4194303) return VDA_ERR_INVALID_ARG;
  // one frame of one batch entry (all heads) is addressed with 32-bit byte offsets
  if ((int64_t)d->height * d->width * d->heads * 128 * 4 > INT32_MAX) return VDA_ERR_INVALID_ARG;
  if (d->d_k < 16 || d->d_k > 128 || d->d_k % 16) return VDA_ERR_INVALID_ARG;
  if (d->d_v < 16 || d->d_v > 128 || d->d_v % 16) return VDA_ERR_INVALID_ARG;
  if (!(d->eps > 0.0f) || !isfinite(d->eps)) return VDA_ERR_INVALID_ARG;
  int64_t x;
  const int64_t units = (int64_t)d->batch * d->heads;
  if (!mul_ok(units * d->frames, (int64_t)d->height * d->width, &x) || !mul_ok(x, 128, &x))
    return VDA_ERR_INVALID_ARG;
  p->batch = d->batch;
  p->H = d->heads;
  p->F = d->frames;
  p->Hl = d->height;
  p->Wl = d->width;
  p->U = d->height * d->width;
  p->dk = d->d_k;
  p->dv = d->d_v;
  p->dtype = d->dtype;
  p->eps = d->eps;
  p->tiles_r = (d->height + 7) / 8;  // 8 x 8 output tiles of the convolution
  p->tiles_c = (d->width + 7) / 8;
  // the feature map's 1-D grid (a K and a V workgroup per unit and tile, each
  // count rounded up to a multiple of 8, then 1024 workgroups of the Q pass):
  // fewer than 2^22 workgroups of 1024 threads
  if (!mul_ok(units, (int64_t)p->tiles_r * p->tiles_c, &x) || x >= (INT64_C(1) << 21) - 1024)
    return VDA_ERR_INVALID_ARG;
  return VDA_OK;
}

}  // namespace
}  // namespace vda

namespace vda {
namespace {

// Workspace of vda_forward_noalloc: a fixed device array in this library's
// code object, one copy per GPU, held until the process ends.  Its name is
// only a host-side handle: host code uses the address hipGetSymbolAddress
// returns for the current device (scratch_ptr below), never the name itself.
__device__ __align__(256) unsigned char scratch[VDA_NOALLOC_MAX_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];  // device address of `scratch`, per device ordinal
std::mutex g_scratch_mu;

// The device address of `scratch` on the device `stream` belongs to (the
// current device for the null stream), looked up once per device with that
// device current.  Returns VDA_ERR_HIP when the device cannot be queried or
// the lookup fails.
int scratch_ptr(hipStream_t stream, void** out) {
  int dev = -1;
  if (stream ? hipStreamGetDevice(stream, &dev) != hipSuccess : hipGetDevice(&dev) != hipSuccess)
    return VDA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return VDA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return VDA_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return VDA_ERR_HIP;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return VDA_ERR_HIP;
    if (e != hipSuccess || !ptr) return VDA_ERR_HIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return VDA_OK;
}

}  // namespace
}  // namespace vda

using vda::Plan;
using vda::WsPtrs;

extern "C" {

size_t vda_workspace_bytes(const vda_desc_t* desc) {
  Plan p;
  if (vda::make_plan(desc, &p) != VDA_OK) return 0;
  return p.total;
}

int vda_check_desc(const vda_desc_t* desc) {
  Plan p;
  return vda::make_plan(desc, &p);
}

int vda_forward(const vda_desc_t* desc, const void* q, const void* k, const void* v,
                const float* beta, const void* gate, const void* text_k, const void* text_v,
                const float* text_beta, const float* rms_weight, void* out, void* workspace,
                size_t workspace_bytes, vda_stream_t stream) {
  return vda::forward_impl(desc, q, k, v, beta, nullptr, gate, text_k, text_v, text_beta,
                           rms_weight, out, workspace, workspace_bytes, stream, nullptr);
}

int vda_forward_noalloc(const vda_desc_t* desc, const void* q, const void* k, const void* v,
                        const float* beta, const void* gate, const void* text_k,
                        const void* text_v, const float* text_beta, const float* rms_weight,
                        void* out, vda_stream_t stream) {
  Plan p;
  int st = vda::make_plan(desc, &p);
  if (st != VDA_OK) return st;
  if (p.total > (size_t)VDA_NOALLOC_MAX_BYTES) return VDA_ERR_SCRATCH_TOO_SMALL;
  st = vda::check_state_tensors(p, k, v, beta, text_k, text_v, text_beta);
  if (st != VDA_OK) return st;
  st = vda::check_readout_tensors(p, q, gate, rms_weight, out);
  if (st != VDA_OK) return st;
  if (p.total == 0) return VDA_OK;  // an empty problem enqueues nothing
  void* ws = nullptr;
  st = vda::scratch_ptr(reinterpret_cast<hipStream_t>(stream), &ws);
  if (st != VDA_OK) return st;
  // every workspace section the pipeline reads is written earlier in the same
  // call (no counters, no accumulation), so the array needs no clearing
  return vda::launch_forward(p, q, k, v, beta, nullptr, gate, text_k, text_v, text_beta,
                             rms_weight, out, ws, stream, nullptr);
}

int vda_forward_timed(const vda_desc_t* desc, const void* q, const void* k, const void* v,
                      const float* beta, const float* alpha, const void* gate,
                      const void* text_k, const void* text_v, const float* text_beta,
                      const float* rms_weight, void* out, void* workspace, size_t workspace_bytes,
                      vda_stream_t stream, void* const* stage_events, int n_events) {
  if (!stage_events || n_events != 6) return VDA_ERR_INVALID_ARG;
  if (alpha) {
    const int st = vda::check_decay(desc, alpha);
    if (st != VDA_OK) return st;
  }
  return vda::forward_impl(desc, q, k, v, beta, alpha, gate, text_k, text_v, text_beta,
                           rms_weight, out, workspace, workspace_bytes, stream,
                           reinterpret_cast<hipEvent_t const*>(stage_events));
}

int vda_forward_decay(const vda_desc_t* desc, const void* q, const void* k, const void* v,
                      const float* beta, const float* alpha, const void* gate,
                      const void* text_k, const void* text_v, const float* text_beta,
                      const float* rms_weight, void* out, void* workspace, size_t workspace_bytes,
                      vda_stream_t stream) {
  const int st = vda::check_decay(desc, alpha);
  if (st != VDA_OK) return st;
  return vda::forward_impl(desc, q, k, v, beta, alpha, gate, text_k, text_v, text_beta,
                           rms_weight, out, workspace, workspace_bytes, stream, nullptr);
}

int vda_debug_stats(const vda_desc_t* desc, const void* k, const void* v, const float* beta,
                    const void* text_k, const void* text_v, const float* text_beta, float* A_out,
                    float* B_out, void* workspace, size_t workspace_bytes, vda_stream_t stream) {
  Plan p;
  int st = vda::make_plan(desc, &p);
  if (st != VDA_OK) return st;
  st = vda::check_state_inputs(p, k, v, beta, text_k, text_v, text_beta, workspace,
                               workspace_bytes);
  if (st != VDA_OK) return st;
  if (p.units == 0 || p.F == 0) return VDA_OK;
  if (!A_out || !B_out) return VDA_ERR_INVALID_ARG;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const WsPtrs w = vda::carve(p, workspace);
  p.full_stats = true;  // the tap returns whole matrices
  st = vda::run_states(p, k, v, beta, text_k, text_v, text_beta, w, s, 1);
  if (st != VDA_OK) return st;
  const size_t fr = (size_t)p.units * (p.F + 1);
  if (hipMemcpyAsync(A_out, w.A, fr * p.dk * p.dk * 4, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return VDA_ERR_HIP;
  return vda::hip_status(
      hipMemcpyAsync(B_out, w.B, fr * p.dv * p.dk * 4, hipMemcpyDeviceToDevice, s));
}

int vda_debug_solve(const vda_desc_t* desc, const void* k, const void* v, const float* beta,
                    const void* text_k, const void* text_v, const float* text_beta, float* M_out,
                    float* seed_out, void* workspace, size_t workspace_bytes, vda_stream_t stream) {
  Plan p;
  int st = vda::make_plan(desc, &p);
  if (st != VDA_OK) return st;
  st = vda::check_state_inputs(p, k, v, beta, text_k, text_v, text_beta, workspace,
                               workspace_bytes);
  if (st != VDA_OK) return st;
  if (p.units == 0 || p.F == 0) return VDA_OK;
  if (!M_out || !seed_out) return VDA_ERR_INVALID_ARG;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const WsPtrs w = vda::carve(p, workspace);
  st = vda::run_states(p, k, v, beta, text_k, text_v, text_beta, w, s, 3);  // seed: compose
  if (st != VDA_OK) return st;
  const size_t fr = (size_t)p.units * (p.F + 1);
  if (hipMemcpyAsync(M_out, w.M, fr * p.dk * p.dk * 4, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return VDA_ERR_HIP;
  const size_t SSb = (size_t)p.dv * p.dk * 4;
  return vda::hip_status(hipMemcpy2DAsync(seed_out, SSb, w.ST, 2 * (p.n + 1) * SSb, SSb, p.units,
                                          hipMemcpyDeviceToDevice, s));
}

int vda_debug_frame_maps(const vda_desc_t* desc, const void* k, const void* v, const float* beta,
                         const void* text_k, const void* text_v, const float* text_beta,
                         float* M_out, float* J_out, int* not_spd, void* workspace,
                         size_t workspace_bytes, vda_stream_t stream) {
  Plan p;
  int st = vda::make_plan(desc, &p);
  if (st != VDA_OK) return st;
  if (p.rule != 0) return VDA_ERR_INVALID_ARG;
  st = vda::check_state_inputs(p, k, v, beta, text_k, text_v, text_beta, workspace,
                               workspace_bytes);
  if (st != VDA_OK) return st;
  if (p.units == 0 || p.F == 0) return VDA_OK;
  if (!M_out || !J_out) return VDA_ERR_INVALID_ARG;
  if (!vda::aligned(not_spd, 4)) return VDA_ERR_MISALIGNED;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const WsPtrs w = vda::carve(p, workspace);
  st = vda::run_states(p, k, v, beta, text_k, text_v, text_beta, w, s, 1);
  if (st != VDA_OK) return st;
  if (vda::launch_solve(p, w, s, not_spd) != hipSuccess ||
      vda::launch_frame_injections(p, w, J_out, s) != hipSuccess)
    return VDA_ERR_HIP;
  const size_t fr = (size_t)p.units * (p.F + 1);
  return vda::hip_status(
      hipMemcpyAsync(M_out, w.M, fr * p.dk * p.dk * 4, hipMemcpyDeviceToDevice, s));
}

int vda_debug_chunks(const vda_desc_t* desc, const void* k, const void* v, const float* beta,
                     const void* text_k, const void* text_v, const float* text_beta, float* Mc_out,
                     float* Jf_out, float* Jr_out, void* workspace, size_t workspace_bytes,
                     vda_stream_t stream) {
  return vda::chunks_impl(desc, k, v, beta, nullptr, text_k, text_v, text_beta, Mc_out, nullptr,
                          false, Jf_out, Jr_out, workspace, workspace_bytes, stream);
}

int vda_debug_chunks_decay(const vda_desc_t* desc, const void* k, const void* v,
                           const float* beta, const float* alpha, const void* text_k,
                           const void* text_v, const float* text_beta, float* Mc_out,
                           float* Mr_t_out, float* Jf_out, float* Jr_out, void* workspace,
                           size_t workspace_bytes, vda_stream_t stream) {
  const int st = vda::check_decay(desc, alpha);
  if (st != VDA_OK) return st;
  return vda::chunks_impl(desc, k, v, beta, alpha, text_k, text_v, text_beta, Mc_out, Mr_t_out,
                          true, Jf_out, Jr_out, workspace, workspace_bytes, stream);
}

int vda_debug_states(const vda_desc_t* desc, const void* k, const void* v, const float* beta,
                     const void* text_k, const void* text_v, const float* text_beta, float* P_out,
                     float* R_out, void* workspace, size_t workspace_bytes, vda_stream_t stream) {
  return vda::states_impl(desc, k, v, beta, nullptr, text_k, text_v, text_beta, P_out, R_out,
                          workspace, workspace_bytes, stream);
}

int vda_debug_states_decay(const vda_desc_t* desc, const void* k, const void* v,
                           const float* beta, const float* alpha, const void* text_k,
                           const void* text_v, const float* text_beta, float* P_out,
                           float* R_out, void* workspace, size_t workspace_bytes,
                           vda_stream_t stream) {
  const int st = vda::check_decay(desc, alpha);
  if (st != VDA_OK) return st;
  return vda::states_impl(desc, k, v, beta, alpha, text_k, text_v, text_beta, P_out, R_out,
                          workspace, workspace_bytes, stream);
}

int vda_prep_check_desc(const vda_prep_desc_t* desc) {
  vda::PrepPlan p;
  return vda::make_prep_plan(desc, &p);
}

int vda_prep(const vda_prep_desc_t* desc, const void* q, const void* k, const void* v,
             const float* wk_s, const float* wk_t, const float* wv_s, const float* wv_t,
             void* q_out, void* k_out, void* v_out, vda_stream_t stream) {
  vda::PrepPlan p;
  const int st = vda::make_prep_plan(desc, &p);
  if (st != VDA_OK) return st;
  const int64_t rows = (int64_t)p.batch * p.H * p.F * p.U;
  if (rows == 0) return VDA_OK;
  // q and q_out both NULL: K' and V' only (the query map runs in the readout)
  if ((q == nullptr) != (q_out == nullptr)) return VDA_ERR_INVALID_ARG;
  if (!k || !v || !k_out || !v_out || !wk_s || !wk_t || !wv_s || !wv_t) return VDA_ERR_INVALID_ARG;
  for (const void* ptr : {q, k, v, static_cast<const void*>(q_out), static_cast<const void*>(k_out),
                          static_cast<const void*>(v_out)})
    if (ptr && !vda::aligned(ptr, 16)) return VDA_ERR_MISALIGNED;
  for (const float* ptr : {wk_s, wk_t, wv_s, wv_t})
    if (!vda::aligned(ptr, 4)) return VDA_ERR_MISALIGNED;
  return vda::hip_status(vda::launch_prep(p, q, k, v, wk_s, wk_t, wv_s, wv_t, q_out, k_out, v_out,
                                          reinterpret_cast<hipStream_t>(stream)));
}

const char* vda_status_string(int status) {
  switch (status) {
    case VDA_OK: return "ok";
    case VDA_ERR_INVALID_ARG: return "invalid argument";
    case VDA_ERR_BAD_DTYPE: return "unsupported dtype";
    case VDA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case VDA_ERR_MISALIGNED: return "misaligned pointer";
    case VDA_ERR_HIP: return "HIP launch or copy failed";
    case VDA_ERR_SCRATCH_TOO_SMALL:
      return "problem needs more workspace than vda_forward_noalloc's fixed scratch";
    case VDA_ERR_NOT_SPD:
      return "some I + A_t is not numerically positive definite (a pivot <= 0 or NaN: beta < 0?)";
    default: return "unknown status";
  }
}

}  // extern "C"
