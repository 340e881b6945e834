/*
 * vda.h -- C ABI of the Video Delta Attention (VDA) forward library for
 * AMD Instinct MI355X (gfx950).
 *
 * VDA is the bidirectional, frame-wise delta-rule linear-memory branch of
 * "Video DeltaNet: A Video-Native Hybrid Attention for Livestream Video
 * Generation" (arXiv 2609.20744), cited here as [VDN].  For every unit
 * (one batch x head pair; units are independent) the library computes:
 *
 *   1. frame statistics ([VDN] Sec. 3.1 Eq. (3b)), per latent frame t:
 *        A_t = K_t^T Diag(beta_t) K_t   (d_k x d_k)
 *        B_t = V_t^T Diag(beta_t) K_t   (d_v x d_k)
 *      and the same for the text tokens, taken as one more frame placed before
 *      the first latent frame
 *      ([VDN] Sec. 5, "Chunk-wise scans");
 *   2. the frame-wise update ([VDN] Sec. 3.2 Eq. (5), decay alpha = 1):
 *        S_t = (S_{t-1} + B_t) (I + A_t)^{-1}
 *      through symmetric Gauss-Jordan elimination of the SPD matrix I + A_t,
 *      giving the transition M_t = (I + A_t)^{-1} ([VDN] App. A.1 Eq. (A.1));
 *   3. the text seed ([VDN] Sec. 2.2 Eq. (1b)): S_T = B_T (I + A_T)^{-1} and
 *      both scans start at S_T / 2 (seed_mode 0), or at the text written from
 *      zero at beta / 2 (seed_mode 1);
 *   4. per chunk of `chunk` frames, the composed affine map
 *      S_out = S_in M_chunk + J_chunk in both directions ([VDN] Sec. 5), and a
 *      scan over chunk boundaries in both directions that keeps the forward
 *      states P[j] (frames [0, j*chunk)) and reverse states R[j] (frames
 *      [j*chunk, F)), with P[0] = R[n] = seed;
 *   5. the readout ([VDN] Eq. (1a), App. A.3 Eq. (A.4) with alpha = 1, Eq. (1c)):
 *      a query of chunk c reads S~ = P[max(c - radius, 0)] + R[min(c + radius + 1, n)],
 *      o = S~ q, y = w * o / sqrt(mean(o^2) + eps), out = sigmoid(g) * y.
 *      With desc->q_l2_eps > 0 the query is first normalised to unit L2 norm,
 *      q' = q / max(||q||_2, q_l2_eps) (the feature map's query map, [VDN]
 *      Sec. 2.3); o is linear in q and the RMSNorm undoes any scale but its
 *      eps, so the readout forms o = S~ q from the raw query and takes
 *      y = w * o / sqrt(mean(o^2) + eps * max(||q||^2, q_l2_eps^2)), which
 *      equals the normalised query's result up to rounding.
 *
 * With channel-wise decay (vda_forward_decay; [VDN] Sec. 3.1 Eq. (2), App. A.1
 * Eq. (A.1) and App. A.3 Eq. (A.4)), frame t carries gates alpha_t in [0, 1]^d_k:
 * entering frame t, either scan decays the state it inherits, S Diag(alpha_t),
 * before the update (M_t = Diag(alpha_t) (I + A_t)^{-1}), and a query of frame t
 * in chunk c, whose window [c - radius, c + radius] spans frames [l, h] of the
 * clip, reads the bridged state
 *      S~_t = P[max(c - radius, 0)] Diag(prod_{s=l}^{t} alpha_s)
 *           + R[min(c + radius + 1, n)] Diag(prod_{s=t}^{h} alpha_s).
 * The text seed is unchanged (the text state starts from zero).
 *
 * Boundary anchors (desc->anchors = 1; [VDN] Sec. 2.1, Sec. 2.2, App. A.3 and
 * Algorithm 1 steps 2 and 7): frames 0 and F - 1 are left out of both scans
 * (their k, v, beta and alpha are never read), so the states are those of the
 * interior frames 1..F-2 with P_0 = R_{F-1} = seed, a query's window is
 * clipped to the interior frames, the anchor rows of `out` are zero, and so is
 * every row whose window (chunks c - radius .. c + radius) spans the whole clip
 * (the linear path is bypassed there); a clip of at most two frames has only
 * zero rows.  An anchor frame therefore acts on the states as the identity.
 *
 * Comparison rules (desc->rule; [VDN] Sec. 3.1 Eq. (3a)/(3c), App. A.2): rule 1
 * replaces the frame-wise update of step 2 everywhere (both scans and the text
 * frame) by SANA-WM's frozen-state batched update S_t = S_{t-1} (I - A_t) + B_t;
 * rule 2 adds its frame-size key scaling (every key of a frame of N tokens
 * scaled by 1/sqrt(N): A -> A / N, B -> B / sqrt(N); N = tokens, T for the text
 * frame).  Their factor I - A is not non-expansive once an eigenvalue of A
 * passes 2 (rule 1 can overflow on real inputs); they exist for comparison and
 * run without decay (the decay entry points reject rule != 0).
 *
 * Layouts (row-major, last index fastest, all tensors contiguous):
 *   q     [units][frames][tokens][d_k]   in_dtype (desc->q_heads <= 1), or with
 *         q_heads = H > 1 [units / H][frames][tokens][H][d_k]: the QKV projection's
 *         layout, heads interleaved per token (vda_prep's input order with
 *         tokens = height x width), unit u = b x H + h reading head h of entry b
 *   k     [units][frames][tokens][d_k]   in_dtype (prepared features)
 *   v     [units][frames][tokens][d_v]   in_dtype
 *   beta  [units][frames][tokens]        float32, >= 0 (write strengths)
 *   gate  [units][frames][tokens][d_v]   in_dtype (gate logits)
 *   text_k [units][text_tokens][d_k]     in_dtype
 *   text_v [units][text_tokens][d_v]     in_dtype
 *   text_beta [units][text_tokens]       float32, >= 0
 *   rms_weight [d_v]                     float32 (shared by all units)
 *   alpha [units][frames][d_k]           float32 in [0, 1] (decay gates, optional)
 *   out   [units][frames][tokens][d_v]   out_dtype (== in_dtype)
 *
 * Ownership: the caller owns every buffer.  All pointers are device pointers
 * (HBM), except the descriptor, which is a host pointer read during the call.
 * The library never allocates or frees memory; it writes only `out` (fully
 * overwritten) and the caller's workspace (vda_forward_noalloc: its own fixed
 * scratch instead).  Inputs are read-only.
 *
 * Streams: every call only enqueues kernels (and, for the debug taps,
 * device-to-device copies) on `stream`; it never synchronises.  Execution
 * errors surface at the caller's next synchronisation.  Apart from
 * vda_forward_noalloc's per-GPU scratch (below), the library holds no mutable
 * global state; calls are reentrant.  Calls that share a workspace must be
 * ordered on one stream.
 *
 * Errors: functions return VDA_OK (0) or a negative vda_status_t.  Argument
 * checks happen on the host before anything is enqueued, so a failed check
 * leaves every buffer untouched.  No exceptions cross the ABI.
 */
#ifndef VDA_H_
#define VDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* vda_stream_t; /* a hipStream_t; NULL = default stream */

typedef enum vda_status {
  VDA_OK = 0,
  VDA_ERR_INVALID_ARG = -1,         /* null pointer, size out of range, bad chunk/radius/eps */
  VDA_ERR_BAD_DTYPE = -2,           /* unsupported in_dtype/out_dtype combination */
  VDA_ERR_WORKSPACE_TOO_SMALL = -3, /* workspace_bytes < vda_workspace_bytes(desc) */
  VDA_ERR_MISALIGNED = -4,          /* a tensor is not 16-byte aligned, workspace not 256-byte */
  VDA_ERR_HIP = -5,                 /* a kernel launch or copy failed (hipGetLastError) */
  VDA_ERR_SCRATCH_TOO_SMALL = -6,   /* vda_forward_noalloc: workspace > VDA_NOALLOC_MAX_BYTES */
  VDA_ERR_NOT_SPD = -7              /* debug only: the value vda_debug_frame_maps writes to its
                                       device flag when some I + A_t is not numerically SPD */
} vda_status_t;

typedef enum vda_dtype {
  VDA_DTYPE_F32 = 0,  /* fp32 features, fp32 arithmetic throughout */
  VDA_DTYPE_BF16 = 1  /* bf16 features, bf16 x bf16 MFMA with fp32 accumulation, fp32 state */
} vda_dtype_t;

typedef struct vda_desc {
  int32_t units;       /* batch x heads, 0..65535 */
  int32_t frames;      /* latent frames F, 0..2^20; units x (F + 1) <= 2^30 */
  int32_t tokens;      /* tokens per frame U, 0..4194303 */
  int32_t text_tokens; /* text tokens T, 0..4194303 (0: zero seed) */
  int32_t d_k;         /* key channels, multiple of 16, 16..128 */
  int32_t d_v;         /* value channels, multiple of 16, 16..128 */
  int32_t chunk;       /* frames per chunk C, >= 1 ([VDN] uses 5) */
  int32_t radius;      /* window radius in chunks r, >= 0 ([VDN] uses 1) */
  float rms_eps;       /* RMSNorm epsilon, finite and >= 0 */
  int32_t seed_mode;   /* 0: seed = S_T / 2 ([VDN] Eq. (1b)); 1: text written at beta / 2 */
  int32_t in_dtype;    /* vda_dtype_t of q, k, v, gate, text_k, text_v */
  int32_t out_dtype;   /* vda_dtype_t of out; must equal in_dtype */
  int32_t anchors;     /* 0: no anchors; 1: boundary anchors (see above) */
  int32_t rule;        /* 0: the frame-wise delta rule; 1, 2: batched comparison rules (above) */
  int32_t fp32_products; /* bf16 features: 0 = the composition and the scan multiply their
                            fp32 maps with split-bf16 MFMA (hi/lo operands, about 2^-16
                            relative per product, the fast default); 1 = with fp32 MFMA
                            (exact fp32 products, the fp32 state updates of [VDN] Sec. 5).
                            fp32 features always use fp32 products. */
  int32_t solver;      /* frame-wise rule: 0 = symmetric Gauss-Jordan elimination of I + A_t
                          (block sweep, the default); 1 = blocked Cholesky factorisation
                          I + A_t = L L^T, then M_t = L^-T L^-1 (same result to rounding);
                          rules 1, 2 take 0 only */
  int32_t q_heads;     /* 0 or 1: q in the unit layout; H > 1 (dividing units, <= 65535):
                          q in the projection layout with H heads per token (above) */
  float q_l2_eps;      /* 0: q read as given; > 0 (finite): each query row normalised to
                          unit L2 norm with this floor inside the readout (above), so
                          the feature map's query pass can be skipped (vda_prep with
                          q = q_out = NULL) */
} vda_desc_t;

/* Bytes of device workspace vda_forward and the debug taps need for `desc`
 * (fp32 frame statistics, transitions, chunk maps and boundary states; with bf16
 * features and d_k = d_v = 128 also each chunk's gathered readout state split into
 * bf16 high and low parts, 69632 bytes per (unit, chunk)).
 * Returns 0 when desc is NULL or invalid. Host-only; never touches the GPU. */
size_t vda_workspace_bytes(const vda_desc_t* desc);

/* Checks desc alone (host-only).  Returns VDA_OK or the error vda_forward
 * would return for it.  Besides the field ranges above, the launch grids must
 * fit: units x ceil(frames / chunk) x ceil(chunk x tokens / R) < 2^22 with R =
 * 1024 (bf16; 2^24 and R = 64 for fp32), and units x (3 ceil(frames / chunk) +
 * 1) <= 2^22.  The decay entry points also need units x frames x
 * ceil(tokens / R) below the same bound and units x (4 ceil(frames / chunk) +
 * 1) <= 2^22. */
int vda_check_desc(const vda_desc_t* desc);

/* The VDA forward pass described at the top of this file.  q, k, v, gate,
 * out, text_k, text_v and rms_weight must be 16-byte aligned, beta and
 * text_beta 4-byte aligned, workspace 256-byte aligned.  Pointers to empty
 * tensors (size 0) may be NULL.  beta and text_beta must be >= 0 (I + A must
 * be SPD); this is not checked (negative values give undefined results). */
int vda_forward(const vda_desc_t* desc, const void* q, const void* k, const void* v,
                const float* beta, const void* gate, const void* text_k, const void* text_v,
                const float* text_beta, const float* rms_weight, void* out, void* workspace,
                size_t workspace_bytes, vda_stream_t stream);

/* Bytes of the fixed device scratch vda_forward_noalloc works in (64 MiB). */
#define VDA_NOALLOC_MAX_BYTES (64u << 20)

/* vda_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same pass with the same arguments minus the workspace, computed in a fixed
 * array of VDA_NOALLOC_MAX_BYTES in the library's own device memory (one copy
 * per GPU, created with the library's code object on that GPU and held until
 * the process ends).  The call allocates and frees nothing.  Problems whose
 * vda_workspace_bytes(desc) exceeds VDA_NOALLOC_MAX_BYTES are refused with
 * VDA_ERR_SCRATCH_TOO_SMALL before anything is enqueued (the small and tiny
 * workloads fit; the 768p head share, 420 MB, does not: use vda_forward).  The
 * first call on a GPU looks up the array's device address with that GPU
 * current (VDA_ERR_HIP if that fails); later calls reuse it.  The work runs on
 * the GPU `stream` belongs to.  Every call on one GPU shares that GPU's array,
 * which keeps the last call's contents; nothing in it needs to start at zero.
 * Calls that overlap on one GPU (on different streams, or from several host
 * threads without ordering) race on the array and give undefined results:
 * order them on one stream.  Results are bit-identical to vda_forward. */
int vda_forward_noalloc(const vda_desc_t* desc, const void* q, const void* k, const void* v,
                        const float* beta, const void* gate, const void* text_k,
                        const void* text_v, const float* text_beta, const float* rms_weight,
                        void* out, vda_stream_t stream);

/* vda_forward (alpha NULL) or vda_forward_decay (alpha non-NULL) that also
 * records caller-created HIP events (hipEvent_t, cast to void*) on `stream`
 * at the stage boundaries, for per-kernel timing: stage_events[0] before the
 * statistics kernels, [1] before the solve, [2] before the chunk composition,
 * [3] before the scan, [4] before the readout and [5] after it.  n_events
 * must be 6; a NULL entry skips that boundary (each recorded event is a
 * stream marker that adds a few microseconds between the kernels it
 * separates, so timing one stage needs only its two events).  Results are
 * identical to the untimed entry point. */
int vda_forward_timed(const vda_desc_t* desc, const void* q, const void* k, const void* v,
                      const float* beta, const float* alpha, const void* gate,
                      const void* text_k, const void* text_v, const float* text_beta,
                      const float* rms_weight, void* out, void* workspace, size_t workspace_bytes,
                      vda_stream_t stream, void* const* stage_events, int n_events);

/* The forward pass with channel-wise decay described at the top of this file;
 * alpha [units][frames][d_k] float32 in [0, 1], 16-byte aligned, required
 * (VDA_ERR_INVALID_ARG when NULL and units x frames > 0).  Gates outside
 * [0, 1] are not checked (they break Prop. 1's contraction bound, not the
 * arithmetic).  Other arguments as in vda_forward; the same workspace size.
 * Returns VDA_ERR_INVALID_ARG also when the per-frame launch grids do not fit
 * (see vda_check_desc). */
int vda_forward_decay(const vda_desc_t* desc, const void* q, const void* k, const void* v,
                      const float* beta, const float* alpha, const void* gate,
                      const void* text_k, const void* text_v, const float* text_beta,
                      const float* rms_weight, void* out, void* workspace, size_t workspace_bytes,
                      vda_stream_t stream);

/* ---- feature map (VDA-Prep; [VDN] Sec. 2.3, fused as in Sec. 5) ----
 * From the QKV projection outputs to the prepared features vda_forward takes:
 *   K' = L2(SiLU(conv_k(K))),  V' = SiLU(conv_v(V)),  Q' = L2(Q)
 * conv: depthwise (one filter per head and channel) separable short
 * convolution -- a 5 x 5 spatial filter w_s and a five-tap temporal filter
 * w_t -- applied as the centred correlation
 *   y[t][i][j] = sum_{tau,a,b} w_t[tau] w_s[a][b] x[t+tau-2][i+a-2][j+b-2]
 * with zero padding at the clip's and the frame's borders; SiLU(x) =
 * x sigmoid(x); L2(x) = x / max(||x||_2, eps) over the d channels of one
 * (token, head).  Layouts:
 *   q, k in   [batch][frames][height][width][heads][d_k]   dtype
 *   v in      [batch][frames][height][width][heads][d_v]   dtype
 *   wk_s [heads][d_k][5][5], wk_t [heads][d_k][5], wv_s [heads][d_v][5][5],
 *   wv_t [heads][d_v][5]                                   float32
 *   q, k out  [batch * heads][frames][height * width][d_k] dtype (unit = b * heads + h)
 *   v out     [batch * heads][frames][height * width][d_v] dtype
 * The outputs are exactly the q, k, v layouts of vda_forward (tokens =
 * height * width).  Outputs must not overlap inputs.  q and q_out may both be
 * NULL: then only K' and V' are formed (the query map is left to vda_forward,
 * which takes the raw projection q with q_heads = heads and q_l2_eps = eps and
 * normalises each query inside its readout, saving the query pass's read and
 * write of q; one NULL without the other is VDA_ERR_INVALID_ARG).  Arithmetic is fp32;
 * with bf16 features the spatial filter runs on the matrix cores with each tap
 * split into bf16 hi + lo (the tap to about 2^-17 relative, every product
 * exact, fp32 accumulation). */
typedef struct vda_prep_desc {
  int32_t batch;  /* >= 0 */
  int32_t heads;  /* >= 0; batch x heads <= 65535 */
  int32_t frames; /* 0..2^20 */
  int32_t height; /* latent rows H_l >= 0 */
  int32_t width;  /* latent columns W_l >= 0; height, width and height x width each
                     <= 4194303, height x width x heads x 512 <= 2^31 - 1, and batch x
                     heads x ceil(height / 8) x ceil(width / 8) < 2^21 - 1024 */
  int32_t d_k;    /* channels of q and k: multiple of 16, 16..128 */
  int32_t d_v;    /* channels of v: multiple of 16, 16..128 */
  float eps;      /* L2 normalisation floor: finite, > 0 */
  int32_t dtype;  /* vda_dtype_t of q, k, v in and out */
} vda_prep_desc_t;

/* Checks desc alone (host-only); VDA_OK or the error vda_prep would return. */
int vda_prep_check_desc(const vda_prep_desc_t* desc);

/* Enqueues the feature map on `stream`.  Tensors 16-byte aligned, filters
 * 4-byte aligned; pointers of empty tensors may be NULL.  The caller owns
 * every buffer; nothing is allocated. */
int vda_prep(const vda_prep_desc_t* desc, const void* q, const void* k, const void* v,
             const float* wk_s, const float* wk_t, const float* wv_s, const float* wv_t,
             void* q_out, void* k_out, void* v_out, vda_stream_t stream);

/* ---- debug taps (tests only).  Each runs the pipeline up to the named stage in
 * the caller's workspace and copies that stage's fp32 results to caller
 * buffers (device pointers, row-major, contiguous). ---- */

/* Frame statistics, [VDN] Eq. (3b).  Frame index 0 is the text frame (its beta
 * already halved in seed_mode 1), frame f + 1 is latent frame f.
 * A_out [units][frames + 1][d_k][d_k], B_out [units][frames + 1][d_v][d_k]. */
int vda_debug_stats(const vda_desc_t* desc, const void* k, const void* v, const float* beta,
                    const void* text_k, const void* text_v, const float* text_beta,
                    float* A_out, float* B_out, void* workspace, size_t workspace_bytes,
                    vda_stream_t stream);

/* Transitions M_t = (I + A_t)^{-1} ([VDN] Eq. (A.1)) and the seed ([VDN] Eq. (1b)).
 * Runs the pipeline through the chunk composition, which applies the text
 * frame's map to form the seed.
 * M_out [units][frames + 1][d_k][d_k] (index 0: text frame), seed_out [units][d_v][d_k]. */
int vda_debug_solve(const vda_desc_t* desc, const void* k, const void* v, const float* beta,
                    const void* text_k, const void* text_v, const float* text_beta,
                    float* M_out, float* seed_out, void* workspace, size_t workspace_bytes,
                    vda_stream_t stream);

/* Per-frame maps of the frame-wise rule ([VDN] App. A.1 Eq. (A.1): the update
 * S_t = (S_{t-1} + B_t) M_t written as the affine map S_t = S_{t-1} M_t + J_t):
 * M_t = (I + A_t)^{-1} and J_t = B_t M_t for every frame, text frame at index 0.
 * The forward pass never forms J_t (the chunk composition folds B_t in); this
 * tap computes it from the same B_t and M_t with an fp32 product.
 * M_out [units][frames + 1][d_k][d_k], J_out [units][frames + 1][d_v][d_k].
 * not_spd (device int, may be NULL): the solve writes VDA_ERR_NOT_SPD there when
 * a pivot of some I + A_t is not positive or not a number, i.e. the inputs broke
 * the beta >= 0 precondition of the frame statistics (a negative beta makes
 * sqrt(beta) a NaN); it is never written otherwise, so the caller sets it to
 * VDA_OK first and reads it after synchronising.  The frame-wise rule only
 * (rules 1, 2: VDA_ERR_INVALID_ARG). */
int vda_debug_frame_maps(const vda_desc_t* desc, const void* k, const void* v, const float* beta,
                         const void* text_k, const void* text_v, const float* text_beta,
                         float* M_out, float* J_out, int* not_spd, void* workspace,
                         size_t workspace_bytes, vda_stream_t stream);

/* Composed chunk maps ([VDN] Sec. 5): forward S_out = S_in Mc + Jf over the
 * chunk's frames in order, reverse S_out = S_in Mc^T + Jr over them in
 * reverse order (each M_t is symmetric).  n = ceil(frames / chunk).
 * Mc_out [units][n][d_k][d_k], Jf_out and Jr_out [units][n][d_v][d_k]. */
int vda_debug_chunks(const vda_desc_t* desc, const void* k, const void* v, const float* beta,
                     const void* text_k, const void* text_v, const float* text_beta,
                     float* Mc_out, float* Jf_out, float* Jr_out, void* workspace,
                     size_t workspace_bytes, vda_stream_t stream);

/* Boundary states of both scans: P_out[u][j] = forward state after frames
 * [0, j*chunk), R_out[u][j] = reverse state after frames [j*chunk, F),
 * j = 0..n, with P[0] = R[n] = seed.  P_out, R_out [units][n + 1][d_v][d_k]. */
int vda_debug_states(const vda_desc_t* desc, const void* k, const void* v, const float* beta,
                     const void* text_k, const void* text_v, const float* text_beta,
                     float* P_out, float* R_out, void* workspace, size_t workspace_bytes,
                     vda_stream_t stream);

/* Chunk maps with decay: forward S_out = S_in Mc + Jf over the chunk's frames in
 * order, reverse S_out = S_in Mr + Jr over them in reverse order, where each
 * frame contributes Diag(alpha_t) (I + A_t)^{-1}; Mr is returned transposed
 * (Mr_t_out = Mr^T, the layout the reverse scan reads).  alpha as in
 * vda_forward_decay (required).
 * Mc_out, Mr_t_out [units][n][d_k][d_k], Jf_out and Jr_out [units][n][d_v][d_k]. */
int vda_debug_chunks_decay(const vda_desc_t* desc, const void* k, const void* v,
                           const float* beta, const float* alpha, const void* text_k,
                           const void* text_v, const float* text_beta, float* Mc_out,
                           float* Mr_t_out, float* Jf_out, float* Jr_out, void* workspace,
                           size_t workspace_bytes, vda_stream_t stream);

/* Boundary states of both scans with decay (layout as vda_debug_states). */
int vda_debug_states_decay(const vda_desc_t* desc, const void* k, const void* v,
                           const float* beta, const float* alpha, const void* text_k,
                           const void* text_v, const float* text_beta, float* P_out,
                           float* R_out, void* workspace, size_t workspace_bytes,
                           vda_stream_t stream);

/* Static, human-readable text for a vda_status_t (never NULL). */
const char* vda_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* VDA_H_ */
