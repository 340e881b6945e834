/* One VDA forward pass driven from plain C99 through the C ABI and the HIP
 * runtime's C API: deterministic bf16 inputs (a small xorshift generator),
 * device buffers from hipMalloc, vda_forward on the default stream, the output
 * copied back.  Writes the inputs and the output to the file named by argv[1]
 * (layout below) so that tests/test_c_abi_gpu.py can compare them with the
 * fp64 oracle.  Exit status 0 on success.
 *
 * File: int32 units, frames, tokens, text_tokens, d_k, d_v, chunk, radius;
 * then q, k, v, gate (bf16 bits), beta (fp32), text_k, text_v (bf16 bits),
 * text_beta (fp32), rms_weight (fp32), out (bf16 bits), in that order. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "vda.h"

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static double uniform(void) { /* xorshift64*, in (0, 1) */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return ((rng_state * 2685821657736338717ull) >> 11) * (1.0 / 9007199254740992.0) + 1e-17;
}
static double normal(void) { return sqrt(-2.0 * log(uniform())) * cos(6.283185307179586 * uniform()); }

static uint16_t to_bf16(float x) { /* round to nearest even (finite inputs) */
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

#define HIP(call)                                                        \
  do {                                                                   \
    hipError_t e_ = (call);                                              \
    if (e_ != hipSuccess) {                                              \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_)); \
      return 1;                                                          \
    }                                                                    \
  } while (0)

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s OUTFILE\n", argv[0]);
    return 2;
  }
  const int32_t dims[8] = {2, 11, 40, 7, 64, 48, 5, 1}; /* units F U T dk dv chunk radius */
  const size_t units = dims[0], F = dims[1], U = dims[2], T = dims[3], dk = dims[4], dv = dims[5];
  const size_t nq = units * F * U * dk, nv = units * F * U * dv, nb = units * F * U;
  const size_t ntk = units * T * dk, ntv = units * T * dv, ntb = units * T;
  uint16_t *q = malloc(nq * 2), *k = malloc(nq * 2), *v = malloc(nv * 2), *g = malloc(nv * 2);
  uint16_t *tk = malloc(ntk * 2), *tv = malloc(ntv * 2), *out = malloc(nv * 2);
  float *beta = malloc(nb * 4), *tb = malloc(ntb * 4), *w = malloc(dv * 4);
  if (!q || !k || !v || !g || !tk || !tv || !out || !beta || !tb || !w) return 1;
  for (size_t i = 0; i < nq; ++i) q[i] = to_bf16((float)normal());
  for (size_t r = 0; r < nb; ++r) { /* unit keys */
    double x[128], ss = 0.0;
    for (size_t c = 0; c < dk; ++c) {
      x[c] = normal();
      ss += x[c] * x[c];
    }
    for (size_t c = 0; c < dk; ++c) k[r * dk + c] = to_bf16((float)(x[c] / sqrt(ss)));
  }
  for (size_t i = 0; i < nv; ++i) v[i] = to_bf16((float)normal());
  for (size_t i = 0; i < nv; ++i) g[i] = to_bf16((float)normal());
  for (size_t i = 0; i < nb; ++i) beta[i] = (float)(1.0 / (1.0 + exp(-normal())));
  for (size_t r = 0; r < units * T; ++r) {
    double x[128], ss = 0.0;
    for (size_t c = 0; c < dk; ++c) {
      x[c] = normal();
      ss += x[c] * x[c];
    }
    for (size_t c = 0; c < dk; ++c) tk[r * dk + c] = to_bf16((float)(x[c] / sqrt(ss)));
  }
  for (size_t i = 0; i < ntv; ++i) tv[i] = to_bf16((float)normal());
  for (size_t i = 0; i < ntb; ++i) tb[i] = (float)(1.0 / (1.0 + exp(-normal())));
  for (size_t i = 0; i < dv; ++i) w[i] = 1.0f;

  vda_desc_t d;
  memset(&d, 0, sizeof d);
  d.units = dims[0];
  d.frames = dims[1];
  d.tokens = dims[2];
  d.text_tokens = dims[3];
  d.d_k = dims[4];
  d.d_v = dims[5];
  d.chunk = dims[6];
  d.radius = dims[7];
  d.rms_eps = 1e-6f;
  d.in_dtype = VDA_DTYPE_BF16;
  d.out_dtype = VDA_DTYPE_BF16;
  const size_t ws_bytes = vda_workspace_bytes(&d);
  if (ws_bytes == 0) return 1;

  void *dq, *dk_, *dv_, *dg, *dtk, *dtv, *dout, *dws;
  float *dbeta, *dtb, *dw;
  HIP(hipMalloc(&dq, nq * 2));
  HIP(hipMalloc(&dk_, nq * 2));
  HIP(hipMalloc(&dv_, nv * 2));
  HIP(hipMalloc(&dg, nv * 2));
  HIP(hipMalloc(&dtk, ntk * 2));
  HIP(hipMalloc(&dtv, ntv * 2));
  HIP(hipMalloc(&dout, nv * 2));
  HIP(hipMalloc((void**)&dbeta, nb * 4));
  HIP(hipMalloc((void**)&dtb, ntb * 4));
  HIP(hipMalloc((void**)&dw, dv * 4));
  HIP(hipMalloc(&dws, ws_bytes));
  HIP(hipMemcpy(dq, q, nq * 2, hipMemcpyHostToDevice));
  HIP(hipMemcpy(dk_, k, nq * 2, hipMemcpyHostToDevice));
  HIP(hipMemcpy(dv_, v, nv * 2, hipMemcpyHostToDevice));
  HIP(hipMemcpy(dg, g, nv * 2, hipMemcpyHostToDevice));
  HIP(hipMemcpy(dtk, tk, ntk * 2, hipMemcpyHostToDevice));
  HIP(hipMemcpy(dtv, tv, ntv * 2, hipMemcpyHostToDevice));
  HIP(hipMemcpy(dbeta, beta, nb * 4, hipMemcpyHostToDevice));
  HIP(hipMemcpy(dtb, tb, ntb * 4, hipMemcpyHostToDevice));
  HIP(hipMemcpy(dw, w, dv * 4, hipMemcpyHostToDevice));

  const int st = vda_forward(&d, dq, dk_, dv_, dbeta, dg, dtk, dtv, dtb, dw, dout, dws, ws_bytes,
                             NULL);
  if (st != VDA_OK) {
    fprintf(stderr, "vda_forward: %s\n", vda_status_string(st));
    return 1;
  }
  HIP(hipDeviceSynchronize());
  HIP(hipMemcpy(out, dout, nv * 2, hipMemcpyDeviceToHost));

  FILE* f = fopen(argv[1], "wb");
  if (!f) return 1;
  fwrite(dims, 4, 8, f);
  fwrite(q, 2, nq, f);
  fwrite(k, 2, nq, f);
  fwrite(v, 2, nv, f);
  fwrite(g, 2, nv, f);
  fwrite(beta, 4, nb, f);
  fwrite(tk, 2, ntk, f);
  fwrite(tv, 2, ntv, f);
  fwrite(tb, 4, ntb, f);
  fwrite(w, 4, dv, f);
  fwrite(out, 2, nv, f);
  fclose(f);
  hipFree(dq);
  hipFree(dk_);
  hipFree(dv_);
  hipFree(dg);
  hipFree(dtk);
  hipFree(dtv);
  hipFree(dout);
  hipFree(dbeta);
  hipFree(dtb);
  hipFree(dw);
  hipFree(dws);
  printf("ok\n");
  return 0;
}
