/* Host-side descriptor fuzzing of the C ABI: a fixed-seed stream of
 * descriptors whose fields are drawn mostly from their valid ranges and
 * otherwise from range edges (the documented limits and one past them,
 * INT32_MIN/INT32_MAX, NaN and infinities) goes through every host-only path: the descriptor checks, workspace sizing, and
 * the forward / feature-map entry points with NULL pointers (refused before
 * anything is enqueued, or accepted as an empty problem, which enqueues
 * nothing).  Built with the host sanitizers by tests/test_host_sanitizers.py,
 * where any overflow in the size arithmetic or an out-of-bounds read stops the
 * run; prints "ok" when every consistency check holds. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "vda.h"

static uint64_t state = 0x9E3779B97F4A7C15ull;

static uint32_t next_u32(void) { /* xorshift64* (Vigna 2016) */
  state ^= state >> 12;
  state ^= state << 25;
  state ^= state >> 27;
  return (uint32_t)((state * 0x2545F4914F6CDD1Dull) >> 32);
}

static int32_t pick(const int32_t* v, int n) { return v[next_u32() % (uint32_t)n]; }

#define N(a) ((int)(sizeof(a) / sizeof((a)[0])))

/* Each field: seven times in eight a value from its valid range (so that a
 * useful share of descriptors passes every check), else a range edge. */
static const int32_t kCountOk[] = {0, 1, 2, 3, 16, 255, 256, 4032};
static const int32_t kCountEdge[] = {65535, 65536, 1 << 20, (1 << 20) + 1, 4194303, 4194304,
                                     INT32_MAX, -1, INT32_MIN};
static const int32_t kDimOk[] = {16, 32, 48, 64, 112, 128};
static const int32_t kDimEdge[] = {0, 8, 15, 24, 129, 144, 256, -16, INT32_MAX};
static const int32_t kChunkOk[] = {1, 2, 3, 5, 7, 90};
static const int32_t kRadiusOk[] = {0, 1, 2, 3};
static const int32_t kSmallEdge[] = {0, 1 << 24, INT32_MAX, -1, INT32_MIN};
static const int32_t kFlagOk[] = {0, 1};
static const int32_t kFlagEdge[] = {2, -1, INT32_MAX};

static int32_t draw(const int32_t* ok, int nok, const int32_t* edge, int nedge) {
  return (next_u32() & 7u) ? pick(ok, nok) : pick(edge, nedge);
}

#define DRAW(ok, edge) draw(ok, N(ok), edge, N(edge))

static float pick_eps(void) {
  const float ok[] = {1e-6f, 1.0f, 0.0f};
  const float edge[] = {-1e-6f, NAN, INFINITY, -INFINITY, 1e30f};
  return (next_u32() & 7u) ? ok[next_u32() % 3u] : edge[next_u32() % 5u];
}

int main(void) {
  int failures = 0;
  int accepted = 0, prep_accepted = 0;
  for (int it = 0; it < 200000; ++it) {
    vda_desc_t d;
    memset(&d, 0, sizeof d);
    d.units = DRAW(kCountOk, kCountEdge);
    d.frames = DRAW(kCountOk, kCountEdge);
    d.tokens = DRAW(kCountOk, kCountEdge);
    d.text_tokens = DRAW(kCountOk, kCountEdge);
    d.d_k = DRAW(kDimOk, kDimEdge);
    d.d_v = DRAW(kDimOk, kDimEdge);
    d.chunk = DRAW(kChunkOk, kSmallEdge);
    d.radius = DRAW(kRadiusOk, kSmallEdge);
    d.rms_eps = pick_eps();
    d.seed_mode = DRAW(kFlagOk, kFlagEdge);
    d.in_dtype = DRAW(kFlagOk, kFlagEdge);
    d.out_dtype = (next_u32() & 7u) ? d.in_dtype : DRAW(kFlagOk, kFlagEdge);
    d.anchors = DRAW(kFlagOk, kFlagEdge);
    d.rule = DRAW(kFlagOk, kFlagEdge);
    d.fp32_products = DRAW(kFlagOk, kFlagEdge);
    d.solver = DRAW(kFlagOk, kFlagEdge);
    d.q_heads = (next_u32() & 3u) ? 0 : DRAW(kChunkOk, kSmallEdge);
    d.q_l2_eps = (next_u32() & 3u) ? 0.0f : pick_eps();
    const int st = vda_check_desc(&d);
    const size_t ws = vda_workspace_bytes(&d);
    if (st != VDA_OK && ws != 0) {
      fprintf(stderr, "iteration %d: invalid descriptor (%d) sized %zu bytes\n", it, st, ws);
      ++failures;
    }
    if (st == VDA_OK) {
      ++accepted;
      const int empty = d.units == 0 || d.frames == 0;
      if (empty != (ws == 0)) {
        fprintf(stderr, "iteration %d: workspace %zu for an %s problem\n", it, ws,
                empty ? "empty" : "non-empty");
        ++failures;
      }
      /* every tensor pointer NULL: only an empty problem (no rows to write and
       * no state to build) may be accepted */
      const int rows = d.units != 0 && d.frames != 0 && d.tokens != 0;
      const int f = vda_forward(&d, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                                NULL, 0, NULL);
      if (rows && f == VDA_OK) {
        fprintf(stderr, "iteration %d: NULL tensors accepted\n", it);
        ++failures;
      }
      const int g = vda_forward_noalloc(&d, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                                        NULL, NULL);
      if (ws > VDA_NOALLOC_MAX_BYTES ? g != VDA_ERR_SCRATCH_TOO_SMALL : (rows && g == VDA_OK)) {
        fprintf(stderr, "iteration %d: noalloc returned %d for %zu bytes\n", it, g, ws);
        ++failures;
      }
    } else if (vda_forward(&d, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                           0, NULL) != st) {
      fprintf(stderr, "iteration %d: forward and check disagree\n", it);
      ++failures;
    }
    if (vda_status_string(st) == NULL) ++failures;

    vda_prep_desc_t p;
    memset(&p, 0, sizeof p);
    p.batch = DRAW(kRadiusOk, kSmallEdge);
    p.heads = DRAW(kChunkOk, kSmallEdge);
    p.frames = DRAW(kCountOk, kCountEdge);
    p.height = DRAW(kCountOk, kCountEdge);
    p.width = DRAW(kCountOk, kCountEdge);
    p.d_k = DRAW(kDimOk, kDimEdge);
    p.d_v = DRAW(kDimOk, kDimEdge);
    p.eps = pick_eps();
    p.dtype = DRAW(kFlagOk, kFlagEdge);
    const int ps = vda_prep_check_desc(&p);
    prep_accepted += ps == VDA_OK;
    const int pr = vda_prep(&p, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL);
    if (ps != VDA_OK && pr != ps) {
      fprintf(stderr, "iteration %d: prep and its check disagree (%d, %d)\n", it, pr, ps);
      ++failures;
    }
    if (failures > 20) break;
  }
  if (accepted < 10000 || prep_accepted < 10000) {
    fprintf(stderr, "only %d / %d descriptors accepted: the stream misses the valid range\n",
            accepted, prep_accepted);
    ++failures;
  }
  if (failures) return 1;
  printf("ok\n");
  return 0;
}
