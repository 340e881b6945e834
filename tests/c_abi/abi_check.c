/* The C ABI from plain C99: descriptor checks, workspace sizing and status
 * strings (host-only entry points; no device is touched).  Built and run by
 * tests/test_c_abi.py; prints "ok" and exits 0 when every check holds. */
#include <stdio.h>
#include <string.h>

#include "vda.h"

static int failures = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static vda_desc_t base(void) {
  vda_desc_t d;
  memset(&d, 0, sizeof d);
  d.units = 16;
  d.frames = 90;
  d.tokens = 4032;
  d.text_tokens = 512;
  d.d_k = 128;
  d.d_v = 128;
  d.chunk = 5;
  d.radius = 1;
  d.rms_eps = 1e-6f;
  d.seed_mode = 0;
  d.in_dtype = VDA_DTYPE_BF16;
  d.out_dtype = VDA_DTYPE_BF16;
  d.anchors = 0;
  d.rule = 0;
  return d;
}

int main(void) {
  vda_desc_t d = base();
  CHECK(vda_check_desc(&d) == VDA_OK);
  /* A, B, M per (unit, frame + 1); Mc, McT, MrT, Jf, Jr per chunk; P and R */
  {
    const size_t mat = 128 * 128 * 4, U = 16, Fp1 = 91, n = 18;
    const size_t least = U * Fp1 * 3 * mat + U * n * 5 * mat + U * 2 * (n + 1) * mat;
    CHECK(vda_workspace_bytes(&d) >= least);
  }
  d.d_k = 130;
  CHECK(vda_check_desc(&d) == VDA_ERR_INVALID_ARG);
  CHECK(vda_workspace_bytes(&d) == 0);
  d = base();
  d.out_dtype = VDA_DTYPE_F32;
  CHECK(vda_check_desc(&d) == VDA_ERR_BAD_DTYPE);
  d = base();
  d.chunk = 0;
  CHECK(vda_check_desc(&d) == VDA_ERR_INVALID_ARG);
  d = base();
  d.rule = 3;
  CHECK(vda_check_desc(&d) == VDA_ERR_INVALID_ARG);
  CHECK(vda_check_desc(NULL) == VDA_ERR_INVALID_ARG);
  /* an empty problem is valid and needs no workspace */
  d = base();
  d.units = 0;
  CHECK(vda_check_desc(&d) == VDA_OK);
  CHECK(vda_workspace_bytes(&d) == 0);
  /* null pointers are refused before anything is enqueued */
  d = base();
  CHECK(vda_forward(&d, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0,
                    NULL) != VDA_OK);
  /* the allocation-free entry point refuses what its fixed scratch cannot hold
   * (the 768p head share), and checks pointers first on smaller problems */
  CHECK(vda_workspace_bytes(&d) > VDA_NOALLOC_MAX_BYTES);
  CHECK(vda_forward_noalloc(&d, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                            NULL) == VDA_ERR_SCRATCH_TOO_SMALL);
  d.units = 1;
  d.frames = 10;
  d.tokens = 256;
  CHECK(vda_workspace_bytes(&d) <= VDA_NOALLOC_MAX_BYTES);
  CHECK(vda_forward_noalloc(&d, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                            NULL) == VDA_ERR_INVALID_ARG);
  d = base();
  {
    vda_prep_desc_t p;
    memset(&p, 0, sizeof p);
    p.batch = 2;
    p.heads = 8;
    p.frames = 90;
    p.height = 48;
    p.width = 84;
    p.d_k = 128;
    p.d_v = 128;
    p.eps = 1e-6f;
    p.dtype = VDA_DTYPE_BF16;
    CHECK(vda_prep_check_desc(&p) == VDA_OK);
    p.eps = 0.0f;
    CHECK(vda_prep_check_desc(&p) == VDA_ERR_INVALID_ARG);
  }
  {
    const int codes[] = {VDA_OK, VDA_ERR_INVALID_ARG, VDA_ERR_BAD_DTYPE,
                         VDA_ERR_WORKSPACE_TOO_SMALL, VDA_ERR_MISALIGNED, VDA_ERR_HIP, -99};
    for (size_t i = 0; i < sizeof codes / sizeof codes[0]; ++i) {
      const char* s = vda_status_string(codes[i]);
      CHECK(s != NULL && s[0] != '\0');
    }
  }
  if (failures) return 1;
  printf("ok\n");
  return 0;
}
