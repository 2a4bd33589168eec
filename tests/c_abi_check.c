/* The C ABI used from C (no Python, no torch): buffer sizes, struct sizes and
 * the status codes of argument validation.  Every call below returns before
 * the library makes any HIP call, so this runs on a machine without a GPU.
 * Built and run by tests/test_c_abi_cpu.py; prints one "key value" line per
 * check. */
#include <stdio.h>
#include <string.h>

#include "sage_attn.h"

int main(void) {
  const sage_shape_t shapes[3] = {{2, 3, 300, 700, 128}, {1, 1, 1, 1, 64}, {3, 21845, 33, 70, 64}};
  for (int i = 0; i < 3; ++i)
    for (int w = 0; w < SAGE_BUF_COUNT; ++w) {
      size_t n = 0;
      const int r = sage_buffer_bytes(&shapes[i], w, &n);
      printf("buf_%d_%d %d %zu\n", i, w, r, n);
    }
  for (int i = 0; i < 3; ++i) {
    size_t off = 0;
    const int r = sage_prep_status_offset(&shapes[i], &off);
    printf("status_off_%d %d %zu\n", i, r, off);
  }
  printf("status_off_null %d\n", sage_prep_status_offset(&shapes[0], NULL));
  printf("sizeof_shape %zu\n", sizeof(sage_shape_t));
  printf("sizeof_strides %zu\n", sizeof(sage_strides_t));
  printf("sizeof_quant %zu\n", sizeof(sage_quant_t));

  sage_shape_t s = shapes[0];
  sage_strides_t st;
  memset(&st, 0, sizeof st);
  sage_quant_t q;
  memset(&q, 0, sizeof q);
  size_t n = 0;
  printf("bytes_null_shape %d\n", sage_buffer_bytes(NULL, 0, &n));
  printf("bytes_bad_which %d\n", sage_buffer_bytes(&s, SAGE_BUF_COUNT, &n));
  sage_shape_t bad = s;
  bad.D = 96;
  printf("bytes_bad_headdim %d\n", sage_buffer_bytes(&bad, 0, &n));
  bad = s;
  bad.H = 65536;
  bad.B = 1;
  printf("bytes_too_many_heads %d\n", sage_buffer_bytes(&bad, 0, &n));
  printf("prep_null_inputs %d\n", sage_quant_prep(NULL, NULL, NULL, &s, &st, &q, NULL));
  printf("prep1_null_inputs %d\n", sage_quant_prep_single_pass(NULL, NULL, NULL, &s, &st, &q, NULL));
  printf("prep_bad_shape %d\n", sage_quant_prep((void *)16, (void *)16, (void *)16, &bad, &st, &q, NULL));
  printf("fwd_null_out %d\n", sage_attn_fwd(&q, &s, 0.f, NULL, &st, NULL));
  printf("status_alias %s\n", sage_status_string(SAGE_E_ALIAS));
  printf("status_unknown %s\n", sage_status_string(12345));
  return 0;
}
