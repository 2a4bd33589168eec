/* A caller of the C ABI written in C against the HIP runtime API only (no
 * Python, no torch).  Reads bf16 Q [B,H,Nq,D], K and V [B,H,Nkv,D] (row-major,
 * raw little-endian bf16) from files, allocates every buffer with hipMalloc,
 * runs sage_quant_prep (or the single pass) and sage_attn_fwd on the default
 * stream and writes O [B,H,Nq,D] as raw bf16.  Built and run by
 * tests/test_c_abi_gpu.py.
 *
 *   c_abi_gpu B H Nq Nkv D q.bin k.bin v.bin o.bin single_pass(0|1)
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>

#include "sage_attn.h"

#define HIP_OK(x)                                                            \
  do {                                                                       \
    hipError_t e_ = (x);                                                     \
    if (e_ != hipSuccess) {                                                  \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                \
      return 1;                                                              \
    }                                                                        \
  } while (0)

static int read_exact(const char *path, void *buf, size_t n) {
  FILE *f = fopen(path, "rb");
  if (!f) return 0;
  const size_t got = fread(buf, 1, n, f);
  fclose(f);
  return got == n;
}

int main(int argc, char **argv) {
  if (argc != 11) {
    fprintf(stderr, "usage: %s B H Nq Nkv D q.bin k.bin v.bin o.bin single_pass\n", argv[0]);
    return 2;
  }
  sage_shape_t s = {atoi(argv[1]), atoi(argv[2]), atoi(argv[3]), atoi(argv[4]), atoi(argv[5])};
  const int single_pass = atoi(argv[10]);
  size_t n;
  /* sage_buffer_bytes validates the shape before anything is allocated */
  int r = sage_buffer_bytes(&s, SAGE_BUF_Q_CODES, &n);
  if (r != SAGE_OK) {
    fprintf(stderr, "shape: %s\n", sage_status_string(r));
    return 1;
  }
  const size_t bq = (size_t)s.B * s.H * s.Nq * s.D * 2, bkv = (size_t)s.B * s.H * s.Nkv * s.D * 2;
  void *hq = malloc(bq), *hk = malloc(bkv), *hv = malloc(bkv), *ho = malloc(bq);
  if (!hq || !hk || !hv || !ho) return 1;
  if (!read_exact(argv[6], hq, bq) || !read_exact(argv[7], hk, bkv) || !read_exact(argv[8], hv, bkv)) {
    fprintf(stderr, "short input file\n");
    return 1;
  }
  void *dq, *dk, *dv, *dout;
  HIP_OK(hipMalloc(&dq, bq));
  HIP_OK(hipMalloc(&dk, bkv));
  HIP_OK(hipMalloc(&dv, bkv));
  HIP_OK(hipMalloc(&dout, bq));
  HIP_OK(hipMemcpy(dq, hq, bq, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dk, hk, bkv, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dv, hv, bkv, hipMemcpyHostToDevice));

  void *buf[SAGE_BUF_COUNT];
  for (int i = 0; i < SAGE_BUF_COUNT; ++i) {
    if ((r = sage_buffer_bytes(&s, i, &n)) != SAGE_OK) return 1;
    HIP_OK(hipMalloc(&buf[i], n));
  }
  sage_quant_t quant = {(int8_t *)buf[SAGE_BUF_Q_CODES], (float *)buf[SAGE_BUF_Q_SCALE],
                        (int8_t *)buf[SAGE_BUF_K_CODES], (float *)buf[SAGE_BUF_K_SCALE],
                        (uint8_t *)buf[SAGE_BUF_V_CODES], (float *)buf[SAGE_BUF_V_SCALE],
                        (float *)buf[SAGE_BUF_K_MEAN],    buf[SAGE_BUF_WORKSPACE]};
  sage_strides_t st;
  const int64_t sq[3] = {(int64_t)s.H * s.Nq * s.D, (int64_t)s.Nq * s.D, s.D};
  const int64_t skv[3] = {(int64_t)s.H * s.Nkv * s.D, (int64_t)s.Nkv * s.D, s.D};
  for (int i = 0; i < 3; ++i) {
    st.q[i] = sq[i];
    st.o[i] = sq[i];
    st.k[i] = skv[i];
    st.v[i] = skv[i];
  }
  r = single_pass ? sage_quant_prep_single_pass(dq, dk, dv, &s, &st, &quant, NULL)
                  : sage_quant_prep(dq, dk, dv, &s, &st, &quant, NULL);
  if (r != SAGE_OK) {
    fprintf(stderr, "prep: %s\n", sage_status_string(r));
    return 1;
  }
  r = sage_attn_fwd(&quant, &s, 0.0f, dout, &st, NULL);
  if (r != SAGE_OK) {
    fprintf(stderr, "fwd: %s\n", sage_status_string(r));
    return 1;
  }
  HIP_OK(hipDeviceSynchronize());
  if (single_pass) {
    /* the single pass reports a workgroup that stopped waiting in its status word */
    size_t off = 0;
    uint32_t status = 1;
    if ((r = sage_prep_status_offset(&s, &off)) != SAGE_OK) return 1;
    HIP_OK(hipMemcpy(&status, (char *)quant.workspace + off, sizeof status, hipMemcpyDeviceToHost));
    if (status != 0) {
      fprintf(stderr, "single-pass prep status word %u\n", status);
      return 1;
    }
  }
  HIP_OK(hipMemcpy(ho, dout, bq, hipMemcpyDeviceToHost));
  FILE *f = fopen(argv[9], "wb");
  if (!f || fwrite(ho, 1, bq, f) != bq) return 1;
  fclose(f);
  for (int i = 0; i < SAGE_BUF_COUNT; ++i) HIP_OK(hipFree(buf[i]));
  HIP_OK(hipFree(dq));
  HIP_OK(hipFree(dk));
  HIP_OK(hipFree(dv));
  HIP_OK(hipFree(dout));
  free(hq);
  free(hk);
  free(hv);
  free(ho);
  printf("ok\n");
  return 0;
}
