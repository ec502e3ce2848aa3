/* A C99 program that runs the attention forward on the GPU through include/attn.h and
 * libattn.so, with device memory from the HIP runtime's C API: the library's entry points
 * are called directly, with no Python or torch between the caller and the kernels.
 *
 *   fwd_from_c IN OUT B Hq Hkv Lq Lk D DTYPE SCALE
 *
 * IN holds Q [B,Hq,Lq,D], then K and V [B,Hkv,Lk,D], as raw 16-bit values of type DTYPE
 * (0 fp16, 1 bf16).  OUT receives, as raw bytes:
 *   O [B,Hq,Lq,D] (16-bit) and LSE [B,Hq,Lq] (fp32) of attn_fwd (null stream), then
 *   O and LSE of attn_fwd_ex with the causal mask and the planner's key splits (nsplit = 0,
 *   workspace from hipMalloc, sized by attn_plan_ex).
 * Outputs are filled with 0xFF bytes (NaN) before each call, so an element the kernels do
 * not write shows up.  It also checks that a refused call returns the documented code.
 * Prints one line per step and "fwd_from_c: ok" at the end; returns 0 on success. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "attn.h"

static int fail(const char* what, long code) {
  fprintf(stderr, "fwd_from_c: %s failed (%ld)\n", what, code);
  return 1;
}

#define HIP_OK(call)                                   \
  do {                                                 \
    hipError_t e_ = (call);                            \
    if (e_ != hipSuccess) return fail(#call, (long)e_); \
  } while (0)

int main(int argc, char** argv) {
  if (argc != 11) {
    fprintf(stderr, "usage: %s IN OUT B Hq Hkv Lq Lk D DTYPE SCALE\n", argv[0]);
    return 2;
  }
  const int64_t B = atoll(argv[3]), Hq = atoll(argv[4]), Hkv = atoll(argv[5]);
  const int64_t Lq = atoll(argv[6]), Lk = atoll(argv[7]), D = atoll(argv[8]);
  const int dtype = atoi(argv[9]);
  const float scale = (float)atof(argv[10]);
  const size_t qbytes = (size_t)(B * Hq * Lq * D) * 2, kvbytes = (size_t)(B * Hkv * Lk * D) * 2;
  const size_t lbytes = (size_t)(B * Hq * Lq) * 4;

  char* host = (char*)malloc(qbytes + 2 * kvbytes);
  char* out = (char*)malloc(2 * (qbytes + lbytes));
  if (!host || !out) return fail("malloc", 0);
  FILE* f = fopen(argv[1], "rb");
  if (!f || fread(host, 1, qbytes + 2 * kvbytes, f) != qbytes + 2 * kvbytes)
    return fail("read IN", 0);
  fclose(f);

  void *q, *k, *v, *o;
  float* lse;
  HIP_OK(hipMalloc(&q, qbytes));
  HIP_OK(hipMalloc(&k, kvbytes));
  HIP_OK(hipMalloc(&v, kvbytes));
  HIP_OK(hipMalloc(&o, qbytes));
  HIP_OK(hipMalloc((void**)&lse, lbytes));
  HIP_OK(hipMemcpy(q, host, qbytes, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(k, host + qbytes, kvbytes, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(v, host + qbytes + kvbytes, kvbytes, hipMemcpyHostToDevice));

  /* a refused call: unsupported head dimension, nothing enqueued */
  int rc = attn_fwd(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, 64, scale, dtype);
  if (rc != ATTN_E_HEADDIM) return fail("attn_fwd with D = 64 (expected ATTN_E_HEADDIM)", rc);
  printf("refused call: %s\n", attn_strerror(rc));

  /* 1. attn_fwd on the null stream */
  HIP_OK(hipMemset(o, 0xFF, qbytes));
  HIP_OK(hipMemset(lse, 0xFF, lbytes));
  HIP_OK(hipDeviceSynchronize());
  rc = attn_fwd(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, scale, dtype);
  if (rc != ATTN_OK) return fail(attn_strerror(rc), rc);
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(out, o, qbytes, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(out + qbytes, lse, lbytes, hipMemcpyDeviceToHost));
  printf("attn_fwd: ok\n");

  /* 2. attn_fwd_ex, causal, planner's split count, caller-allocated workspace */
  attn_plan_t plan;
  rc = attn_plan_ex(B, Hq, Hkv, Lq, Lk, D, dtype, ATTN_CAUSAL, &plan);
  if (rc != ATTN_OK) return fail("attn_plan_ex", rc);
  void* ws = NULL;
  if (plan.workspace_bytes > 0) HIP_OK(hipMalloc(&ws, (size_t)plan.workspace_bytes));
  HIP_OK(hipMemset(o, 0xFF, qbytes));
  HIP_OK(hipMemset(lse, 0xFF, lbytes));
  HIP_OK(hipDeviceSynchronize());
  rc = attn_fwd_ex(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, scale, dtype, ATTN_CAUSAL, 0, ws,
                   plan.workspace_bytes, NULL);
  if (rc != ATTN_OK) return fail(attn_strerror(rc), rc);
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(out + qbytes + lbytes, o, qbytes, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(out + 2 * qbytes + lbytes, lse, lbytes, hipMemcpyDeviceToHost));
  printf("attn_fwd_ex causal: ok (%s, nsplit %d)\n", plan.kernel, (int)plan.nsplit);

  if (ws) HIP_OK(hipFree(ws));
  HIP_OK(hipFree(q));
  HIP_OK(hipFree(k));
  HIP_OK(hipFree(v));
  HIP_OK(hipFree(o));
  HIP_OK(hipFree(lse));
  f = fopen(argv[2], "wb");
  if (!f || fwrite(out, 1, 2 * (qbytes + lbytes), f) != 2 * (qbytes + lbytes))
    return fail("write OUT", 0);
  fclose(f);
  free(host);
  free(out);
  printf("fwd_from_c: ok\n");
  return 0;
}
