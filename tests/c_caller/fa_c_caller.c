/*
 * A plain C caller of libfa: no Python, no torch, only the HIP runtime's C
 * API for device memory and a stream.  It shows that the boundary declared
 * in include/fa.h is usable as it stands, and the GPU test that runs it
 * checks the results against the fp64 oracle.
 *
 * usage: fa_c_caller DIR
 *   DIR/args.txt   "B Hq Hkv N d causal window_left scale"
 *   DIR/q.bin, DIR/k.bin, DIR/v.bin, DIR/do.bin
 *                  bfloat16 bit patterns, [B][H][N][d] (little endian)
 * writes DIR/o.bin (bfloat16), DIR/lse.bin (float32 [B][Hq][N]) from
 * fa_fwd_bf16, and DIR/dq.bin, DIR/dk.bin, DIR/dv.bin (bfloat16) from
 * fa_bwd_bf16 on that o and lse; then checks that two invalid calls are
 * refused with the documented status before anything is enqueued.
 * Exit status 0 on success, 1 on any failure (with a message on stderr).
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fa.h"

#define HIP_OK(call)                                                        \
  do {                                                                      \
    hipError_t e_ = (call);                                                 \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));     \
      return 1;                                                             \
    }                                                                       \
  } while (0)

static int read_file(const char* dir, const char* name, void* dst, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", path);
    return 1;
  }
  size_t got = fread(dst, 1, bytes, f);
  fclose(f);
  if (got != bytes) {
    fprintf(stderr, "%s: read %zu of %zu bytes\n", path, got, bytes);
    return 1;
  }
  return 0;
}

static int write_file(const char* dir, const char* name, const void* src, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(src, 1, bytes, f) != bytes) {
    fprintf(stderr, "cannot write %s\n", path);
    if (f) fclose(f);
    return 1;
  }
  fclose(f);
  return 0;
}

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s DIR\n", argv[0]);
    return 1;
  }
  const char* dir = argv[1];
  char path[4096];
  snprintf(path, sizeof path, "%s/args.txt", dir);
  FILE* fa = fopen(path, "r");
  int B, Hq, Hkv, N, d, causal, wl;
  float scale;
  if (!fa || fscanf(fa, "%d %d %d %d %d %d %d %f", &B, &Hq, &Hkv, &N, &d, &causal, &wl, &scale) != 8) {
    fprintf(stderr, "cannot read %s\n", path);
    if (fa) fclose(fa);
    return 1;
  }
  fclose(fa);
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || d <= 0) {
    fprintf(stderr, "sizes must be positive\n");
    return 1;
  }
  const size_t nq = (size_t)B * Hq * N * d, nkv = (size_t)B * Hkv * N * d, nl = (size_t)B * Hq * N;
  unsigned short* hq = malloc(nq * 2);
  unsigned short* hk = malloc(nkv * 2);
  unsigned short* hv = malloc(nkv * 2);
  unsigned short* hdo = malloc(nq * 2);
  unsigned short* hbuf = malloc((nq > nkv ? nq : nkv) * 2);
  float* hl = malloc(nl * sizeof(float));
  if (!hq || !hk || !hv || !hdo || !hbuf || !hl) {
    fprintf(stderr, "out of host memory\n");
    return 1;
  }
  if (read_file(dir, "q.bin", hq, nq * 2) || read_file(dir, "k.bin", hk, nkv * 2) ||
      read_file(dir, "v.bin", hv, nkv * 2) || read_file(dir, "do.bin", hdo, nq * 2))
    return 1;

  void *q, *k, *v, *o, *dout, *dq, *dk, *dv;
  float *lse, *work;
  const size_t work_bytes = fa_bwd_workspace_size(B, Hq, N);
  HIP_OK(hipMalloc(&q, nq * 2));
  HIP_OK(hipMalloc(&k, nkv * 2));
  HIP_OK(hipMalloc(&v, nkv * 2));
  HIP_OK(hipMalloc(&o, nq * 2));
  HIP_OK(hipMalloc(&dout, nq * 2));
  HIP_OK(hipMalloc(&dq, nq * 2));
  HIP_OK(hipMalloc(&dk, nkv * 2));
  HIP_OK(hipMalloc(&dv, nkv * 2));
  HIP_OK(hipMalloc((void**)&lse, nl * sizeof(float)));
  HIP_OK(hipMalloc((void**)&work, work_bytes > 0 ? work_bytes : 16));
  HIP_OK(hipMemcpy(q, hq, nq * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(k, hk, nkv * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(v, hv, nkv * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dout, hdo, nq * 2, hipMemcpyHostToDevice));
  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));

  int st = fa_fwd_bf16(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, wl, scale, stream);
  if (st != FA_OK) {
    fprintf(stderr, "fa_fwd_bf16: %s (%s)\n", fa_status_string(st), fa_last_error());
    return 1;
  }
  st = fa_bwd_bf16(q, k, v, o, lse, dout, dq, dk, dv, work, B, Hq, Hkv, N, d, causal, wl, scale, stream);
  if (st != FA_OK) {
    fprintf(stderr, "fa_bwd_bf16: %s (%s)\n", fa_status_string(st), fa_last_error());
    return 1;
  }
  HIP_OK(hipStreamSynchronize(stream));

  HIP_OK(hipMemcpy(hbuf, o, nq * 2, hipMemcpyDeviceToHost));
  if (write_file(dir, "o.bin", hbuf, nq * 2)) return 1;
  HIP_OK(hipMemcpy(hl, lse, nl * sizeof(float), hipMemcpyDeviceToHost));
  if (write_file(dir, "lse.bin", hl, nl * sizeof(float))) return 1;
  HIP_OK(hipMemcpy(hbuf, dq, nq * 2, hipMemcpyDeviceToHost));
  if (write_file(dir, "dq.bin", hbuf, nq * 2)) return 1;
  HIP_OK(hipMemcpy(hbuf, dk, nkv * 2, hipMemcpyDeviceToHost));
  if (write_file(dir, "dk.bin", hbuf, nkv * 2)) return 1;
  HIP_OK(hipMemcpy(hbuf, dv, nkv * 2, hipMemcpyDeviceToHost));
  if (write_file(dir, "dv.bin", hbuf, nkv * 2)) return 1;

  /* refused on the host, before any launch */
  st = fa_fwd_bf16(q, k, v, o, lse, B, Hq, Hq + 1, N, d, causal, wl, scale, stream);
  if (st != FA_ERR_INVALID_ARG || strlen(fa_last_error()) == 0) {
    fprintf(stderr, "a head count that does not divide Hq gave %d\n", st);
    return 1;
  }
  st = fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, wl, scale, stream, 7);
  if (st != FA_ERR_UNSUPPORTED) {
    fprintf(stderr, "an unknown element type gave %d\n", st);
    return 1;
  }

  HIP_OK(hipStreamDestroy(stream));
  HIP_OK(hipFree(q));
  HIP_OK(hipFree(k));
  HIP_OK(hipFree(v));
  HIP_OK(hipFree(o));
  HIP_OK(hipFree(dout));
  HIP_OK(hipFree(dq));
  HIP_OK(hipFree(dk));
  HIP_OK(hipFree(dv));
  HIP_OK(hipFree(lse));
  HIP_OK(hipFree(work));
  free(hq);
  free(hk);
  free(hv);
  free(hdo);
  free(hbuf);
  free(hl);
  printf("fa_c_caller: ok (fa_version %d)\n", fa_version());
  return 0;
}
