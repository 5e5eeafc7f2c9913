/*
 * c_client.c -- a plain C caller of the library's C ABI (include/sgemm.h),
 * with no Python and no torch: device memory comes from the HIP runtime.
 *
 * Usage: c_client M N K alpha beta in.bin out.bin
 *
 * in.bin holds A (M x K), B (K x N) and C (M x N) as row-major float32, one
 * after the other.  The program computes C = alpha*A*B + beta*C three times
 * on the current device -- through sgemm() on the default stream, through
 * sgemm_strided_batched_ws() with a zero-filled workspace of the size
 * sgemm_workspace_size() reports, and through
 * sgemm_strided_batched_noalloc() -- and writes the three results, each
 * M x N float32, one after the other to out.bin.  It also checks that a
 * negative dimension is refused with SGEMM_ERR_DIM before any HIP call.
 * Exit status 0 on success; any failed status or HIP error is printed and
 * exits with 1.
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>

#include "sgemm.h"

static int hip_ok(hipError_t e, const char *what) {
  if (e != hipSuccess) {
    fprintf(stderr, "%s: HIP error %d (%s)\n", what, (int)e, hipGetErrorString(e));
    return 0;
  }
  return 1;
}

static int st_ok(int st, const char *what) {
  if (st != SGEMM_OK) {
    fprintf(stderr, "%s: status %d (%s)\n", what, st, sgemm_status_string(st));
    return 0;
  }
  return 1;
}

int main(int argc, char **argv) {
  if (argc != 8) {
    fprintf(stderr, "usage: %s M N K alpha beta in.bin out.bin\n", argv[0]);
    return 2;
  }
  const int M = atoi(argv[1]), N = atoi(argv[2]), K = atoi(argv[3]);
  const float alpha = (float)atof(argv[4]), beta = (float)atof(argv[5]);
  const size_t na = (size_t)M * K, nb = (size_t)K * N, nc = (size_t)M * N;

  /* refused on the host, before any device work */
  if (sgemm(-1, N, K, alpha, NULL, K, NULL, N, beta, NULL, N, NULL) != SGEMM_ERR_DIM) {
    fprintf(stderr, "negative M was not refused with SGEMM_ERR_DIM\n");
    return 1;
  }

  float *host = (float *)malloc((na + nb + nc) * sizeof(float));
  float *out = (float *)malloc(3 * nc * sizeof(float));
  if (host == NULL || out == NULL) return 1;
  FILE *f = fopen(argv[6], "rb");
  if (f == NULL || fread(host, sizeof(float), na + nb + nc, f) != na + nb + nc) {
    fprintf(stderr, "cannot read %s\n", argv[6]);
    return 1;
  }
  fclose(f);

  float *dA = NULL, *dB = NULL, *dC = NULL;
  void *ws = NULL;
  const long long ws_bytes = sgemm_workspace_size(SGEMM_OP_N, SGEMM_OP_N, M, N, K, 1);
  if (ws_bytes < 0) return st_ok((int)ws_bytes, "sgemm_workspace_size") ? 0 : 1;
  int ok = hip_ok(hipMalloc((void **)&dA, na * sizeof(float) + 16), "hipMalloc A") &&
           hip_ok(hipMalloc((void **)&dB, nb * sizeof(float) + 16), "hipMalloc B") &&
           hip_ok(hipMalloc((void **)&dC, nc * sizeof(float) + 16), "hipMalloc C") &&
           hip_ok(hipMalloc(&ws, ws_bytes > 0 ? (size_t)ws_bytes : 16), "hipMalloc workspace") &&
           hip_ok(hipMemset(ws, 0, ws_bytes > 0 ? (size_t)ws_bytes : 16), "hipMemset workspace") &&
           hip_ok(hipMemcpy(dA, host, na * sizeof(float), hipMemcpyHostToDevice), "copy A") &&
           hip_ok(hipMemcpy(dB, host + na, nb * sizeof(float), hipMemcpyHostToDevice), "copy B");

  for (int form = 0; ok && form < 3; ++form) {
    ok = hip_ok(hipMemcpy(dC, host + na + nb, nc * sizeof(float), hipMemcpyHostToDevice), "copy C");
    if (!ok) break;
    int st;
    if (form == 0) {
      st = sgemm(M, N, K, alpha, dA, K, dB, N, beta, dC, N, NULL);
    } else if (form == 1) {
      st = sgemm_strided_batched_ws(SGEMM_OP_N, SGEMM_OP_N, M, N, K, alpha, dA, K, 0, dB, N, 0, beta, dC, N,
                                    0, 1, ws, (unsigned long long)(ws_bytes > 0 ? ws_bytes : 0), NULL);
    } else {
      st = sgemm_strided_batched_noalloc(SGEMM_OP_N, SGEMM_OP_N, M, N, K, alpha, dA, K, 0, dB, N, 0, beta, dC,
                                         N, 0, 1, NULL);
    }
    ok = st_ok(st, form == 0 ? "sgemm" : (form == 1 ? "sgemm_strided_batched_ws" : "sgemm_strided_batched_noalloc")) &&
         hip_ok(hipDeviceSynchronize(), "synchronize") &&
         hip_ok(hipMemcpy(out + form * nc, dC, nc * sizeof(float), hipMemcpyDeviceToHost), "copy back");
  }
  hipFree(dA);
  hipFree(dB);
  hipFree(dC);
  hipFree(ws);
  if (!ok) return 1;

  f = fopen(argv[7], "wb");
  if (f == NULL || fwrite(out, sizeof(float), 3 * nc, f) != 3 * nc) {
    fprintf(stderr, "cannot write %s\n", argv[7]);
    return 1;
  }
  fclose(f);
  printf("c_client: %dx%dx%d, workspace %lld bytes, three forms ok\n", M, N, K, ws_bytes);
  free(host);
  free(out);
  return 0;
}
