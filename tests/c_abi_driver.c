/*
 * c_abi_driver.c -- exercises liblrs.so from plain C, the way a caller with no
 * Python or PyTorch would: device buffers from hipMalloc, a stream of its own,
 * the workspace sized by the query, error returns checked before the real
 * calls, then lrs_scan_fwd and lrs_scan_bwd on [B,D,T] fp32 arrays.
 *
 * usage: c_abi_driver B D T in.bin out.bin
 *   in.bin : a, b, grad_h (B*D*T floats each, [B,D,T]) then h0 (B*D floats)
 *   out.bin: h, grad_a, grad_b (B*D*T floats each) then grad_h0 (B*D floats)
 * Exit status 0 on success; 2 for a HIP error, 3 for an unexpected return
 * code of the library, 1 for bad usage or I/O.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "lrs.h"

#define CK(x)                                                                  \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                  \
      return 2;                                                                \
    }                                                                          \
  } while (0)

#define LK(x, want)                                                            \
  do {                                                                         \
    int r_ = (x);                                                              \
    if (r_ != (want)) {                                                        \
      fprintf(stderr, "%s returned %d (%s), expected %d\n", #x, r_,            \
              lrs_status_string(r_), (want));                                  \
      return 3;                                                                \
    }                                                                          \
  } while (0)

int main(int argc, char **argv) {
  if (argc != 6) {
    fprintf(stderr, "usage: %s B D T in.bin out.bin\n", argv[0]);
    return 1;
  }
  const int64_t B = atoll(argv[1]), D = atoll(argv[2]), T = atoll(argv[3]);
  if (B < 1 || D < 1 || T < 1) return 1;
  const int64_t C = B * D, N = C * T;
  const size_t nb = (size_t)N * sizeof(float), cb = (size_t)C * sizeof(float);

  float *host = (float *)malloc(6 * nb + 2 * cb);
  if (!host) return 1;
  float *a = host, *b = a + N, *g = b + N, *h0 = g + N;
  FILE *f = fopen(argv[4], "rb");
  if (!f || fread(host, 1, 3 * nb + cb, f) != 3 * nb + cb) return 1;
  fclose(f);

  hipStream_t st;
  CK(hipStreamCreate(&st));
  float *da, *db, *dg, *dh0, *dh, *dga, *dgb, *dgh0;
  CK(hipMalloc((void **)&da, nb));
  CK(hipMalloc((void **)&db, nb));
  CK(hipMalloc((void **)&dg, nb));
  CK(hipMalloc((void **)&dh, nb));
  CK(hipMalloc((void **)&dga, nb));
  CK(hipMalloc((void **)&dgb, nb));
  CK(hipMalloc((void **)&dh0, cb));
  CK(hipMalloc((void **)&dgh0, cb));
  CK(hipMemcpy(da, a, nb, hipMemcpyHostToDevice));
  CK(hipMemcpy(db, b, nb, hipMemcpyHostToDevice));
  CK(hipMemcpy(dg, g, nb, hipMemcpyHostToDevice));
  CK(hipMemcpy(dh0, h0, cb, hipMemcpyHostToDevice));

  const size_t ws = lrs_scan_workspace_bytes(B, D, T, LRS_LAYOUT_BDT, LRS_F32);
  void *dws = NULL;
  if (ws) CK(hipMalloc(&dws, ws));

  /* rejected before any launch */
  LK(lrs_scan_fwd(NULL, db, dh0, dh, B, D, T, LRS_LAYOUT_BDT, LRS_F32, dws, ws, st),
     LRS_ERR_INVALID_ARG);
  LK(lrs_scan_fwd(da, db, dh0, da, B, D, T, LRS_LAYOUT_BDT, LRS_F32, dws, ws, st),
     LRS_ERR_INVALID_ARG);  /* h aliases a */
  LK(lrs_scan_fwd(da, db, dh0, dh, B, D, -T, LRS_LAYOUT_BDT, LRS_F32, dws, ws, st),
     LRS_ERR_INVALID_ARG);
  if (ws)
    LK(lrs_scan_fwd(da, db, dh0, dh, B, D, T, LRS_LAYOUT_BDT, LRS_F32, NULL, 0, st),
       LRS_ERR_WORKSPACE);

  LK(lrs_scan_fwd(da, db, dh0, dh, B, D, T, LRS_LAYOUT_BDT, LRS_F32, dws, ws, st), LRS_OK);
  LK(lrs_scan_bwd(da, dh, dh0, dg, dga, dgb, dgh0, B, D, T, LRS_LAYOUT_BDT, LRS_F32, dws, ws, st),
     LRS_OK);
  CK(hipStreamSynchronize(st));

  float *h = h0 + C, *ga = h + N, *gb = ga + N, *gh0 = gb + N;
  CK(hipMemcpy(h, dh, nb, hipMemcpyDeviceToHost));
  CK(hipMemcpy(ga, dga, nb, hipMemcpyDeviceToHost));
  CK(hipMemcpy(gb, dgb, nb, hipMemcpyDeviceToHost));
  CK(hipMemcpy(gh0, dgh0, cb, hipMemcpyDeviceToHost));
  f = fopen(argv[5], "wb");
  if (!f || fwrite(h, 1, 3 * nb + cb, f) != 3 * nb + cb) return 1;
  fclose(f);

  if (dws) CK(hipFree(dws));
  CK(hipFree(da));
  CK(hipFree(db));
  CK(hipFree(dg));
  CK(hipFree(dh));
  CK(hipFree(dga));
  CK(hipFree(dgb));
  CK(hipFree(dh0));
  CK(hipFree(dgh0));
  CK(hipStreamDestroy(st));
  free(host);
  return 0;
}
