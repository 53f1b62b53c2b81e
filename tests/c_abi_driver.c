/*
 * c_abi_driver.c -- exercises liblrs.so from plain C, the way a caller with no
 * Python or PyTorch would: device buffers from hipMalloc, a stream of its own,
 * workspaces sized by the queries, error returns checked before the real
 * calls.  Four modes:
 *
 *   c_abi_driver scan B D T in.bin out.bin
 *     lrs_scan_fwd + lrs_scan_bwd on [B,D,T] fp32 arrays, and lrs_scan_fwd_ex
 *     with default options, which must give the same bits as lrs_scan_fwd.
 *     in.bin : a, b, grad_h (B*D*T floats each) then h0 (B*D floats)
 *     out.bin: h, grad_a, grad_b (B*D*T floats each) then grad_h0 (B*D floats)
 *
 *   c_abi_driver scan16 B D T in.bin out.bin
 *     the same with bf16 arrays: a, b, grad_h, h, grad_a, grad_b as bf16 bit
 *     patterns (2 bytes per element), h0 and grad_h0 fp32.
 *
 *   c_abi_driver sru T B D in.bin out.bin
 *     lrs_sru_fwd with bf16 I/O on [T,B,D] arrays, c_T requested.
 *     in.bin : z_f, z_r, z_x (T*B*D bf16 bit patterns each) then bias_f,
 *              bias_r (D floats each)
 *     out.bin: h (T*B*D bf16) then c_last (B*D floats)
 *
 *   c_abi_driver deer B D T in.bin out.bin
 *     lrs_deer_solve (eps 1e-5, k_max 5, host record) on [B,D,T] fp32.
 *     in.bin : w (D floats), u (B*D*T floats), h0 (B*D floats)
 *     out.bin: h (B*D*T floats), iterations (int32), converged (int32),
 *              deltas (5 floats), then lrs_deer_eps_schedule(0..4 of 5,
 *              1e-4, 1e-6) (5 floats), then the sequential loop's h
 *              (lrs_rnn_seq, B*D*T floats)
 *
 * Exit status 0 on success; 2 for a HIP error, 3 for an unexpected return
 * code of the library, 4 for a mismatch between lrs_scan_fwd and
 * lrs_scan_fwd_ex, 1 for bad usage or I/O.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

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

static int read_file(const char *path, void *buf, size_t n) {
  FILE *f = fopen(path, "rb");
  if (!f) return 1;
  const size_t got = fread(buf, 1, n, f);
  fclose(f);
  return got == n ? 0 : 1;
}

static int write_file(const char *path, const void *buf, size_t n) {
  FILE *f = fopen(path, "wb");
  if (!f) return 1;
  const size_t put = fwrite(buf, 1, n, f);
  fclose(f);
  return put == n ? 0 : 1;
}

static int run_scan(int64_t B, int64_t D, int64_t T, int dtype, const char *in,
                    const char *out) {
  const int64_t C = B * D, N = C * T;
  const size_t es = dtype == LRS_BF16 ? 2 : 4;
  const size_t nb = (size_t)N * es, cb = (size_t)C * sizeof(float);
  char *host = (char *)malloc(7 * nb + 2 * cb);
  if (!host) return 1;
  char *a = host, *b = a + nb, *g = b + nb;
  float *h0 = (float *)(g + nb);
  if (read_file(in, host, 3 * nb + cb)) return 1;

  hipStream_t st;
  CK(hipStreamCreate(&st));
  void *da, *db, *dg, *dh, *dh2, *dga, *dgb;
  float *dh0, *dgh0;
  CK(hipMalloc(&da, nb));
  CK(hipMalloc(&db, nb));
  CK(hipMalloc(&dg, nb));
  CK(hipMalloc(&dh, nb));
  CK(hipMalloc(&dh2, nb));
  CK(hipMalloc(&dga, nb));
  CK(hipMalloc(&dgb, nb));
  CK(hipMalloc((void **)&dh0, cb));
  CK(hipMalloc((void **)&dgh0, cb));
  CK(hipMemcpy(da, a, nb, hipMemcpyHostToDevice));
  CK(hipMemcpy(db, b, nb, hipMemcpyHostToDevice));
  CK(hipMemcpy(dg, g, nb, hipMemcpyHostToDevice));
  CK(hipMemcpy(dh0, h0, cb, hipMemcpyHostToDevice));

  const size_t ws = lrs_scan_workspace_bytes(B, D, T, LRS_LAYOUT_BDT, dtype);
  void *dws = NULL;
  if (ws) CK(hipMalloc(&dws, ws));

  /* rejected before any launch */
  LK(lrs_scan_fwd(NULL, db, dh0, dh, B, D, T, LRS_LAYOUT_BDT, dtype, dws, ws, st),
     LRS_ERR_INVALID_ARG);
  LK(lrs_scan_fwd(da, db, dh0, da, B, D, T, LRS_LAYOUT_BDT, dtype, dws, ws, st),
     LRS_ERR_INVALID_ARG);  /* h aliases a */
  LK(lrs_scan_fwd(da, db, dh0, dh, B, D, -T, LRS_LAYOUT_BDT, dtype, dws, ws, st),
     LRS_ERR_INVALID_ARG);
  LK(lrs_scan_fwd(da, db, dh0, dh, B, D, T, LRS_LAYOUT_BDT, 7, dws, ws, st),
     LRS_ERR_INVALID_ARG);  /* unknown element type */
  if (ws)
    LK(lrs_scan_fwd(da, db, dh0, dh, B, D, T, LRS_LAYOUT_BDT, dtype, NULL, 0, st),
       LRS_ERR_WORKSPACE);

  LK(lrs_scan_fwd(da, db, dh0, dh, B, D, T, LRS_LAYOUT_BDT, dtype, dws, ws, st), LRS_OK);
  LK(lrs_scan_bwd(da, dh, dh0, dg, dga, dgb, dgh0, B, D, T, LRS_LAYOUT_BDT, dtype, dws, ws, st),
     LRS_OK);
  /* the same forward through the options entry point, default options */
  lrs_options opt;
  lrs_options_default(&opt);
  LK(lrs_scan_fwd_ex(da, db, dh0, dh2, B, D, T, LRS_LAYOUT_BDT, dtype, dws, ws, st, &opt),
     LRS_OK);
  CK(hipStreamSynchronize(st));

  char *h = (char *)(h0 + C), *ga = h + nb, *gb = ga + nb;
  float *gh0 = (float *)(gb + nb);
  char *h2 = (char *)(gh0 + C);
  CK(hipMemcpy(h, dh, nb, hipMemcpyDeviceToHost));
  CK(hipMemcpy(ga, dga, nb, hipMemcpyDeviceToHost));
  CK(hipMemcpy(gb, dgb, nb, hipMemcpyDeviceToHost));
  CK(hipMemcpy(gh0, dgh0, cb, hipMemcpyDeviceToHost));
  CK(hipMemcpy(h2, dh2, nb, hipMemcpyDeviceToHost));
  if (memcmp(h, h2, nb) != 0) {
    fprintf(stderr, "lrs_scan_fwd_ex with default options differs from lrs_scan_fwd\n");
    return 4;
  }
  if (write_file(out, h, 3 * nb + cb)) return 1;

  if (dws) CK(hipFree(dws));
  CK(hipFree(da));
  CK(hipFree(db));
  CK(hipFree(dg));
  CK(hipFree(dh));
  CK(hipFree(dh2));
  CK(hipFree(dga));
  CK(hipFree(dgb));
  CK(hipFree(dh0));
  CK(hipFree(dgh0));
  CK(hipStreamDestroy(st));
  free(host);
  return 0;
}

static int run_sru(int64_t T, int64_t B, int64_t D, const char *in, const char *out) {
  const int64_t C = B * D, N = T * C;
  const size_t zb = (size_t)N * 2, db_ = (size_t)D * sizeof(float), cb = (size_t)C * sizeof(float);
  char *host = (char *)malloc(4 * zb + 2 * db_ + cb);
  if (!host) return 1;
  if (read_file(in, host, 3 * zb + 2 * db_)) return 1;

  hipStream_t st;
  CK(hipStreamCreate(&st));
  void *dz, *dh;
  float *dbias, *dcl;
  CK(hipMalloc(&dz, 3 * zb));
  CK(hipMalloc(&dh, zb));
  CK(hipMalloc((void **)&dbias, 2 * db_));
  CK(hipMalloc((void **)&dcl, cb));
  CK(hipMemcpy(dz, host, 3 * zb, hipMemcpyHostToDevice));
  CK(hipMemcpy(dbias, host + 3 * zb, 2 * db_, hipMemcpyHostToDevice));
  const char *zf = (const char *)dz, *zr = zf + zb, *zx = zr + zb;

  const size_t ws = lrs_sru_workspace_bytes(T, B, D);
  void *dws = NULL;
  if (ws) CK(hipMalloc(&dws, ws));
  /* rejected before any launch: a missing input, an unknown I/O type */
  LK(lrs_sru_fwd(zf, NULL, zx, dbias, dbias + D, NULL, dh, dcl, NULL, T, B, D, LRS_BF16, dws, ws,
                 st),
     LRS_ERR_INVALID_ARG);
  LK(lrs_sru_fwd(zf, zr, zx, dbias, dbias + D, NULL, dh, dcl, NULL, T, B, D, 7, dws, ws, st),
     LRS_ERR_INVALID_ARG);
  LK(lrs_sru_fwd(zf, zr, zx, dbias, dbias + D, NULL, dh, dcl, NULL, T, B, D, LRS_BF16, dws, ws, st),
     LRS_OK);
  CK(hipStreamSynchronize(st));
  char *h = host + 3 * zb + 2 * db_;
  CK(hipMemcpy(h, dh, zb, hipMemcpyDeviceToHost));
  CK(hipMemcpy(h + zb, dcl, cb, hipMemcpyDeviceToHost));
  if (write_file(out, h, zb + cb)) return 1;

  if (dws) CK(hipFree(dws));
  CK(hipFree(dz));
  CK(hipFree(dh));
  CK(hipFree(dbias));
  CK(hipFree(dcl));
  CK(hipStreamDestroy(st));
  free(host);
  return 0;
}

static int run_deer(int64_t B, int64_t D, int64_t T, const char *in, const char *out) {
  enum { KMAX = 5 };
  const int64_t C = B * D, N = C * T;
  const size_t nb = (size_t)N * sizeof(float), cb = (size_t)C * sizeof(float);
  const size_t wb = (size_t)D * sizeof(float);
  const size_t ob = 2 * nb + 2 * sizeof(int32_t) + 2 * KMAX * sizeof(float);
  char *host = (char *)malloc(wb + nb + cb + ob);
  if (!host) return 1;
  if (read_file(in, host, wb + nb + cb)) return 1;

  hipStream_t st;
  CK(hipStreamCreate(&st));
  float *dw, *du, *dh0, *dh;
  CK(hipMalloc((void **)&dw, wb));
  CK(hipMalloc((void **)&du, nb));
  CK(hipMalloc((void **)&dh0, cb));
  CK(hipMalloc((void **)&dh, nb));
  CK(hipMemcpy(dw, host, wb, hipMemcpyHostToDevice));
  CK(hipMemcpy(du, host + wb, nb, hipMemcpyHostToDevice));
  CK(hipMemcpy(dh0, host + wb + nb, cb, hipMemcpyHostToDevice));

  const size_t ws = lrs_deer_workspace_bytes(B, D, T, KMAX);
  void *dws = NULL;
  CK(hipMalloc(&dws, ws));
  int iters = 0, conv = 0;
  float deltas[KMAX];
  /* rejected before any launch: k_max < 1, a workspace that is too small */
  LK(lrs_deer_solve(dw, du, dh0, NULL, dh, B, D, T, 1e-5f, 0, &iters, deltas, &conv, dws, ws, st),
     LRS_ERR_INVALID_ARG);
  LK(lrs_deer_solve(dw, du, dh0, NULL, dh, B, D, T, 1e-5f, KMAX, &iters, deltas, &conv, dws,
                    ws / 2, st),
     LRS_ERR_WORKSPACE);
  LK(lrs_deer_solve(dw, du, dh0, NULL, dh, B, D, T, 1e-5f, KMAX, &iters, deltas, &conv, dws, ws,
                    st),
     LRS_OK);
  char *o = host + wb + nb + cb;
  CK(hipMemcpy(o, dh, nb, hipMemcpyDeviceToHost));
  int32_t rec[2] = {iters, conv};
  memcpy(o + nb, rec, sizeof(rec));
  memcpy(o + nb + sizeof(rec), deltas, sizeof(deltas));
  float sched[KMAX];
  for (int i = 0; i < KMAX; ++i) sched[i] = lrs_deer_eps_schedule(i, KMAX, 1e-4f, 1e-6f);
  memcpy(o + nb + sizeof(rec) + sizeof(deltas), sched, sizeof(sched));
  /* the sequential loop: a null input and an output on top of u are rejected */
  LK(lrs_rnn_seq(dw, NULL, dh0, dh, B, D, T, st), LRS_ERR_INVALID_ARG);
  LK(lrs_rnn_seq(dw, du, dh0, du, B, D, T, st), LRS_ERR_INVALID_ARG);
  LK(lrs_rnn_seq(dw, du, dh0, dh, B, D, T, st), LRS_OK);
  CK(hipStreamSynchronize(st));
  CK(hipMemcpy(o + nb + sizeof(rec) + sizeof(deltas) + sizeof(sched), dh, nb,
               hipMemcpyDeviceToHost));
  if (write_file(out, o, ob)) return 1;

  CK(hipFree(dws));
  CK(hipFree(dw));
  CK(hipFree(du));
  CK(hipFree(dh0));
  CK(hipFree(dh));
  CK(hipStreamDestroy(st));
  free(host);
  return 0;
}

int main(int argc, char **argv) {
  if (argc != 7) {
    fprintf(stderr, "usage: %s scan|scan16|sru|deer N1 N2 N3 in.bin out.bin\n", argv[0]);
    return 1;
  }
  const int64_t n1 = atoll(argv[2]), n2 = atoll(argv[3]), n3 = atoll(argv[4]);
  if (n1 < 1 || n2 < 1 || n3 < 1) return 1;
  if (strcmp(argv[1], "scan") == 0) return run_scan(n1, n2, n3, LRS_F32, argv[5], argv[6]);
  if (strcmp(argv[1], "scan16") == 0) return run_scan(n1, n2, n3, LRS_BF16, argv[5], argv[6]);
  if (strcmp(argv[1], "sru") == 0) return run_sru(n1, n2, n3, argv[5], argv[6]);
  if (strcmp(argv[1], "deer") == 0) return run_deer(n1, n2, n3, argv[5], argv[6]);
  fprintf(stderr, "unknown mode %s\n", argv[1]);
  return 1;
}
