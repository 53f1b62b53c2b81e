// common.hip -- small helper kernels shared by the entry points.
#include "lrs_device.hpp"
#include "lrs_internal.hpp"

namespace lrs {

// Status words are written in pairs with 16-byte stores when the array is
// 16-byte aligned (workspace carving aligns every array to 256 bytes).
__global__ __launch_bounds__(256) void k_reset(uint64_t* __restrict__ status, int64_t nstatus,
                                               unsigned* __restrict__ tickets, int64_t ntickets,
                                               uint32_t* __restrict__ zero, int64_t nzero) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (((uintptr_t)status & 15) == 0) {
    uint4* s2 = reinterpret_cast<uint4*>(status);
    const uint4 empty = make_uint4(~0u, ~0u, ~0u, ~0u);
    for (int64_t i = tid; i < nstatus / 2; i += stride) s2[i] = empty;
    if ((nstatus & 1) && tid == 0) status[nstatus - 1] = kStatusEmpty;
  } else {
    for (int64_t i = tid; i < nstatus; i += stride) status[i] = kStatusEmpty;
  }
  for (int64_t i = tid; i < ntickets; i += stride) tickets[i] = 0u;
  for (int64_t i = tid; i < nzero; i += stride) zero[i] = 0u;
}

hipError_t launch_reset(uint64_t* status, int64_t nstatus, unsigned* tickets, int64_t ntickets,
                        uint32_t* zero, int64_t nzero, hipStream_t stream) {
  int64_t n = (nstatus + 1) / 2;
  if (ntickets > n) n = ntickets;
  if (nzero > n) n = nzero;
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(k_reset, dim3((unsigned)blocks), dim3(256), 0, stream, status, nstatus,
                     tickets, ntickets, zero, nzero);
  return hipGetLastError();
}

// Column sums of nmat consecutive [R, D] fp32 matrices (gridDim.y = nmat), in
// two fixed-order stages accumulated in fp64 (a parameter gradient adds up
// B*T terms).  Stage 1: block (x, y, z) adds rows [z*rpb, (z+1)*rpb) of matrix
// y for 64 columns (sixteen waves take every sixteenth row, then their sums are
// added in wave order) and writes one double per column to
// acc[(y * nrb + z) * D + d].  Stage 2 adds the nrb doubles of each column in
// order.  Results do not depend on scheduling.
__global__ __launch_bounds__(1024) void k_col_sum_part(const float* __restrict__ part,
                                                       double* __restrict__ acc, int64_t R,
                                                       int64_t D, int64_t rpb) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const int64_t d = (int64_t)blockIdx.x * kWave + lane;
  const float* m = part + (int64_t)blockIdx.y * R * D;
  const int64_t r0 = (int64_t)blockIdx.z * rpb;
  const int64_t r1 = r0 + rpb < R ? r0 + rpb : R;
  __shared__ double red[16][kWave];
  double a = 0.0;
  if (d < D)
    for (int64_t r = r0 + wid; r < r1; r += 16) a += (double)m[r * D + d];
  red[wid][lane] = a;
  __syncthreads();
  if (wid == 0 && d < D) {
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < 16; ++w) t += red[w][lane];
    acc[((int64_t)blockIdx.y * gridDim.z + blockIdx.z) * D + d] = t;
  }
}

__global__ __launch_bounds__(256) void k_col_sum_final(const double* __restrict__ acc,
                                                       float* __restrict__ out0,
                                                       float* __restrict__ out1, int nrb,
                                                       int64_t D, int nmat) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // 0 .. nmat*D-1
  if (i >= nmat * D) return;
  const int64_t y = i / D, d = i - y * D;
  double t = 0.0;
  for (int z = 0; z < nrb; ++z) t += acc[(y * nrb + z) * D + d];
  (y == 0 ? out0 : out1)[d] = (float)t;
}

int64_t col_sum_blocks(int64_t R) {
  int64_t nrb = (R + 63) / 64;
  if (nrb > 4096) nrb = 4096;
  return nrb < 1 ? 1 : nrb;
}

hipError_t launch_col_sums(const float* part, int nmat, int64_t R, int64_t D, double* acc,
                           float* out0, float* out1, hipStream_t stream) {
  if (R <= 0 || D <= 0) return hipSuccess;
  const int64_t nrb = col_sum_blocks(R), rpb = (R + nrb - 1) / nrb;
  hipLaunchKernelGGL(k_col_sum_part,
                     dim3((unsigned)((D + kWave - 1) / kWave), (unsigned)nmat, (unsigned)nrb),
                     dim3(1024), 0, stream, part, acc, R, D, rpb);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_col_sum_final, dim3((unsigned)((nmat * D + 255) / 256)), dim3(256), 0,
                     stream, acc, out0, out1, (int)nrb, D, nmat);
  return hipGetLastError();
}

int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && cache[dev] > 0) return cache[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < 64) cache[dev] = n;
  return n;
}

}  // namespace lrs
