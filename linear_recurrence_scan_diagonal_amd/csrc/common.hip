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
// B*T terms).  Stage 1: block (x, y, z) takes rows [z*rpb, (z+1)*rpb) of
// matrix y for 256 columns, four per lane (one 1 KiB row piece per wave and
// load); its four waves take every fourth row and their sums are added in wave
// order.  With one row block the result is final and goes straight to out0 /
// out1; otherwise it is written to acc[(y * D + d) * nrb + z], so that the nrb
// partials of a column are contiguous.  Stage 2: one wave per column; lane l
// adds partials l, l + 64, ... in order and a fixed butterfly adds the lanes.
// Results do not depend on scheduling.
template <bool VEC>
__global__ __launch_bounds__(256) void k_col_sum_part(const float* __restrict__ part,
                                                      double* __restrict__ acc,
                                                      float* __restrict__ out0,
                                                      float* __restrict__ out1, int64_t R,
                                                      int64_t D, int64_t rpb, int nrb) {
  constexpr int kCols = 4 * kWave;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const int64_t d0 = (int64_t)blockIdx.x * kCols + lane * 4;
  const float* m = part + (int64_t)blockIdx.y * R * D;
  const int64_t r0 = (int64_t)blockIdx.z * rpb;
  const int64_t r1 = r0 + rpb < R ? r0 + rpb : R;
  double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
  if (VEC) {
    if (d0 < D) {
#pragma unroll 8
      for (int64_t r = r0 + wid; r < r1; r += 4) {
        const float4 v = *reinterpret_cast<const float4*>(m + r * D + d0);
        s0 += (double)v.x;
        s1 += (double)v.y;
        s2 += (double)v.z;
        s3 += (double)v.w;
      }
    }
  } else {
#pragma unroll 4
    for (int64_t r = r0 + wid; r < r1; r += 4) {
      const float* row = m + r * D;
      if (d0 < D) s0 += (double)row[d0];
      if (d0 + 1 < D) s1 += (double)row[d0 + 1];
      if (d0 + 2 < D) s2 += (double)row[d0 + 2];
      if (d0 + 3 < D) s3 += (double)row[d0 + 3];
    }
  }
  __shared__ double red[4][kCols];
  red[wid][lane * 4 + 0] = s0;
  red[wid][lane * 4 + 1] = s1;
  red[wid][lane * 4 + 2] = s2;
  red[wid][lane * 4 + 3] = s3;
  __syncthreads();
  const int t = threadIdx.x;
  const int64_t d = (int64_t)blockIdx.x * kCols + t;
  if (d < D) {
    const double v = ((red[0][t] + red[1][t]) + red[2][t]) + red[3][t];
    if (nrb == 1)
      (blockIdx.y == 0 ? out0 : out1)[d] = (float)v;
    else
      acc[((int64_t)blockIdx.y * D + d) * nrb + blockIdx.z] = v;
  }
}

__global__ __launch_bounds__(256) void k_col_sum_final(const double* __restrict__ acc,
                                                       float* __restrict__ out0,
                                                       float* __restrict__ out1, int nrb,
                                                       int64_t D, int nmat) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t w = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (w >= nmat * D) return;  // whole waves
  const double* p = acc + w * nrb;
  double t = 0.0;
  for (int z = lane; z < nrb; z += kWave) t += p[z];
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) t += __shfl_xor(t, o);
  if (lane == 0) {
    const int64_t y = w / D, d = w - y * D;
    (y == 0 ? out0 : out1)[d] = (float)t;
  }
}

// Rows per stage-1 block: 32 (eight per wave), so that a few thousand rows
// give hundreds of blocks; at most 4096 blocks per column.
int64_t col_sum_blocks(int64_t R) {
  int64_t nrb = (R + 31) / 32;
  if (nrb > 4096) nrb = 4096;
  return nrb < 1 ? 1 : nrb;
}

hipError_t launch_col_sums(const float* part, int nmat, int64_t R, int64_t D, double* acc,
                           float* out0, float* out1, hipStream_t stream) {
  if (R <= 0 || D <= 0) return hipSuccess;
  const int64_t nrb = col_sum_blocks(R), rpb = (R + nrb - 1) / nrb;
  const dim3 grid((unsigned)((D + 4 * kWave - 1) / (4 * kWave)), (unsigned)nmat, (unsigned)nrb);
  if (D % 4 == 0)
    hipLaunchKernelGGL(k_col_sum_part<true>, grid, dim3(256), 0, stream, part, acc, out0, out1, R,
                       D, rpb, (int)nrb);
  else
    hipLaunchKernelGGL(k_col_sum_part<false>, grid, dim3(256), 0, stream, part, acc, out0, out1,
                       R, D, rpb, (int)nrb);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || nrb == 1) return e;
  hipLaunchKernelGGL(k_col_sum_final, dim3((unsigned)((nmat * D + 3) / 4)), dim3(256), 0, stream,
                     acc, out0, out1, (int)nrb, D, nmat);
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
