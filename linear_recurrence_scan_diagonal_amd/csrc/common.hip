// common.hip -- small helper kernels shared by the entry points.
#include "lrs_device.hpp"
#include "lrs_internal.hpp"

namespace lrs {

__global__ __launch_bounds__(256) void k_reset(uint64_t* __restrict__ status, int64_t nstatus,
                                               unsigned* __restrict__ tickets, int64_t ntickets,
                                               uint32_t* __restrict__ zero, int64_t nzero) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nstatus; i += stride)
    status[i] = kStatusEmpty;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < ntickets; i += stride)
    tickets[i] = 0u;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nzero; i += stride)
    zero[i] = 0u;
}

hipError_t launch_reset(uint64_t* status, int64_t nstatus, unsigned* tickets, int64_t ntickets,
                        uint32_t* zero, int64_t nzero, hipStream_t stream) {
  int64_t n = nstatus;
  if (ntickets > n) n = ntickets;
  if (nzero > n) n = nzero;
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(k_reset, dim3((unsigned)blocks), dim3(256), 0, stream, status, nstatus,
                     tickets, ntickets, zero, nzero);
  return hipGetLastError();
}

}  // namespace lrs
