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

}  // namespace lrs
