// scan_serial.hip -- sequential per-channel scans for short channels
// ([B, D, T] layout): one lane walks one channel from its first step to its
// last (the backward from its last to its first), with no cross-lane work.
//
// Page "CUDA并行化RNN训练：从O(T)到O(log T)的工程实践与参数调优", checklist item 3
// and the pages' applicability notes: below some sequence length the plain
// sequential recurrence beats the parallel scan, whose per-chunk combine and
// per-workgroup overhead do not pay off.  The parallel kernels give a short
// channel a whole workgroup of 64 or more lanes, most of them idle; here 256
// channels share a workgroup.  Where the two cross over is measured, not
// assumed (plan_scan_*_rows).
//
// A lane reads its channel in groups of 4 elements (16 bytes of fp32, 8 of
// bf16) when the rows allow it (T a multiple of 4 and aligned arrays), else
// element by element; the
// lanes of a wave read 64 consecutive rows, so a wave's accesses cover one
// contiguous stretch of 64*T elements per array.
#include "lrs_device.hpp"
#include "lrs_internal.hpp"

namespace lrs {

constexpr int kSerialThreads = 256;

template <typename IO, bool VEC>
__global__ __launch_bounds__(kSerialThreads) void k_scan_fwd_serial(
    const IO* __restrict__ a, const IO* __restrict__ b, const float* __restrict__ h0,
    IO* __restrict__ h, int64_t T, int64_t C) {
  const int64_t ch = (int64_t)blockIdx.x * kSerialThreads + threadIdx.x;
  if (ch >= C) return;
  const int64_t row = ch * T;
  float x = h0 ? h0[ch] : 0.0f;
  if (VEC) {
    const IO* ar = a + row;
    const IO* br = b + row;
    IO* hr = h + row;
    const int64_t ng = T / 4;
#pragma unroll 4
    for (int64_t i = 0; i < ng; ++i) {
      const float4 av = load_group_full(ar, 4 * i), bv = load_group_full(br, 4 * i);
      float4 o;
      x = __builtin_fmaf(av.x, x, bv.x); o.x = x;
      x = __builtin_fmaf(av.y, x, bv.y); o.y = x;
      x = __builtin_fmaf(av.z, x, bv.z); o.z = x;
      x = __builtin_fmaf(av.w, x, bv.w); o.w = x;
      store_group_full(hr, 4 * i, o);
    }
  } else {
#pragma unroll 4
    for (int64_t t = 0; t < T; ++t) {
      x = __builtin_fmaf(io_ld(a, row + t), x, io_ld(b, row + t));
      io_st(h, row + t, x);
    }
  }
}

// lam_t = g_t + a_{t+1} lam_{t+1} (a_{T+1} = 0), grad_b = lam,
// grad_a_t = lam_t h_{t-1} (h0 at t = 1), grad_h0 = a_1 lam_1.  grad_b may
// alias g: each element of g is read before the same element of grad_b is
// written, by the same lane.
template <typename IO, bool VEC>
__global__ __launch_bounds__(kSerialThreads) void k_scan_bwd_serial(
    const IO* __restrict__ a, const IO* __restrict__ h, const float* __restrict__ h0,
    const IO* g, IO* __restrict__ da, IO* db, float* __restrict__ dh0, int64_t T,
    int64_t C) {
  const int64_t ch = (int64_t)blockIdx.x * kSerialThreads + threadIdx.x;
  if (ch >= C) return;
  const int64_t row = ch * T;
  const float x0 = h0 ? h0[ch] : 0.0f;
  float lam = 0.0f, a_next = 0.0f;  // lam_{t+1} and a_{t+1} past the group
  // Blocks of kU groups: every load of a block is issued before its first
  // store (grad_b may alias g, so the compiler may not move loads past stores).
  constexpr int kU = 4;
  if (VEC) {
    const IO* ar = a + row;
    const IO* hr = h + row;
    const IO* gr = g + row;
    IO* dar = da + row;
    IO* dbr = db + row;
    int64_t i = T / 4 - 1;  // group index, descending
    for (; i >= kU - 1; i -= kU) {
      float4 av[kU], hh[kU], gv[kU];
#pragma unroll
      for (int k = 0; k < kU; ++k) {
        av[k] = load_group_full(ar, 4 * (i - k));
        hh[k] = load_group_full(hr, 4 * (i - k));
        gv[k] = load_group_full(gr, 4 * (i - k));
      }
      const int64_t first = i - (kU - 1);
      const float hp_last = (first > 0) ? io_ld(hr, 4 * first - 1) : x0;
#pragma unroll
      for (int k = 0; k < kU; ++k) {
        const float hp = (k < kU - 1) ? hh[k + 1].w : hp_last;
        const float l3 = __builtin_fmaf(a_next, lam, gv[k].w);
        const float l2 = __builtin_fmaf(av[k].w, l3, gv[k].z);
        const float l1 = __builtin_fmaf(av[k].z, l2, gv[k].y);
        const float l0 = __builtin_fmaf(av[k].y, l1, gv[k].x);
        store_group_full(dar, 4 * (i - k), make_float4(l0 * hp, l1 * hh[k].x, l2 * hh[k].y, l3 * hh[k].z));
        store_group_full(dbr, 4 * (i - k), make_float4(l0, l1, l2, l3));
        lam = l0;
        a_next = av[k].x;
      }
    }
    for (; i >= 0; --i) {
      const float4 av = load_group_full(ar, 4 * i), hh = load_group_full(hr, 4 * i),
                   gv = load_group_full(gr, 4 * i);
      const float hp = (i > 0) ? io_ld(hr, 4 * i - 1) : x0;
      const float l3 = __builtin_fmaf(a_next, lam, gv.w);
      const float l2 = __builtin_fmaf(av.w, l3, gv.z);
      const float l1 = __builtin_fmaf(av.z, l2, gv.y);
      const float l0 = __builtin_fmaf(av.y, l1, gv.x);
      store_group_full(dar, 4 * i, make_float4(l0 * hp, l1 * hh.x, l2 * hh.y, l3 * hh.z));
      store_group_full(dbr, 4 * i, make_float4(l0, l1, l2, l3));
      lam = l0;
      a_next = av.x;
    }
  } else {
    int64_t t = T - 1;  // step index, descending
    for (; t >= kU - 1; t -= kU) {
      float av[kU], hp[kU], gv[kU];
#pragma unroll
      for (int k = 0; k < kU; ++k) {
        av[k] = io_ld(a, row + t - k);
        gv[k] = io_ld(g, row + t - k);
        hp[k] = (t - k > 0) ? io_ld(h, row + t - k - 1) : x0;
      }
#pragma unroll
      for (int k = 0; k < kU; ++k) {
        lam = __builtin_fmaf(a_next, lam, gv[k]);
        io_st(da, row + t - k, lam * hp[k]);
        io_st(db, row + t - k, lam);
        a_next = av[k];
      }
    }
    for (; t >= 0; --t) {
      const float at = io_ld(a, row + t), gt = io_ld(g, row + t);
      const float hp = (t > 0) ? io_ld(h, row + t - 1) : x0;
      lam = __builtin_fmaf(a_next, lam, gt);
      io_st(da, row + t, lam * hp);
      io_st(db, row + t, lam);
      a_next = at;
    }
  }
  if (dh0) dh0[ch] = a_next * lam;
}

template <typename IO>
static void scan_fwd_serial_io(const IO* a, const IO* b, const float* h0, IO* h, int64_t C,
                               int64_t T, int vec, hipStream_t stream) {
  const dim3 grid((unsigned)((C + kSerialThreads - 1) / kSerialThreads));
  if (vec)
    hipLaunchKernelGGL((k_scan_fwd_serial<IO, true>), grid, dim3(kSerialThreads), 0, stream, a, b,
                       h0, h, T, C);
  else
    hipLaunchKernelGGL((k_scan_fwd_serial<IO, false>), grid, dim3(kSerialThreads), 0, stream, a, b,
                       h0, h, T, C);
}

template <typename IO>
static void scan_bwd_serial_io(const IO* a, const IO* h, const float* h0, const IO* g, IO* da,
                               IO* db, float* dh0, int64_t C, int64_t T, int vec,
                               hipStream_t stream) {
  const dim3 grid((unsigned)((C + kSerialThreads - 1) / kSerialThreads));
  if (vec)
    hipLaunchKernelGGL((k_scan_bwd_serial<IO, true>), grid, dim3(kSerialThreads), 0, stream, a, h,
                       h0, g, da, db, dh0, T, C);
  else
    hipLaunchKernelGGL((k_scan_bwd_serial<IO, false>), grid, dim3(kSerialThreads), 0, stream, a, h,
                       h0, g, da, db, dh0, T, C);
}

hipError_t launch_scan_fwd_serial(const void* a, const void* b, const float* h0, void* h, int io,
                                  int64_t C, int64_t T, int vec, hipStream_t stream) {
  if (io == kIoBf16)
    scan_fwd_serial_io((const uint16_t*)a, (const uint16_t*)b, h0, (uint16_t*)h, C, T, vec,
                       stream);
  else
    scan_fwd_serial_io((const float*)a, (const float*)b, h0, (float*)h, C, T, vec, stream);
  return hipGetLastError();
}

hipError_t launch_scan_bwd_serial(const void* a, const void* h, const float* h0, const void* g,
                                  void* da, void* db, float* dh0, int io, int64_t C, int64_t T,
                                  int vec, hipStream_t stream) {
  if (io == kIoBf16)
    scan_bwd_serial_io((const uint16_t*)a, (const uint16_t*)h, h0, (const uint16_t*)g,
                       (uint16_t*)da, (uint16_t*)db, dh0, C, T, vec, stream);
  else
    scan_bwd_serial_io((const float*)a, (const float*)h, h0, (const float*)g, (float*)da,
                       (float*)db, dh0, C, T, vec, stream);
  return hipGetLastError();
}

}  // namespace lrs
