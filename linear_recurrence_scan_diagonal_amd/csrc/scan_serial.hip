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
// A lane reads its channel in 16-byte groups when the rows allow it (T a
// multiple of 4 and 16-byte aligned arrays), else element by element; the
// lanes of a wave read 64 consecutive rows, so a wave's accesses cover one
// contiguous stretch of 64*T elements per array.
#include "lrs_device.hpp"
#include "lrs_internal.hpp"

namespace lrs {

constexpr int kSerialThreads = 256;

template <bool VEC>
__global__ __launch_bounds__(kSerialThreads) void k_scan_fwd_serial(
    const float* __restrict__ a, const float* __restrict__ b, const float* __restrict__ h0,
    float* __restrict__ h, int64_t T, int64_t C) {
  const int64_t ch = (int64_t)blockIdx.x * kSerialThreads + threadIdx.x;
  if (ch >= C) return;
  const int64_t row = ch * T;
  float x = h0 ? h0[ch] : 0.0f;
  if (VEC) {
    const float4* a4 = reinterpret_cast<const float4*>(a + row);
    const float4* b4 = reinterpret_cast<const float4*>(b + row);
    float4* h4 = reinterpret_cast<float4*>(h + row);
    const int64_t ng = T / 4;
#pragma unroll 4
    for (int64_t i = 0; i < ng; ++i) {
      const float4 av = a4[i], bv = b4[i];
      float4 o;
      x = __builtin_fmaf(av.x, x, bv.x); o.x = x;
      x = __builtin_fmaf(av.y, x, bv.y); o.y = x;
      x = __builtin_fmaf(av.z, x, bv.z); o.z = x;
      x = __builtin_fmaf(av.w, x, bv.w); o.w = x;
      h4[i] = o;
    }
  } else {
#pragma unroll 4
    for (int64_t t = 0; t < T; ++t) {
      x = __builtin_fmaf(a[row + t], x, b[row + t]);
      h[row + t] = x;
    }
  }
}

// lam_t = g_t + a_{t+1} lam_{t+1} (a_{T+1} = 0), grad_b = lam,
// grad_a_t = lam_t h_{t-1} (h0 at t = 1), grad_h0 = a_1 lam_1.  grad_b may
// alias g: each element of g is read before the same element of grad_b is
// written, by the same lane.
template <bool VEC>
__global__ __launch_bounds__(kSerialThreads) void k_scan_bwd_serial(
    const float* __restrict__ a, const float* __restrict__ h, const float* __restrict__ h0,
    const float* g, float* __restrict__ da, float* db, float* __restrict__ dh0, int64_t T,
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
    const float4* a4 = reinterpret_cast<const float4*>(a + row);
    const float4* hv = reinterpret_cast<const float4*>(h + row);
    const float4* g4 = reinterpret_cast<const float4*>(g + row);
    float4* da4 = reinterpret_cast<float4*>(da + row);
    float4* db4 = reinterpret_cast<float4*>(db + row);
    int64_t i = T / 4 - 1;  // group index, descending
    for (; i >= kU - 1; i -= kU) {
      float4 av[kU], hh[kU], gv[kU];
#pragma unroll
      for (int k = 0; k < kU; ++k) {
        av[k] = a4[i - k];
        hh[k] = hv[i - k];
        gv[k] = g4[i - k];
      }
      const int64_t first = i - (kU - 1);
      const float hp_last = (first > 0) ? h[row + 4 * first - 1] : x0;
#pragma unroll
      for (int k = 0; k < kU; ++k) {
        const float hp = (k < kU - 1) ? hh[k + 1].w : hp_last;
        const float l3 = __builtin_fmaf(a_next, lam, gv[k].w);
        const float l2 = __builtin_fmaf(av[k].w, l3, gv[k].z);
        const float l1 = __builtin_fmaf(av[k].z, l2, gv[k].y);
        const float l0 = __builtin_fmaf(av[k].y, l1, gv[k].x);
        da4[i - k] = make_float4(l0 * hp, l1 * hh[k].x, l2 * hh[k].y, l3 * hh[k].z);
        db4[i - k] = make_float4(l0, l1, l2, l3);
        lam = l0;
        a_next = av[k].x;
      }
    }
    for (; i >= 0; --i) {
      const float4 av = a4[i], hh = hv[i], gv = g4[i];
      const float hp = (i > 0) ? h[row + 4 * i - 1] : x0;
      const float l3 = __builtin_fmaf(a_next, lam, gv.w);
      const float l2 = __builtin_fmaf(av.w, l3, gv.z);
      const float l1 = __builtin_fmaf(av.z, l2, gv.y);
      const float l0 = __builtin_fmaf(av.y, l1, gv.x);
      da4[i] = make_float4(l0 * hp, l1 * hh.x, l2 * hh.y, l3 * hh.z);
      db4[i] = make_float4(l0, l1, l2, l3);
      lam = l0;
      a_next = av.x;
    }
  } else {
    int64_t t = T - 1;  // step index, descending
    for (; t >= kU - 1; t -= kU) {
      float av[kU], hp[kU], gv[kU];
#pragma unroll
      for (int k = 0; k < kU; ++k) {
        av[k] = a[row + t - k];
        gv[k] = g[row + t - k];
        hp[k] = (t - k > 0) ? h[row + t - k - 1] : x0;
      }
#pragma unroll
      for (int k = 0; k < kU; ++k) {
        lam = __builtin_fmaf(a_next, lam, gv[k]);
        da[row + t - k] = lam * hp[k];
        db[row + t - k] = lam;
        a_next = av[k];
      }
    }
    for (; t >= 0; --t) {
      const float at = a[row + t], gt = g[row + t];
      const float hp = (t > 0) ? h[row + t - 1] : x0;
      lam = __builtin_fmaf(a_next, lam, gt);
      da[row + t] = lam * hp;
      db[row + t] = lam;
      a_next = at;
    }
  }
  if (dh0) dh0[ch] = a_next * lam;
}

hipError_t launch_scan_fwd_serial(const float* a, const float* b, const float* h0, float* h,
                                  int64_t C, int64_t T, int vec, hipStream_t stream) {
  const dim3 grid((unsigned)((C + kSerialThreads - 1) / kSerialThreads));
  if (vec)
    hipLaunchKernelGGL(k_scan_fwd_serial<true>, grid, dim3(kSerialThreads), 0, stream, a, b, h0,
                       h, T, C);
  else
    hipLaunchKernelGGL(k_scan_fwd_serial<false>, grid, dim3(kSerialThreads), 0, stream, a, b, h0,
                       h, T, C);
  return hipGetLastError();
}

hipError_t launch_scan_bwd_serial(const float* a, const float* h, const float* h0, const float* g,
                                  float* da, float* db, float* dh0, int64_t C, int64_t T, int vec,
                                  hipStream_t stream) {
  const dim3 grid((unsigned)((C + kSerialThreads - 1) / kSerialThreads));
  if (vec)
    hipLaunchKernelGGL(k_scan_bwd_serial<true>, grid, dim3(kSerialThreads), 0, stream, a, h, h0,
                       g, da, db, dh0, T, C);
  else
    hipLaunchKernelGGL(k_scan_bwd_serial<false>, grid, dim3(kSerialThreads), 0, stream, a, h, h0,
                       g, da, db, dh0, T, C);
  return hipGetLastError();
}

}  // namespace lrs
