// scan_bdt.hip -- time-contiguous kernels: one channel is one row of T values
// ([B, D, T] layout, "stored contiguously along time" as the DEER page's
// engineering section recommends for the input, state and Jacobian arrays).
//
// Work decomposition (same for all three kernels):
//   * a workgroup of NT threads owns one chunk of NT*K consecutive steps of one
//     channel; lane-contiguous strips of K steps are folded serially in
//     registers, then scanned across the wave (DPP) and across waves (LDS);
//   * a channel longer than one chunk is split into chunks (the page's
//     T = N*S sub-sequence split, one block per sub-sequence); the state entering
//     a chunk comes from a decoupled look-back over per-chunk status words, and
//     chunk order comes from a per-channel ticket so the wait always terminates;
//   * every input byte is read once and every output byte written once.
//
// Kernels:
//   k_scan_fwd_bdt : h_t = a_t h_{t-1} + b_t
//   k_scan_bwd_bdt : reverse-time adjoint, lam_t = g_t + a_{t+1} lam_{t+1},
//                    da_t = lam_t h_{t-1}, db_t = lam_t, dh0 = a_1 lam_1
//   k_deer_iter    : one fused DEER Newton iteration for h_t = tanh(w h_{t-1}+u_t)
#include "lrs_device.hpp"
#include "lrs_internal.hpp"

namespace lrs {

template <int NT>
struct BlockShared {
  float wA[NT / kWave];
  float wB[NT / kWave];
  uint32_t wmax[NT / kWave];
  float carry;
  int chunk;
};

// Combine per-wave inclusive results: every thread gets the composition of the
// waves before its own (PA, PB) and of the whole block (TA, TB).
template <int NT>
__device__ __forceinline__ void block_combine(float A, float B, BlockShared<NT>& s, float& PA,
                                              float& PB, float& TA, float& TB) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  if (lane == kWave - 1) {
    s.wA[wid] = A;
    s.wB[wid] = B;
  }
  __syncthreads();
  PA = 1.0f; PB = 0.0f; TA = 1.0f; TB = 0.0f;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) {
    const float wa = s.wA[w], wb = s.wB[w];
    if (w < wid) {
      PB = __builtin_fmaf(wa, PB, wb);
      PA = PA * wa;
    }
    TB = __builtin_fmaf(wa, TB, wb);
    TA = TA * wa;
  }
}

// State entering logical chunk c of a channel.  Single-chunk channels use x0
// directly; otherwise thread 0 publishes this chunk's aggregate, looks back,
// publishes the inclusive state and shares the carry through LDS.
template <int NT>
__device__ __forceinline__ float chunk_carry(bool multi, int c, float TA, float TB, float x0,
                                             uint64_t* st, BlockShared<NT>& s) {
  if (!multi) return x0;
  if (threadIdx.x == 0) {
    float x_in = x0;
    if (c > 0) {
      status_store(st + c, pack_agg(TA, TB));
      x_in = lookback_carry(st, c, 1);
    }
    status_store(st + c, pack_inc(__builtin_fmaf(TA, x_in, TB)));
    s.carry = x_in;
  }
  __syncthreads();
  return s.carry;
}

template <int NT>
__device__ __forceinline__ int chunk_ticket(bool multi, unsigned* tickets, int64_t ch,
                                            BlockShared<NT>& s) {
  if (!multi) return 0;
  if (threadIdx.x == 0) s.chunk = (int)take_ticket(tickets + ch);
  __syncthreads();
  return s.chunk;
}

// ---------------------------------------------------------------------------
// forward scan
// ---------------------------------------------------------------------------
template <int NT, int K>
__global__ __launch_bounds__(NT) void k_scan_fwd_bdt(const float* __restrict__ a,
                                                     const float* __restrict__ b,
                                                     const float* __restrict__ h0,
                                                     float* __restrict__ h, int64_t T, int64_t C,
                                                     int nchunk, int vec,
                                                     uint64_t* __restrict__ status,
                                                     unsigned* __restrict__ tickets) {
  __shared__ BlockShared<NT> s;
  const bool multi = nchunk > 1;
  const int64_t ch = multi ? (int64_t)(blockIdx.x % (uint64_t)C) : (int64_t)blockIdx.x;
  const int c = chunk_ticket<NT>(multi, tickets, ch, s);
  const int64_t t0 = (int64_t)c * (NT * K) + (int64_t)threadIdx.x * K;
  const float* arow = a + ch * T;
  const float* brow = b + ch * T;

  float av[K], bv[K];
  load_strip<K>(arow, t0, T, vec, 1.0f, av);
  load_strip<K>(brow, t0, T, vec, 0.0f, bv);

  float A = av[0], B = bv[0];
#pragma unroll
  for (int j = 1; j < K; ++j) {
    B = __builtin_fmaf(av[j], B, bv[j]);
    A = A * av[j];
  }
  wave_scan(A, B);
  float PA, PB, TA, TB;
  block_combine<NT>(A, B, s, PA, PB, TA, TB);
  const float x0 = h0 ? h0[ch] : 0.0f;
  const float x_in = chunk_carry<NT>(multi, c, TA, TB, x0, status + ch * nchunk, s);

  const float xw = __builtin_fmaf(PA, x_in, PB);  // state entering this wave
  const float xe = __builtin_fmaf(A, xw, B);      // state at the end of this lane's strip
  float x = wave_shift_up(xe, xw);                // state entering this lane's strip
#pragma unroll
  for (int j = 0; j < K; ++j) {
    x = __builtin_fmaf(av[j], x, bv[j]);
    bv[j] = x;
  }
  store_strip<K>(h + ch * T, t0, T, vec, bv);
}

// ---------------------------------------------------------------------------
// backward (reverse-time) scan.  Logical chunk 0 is the last physical chunk and
// lane order runs backwards in time, so the same forward combine applies.
// grad_b may alias grad_h: each thread reads its own g strip before writing.
// ---------------------------------------------------------------------------
template <int NT, int K>
__global__ __launch_bounds__(NT) void k_scan_bwd_bdt(const float* __restrict__ a,
                                                     const float* __restrict__ h,
                                                     const float* __restrict__ h0, const float* g,
                                                     float* __restrict__ da, float* db,
                                                     float* __restrict__ dh0, int64_t T, int64_t C,
                                                     int nchunk, int vec,
                                                     uint64_t* __restrict__ status,
                                                     unsigned* __restrict__ tickets) {
  __shared__ BlockShared<NT> s;
  const bool multi = nchunk > 1;
  const int64_t ch = multi ? (int64_t)(blockIdx.x % (uint64_t)C) : (int64_t)blockIdx.x;
  const int c = chunk_ticket<NT>(multi, tickets, ch, s);
  const int pc = nchunk - 1 - c;
  const int64_t t0 = (int64_t)pc * (NT * K) + (int64_t)(NT - 1 - (int)threadIdx.x) * K;
  const float* arow = a + ch * T;
  const float* hrow = h + ch * T;
  const float* grow = g + ch * T;

  float av[K], hv[K], gv[K];
  load_strip<K>(arow, t0, T, vec, 1.0f, av);
  load_strip<K>(hrow, t0, T, vec, 0.0f, hv);
  load_strip<K>(grow, t0, T, vec, 0.0f, gv);
  const float x0h = h0 ? h0[ch] : 0.0f;
  // halo: a_{t+1} for the strip's last step, h_{t-1} for its first step
  const float a_next = (t0 + K < T) ? arow[t0 + K] : (t0 + K == T ? 0.0f : 1.0f);
  const float h_prev = (t0 > 0 && t0 <= T) ? hrow[t0 - 1] : x0h;

  // alpha_i = a_{t0+i+1}: zero at the last real step, identity past the end
  float al[K];
#pragma unroll
  for (int i = 0; i < K - 1; ++i) al[i] = av[i + 1];
  al[K - 1] = a_next;
  if (t0 + K > T - 1) {
#pragma unroll
    for (int i = 0; i < K - 1; ++i)
      if (t0 + i + 1 == T) al[i] = 0.0f;
  }

  // fold the strip in scan order (descending time)
  float A = al[K - 1], B = gv[K - 1];
#pragma unroll
  for (int i = K - 2; i >= 0; --i) {
    B = __builtin_fmaf(al[i], B, gv[i]);
    A = A * al[i];
  }
  wave_scan(A, B);
  float PA, PB, TA, TB;
  block_combine<NT>(A, B, s, PA, PB, TA, TB);
  const float x_in = chunk_carry<NT>(multi, c, TA, TB, 0.0f, status + ch * nchunk, s);

  const float xw = __builtin_fmaf(PA, x_in, PB);
  const float xe = __builtin_fmaf(A, xw, B);
  float x = wave_shift_up(xe, xw);  // lam entering this strip from the right
  float dav[K];
#pragma unroll
  for (int i = K - 1; i >= 0; --i) {
    x = __builtin_fmaf(al[i], x, gv[i]);
    const float hp = (i > 0) ? hv[i - 1] : h_prev;
    dav[i] = x * hp;
    gv[i] = x;
  }
  if (dh0 && t0 == 0) dh0[ch] = av[0] * x;
  store_strip<K>(da + ch * T, t0, T, vec, dav);
  store_strip<K>(db + ch * T, t0, T, vec, gv);
}

// ---------------------------------------------------------------------------
// DEER iteration: from the iterate y (NULL = all zero) build
//   z_t = tanh(w y_{t-1} + u_t), J_t = w (1 - z_t^2), rhs_t = z_t - J_t y_{t-1}
// (DEER page, core principle: evaluate f and its Jacobian, multiply by the
// Jacobian, apply the inverse operator = linear recurrence with an initial
// condition), solve y'_t = J_t y'_{t-1} + rhs_t by the scan, and fold
// max |y' - y| into delta_bits[iter] (non-negative floats order like their
// bit patterns; NaN sorts above every finite value).
// The kernel returns at once when the previous iteration already met the stop
// rule delta < eps (DEER page, engineering section); a skipped iteration
// leaves its slot at 0, so later ones skip as well.
// ---------------------------------------------------------------------------
template <int NT, int K>
__global__ __launch_bounds__(NT) void k_deer_iter(const float* __restrict__ w,
                                                  const float* __restrict__ u,
                                                  const float* __restrict__ y,
                                                  const float* __restrict__ h0,
                                                  float* __restrict__ yn, int64_t T, int64_t C,
                                                  int64_t D, int nchunk, int vec,
                                                  uint64_t* __restrict__ status,
                                                  unsigned* __restrict__ tickets,
                                                  uint32_t* __restrict__ delta_bits, int iter,
                                                  float eps) {
  if (iter > 0) {
    const uint32_t prev = __hip_atomic_load(delta_bits + iter - 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
    if (as_f32(prev) < eps) return;
  }
  __shared__ BlockShared<NT> s;
  const bool multi = nchunk > 1;
  const int64_t ch = multi ? (int64_t)(blockIdx.x % (uint64_t)C) : (int64_t)blockIdx.x;
  const int c = chunk_ticket<NT>(multi, tickets, ch, s);
  const int64_t t0 = (int64_t)c * (NT * K) + (int64_t)threadIdx.x * K;
  const float wd = w[ch % D];
  const float x0 = h0 ? h0[ch] : 0.0f;

  float uv[K], yv[K];
  load_strip<K>(u + ch * T, t0, T, vec, 0.0f, uv);
  if (y) {
    load_strip<K>(y + ch * T, t0, T, vec, 0.0f, yv);
  } else {
#pragma unroll
    for (int j = 0; j < K; ++j) yv[j] = 0.0f;
  }
  const float y_prev = (t0 > 0 && t0 <= T) ? (y ? y[ch * T + t0 - 1] : 0.0f) : x0;

  float Jv[K], rv[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const float yp = (j > 0) ? yv[j - 1] : y_prev;
    const float z = tanh_fast(__builtin_fmaf(wd, yp, uv[j]));
    const float J = wd * __builtin_fmaf(-z, z, 1.0f);
    Jv[j] = J;
    rv[j] = __builtin_fmaf(-J, yp, z);
  }
  if (t0 + K > T) {
#pragma unroll
    for (int j = 0; j < K; ++j)
      if (t0 + j >= T) { Jv[j] = 1.0f; rv[j] = 0.0f; }
  }

  float A = Jv[0], B = rv[0];
#pragma unroll
  for (int j = 1; j < K; ++j) {
    B = __builtin_fmaf(Jv[j], B, rv[j]);
    A = A * Jv[j];
  }
  wave_scan(A, B);
  float PA, PB, TA, TB;
  block_combine<NT>(A, B, s, PA, PB, TA, TB);
  const float x_in = chunk_carry<NT>(multi, c, TA, TB, x0, status + ch * nchunk, s);

  const float xw = __builtin_fmaf(PA, x_in, PB);
  const float xe = __builtin_fmaf(A, xw, B);
  float x = wave_shift_up(xe, xw);
  uint32_t dmax = 0;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    x = __builtin_fmaf(Jv[j], x, rv[j]);
    const uint32_t d = as_u32(fabsf(x - yv[j]));
    if (t0 + j < T) dmax = d > dmax ? d : dmax;
    rv[j] = x;
  }
  store_strip<K>(yn + ch * T, t0, T, vec, rv);

  dmax = wave_max_u32(dmax);
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  if (lane == 0) s.wmax[wid] = dmax;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < NT / kWave; ++i) m = s.wmax[i] > m ? s.wmax[i] : m;
    __hip_atomic_fetch_max(delta_bits + iter, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
namespace {
constexpr int kNT = 256;

template <int K>
constexpr int chunk_of() { return kNT * K; }

}  // namespace

RowPlan plan_rows(int64_t T, int kmax_strip) {
  RowPlan p;
  p.nt = kNT;
  int K = 4;
  while (K < kmax_strip && (int64_t)kNT * K < T) K *= 2;
  p.k = K;
  const int64_t chunk = (int64_t)kNT * K;
  p.nchunk = (T + chunk - 1) / chunk;
  if (p.nchunk < 1) p.nchunk = 1;
  return p;
}

#define LRS_DISPATCH_K(K_, ...)                        \
  switch (K_) {                                        \
    case 4: { constexpr int KK = 4; __VA_ARGS__; } break;   \
    case 8: { constexpr int KK = 8; __VA_ARGS__; } break;   \
    case 16: { constexpr int KK = 16; __VA_ARGS__; } break; \
    case 32: { constexpr int KK = 32; __VA_ARGS__; } break; \
    default: return hipErrorInvalidValue;              \
  }

hipError_t launch_scan_fwd_bdt(const float* a, const float* b, const float* h0, float* h,
                               int64_t C, int64_t T, const RowPlan& p, int vec,
                               uint64_t* status, unsigned* tickets, hipStream_t stream) {
  const uint64_t grid = (uint64_t)C * (uint64_t)p.nchunk;
  LRS_DISPATCH_K(p.k, hipLaunchKernelGGL((k_scan_fwd_bdt<kNT, KK>), dim3((unsigned)grid),
                                         dim3(kNT), 0, stream, a, b, h0, h, T, C, (int)p.nchunk,
                                         vec, status, tickets));
  return hipGetLastError();
}

hipError_t launch_scan_bwd_bdt(const float* a, const float* h, const float* h0, const float* g,
                               float* da, float* db, float* dh0, int64_t C, int64_t T,
                               const RowPlan& p, int vec, uint64_t* status, unsigned* tickets,
                               hipStream_t stream) {
  const uint64_t grid = (uint64_t)C * (uint64_t)p.nchunk;
  LRS_DISPATCH_K(p.k, hipLaunchKernelGGL((k_scan_bwd_bdt<kNT, KK>), dim3((unsigned)grid),
                                         dim3(kNT), 0, stream, a, h, h0, g, da, db, dh0, T, C,
                                         (int)p.nchunk, vec, status, tickets));
  return hipGetLastError();
}

hipError_t launch_deer_iter(const float* w, const float* u, const float* y, const float* h0,
                            float* yn, int64_t C, int64_t D, int64_t T, const RowPlan& p, int vec,
                            uint64_t* status, unsigned* tickets, uint32_t* delta_bits, int iter,
                            float eps, hipStream_t stream) {
  const uint64_t grid = (uint64_t)C * (uint64_t)p.nchunk;
  LRS_DISPATCH_K(p.k, hipLaunchKernelGGL((k_deer_iter<kNT, KK>), dim3((unsigned)grid), dim3(kNT),
                                         0, stream, w, u, y, h0, yn, T, C, D, (int)p.nchunk, vec,
                                         status, tickets, delta_bits, iter, eps));
  return hipGetLastError();
}

}  // namespace lrs
