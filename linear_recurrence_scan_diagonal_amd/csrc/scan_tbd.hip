// scan_tbd.hip -- feature-contiguous kernels ([T, B, D] layout): consecutive
// lanes own consecutive channels, so every load and store of a time row is a
// contiguous, fully coalesced access, and time runs serially inside a thread.
//
// Work decomposition:
//   * a workgroup of NW waves owns a block of CW = 64*CPT channels over a
//     block of TW = NW*L time steps; wave w takes L consecutive steps, each
//     lane CPT consecutive channels;
//   * per channel, each thread folds its L steps into one affine map, the
//     waves' maps are combined through LDS, and the state entering the time
//     block comes from a lane-parallel decoupled look-back over per-channel
//     status words (one 64-bit word per channel and time block); time-block
//     order comes from a per-channel-block ticket;
//   * every input byte is read once and every output byte written once
//     (the backward kernel also reads one halo row above and below each
//     thread's steps; those hit in cache).
//
// Kernels:
//   k_scan_fwd_tbd : h_t = a_t h_{t-1} + b_t
//   k_scan_bwd_tbd : reverse-time adjoint (see k_scan_bwd_bdt)
//   k_sru_fwd      : SRU layer, gates + cell-state scan + highway output fused
//                    (page "CUDA并行化RNN训练：从O(T)到O(log T)的工程实践与参数调优",
//                    SRU paragraph and checklist item 2: one kernel for every
//                    element-wise operation)
#include "lrs_device.hpp"
#include "lrs_internal.hpp"

namespace lrs {

template <int NW, int CPT>
struct ColShared {
  float A[NW][kWave * CPT];
  float B[NW][kWave * CPT];
  float carry[kWave * CPT];
  int chunk;
};

// ---- CPT-wide row access --------------------------------------------------

template <int CPT>
__device__ __forceinline__ void load_row(const float* __restrict__ p, int nvalid, bool vec,
                                         float fill, float (&v)[CPT]) {
  if (vec && nvalid == CPT) {
    if constexpr (CPT == 4) {
      const float4 x = *reinterpret_cast<const float4*>(p);
      v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    } else if constexpr (CPT == 2) {
      const float2 x = *reinterpret_cast<const float2*>(p);
      v[0] = x.x; v[1] = x.y;
    } else {
#pragma unroll
      for (int k = 0; k < CPT; ++k) v[k] = p[k];
    }
  } else {
#pragma unroll
    for (int k = 0; k < CPT; ++k) v[k] = (k < nvalid) ? p[k] : fill;
  }
}

template <int CPT>
__device__ __forceinline__ void store_row(float* __restrict__ p, int nvalid, bool vec,
                                          const float (&v)[CPT]) {
  if (vec && nvalid == CPT) {
    if constexpr (CPT == 4) {
      *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    } else if constexpr (CPT == 2) {
      *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
    } else {
#pragma unroll
      for (int k = 0; k < CPT; ++k) p[k] = v[k];
    }
  } else {
#pragma unroll
    for (int k = 0; k < CPT; ++k)
      if (k < nvalid) p[k] = v[k];
  }
}

// bf16 rows: raw 16-bit patterns, widened exactly to fp32 on use.
template <int CPT>
__device__ __forceinline__ void load_row_bf16(const uint16_t* __restrict__ p, int nvalid, bool vec,
                                              uint16_t (&v)[CPT]) {
  if (vec && nvalid == CPT) {
    if constexpr (CPT == 4) {
      const uint2 x = *reinterpret_cast<const uint2*>(p);
      v[0] = (uint16_t)x.x; v[1] = (uint16_t)(x.x >> 16);
      v[2] = (uint16_t)x.y; v[3] = (uint16_t)(x.y >> 16);
    } else if constexpr (CPT == 8) {
      const uint4 x = *reinterpret_cast<const uint4*>(p);
      v[0] = (uint16_t)x.x; v[1] = (uint16_t)(x.x >> 16);
      v[2] = (uint16_t)x.y; v[3] = (uint16_t)(x.y >> 16);
      v[4] = (uint16_t)x.z; v[5] = (uint16_t)(x.z >> 16);
      v[6] = (uint16_t)x.w; v[7] = (uint16_t)(x.w >> 16);
    } else {
#pragma unroll
      for (int k = 0; k < CPT; ++k) v[k] = p[k];
    }
  } else {
#pragma unroll
    for (int k = 0; k < CPT; ++k) v[k] = (k < nvalid) ? p[k] : (uint16_t)0;
  }
}

__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return as_f32((uint32_t)v << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Round pairs of fp32 to bf16 (nearest-even, gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  const bf16x2_t b = __builtin_convertvector(f, bf16x2_t);
  return __builtin_bit_cast(uint32_t, b);
}

template <int CPT>
__device__ __forceinline__ void store_row_bf16(uint16_t* __restrict__ p, int nvalid, bool vec,
                                               const float (&v)[CPT]) {
  static_assert(CPT % 2 == 0, "bf16 rows hold an even number of channels");
  uint32_t w[CPT / 2];
#pragma unroll
  for (int k = 0; k < CPT / 2; ++k) w[k] = pack_bf16x2(v[2 * k], v[2 * k + 1]);
  if (vec && nvalid == CPT) {
    if constexpr (CPT == 4) {
      *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
    } else if constexpr (CPT == 8) {
      *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
#pragma unroll
      for (int k = 0; k < CPT / 2; ++k) reinterpret_cast<uint32_t*>(p)[k] = w[k];
    }
  } else {
#pragma unroll
    for (int k = 0; k < CPT; ++k)
      if (k < nvalid) p[k] = (uint16_t)(w[k / 2] >> (16 * (k & 1)));
  }
}

// ---- block-level pieces ----------------------------------------------------

// Per channel: composition of the waves before this one (PA, PB) and of the
// whole block (TA, TB).  Wave order is scan order.
template <int NW, int CPT>
__device__ __forceinline__ void col_block_combine(const float (&A)[CPT], const float (&B)[CPT],
                                                  ColShared<NW, CPT>& s, float (&PA)[CPT],
                                                  float (&PB)[CPT], float (&TA)[CPT],
                                                  float (&TB)[CPT]) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    s.A[wid][lane * CPT + k] = A[k];
    s.B[wid][lane * CPT + k] = B[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    PA[k] = 1.0f; PB[k] = 0.0f; TA[k] = 1.0f; TB[k] = 0.0f;
  }
#pragma unroll
  for (int w = 0; w < NW; ++w) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const float wa = s.A[w][lane * CPT + k], wb = s.B[w][lane * CPT + k];
      if (w < wid) {
        PB[k] = __builtin_fmaf(wa, PB[k], wb);
        PA[k] = PA[k] * wa;
      }
      TB[k] = __builtin_fmaf(wa, TB[k], wb);
      TA[k] = TA[k] * wa;
    }
  }
}

// State entering logical time block tb for each of this lane's channels.
// Wave 0 publishes aggregates, looks back and publishes inclusive states.
// st points at this channel block's status row for time block 0; time blocks
// are CW words apart.
template <int NW, int CPT>
__device__ __forceinline__ void col_chunk_carry(bool multi, int tb, int nvc,
                                                const float (&TA)[CPT], const float (&TB)[CPT],
                                                const float (&x0)[CPT], uint64_t* st,
                                                ColShared<NW, CPT>& s, float (&carry)[CPT]) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  constexpr int CW = kWave * CPT;
  if (!multi) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) carry[k] = x0[k];
    return;
  }
  if (wid == 0) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int j = lane * CPT + k;
      float x_in = x0[k];
      if (k < nvc) {
        if (tb > 0) {
          status_store(st + (int64_t)tb * CW + j, pack_agg(TA[k], TB[k]));
          x_in = lookback_carry(st + j, tb, CW);
        }
        status_store(st + (int64_t)tb * CW + j, pack_inc(__builtin_fmaf(TA[k], x_in, TB[k])));
      }
      s.carry[j] = x_in;
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < CPT; ++k) carry[k] = s.carry[lane * CPT + k];
}

template <int NW, int CPT>
__device__ __forceinline__ int col_ticket(bool multi, unsigned* tickets, int cb,
                                          ColShared<NW, CPT>& s) {
  if (!multi) return 0;
  if (threadIdx.x == 0) s.chunk = (int)take_ticket(tickets + cb);
  __syncthreads();
  return s.chunk;
}

__device__ __forceinline__ int clamp_valid(int64_t n, int cpt) {
  return n <= 0 ? 0 : (n >= cpt ? cpt : (int)n);
}

// ---------------------------------------------------------------------------
// forward scan, [T, B, D]
// ---------------------------------------------------------------------------
template <int NW, int L, int CPT>
__global__ __launch_bounds__(NW* kWave) void k_scan_fwd_tbd(
    const float* __restrict__ a, const float* __restrict__ b, const float* __restrict__ h0,
    float* __restrict__ h, int64_t T, int64_t C, int ncb, int ntb, int vec,
    uint64_t* __restrict__ status, unsigned* __restrict__ tickets) {
  constexpr int CW = kWave * CPT, TW = NW * L;
  __shared__ ColShared<NW, CPT> s;
  const bool multi = ntb > 1;
  const int cb = (int)(blockIdx.x % (unsigned)ncb);
  const int tb = col_ticket<NW, CPT>(multi, tickets, cb, s);
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const int64_t c0 = (int64_t)cb * CW + lane * CPT;
  const int nvc = clamp_valid(C - c0, CPT);
  const int64_t tw0 = (int64_t)tb * TW + (int64_t)wid * L;

  float av[L][CPT], bv[L][CPT];
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int nv = (tw0 + i < T) ? nvc : 0;
    const int64_t off = (tw0 + i) * C + c0;
    load_row<CPT>(a + off, nv, vec, 1.0f, av[i]);
    load_row<CPT>(b + off, nv, vec, 0.0f, bv[i]);
  }
  float A[CPT], B[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    A[k] = av[0][k];
    B[k] = bv[0][k];
#pragma unroll
    for (int i = 1; i < L; ++i) {
      B[k] = __builtin_fmaf(av[i][k], B[k], bv[i][k]);
      A[k] = A[k] * av[i][k];
    }
  }
  float PA[CPT], PB[CPT], TA[CPT], TB[CPT], x0[CPT], x[CPT];
  col_block_combine<NW, CPT>(A, B, s, PA, PB, TA, TB);
#pragma unroll
  for (int k = 0; k < CPT; ++k) x0[k] = (h0 && k < nvc) ? h0[c0 + k] : 0.0f;
  col_chunk_carry<NW, CPT>(multi, tb, nvc, TA, TB, x0, status + (int64_t)cb * ntb * CW, s, x);
#pragma unroll
  for (int k = 0; k < CPT; ++k) x[k] = __builtin_fmaf(PA[k], x[k], PB[k]);
#pragma unroll
  for (int i = 0; i < L; ++i) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      x[k] = __builtin_fmaf(av[i][k], x[k], bv[i][k]);
      bv[i][k] = x[k];
    }
    const int nv = (tw0 + i < T) ? nvc : 0;
    store_row<CPT>(h + (tw0 + i) * C + c0, nv, vec, bv[i]);
  }
}

// ---------------------------------------------------------------------------
// backward scan, [T, B, D]: logical time block 0 is the last physical block,
// wave 0 takes the latest steps of the block, each thread runs time backwards.
// ---------------------------------------------------------------------------
template <int NW, int L, int CPT>
__global__ __launch_bounds__(NW* kWave) void k_scan_bwd_tbd(
    const float* __restrict__ a, const float* __restrict__ h, const float* __restrict__ h0,
    const float* g, float* __restrict__ da, float* db, float* __restrict__ dh0, int64_t T,
    int64_t C, int ncb, int ntb, int vec, uint64_t* __restrict__ status,
    unsigned* __restrict__ tickets) {
  constexpr int CW = kWave * CPT, TW = NW * L;
  __shared__ ColShared<NW, CPT> s;
  const bool multi = ntb > 1;
  const int cb = (int)(blockIdx.x % (unsigned)ncb);
  const int tb = col_ticket<NW, CPT>(multi, tickets, cb, s);
  const int ptb = ntb - 1 - tb;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const int64_t c0 = (int64_t)cb * CW + lane * CPT;
  const int nvc = clamp_valid(C - c0, CPT);
  const int64_t tw0 = (int64_t)ptb * TW + (int64_t)(NW - 1 - wid) * L;

  float av[L + 1][CPT], hv[L][CPT], gv[L][CPT], hp[CPT];
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int nv = (tw0 + i < T) ? nvc : 0;
    const int64_t off = (tw0 + i) * C + c0;
    load_row<CPT>(a + off, nv, vec, 1.0f, av[i]);
    load_row<CPT>(h + off, nv, vec, 0.0f, hv[i]);
    load_row<CPT>(g + off, nv, vec, 0.0f, gv[i]);
  }
  // halo rows: a at t = tw0+L (0 exactly one past the end, 1 beyond),
  // h at t = tw0-1 (h0 for the first step)
  {
    const int64_t tn = tw0 + L;
    if (tn < T) {
      load_row<CPT>(a + tn * C + c0, nvc, vec, 1.0f, av[L]);
    } else {
#pragma unroll
      for (int k = 0; k < CPT; ++k) av[L][k] = (tn == T) ? 0.0f : 1.0f;
    }
    if (tw0 > 0 && tw0 <= T) {
      load_row<CPT>(h + (tw0 - 1) * C + c0, nvc, vec, 0.0f, hp);
    } else {
#pragma unroll
      for (int k = 0; k < CPT; ++k) hp[k] = (h0 && k < nvc) ? h0[c0 + k] : 0.0f;
    }
  }
  // alpha_i = a_{t+1}; zero at the last real step
  if (tw0 + L > T - 1) {
#pragma unroll
    for (int i = 0; i < L; ++i)
      if (tw0 + i + 1 == T) {
#pragma unroll
        for (int k = 0; k < CPT; ++k) av[i + 1][k] = 0.0f;
      }
  }
  float A[CPT], B[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    A[k] = av[L][k];
    B[k] = gv[L - 1][k];
#pragma unroll
    for (int i = L - 2; i >= 0; --i) {
      B[k] = __builtin_fmaf(av[i + 1][k], B[k], gv[i][k]);
      A[k] = A[k] * av[i + 1][k];
    }
  }
  float PA[CPT], PB[CPT], TA[CPT], TB[CPT], zero[CPT], x[CPT];
  col_block_combine<NW, CPT>(A, B, s, PA, PB, TA, TB);
#pragma unroll
  for (int k = 0; k < CPT; ++k) zero[k] = 0.0f;
  col_chunk_carry<NW, CPT>(multi, tb, nvc, TA, TB, zero, status + (int64_t)cb * ntb * CW, s, x);
#pragma unroll
  for (int k = 0; k < CPT; ++k) x[k] = __builtin_fmaf(PA[k], x[k], PB[k]);
#pragma unroll
  for (int i = L - 1; i >= 0; --i) {
    float dav[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      x[k] = __builtin_fmaf(av[i + 1][k], x[k], gv[i][k]);
      dav[k] = x[k] * (i > 0 ? hv[i - 1][k] : hp[k]);
      gv[i][k] = x[k];
    }
    const int nv = (tw0 + i < T) ? nvc : 0;
    const int64_t off = (tw0 + i) * C + c0;
    store_row<CPT>(da + off, nv, vec, dav);
    store_row<CPT>(db + off, nv, vec, gv[i]);
  }
  if (dh0 && tw0 == 0) {
#pragma unroll
    for (int k = 0; k < CPT; ++k)
      if (k < nvc) dh0[c0 + k] = av[0][k] * x[k];
  }
}

// ---------------------------------------------------------------------------
// fused SRU forward, [T, B, D]:
//   f = sigmoid(zf + bf[d]), r = sigmoid(zr + br[d]),
//   c_t = f c_{t-1} + (1 - f) zx,   h = r tanh(c) + (1 - r) zx
// IO is bf16 (raw uint16) or fp32; gates and state are fp32.
// ---------------------------------------------------------------------------
template <typename IO, int CPT>
struct IoRow;

template <int CPT>
struct IoRow<uint16_t, CPT> {
  uint16_t v[CPT];
  __device__ __forceinline__ void load(const uint16_t* p, int nvalid, bool vec) {
    load_row_bf16<CPT>(p, nvalid, vec, v);
  }
  __device__ __forceinline__ float get(int k) const { return bf16_to_f32(v[k]); }
  static __device__ __forceinline__ void store(uint16_t* p, int nvalid, bool vec,
                                               const float (&x)[CPT]) {
    store_row_bf16<CPT>(p, nvalid, vec, x);
  }
};

template <int CPT>
struct IoRow<float, CPT> {
  float v[CPT];
  __device__ __forceinline__ void load(const float* p, int nvalid, bool vec) {
    load_row<CPT>(p, nvalid, vec, 0.0f, v);
  }
  __device__ __forceinline__ float get(int k) const { return v[k]; }
  static __device__ __forceinline__ void store(float* p, int nvalid, bool vec,
                                               const float (&x)[CPT]) {
    store_row<CPT>(p, nvalid, vec, x);
  }
};

template <typename IO, int NW, int L, int CPT>
__global__ __launch_bounds__(NW* kWave) void k_sru_fwd(
    const IO* __restrict__ zf, const IO* __restrict__ zr, const IO* __restrict__ zx,
    const float* __restrict__ bias_f, const float* __restrict__ bias_r,
    const float* __restrict__ c0p, IO* __restrict__ h, float* __restrict__ c_last, int64_t T,
    int64_t C, int64_t D, int ncb, int ntb, int vec, uint64_t* __restrict__ status,
    unsigned* __restrict__ tickets) {
  constexpr int CW = kWave * CPT, TW = NW * L;
  __shared__ ColShared<NW, CPT> s;
  const bool multi = ntb > 1;
  const int cb = (int)(blockIdx.x % (unsigned)ncb);
  const int tb = col_ticket<NW, CPT>(multi, tickets, cb, s);
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const int64_t c0 = (int64_t)cb * CW + lane * CPT;
  const int nvc = clamp_valid(C - c0, CPT);
  const int64_t tw0 = (int64_t)tb * TW + (int64_t)wid * L;

  float bf[CPT], br[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const int64_t d = (k < nvc) ? (c0 + k) % D : 0;
    bf[k] = bias_f[d];
    br[k] = bias_r[d];
  }

  float av[L][CPT], bv[L][CPT];
  IoRow<IO, CPT> rr[L], xr[L];
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int nv = (tw0 + i < T) ? nvc : 0;
    const int64_t off = (tw0 + i) * C + c0;
    IoRow<IO, CPT> fr;
    fr.load(zf + off, nv, vec);
    rr[i].load(zr + off, nv, vec);
    xr[i].load(zx + off, nv, vec);
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const float f = sigmoid_fast(fr.get(k) + bf[k]);
      const float zxv = xr[i].get(k);
      const bool valid = k < nv;
      av[i][k] = valid ? f : 1.0f;
      bv[i][k] = valid ? __builtin_fmaf(-f, zxv, zxv) : 0.0f;  // (1 - f) * zx
    }
  }
  float A[CPT], B[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    A[k] = av[0][k];
    B[k] = bv[0][k];
#pragma unroll
    for (int i = 1; i < L; ++i) {
      B[k] = __builtin_fmaf(av[i][k], B[k], bv[i][k]);
      A[k] = A[k] * av[i][k];
    }
  }
  float PA[CPT], PB[CPT], TA[CPT], TB[CPT], x0[CPT], x[CPT];
  col_block_combine<NW, CPT>(A, B, s, PA, PB, TA, TB);
#pragma unroll
  for (int k = 0; k < CPT; ++k) x0[k] = (c0p && k < nvc) ? c0p[c0 + k] : 0.0f;
  col_chunk_carry<NW, CPT>(multi, tb, nvc, TA, TB, x0, status + (int64_t)cb * ntb * CW, s, x);
#pragma unroll
  for (int k = 0; k < CPT; ++k) x[k] = __builtin_fmaf(PA[k], x[k], PB[k]);
#pragma unroll
  for (int i = 0; i < L; ++i) {
    float out[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      x[k] = __builtin_fmaf(av[i][k], x[k], bv[i][k]);
      const float r = sigmoid_fast(rr[i].get(k) + br[k]);
      const float zxv = xr[i].get(k);
      out[k] = __builtin_fmaf(r, tanh_fast(x[k]) - zxv, zxv);  // r tanh(c) + (1 - r) zx
    }
    const int nv = (tw0 + i < T) ? nvc : 0;
    IoRow<IO, CPT>::store(h + (tw0 + i) * C + c0, nv, vec, out);
    if (c_last && tw0 + i == T - 1) {
#pragma unroll
      for (int k = 0; k < CPT; ++k)
        if (k < nvc) c_last[c0 + k] = x[k];
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
ColPlan plan_cols(int64_t C, int64_t T, int nw, int l, int cpt) {
  ColPlan p;
  p.nw = nw;
  p.l = l;
  p.cpt = cpt;
  const int64_t cw = (int64_t)kWave * cpt, tw = (int64_t)nw * l;
  p.ncb = (C + cw - 1) / cw;
  p.ntb = (T + tw - 1) / tw;
  if (p.ntb < 1) p.ntb = 1;
  return p;
}

int64_t col_status_words(const ColPlan& p) { return p.ntb > 1 ? p.ncb * p.ntb * kWave * p.cpt : 0; }

// fp32 scans: forward uses 8 waves x 8 steps x 4 channels per lane,
// backward 8 waves x 8 steps x 2 channels per lane (three input streams).
ColPlan plan_scan_fwd_tbd(int64_t C, int64_t T) { return plan_cols(C, T, 8, 8, 4); }
ColPlan plan_scan_bwd_tbd(int64_t C, int64_t T) { return plan_cols(C, T, 8, 8, 2); }
ColPlan plan_sru(int64_t C, int64_t T, int io_dtype) {
  return io_dtype == 1 ? plan_cols(C, T, 8, 8, 4) : plan_cols(C, T, 8, 8, 4);
}

hipError_t launch_scan_fwd_tbd(const float* a, const float* b, const float* h0, float* h,
                               int64_t C, int64_t T, const ColPlan& p, int vec, uint64_t* status,
                               unsigned* tickets, hipStream_t stream) {
  const uint64_t grid = (uint64_t)p.ncb * (uint64_t)p.ntb;
  hipLaunchKernelGGL((k_scan_fwd_tbd<8, 8, 4>), dim3((unsigned)grid), dim3(8 * kWave), 0, stream,
                     a, b, h0, h, T, C, (int)p.ncb, (int)p.ntb, vec, status, tickets);
  return hipGetLastError();
}

hipError_t launch_scan_bwd_tbd(const float* a, const float* h, const float* h0, const float* g,
                               float* da, float* db, float* dh0, int64_t C, int64_t T,
                               const ColPlan& p, int vec, uint64_t* status, unsigned* tickets,
                               hipStream_t stream) {
  const uint64_t grid = (uint64_t)p.ncb * (uint64_t)p.ntb;
  hipLaunchKernelGGL((k_scan_bwd_tbd<8, 8, 2>), dim3((unsigned)grid), dim3(8 * kWave), 0, stream,
                     a, h, h0, g, da, db, dh0, T, C, (int)p.ncb, (int)p.ntb, vec, status,
                     tickets);
  return hipGetLastError();
}

hipError_t launch_sru_fwd(const void* zf, const void* zr, const void* zx, const float* bias_f,
                          const float* bias_r, const float* c0, void* h, float* c_last, int64_t T,
                          int64_t B, int64_t D, int io_dtype, const ColPlan& p, int vec,
                          uint64_t* status, unsigned* tickets, hipStream_t stream) {
  const uint64_t grid = (uint64_t)p.ncb * (uint64_t)p.ntb;
  const int64_t C = B * D;
  if (io_dtype == 1) {
    hipLaunchKernelGGL((k_sru_fwd<uint16_t, 8, 8, 4>), dim3((unsigned)grid), dim3(8 * kWave), 0,
                       stream, (const uint16_t*)zf, (const uint16_t*)zr, (const uint16_t*)zx,
                       bias_f, bias_r, c0, (uint16_t*)h, c_last, T, C, D, (int)p.ncb, (int)p.ntb,
                       vec, status, tickets);
  } else {
    hipLaunchKernelGGL((k_sru_fwd<float, 8, 8, 4>), dim3((unsigned)grid), dim3(8 * kWave), 0,
                       stream, (const float*)zf, (const float*)zr, (const float*)zx, bias_f,
                       bias_r, c0, (float*)h, c_last, T, C, D, (int)p.ncb, (int)p.ntb, vec,
                       status, tickets);
  }
  return hipGetLastError();
}

}  // namespace lrs
