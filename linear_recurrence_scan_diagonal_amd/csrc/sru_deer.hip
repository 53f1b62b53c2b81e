// sru_deer.hip -- SRU layer whose forget gate reads the previous cell state,
// solved by DEER Newton iterations ([T, B, D] layout).
//
// Page "CUDA并行化RNN训练：从O(T)到O(log T)的工程实践与参数调优", SRU paragraph:
// the forget gate is f_t = sigmoid(W_f x_t + v_f (.) c_{t-1} + b_f).  With
// v_f != 0 the cell recurrence c_t = f_t c_{t-1} + (1 - f_t) z_x,t is
// element-wise nonlinear, so the linear scan alone cannot solve it.  The DEER
// page ("cuda-parallel-rnn-training-logt-optimization", core principle)
// solves such a recurrence by Newton's method on the whole sequence: with
// F(c) = f(c) (c - z_x) + z_x and its derivative (the Jacobian is diagonal)
//   J_t = f + (c_{t-1} - z_x) f (1 - f) v_f,
// one iteration from the iterate y is the linear recurrence
//   y'_t = J_t y'_{t-1} + F(y_{t-1}) - J_t y_{t-1},   y'_{-1} = c0,
// solved by the [T,B,D] scan tile (lrs_tbd.hpp), which also folds
// max |y' - y| into the iteration's norm slots.  The stop rule, the norm
// slots and the solve record are those of the tanh RNN solve (engineering
// section: ||y' - y|| < eps or K_max iterations).  k_sru_deer_out then forms
// h = r tanh(c) + (1 - r) z_x from the solution.
#include "lrs_tbd.hpp"

namespace lrs {

template <int NW>
struct DeltaShared {
  uint32_t wmax[NW];
};

// Start of iteration iter > 0: fold the norm of iteration iter - 1 (completed
// by the previous launch) from its slot set; workgroup 0 records it and clears
// the set the next iteration uses (the sets rotate over three iterations).
// True when that norm met the stop rule: the same decision in every workgroup.
template <int NW>
__device__ __forceinline__ bool sru_deer_prev_converged(uint32_t* __restrict__ delta_bits,
                                                        uint32_t* __restrict__ delta_out,
                                                        int iter, float eps,
                                                        DeltaShared<NW>& ds) {
  if (iter == 0) return false;
  constexpr int64_t kSet = kDeltaSlots * kDeltaStride;
  const int lane = threadIdx.x & (kWave - 1);
  if (threadIdx.x < kWave) {
    uint32_t v = delta_bits[((iter - 1) % 3) * kSet + lane * kDeltaStride];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const uint32_t o = (uint32_t)__shfl_xor((int)v, off, kWave);
      v = v > o ? v : o;
    }
    if (blockIdx.x == 0) {
      delta_bits[((iter + 1) % 3) * kSet + lane * kDeltaStride] = 0u;
      if (lane == 0) delta_out[iter - 1] = v;
    }
    if (lane == 0) ds.wmax[0] = v;
  }
  __syncthreads();
  const float prev_delta = as_f32(ds.wmax[0]);
  __syncthreads();
  return prev_delta < eps;
}

// End of an iteration: this workgroup's max |y' - y| (dmax, per lane) into its
// slot of the iteration's set.
template <int NW>
__device__ __forceinline__ void sru_deer_fold_norm(uint32_t dmax, uint32_t* __restrict__ delta_bits,
                                                   int iter, DeltaShared<NW>& ds) {
  constexpr int64_t kSet = kDeltaSlots * kDeltaStride;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)dmax, off, kWave);
    dmax = dmax > o ? dmax : o;
  }
  if (lane == 0) ds.wmax[wid] = dmax;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) m = ds.wmax[w] > m ? ds.wmax[w] : m;
    uint32_t* slot = delta_bits + (iter % 3) * kSet + (blockIdx.x % kDeltaSlots) * kDeltaStride;
    __hip_atomic_fetch_max(slot, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Forget gate of an SRU-by-DEER step, sigmoid(v_f c_{t-1} + z_f + b_f), as
// 1 / (1 + 2^(vs c_{t-1} + zq)) with vs = -log2(e) v_f and
// zq = -log2(e) (z_f + b_f) = fma(z_f, -log2 e, nbf), nbf = -log2(e) b_f: zq
// does not depend on the iterate, so a walk over several Newton iterations
// computes it once per element.
__device__ __forceinline__ float sd_zq(float zf, float nbf) {
  return __builtin_fmaf(zf, -kLog2e, nbf);
}
__device__ __forceinline__ float sd_gate(float vs, float prev, float zq) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(__builtin_fmaf(vs, prev, zq)));
}

template <typename IO, int NW, int L, int CPT, bool FULL, bool NT>
__device__ __forceinline__ void sru_deer_tile(const IO* __restrict__ zf, const IO* __restrict__ zx,
                                              const float* __restrict__ bias_f,
                                              const float* __restrict__ v_f,
                                              const float* __restrict__ c0p,
                                              const float* __restrict__ y, float* __restrict__ yn,
                                              int64_t T, int64_t C, int64_t D, int tb, int cb,
                                              bool multi, uint64_t* st, ColShared<NW, CPT>& s,
                                              uint32_t& dmax) {
  const ColPos q = col_pos<NW, L, CPT>(tb, cb, C);
  const int64_t cbase = (int64_t)cb * (kWave * CPT);
  float nbf[CPT], vf[CPT];
  {
    int64_t d = (q.nvc > 0) ? q.c0 % D : 0;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int64_t dk = (k < q.nvc) ? d : 0;
      nbf[k] = -kLog2e * bias_f[dk];
      vf[k] = v_f[dk];
      d = (d + 1 == D) ? 0 : d + 1;
    }
  }
  // the iterate just before this wave's steps (c0 before the first step; a
  // missing iterate is zero)
  float yp[CPT];
  if (q.row0 == 0) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) yp[k] = (c0p && k < q.nvc) ? c0p[q.c0 + k] : 0.0f;
  } else if (y && q.row0 <= T) {
    load_row<CPT, FULL, false>(y + (q.row0 - 1) * C + cbase, q.off, q.nvc, 0.0f, yp);
  } else {
#pragma unroll
    for (int k = 0; k < CPT; ++k) yp[k] = 0.0f;
  }
  // per step: J and the constant term F(y_{t-1}) - J y_{t-1} of the affine map
  float Jv[L][CPT], Bv[L][CPT], yo[L][CPT];
  {
    const IO* fp = zf + q.row0 * C + cbase;
    const IO* xp = zx + q.row0 * C + cbase;
    const float* yq = y ? y + q.row0 * C + cbase : nullptr;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int nv = (FULL || q.row0 + i < T) ? q.nvc : 0;
      IoRow<IO, CPT> fr, xr;
      fr.template load<FULL, NT>(fp, q.off, nv);
      xr.template load<FULL, NT>(xp, q.off, nv);
      if (yq) {
        load_row<CPT, FULL, NT>(yq, q.off, nv, 0.0f, yo[i]);
        yq += C;
      } else {
#pragma unroll
        for (int k = 0; k < CPT; ++k) yo[i][k] = 0.0f;
      }
      fp += C;
      xp += C;
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        const float prev = (i > 0) ? yo[i - 1][k] : yp[k];
        if (FULL || k < nv) {
          const float f = sd_gate(-kLog2e * vf[k], prev, sd_zq(fr.get(k), nbf[k]));
          const float dx = prev - xr.get(k);
          const float F = __builtin_fmaf(f, dx, xr.get(k));
          const float J = __builtin_fmaf(dx * (f - f * f), vf[k], f);
          Jv[i][k] = J;
          Bv[i][k] = __builtin_fmaf(-J, prev, F);
        } else {  // identity map past the end
          Jv[i][k] = 1.0f;
          Bv[i][k] = 0.0f;
        }
      }
    }
  }
  float A[CPT], B[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    A[k] = Jv[0][k];
    B[k] = Bv[0][k];
#pragma unroll
    for (int i = 1; i < L; ++i) {
      B[k] = __builtin_fmaf(Jv[i][k], B[k], Bv[i][k]);
      A[k] = A[k] * Jv[i][k];
    }
  }
  float x0[CPT], x[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) x0[k] = (c0p && k < q.nvc) ? c0p[q.c0 + k] : 0.0f;
  col_enter_state<NW, CPT>(A, B, multi, tb, x0, c0p, cbase, clamp_valid(C - cbase, kWave * CPT),
                           st, s, x);
  float* op = yn + q.row0 * C + cbase;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const bool row_ok = FULL || q.row0 + i < T;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      x[k] = __builtin_fmaf(Jv[i][k], x[k], Bv[i][k]);
      const uint32_t d = as_u32(fabsf(x[k] - yo[i][k]));
      if (FULL || (row_ok && k < q.nvc)) dmax = d > dmax ? d : dmax;
    }
    store_row<CPT, FULL, NT>(op, q.off, row_ok ? q.nvc : 0, x);
    op += C;
  }
}

// One Newton iteration.  Iteration iter > 0 first folds the norm of
// iteration iter - 1 (completed by the previous launch) and exits when it met
// the stop rule; workgroup 0 records that norm and clears the slot set the next
// iteration uses.  The slot sets rotate over three iterations.
template <typename IO, int NW, int L, int CPT, bool NT>
__global__ __launch_bounds__(NW* kWave) void k_sru_deer_iter(
    const IO* __restrict__ zf, const IO* __restrict__ zx, const float* __restrict__ bias_f,
    const float* __restrict__ v_f, const float* __restrict__ c0p, const float* __restrict__ y,
    float* __restrict__ yn, int64_t T, int64_t C, int64_t D, int ncb, int ntb, int vec,
    uint64_t* __restrict__ status, unsigned* __restrict__ tickets,
    uint32_t* __restrict__ delta_bits, uint32_t* __restrict__ delta_out, int iter, float eps) {
  constexpr int CW = kWave * CPT, TW = NW * L;
  __shared__ ColShared<NW, CPT> s;
  __shared__ DeltaShared<NW> ds;
  if (sru_deer_prev_converged<NW>(delta_bits, delta_out, iter, eps, ds)) return;
  const bool multi = ntb > 1;
  const int cb = (int)(blockIdx.x % (unsigned)ncb);
  const int tb = col_ticket<NW, CPT>(multi, tickets, cb, s);
  uint64_t* st = status + (int64_t)cb * ntb * CW;
  const bool full = vec && ((int64_t)(tb + 1) * TW <= T) && ((int64_t)(cb + 1) * CW <= C);
  uint32_t dmax = 0;
  if (full)
    sru_deer_tile<IO, NW, L, CPT, true, NT>(zf, zx, bias_f, v_f, c0p, y, yn, T, C, D, tb, cb,
                                            multi, st, s, dmax);
  else
    sru_deer_tile<IO, NW, L, CPT, false, NT>(zf, zx, bias_f, v_f, c0p, y, yn, T, C, D, tb, cb,
                                             multi, st, s, dmax);
  sru_deer_fold_norm<NW>(dmax, delta_bits, iter, ds);
}

// ---------------------------------------------------------------------------
// Persistent form of the iteration, used when the channel blocks alone fill the
// GPU: one workgroup per channel block walks every time tile in order with the
// state entering the tile in LDS, loading the next tile's rows while it
// processes the current one.  No look-back state, so no reset kernel between
// iterations.  Same per-step map and norm as sru_deer_tile.
// ---------------------------------------------------------------------------
template <typename IO, int L, int CPT>
struct SdRows {
  IoRow<IO, CPT> f[L], x[L];
  float y[L][CPT];  // the iterate at the rows
  float yp[CPT];    // the iterate just before the first row (c0 before step 0)
};

template <typename IO, int L, int CPT, bool FULL, bool NT>
__device__ __forceinline__ void sru_deer_persist_load(
    const IO* __restrict__ zf, const IO* __restrict__ zx, const float* __restrict__ c0p,
    const float* __restrict__ y, int64_t row0, int64_t T, int64_t C, int64_t cbase, uint32_t off,
    int nvc, SdRows<IO, L, CPT>& w) {
  const IO* fp = zf + row0 * C + cbase;
  const IO* xp = zx + row0 * C + cbase;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int nv = (FULL || row0 + i < T) ? nvc : 0;
    w.f[i].template load<FULL, NT>(fp, off, nv);
    w.x[i].template load<FULL, NT>(xp, off, nv);
    if (y) {
      load_row<CPT, FULL, NT>(y + (row0 + i) * C + cbase, off, nv, 0.0f, w.y[i]);
    } else {
#pragma unroll
      for (int k = 0; k < CPT; ++k) w.y[i][k] = 0.0f;
    }
    fp += C;
    xp += C;
  }
  if (row0 == 0) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) w.yp[k] = (c0p && k < nvc) ? c0p[cbase + off + k] : 0.0f;
  } else if (y && row0 <= T) {
    load_row<CPT, false, false>(y + (row0 - 1) * C + cbase, off, nvc, 0.0f, w.yp);
  } else {
#pragma unroll
    for (int k = 0; k < CPT; ++k) w.yp[k] = 0.0f;
  }
}

// One tile of the walk (PF as in the persistent SRU forward: 0 no prefetch,
// 1 full rows, 2 predicated rows of the next tile; FULL: no predication).
template <typename IO, int NW, int L, int CPT, bool FULL, int PF, bool NT>
__device__ __forceinline__ void sru_deer_persist_tile(
    const IO* __restrict__ zf, const IO* __restrict__ zx, const float* __restrict__ c0p,
    const float* __restrict__ y, float* __restrict__ yn, int64_t row0, int64_t T, int64_t C,
    int64_t cbase, uint32_t off, int nvc, const float (&nbf)[CPT], const float (&vf)[CPT],
    SdRows<IO, L, CPT>& w, PersistShared<NW, CPT>& s, int wid, int par, uint32_t& dmax) {
  constexpr int TW = NW * L;
  float Jv[L][CPT], Bv[L][CPT], yo[L][CPT];
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const bool row_ok = FULL || row0 + i < T;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const float prev = (i > 0) ? w.y[i - 1][k] : w.yp[k];
      yo[i][k] = w.y[i][k];
      if (FULL || (row_ok && k < nvc)) {
        const float xv = w.x[i].get(k);
        const float f = sd_gate(-kLog2e * vf[k], prev, sd_zq(w.f[i].get(k), nbf[k]));
        const float dx = prev - xv;
        const float F = __builtin_fmaf(f, dx, xv);
        const float J = __builtin_fmaf(dx * (f - f * f), vf[k], f);
        Jv[i][k] = J;
        Bv[i][k] = __builtin_fmaf(-J, prev, F);
      } else {  // identity map past the end
        Jv[i][k] = 1.0f;
        Bv[i][k] = 0.0f;
      }
    }
  }
  if (PF == 1)
    sru_deer_persist_load<IO, L, CPT, true, NT>(zf, zx, c0p, y, row0 + TW, T, C, cbase, off, nvc,
                                                w);
  else if (PF == 2)
    sru_deer_persist_load<IO, L, CPT, false, NT>(zf, zx, c0p, y, row0 + TW, T, C, cbase, off, nvc,
                                                 w);
  float A[CPT], B[CPT], x[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    A[k] = Jv[0][k];
    B[k] = Bv[0][k];
#pragma unroll
    for (int i = 1; i < L; ++i) {
      B[k] = __builtin_fmaf(Jv[i][k], B[k], Bv[i][k]);
      A[k] = A[k] * Jv[i][k];
    }
  }
  persist_enter<NW, CPT>(A, B, s, wid, off, x, par);
  float* op = yn + row0 * C + cbase;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const bool row_ok = FULL || row0 + i < T;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      x[k] = __builtin_fmaf(Jv[i][k], x[k], Bv[i][k]);
      const uint32_t d = as_u32(fabsf(x[k] - yo[i][k]));
      if (FULL || (row_ok && k < nvc)) dmax = d > dmax ? d : dmax;
    }
    store_row<CPT, FULL, NT>(op, off, row_ok ? nvc : 0, x);
    op += C;
  }
  persist_advance<NW, CPT>(x, s, wid, off, par);
}

template <typename IO, int NW, int L, int CPT, bool NT>
__global__ __launch_bounds__(NW* kWave) void k_sru_deer_iter_persist(
    const IO* __restrict__ zf, const IO* __restrict__ zx, const float* __restrict__ bias_f,
    const float* __restrict__ v_f, const float* __restrict__ c0p, const float* __restrict__ y,
    float* __restrict__ yn, int64_t T, int64_t C, int64_t D, int vec,
    uint32_t* __restrict__ delta_bits, uint32_t* __restrict__ delta_out, int iter, float eps) {
  constexpr int CW = kWave * CPT, TW = NW * L;
  __shared__ PersistShared<NW, CPT> s;
  __shared__ DeltaShared<NW> ds;
  if (sru_deer_prev_converged<NW>(delta_bits, delta_out, iter, eps, ds)) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t cbase = (int64_t)blockIdx.x * CW;
  const uint32_t off = (uint32_t)(lane * CPT);
  const int64_t c0i = cbase + off;
  const int nvc = clamp_valid(C - c0i, CPT);
  const bool cfull = vec && cbase + CW <= C;
  float nbf[CPT], vf[CPT];
  {
    int64_t d = (nvc > 0) ? c0i % D : 0;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int64_t dk = (k < nvc) ? d : 0;
      nbf[k] = -kLog2e * bias_f[dk];
      vf[k] = v_f[dk];
      d = (d + 1 == D) ? 0 : d + 1;
    }
  }
  for (int j = threadIdx.x; j < CW; j += NW * kWave)
    s.carry[0][j] = (c0p && cbase + j < C) ? c0p[cbase + j] : 0.0f;
  const int64_t ntb = (T + TW - 1) / TW, nfull = T / TW;
  const int64_t w0 = (int64_t)wid * L;
  uint32_t dmax = 0;
  SdRows<IO, L, CPT> w;
#define LRS_SDT(FULLT, PFT, TB)                                                                  \
  sru_deer_persist_tile<IO, NW, L, CPT, FULLT, PFT, NT>(zf, zx, c0p, y, yn, (TB) * TW + w0, T, C, \
                                                        cbase, off, nvc, nbf, vf, w, s, wid,      \
                                                        (int)((TB) & 1), dmax)
  if (cfull && nfull > 0) {
    // full tiles in a straight loop (each loads the next full tile), then the
    // last full tile and the ragged tail, if any
    sru_deer_persist_load<IO, L, CPT, true, NT>(zf, zx, c0p, y, w0, T, C, cbase, off, nvc, w);
    for (int64_t tb = 0; tb + 1 < nfull; ++tb) LRS_SDT(true, 1, tb);
    if (ntb > nfull) {
      LRS_SDT(true, 2, nfull - 1);
      LRS_SDT(false, 0, nfull);
    } else {
      LRS_SDT(true, 0, nfull - 1);
    }
  } else {
    sru_deer_persist_load<IO, L, CPT, false, NT>(zf, zx, c0p, y, w0, T, C, cbase, off, nvc, w);
    for (int64_t tb = 0; tb < ntb; ++tb) {
      if (tb + 1 < ntb) LRS_SDT(false, 2, tb);
      else LRS_SDT(false, 0, tb);
    }
  }
#undef LRS_SDT
  sru_deer_fold_norm<NW>(dmax, delta_bits, iter, ds);
}

// ---------------------------------------------------------------------------
// SRU-by-DEER with the Newton iterations fused into the persistent walk (as
// k_deer_fused does for the tanh RNN): one workgroup per channel block visits
// the time tiles in order and, for each tile, loads z_f, z_x and the starting
// iterate once and computes iterates 1..m, each from the previous one in
// registers.  Iteration k's per-channel state entering the tile sits in LDS
// (ck, two copies that alternate by tile); c_{k-1} at the step before a wave's
// first row is iteration k-1's state entering that wave (for k = 1: the
// starting iterate, from memory inside the tile and from y0c across tiles).
// The wave maps alternate by iteration parity, so each iteration needs one
// barrier, and each tile one more at its end.  Same per-step map and norm as
// sru_deer_persist_tile; only the last iterate is stored.  Pass (sets) and
// redo (rec) forms as in k_deer_fused.
// ---------------------------------------------------------------------------
template <int NW, int CPT>
struct SdFusedShared {
  float A[2][NW][kWave * CPT];                // wave maps, by level parity
  float B[2][NW][kWave * CPT];
  float y0c[kWave * CPT];                     // starting iterate at the last row before the tile
  float ck[2][kDeerFuseMax][kWave * CPT];     // [tile parity][lev - 1]: state entering the tile
  uint32_t dlane[kDeerFuseMax][NW * kWave];  // per-thread max |c_lev - c_{lev-1}|
  uint32_t dm[kDeerFuseMax][NW];             // per-wave max, folded after the walk
};

// Newton iteration lev over one tile of the fused walk: the iterate c_lev
// (yout) from c_{lev-1} (yin) in registers; ent holds c_{lev-1} at the step
// before this wave's first row on entry and c_lev there on exit.  zq and xv:
// the tile's gate inputs (sd_zq) and z_x, unpacked once.  The update norm
// folds |c_lev - c_{lev-1}| into the thread's slot of s.dlane[lev - 1] with
// the NaN-propagating maximum (v_maximum3_f32):
// a non-finite step still reads as the largest update, since the bits of a
// non-negative float or a NaN order as unsigned integers.
template <int NW, int L, int CPT, bool FULL>
__device__ __forceinline__ void sru_deer_fused_level(
    int lev, const float (&zq)[L][CPT], const float (&xv)[L][CPT], const float (&yin)[L][CPT],
    float (&yout)[L][CPT], float (&ent)[CPT], int64_t row0, int64_t T, uint32_t off, int nvc,
    const float (&vf)[CPT], bool keep_start, int tpar, SdFusedShared<NW, CPT>& s, int wid) {
  const int lp = lev & 1;
  float Jv[L][CPT], Bv[L][CPT];
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const bool row_ok = FULL || row0 + i < T;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const float prev = (i > 0) ? yin[i - 1][k] : ent[k];
      if (FULL || (row_ok && k < nvc)) {
        const float f = sd_gate(-kLog2e * vf[k], prev, zq[i][k]);
        const float dx = prev - xv[i][k];
        const float F = __builtin_fmaf(f, dx, xv[i][k]);
        const float J = __builtin_fmaf(dx * (f - f * f), vf[k], f);
        Jv[i][k] = J;
        Bv[i][k] = __builtin_fmaf(-J, prev, F);
      } else {  // identity map past the end
        Jv[i][k] = 1.0f;
        Bv[i][k] = 0.0f;
      }
    }
  }
  float A[CPT], B[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    A[k] = Jv[0][k];
    B[k] = Bv[0][k];
#pragma unroll
    for (int i = 1; i < L; ++i) {
      B[k] = __builtin_fmaf(Jv[i][k], B[k], Bv[i][k]);
      A[k] = A[k] * Jv[i][k];
    }
  }
  // the earlier waves' maps applied in order to iteration lev's state entering the tile
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    s.A[lp][wid][off + k] = A[k];
    s.B[lp][wid][off + k] = B[k];
  }
  __syncthreads();
  float x[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    float xk = s.ck[tpar][lev - 1][off + k];
#pragma unroll
    for (int w = 0; w < NW - 1; ++w)
      if (w < wid) xk = __builtin_fmaf(s.A[lp][w][off + k], xk, s.B[lp][w][off + k]);
    x[k] = xk;
  }
  // every wave has read y0c (before the barrier above): the last wave now
  // keeps the starting iterate at the tile's last row for the next tile
  if (keep_start && wid == NW - 1) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) s.y0c[off + k] = yin[L - 1][k];
  }
  float dmf = 0.0f;
#pragma unroll
  for (int k = 0; k < CPT; ++k) ent[k] = x[k];  // c_lev before this wave's first row
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const bool row_ok = FULL || row0 + i < T;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      x[k] = __builtin_fmaf(Jv[i][k], x[k], Bv[i][k]);
      const float d = __builtin_elementwise_maximum(dmf, fabsf(x[k] - yin[i][k]));
      dmf = (FULL || (row_ok && k < nvc)) ? d : dmf;
      yout[i][k] = x[k];
    }
  }
  __hip_atomic_fetch_max(&s.dlane[lev - 1][threadIdx.x], as_u32(dmf), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_WORKGROUP);
  // the state after the tile goes to the other tile-parity slot, which no wave
  // reads before the barrier that ends this tile; the maps of level lev + 2
  // (same parity) are written after every wave has passed level lev + 1's
  // barrier, so after it has read these
  if (wid == NW - 1) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) s.ck[tpar ^ 1][lev - 1][off + k] = x[k];
  }
}

template <typename IO, int NW, int L, int CPT, bool FULL, bool NT>
__device__ __forceinline__ void sru_deer_fused_tile(
    const IO* __restrict__ zf, const IO* __restrict__ zx, const float* __restrict__ c0p,
    const float* __restrict__ y0, float* __restrict__ out, int64_t row0, int64_t T, int64_t C,
    int64_t cbase, uint32_t off, int nvc, int m, const float (&nbf)[CPT], const float (&vf)[CPT],
    int tpar, SdFusedShared<NW, CPT>& s, int wid) {
  float zq[L][CPT], xv[L][CPT], ya[L][CPT], yb[L][CPT];
  {
    const IO* fp = zf + row0 * C + cbase;
    const IO* xp = zx + row0 * C + cbase;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int nv = (FULL || row0 + i < T) ? nvc : 0;
      IoRow<IO, CPT> fr, xr;
      fr.template load<FULL, NT>(fp, off, nv);
      xr.template load<FULL, NT>(xp, off, nv);
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        zq[i][k] = sd_zq(fr.get(k), nbf[k]);
        xv[i][k] = xr.get(k);
      }
      if (y0) {
        load_row<CPT, FULL, NT>(y0 + (row0 + i) * C + cbase, off, nv, 0.0f, ya[i]);
      } else {
#pragma unroll
        for (int k = 0; k < CPT; ++k) ya[i][k] = 0.0f;
      }
      fp += C;
      xp += C;
    }
  }
  // starting iterate at the step before this wave's first row
  float ent[CPT];
  if (row0 == 0) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) ent[k] = (c0p && k < nvc) ? c0p[cbase + off + k] : 0.0f;
  } else if (!y0) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) ent[k] = 0.0f;
  } else if (wid == 0) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) ent[k] = s.y0c[off + k];
  } else if (row0 <= T) {  // inside the tile: not yet overwritten, even in place
    load_row<CPT, false, false>(y0 + (row0 - 1) * C + cbase, off, nvc, 0.0f, ent);
  } else {  // a wave wholly past the end (its rows are not stored)
#pragma unroll
    for (int k = 0; k < CPT; ++k) ent[k] = 0.0f;
  }
  // iterates alternate between the two register sets
  const bool keep = y0 != nullptr;
  int lev = 1;
#pragma unroll 1
  for (; lev + 1 <= m; lev += 2) {
    sru_deer_fused_level<NW, L, CPT, FULL>(lev, zq, xv, ya, yb, ent, row0, T, off, nvc, vf,
                                           keep && lev == 1, tpar, s, wid);
    sru_deer_fused_level<NW, L, CPT, FULL>(lev + 1, zq, xv, yb, ya, ent, row0, T, off, nvc, vf,
                                           false, tpar, s, wid);
  }
  if (lev <= m) {
    sru_deer_fused_level<NW, L, CPT, FULL>(lev, zq, xv, ya, yb, ent, row0, T, off, nvc, vf,
                                           keep && lev == 1, tpar, s, wid);
#pragma unroll
    for (int i = 0; i < L; ++i)
#pragma unroll
      for (int k = 0; k < CPT; ++k) ya[i][k] = yb[i][k];
  }
  float* op = out + row0 * C + cbase;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    store_row<CPT, FULL, NT>(op, off, (FULL || row0 + i < T) ? nvc : 0, ya[i]);
    op += C;
  }
  // the next tile reads y0c and this tile's states after the tile, and
  // rewrites the wave maps of level 1
  __syncthreads();
}

template <typename IO, int NW, int L, int CPT, bool NT>
__device__ __forceinline__ void sru_deer_fused_body(
    const IO* __restrict__ zf, const IO* __restrict__ zx, const float* __restrict__ bias_f,
    const float* __restrict__ v_f, const float* __restrict__ c0p, const float* __restrict__ y0,
    float* __restrict__ out, int64_t T, int64_t C, int64_t D, int vec, int k_max,
    uint32_t* __restrict__ sets, const int* __restrict__ rec, bool redo,
    SdFusedShared<NW, CPT>& s) {
  constexpr int CW = kWave * CPT, TW = NW * L;
  int m = k_max;
  if (redo) {
    m = rec[0];
    if (m < 1 || m >= k_max) return;  // the pass already holds the answer
  }
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t cbase = (int64_t)blockIdx.x * CW;
  const uint32_t off = (uint32_t)(lane * CPT);
  const int64_t c0i = cbase + off;
  const int nvc = clamp_valid(C - c0i, CPT);
  const bool cfull = vec && cbase + CW <= C;
  float nbf[CPT], vf[CPT];
  {
    int64_t d = (nvc > 0) ? c0i % D : 0;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int64_t dk = (k < nvc) ? d : 0;
      nbf[k] = -kLog2e * bias_f[dk];
      vf[k] = v_f[dk];
      d = (d + 1 == D) ? 0 : d + 1;
    }
  }
  for (int j = threadIdx.x; j < (kDeerFuseMax + 1) * CW; j += NW * kWave) {
    const int c = j % CW, lv = j / CW;
    const float v = (c0p && cbase + c < C) ? c0p[cbase + c] : 0.0f;  // every level starts at c0
    if (lv == 0) s.y0c[c] = v;
    else s.ck[0][lv - 1][c] = v;
  }
#pragma unroll
  for (int j = 0; j < kDeerFuseMax; ++j) s.dlane[j][threadIdx.x] = 0u;
  __syncthreads();
  const int64_t ntb = (T + TW - 1) / TW, nfull = T / TW;
  const int64_t w0 = (int64_t)wid * L;
#pragma unroll 1
  for (int64_t tb = 0; tb < ntb; ++tb) {
    const int tpar = (int)(tb & 1);
    if (cfull && tb < nfull)
      sru_deer_fused_tile<IO, NW, L, CPT, true, NT>(zf, zx, c0p, y0, out, tb * TW + w0, T, C,
                                                    cbase, off, nvc, m, nbf, vf, tpar, s, wid);
    else
      sru_deer_fused_tile<IO, NW, L, CPT, false, NT>(zf, zx, c0p, y0, out, tb * TW + w0, T, C,
                                                     cbase, off, nvc, m, nbf, vf, tpar, s, wid);
  }
  if (redo) return;
  __syncthreads();
  // the wave maxima of each level's slots, then the block's
#pragma unroll 1
  for (int k = 0; k < m; ++k) {
    const uint32_t v = wave_max_u32(s.dlane[k][threadIdx.x]);
    if (lane == 0) s.dm[k][wid] = v;
  }
  __syncthreads();
  if (threadIdx.x < (unsigned)m) {
    const int k = threadIdx.x;
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) v = s.dm[k][i] > v ? s.dm[k][i] : v;
    uint32_t* slot = sets + (int64_t)k * (kDeltaSlots * kDeltaStride) +
                     (blockIdx.x % kDeltaSlots) * kDeltaStride;
    __hip_atomic_fetch_max(slot, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <typename IO, int NW, int L, int CPT, bool NT>
__global__ __launch_bounds__(NW* kWave) void k_sru_deer_fused(
    const IO* __restrict__ zf, const IO* __restrict__ zx, const float* __restrict__ bias_f,
    const float* __restrict__ v_f, const float* __restrict__ c0p, const float* __restrict__ y0,
    float* __restrict__ out, int64_t T, int64_t C, int64_t D, int vec, int k_max,
    uint32_t* __restrict__ sets) {
  __shared__ SdFusedShared<NW, CPT> s;
  sru_deer_fused_body<IO, NW, L, CPT, NT>(zf, zx, bias_f, v_f, c0p, y0, out, T, C, D, vec, k_max,
                                          sets, nullptr, false, s);
}

template <typename IO, int NW, int L, int CPT, bool NT>
__global__ __launch_bounds__(NW* kWave) void k_sru_deer_redo(
    const IO* __restrict__ zf, const IO* __restrict__ zx, const float* __restrict__ bias_f,
    const float* __restrict__ v_f, const float* __restrict__ c0p, const float* __restrict__ y0,
    float* __restrict__ out, int64_t T, int64_t C, int64_t D, int vec, int k_max,
    const int* __restrict__ rec) {
  __shared__ SdFusedShared<NW, CPT> s;
  sru_deer_fused_body<IO, NW, L, CPT, NT>(zf, zx, bias_f, v_f, c0p, y0, out, T, C, D, vec, k_max,
                                          nullptr, rec, true, s);
}

// h = r tanh(c) + (1 - r) z_x with r = sigmoid(z_r + b_r), and c_T, from the
// solved cell states.  Each thread takes groups of 4 consecutive elements
// (16-byte state loads, 8- or 16-byte I/O loads) when VEC, else single
// elements; grid-stride.
template <typename IO>
__device__ __forceinline__ float io_get(const IO* p, int64_t i) {
  if constexpr (sizeof(IO) == 2) return as_f32((uint32_t)p[i] << 16);
  else return p[i];
}

template <typename IO, bool VEC, bool NT>
__global__ __launch_bounds__(256) void k_sru_deer_out(const IO* __restrict__ zr,
                                                      const IO* __restrict__ zx,
                                                      const float* __restrict__ bias_r,
                                                      const float* __restrict__ c,
                                                      IO* __restrict__ h,
                                                      float* __restrict__ c_last, int64_t N,
                                                      int64_t C, int64_t D) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (VEC) {
    // feature index of the group's first element, advanced by the stride
    // without a division per group
    const int64_t dstep = (4 * stride) % D;
    int64_t d0 = (4 * tid) % D;
    for (int64_t j = tid; j < N / 4; j += stride) {
      const int64_t i = 4 * j;
      float r4[4], x4[4];
      if constexpr (sizeof(IO) == 2) {
        const u32x2_t rw = ldv<NT>(reinterpret_cast<const u32x2_t*>(zr + i));
        const u32x2_t xw = ldv<NT>(reinterpret_cast<const u32x2_t*>(zx + i));
        r4[0] = bf16_lo(rw.x); r4[1] = bf16_hi(rw.x); r4[2] = bf16_lo(rw.y); r4[3] = bf16_hi(rw.y);
        x4[0] = bf16_lo(xw.x); x4[1] = bf16_hi(xw.x); x4[2] = bf16_lo(xw.y); x4[3] = bf16_hi(xw.y);
      } else {
        const f32x4_t rv = ldv<NT>(reinterpret_cast<const f32x4_t*>(zr + i));
        const f32x4_t xv = ldv<NT>(reinterpret_cast<const f32x4_t*>(zx + i));
        r4[0] = rv.x; r4[1] = rv.y; r4[2] = rv.z; r4[3] = rv.w;
        x4[0] = xv.x; x4[1] = xv.y; x4[2] = xv.z; x4[3] = xv.w;
      }
      const f32x4_t cv = ldv<NT>(reinterpret_cast<const f32x4_t*>(c + i));
      const float c4[4] = {cv.x, cv.y, cv.z, cv.w};
      float o[4];
      int64_t d = d0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float r = fast_sigmoid(r4[k], -kLog2e * bias_r[d]);
        o[k] = __builtin_fmaf(r, fast_tanh(c4[k]) - x4[k], x4[k]);
        d = (d + 1 == D) ? 0 : d + 1;
      }
      IoRow<IO, 4>::template store<true, NT>(h + i, 0, 4, o);
      if (c_last && i >= N - C) {
#pragma unroll
        for (int k = 0; k < 4; ++k) c_last[i + k - (N - C)] = c4[k];
      }
      d0 += dstep;
      if (d0 >= D) d0 -= D;
    }
  } else {
    for (int64_t i = tid; i < N; i += stride) {
      const float zxv = io_get(zx, i);
      const float r = fast_sigmoid(io_get(zr, i), -kLog2e * bias_r[i % D]);
      const float ci = c[i];
      float o[1] = {__builtin_fmaf(r, fast_tanh(ci) - zxv, zxv)};
      if constexpr (sizeof(IO) == 2) {
        h[i] = (uint16_t)(pack_bf16x2(o[0], 0.0f) & 0xFFFFu);
      } else {
        h[i] = o[0];
      }
      if (c_last && i >= N - C) c_last[i - (N - C)] = ci;
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
namespace {
constexpr int kSdNW = 8, kSdL = 8, kSdCPT = 2;
// persistent walk: 16 steps per lane for bf16 I/O (229 VGPRs), 8 for fp32
constexpr int kSdPNW = 8, kSdPL16 = 16, kSdPL32 = 8, kSdPCPT = 2;
}

ColPlan plan_sru_deer(int64_t C, int64_t T, int io_dtype, bool allow_persist, const Opts& o) {
  ColPlan p = plan_cols(C, T, kSdNW, kSdL, kSdCPT);
  if (allow_persist && p.ncb >= persist_min_blocks(o)) {  // the channel blocks alone fill the GPU
    p = plan_cols(C, T, kSdPNW, io_dtype == 1 ? kSdPL16 : kSdPL32, kSdPCPT);
    p.persist = true;
  }
  // z_f, z_x (io type), the iterate and the next iterate
  p.stream = C * T * (2 * (io_dtype == 1 ? 2 : 4) + 8) >= kStreamFootprint;
  return p;
}

hipError_t launch_sru_deer_iter(const void* zf, const void* zx, const float* bias_f,
                                const float* v_f, const float* c0, const float* y, float* yn,
                                int64_t T, int64_t C, int64_t D, int io_dtype, const ColPlan& p,
                                int vec, uint64_t* status, unsigned* tickets,
                                uint32_t* delta_bits, uint32_t* delta_out, int iter, float eps,
                                hipStream_t stream) {
  if (p.persist) {
#define LRS_SDP(IO, L, NTF)                                                                    \
  hipLaunchKernelGGL((k_sru_deer_iter_persist<IO, kSdPNW, L, kSdPCPT, NTF>),                   \
                     dim3((unsigned)p.ncb), dim3(kSdPNW * kWave), 0, stream, (const IO*)zf,     \
                     (const IO*)zx, bias_f, v_f, c0, y, yn, T, C, D, vec, delta_bits,           \
                     delta_out, iter, eps)
    if (io_dtype == 1) {
      if (p.stream) LRS_SDP(uint16_t, kSdPL16, true);
      else LRS_SDP(uint16_t, kSdPL16, false);
    } else {
      if (p.stream) LRS_SDP(float, kSdPL32, true);
      else LRS_SDP(float, kSdPL32, false);
    }
#undef LRS_SDP
    return hipGetLastError();
  }
  const uint64_t grid = (uint64_t)p.ncb * (uint64_t)p.ntb;
#define LRS_SD(IO, NTF)                                                                        \
  hipLaunchKernelGGL((k_sru_deer_iter<IO, kSdNW, kSdL, kSdCPT, NTF>), dim3((unsigned)grid),   \
                     dim3(kSdNW * kWave), 0, stream, (const IO*)zf, (const IO*)zx, bias_f, v_f, \
                     c0, y, yn, T, C, D, (int)p.ncb, (int)p.ntb, vec, status, tickets,          \
                     delta_bits, delta_out, iter, eps)
  if (io_dtype == 1) {
    if (p.stream) LRS_SD(uint16_t, true);
    else LRS_SD(uint16_t, false);
  } else {
    if (p.stream) LRS_SD(float, true);
    else LRS_SD(float, false);
  }
#undef LRS_SD
  return hipGetLastError();
}

// Tile of the fused SRU-by-DEER walk: 8 waves x kSdFL rows x kSdFCPT channels
// per lane, one workgroup per block of 64 kSdFCPT channels walking all of T.
// Solve time at B=32 D=1024 T=2048 (bf16, with the output kernel), 2 channels
// per lane: 16 rows 442 us, 8 rows 520, 4 rows 682, 2 rows 1036 (192-199 VGPRs
// at 16 rows; 256 workgroups of 8 waves leave 2 waves per SIMD, VALU busy
// 64%).  One channel per lane: 102 VGPRs, 512 workgroups, 4 waves per SIMD,
// 396 instead of 435 us.
constexpr int kSdFL = 16, kSdFCPT = 1;

hipError_t launch_sru_deer_fused(const void* zf, const void* zx, const float* bias_f,
                                 const float* v_f, const float* c0, const float* c_init,
                                 float* out, float* c_states, int64_t T, int64_t C, int64_t D,
                                 int io_dtype, const ColPlan& p, int vec, int k_max, float eps,
                                 uint32_t* sets, uint32_t* delta_out, int* rec,
                                 hipStream_t stream) {
  const dim3 grid((unsigned)((C + kWave * kSdFCPT - 1) / (kWave * kSdFCPT)));
#define LRS_SDF(KER, IO, NTF, OUT, LAST)                                                        \
  hipLaunchKernelGGL((KER<IO, kSdPNW, kSdFL, kSdFCPT, NTF>), grid, dim3(kSdPNW * kWave), 0,    \
                     stream, (const IO*)zf, (const IO*)zx, bias_f, v_f, c0, c_init, OUT, T, C, D, \
                     vec, k_max, LAST)
#define LRS_SDF_IO(KER, OUT, LAST)                                        \
  if (io_dtype == 1) {                                                    \
    if (p.stream) LRS_SDF(KER, uint16_t, true, OUT, LAST);                \
    else LRS_SDF(KER, uint16_t, false, OUT, LAST);                        \
  } else {                                                                \
    if (p.stream) LRS_SDF(KER, float, true, OUT, LAST);                   \
    else LRS_SDF(KER, float, false, OUT, LAST);                           \
  }
  LRS_SDF_IO(k_sru_deer_fused, out, sets)
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = launch_deer_fused_finish(sets, delta_out, rec, k_max, eps, stream)) != hipSuccess)
    return e;
  LRS_SDF_IO(k_sru_deer_redo, c_states, (const int*)rec)
#undef LRS_SDF_IO
#undef LRS_SDF
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return launch_deer_fused_select(out, c_states, C * T, rec, k_max, stream);
}

hipError_t launch_sru_deer_out(const void* zr, const void* zx, const float* bias_r,
                               const float* c, void* h, float* c_last, int64_t N, int64_t C,
                               int64_t D, int io_dtype, int vec, hipStream_t stream) {
  int64_t blocks = ((vec ? N / 4 : N) + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  if (blocks < 1) blocks = 1;
  // z_r, z_x, h in the I/O type and the fp32 cell states
  const bool nt = N * (3 * (io_dtype == 1 ? 2 : 4) + 4) >= kStreamFootprint;
#define LRS_SDO(IO, V, NTF)                                                                      \
  hipLaunchKernelGGL((k_sru_deer_out<IO, V, NTF>), dim3((unsigned)blocks), dim3(256), 0, stream, \
                     (const IO*)zr, (const IO*)zx, bias_r, c, (IO*)h, c_last, N, C, D)
  if (io_dtype == 1) {
    if (vec) { if (nt) LRS_SDO(uint16_t, true, true); else LRS_SDO(uint16_t, true, false); }
    else LRS_SDO(uint16_t, false, false);
  } else {
    if (vec) { if (nt) LRS_SDO(float, true, true); else LRS_SDO(float, true, false); }
    else LRS_SDO(float, false, false);
  }
#undef LRS_SDO
  return hipGetLastError();
}

}  // namespace lrs
