// scan_tbd.hip -- feature-contiguous kernels ([T, B, D] layout): consecutive
// lanes own consecutive channels, so every load and store of a time row is a
// contiguous, fully coalesced access, and time runs serially inside a thread.
//
// Work decomposition:
//   * a workgroup of NW waves owns a tile of CW = 64*CPT channels by TW = NW*L
//     time steps; wave w takes L consecutive steps, each lane CPT consecutive
//     channels;
//   * per channel, each thread folds its L steps into one affine map, the
//     waves' maps are combined through LDS, and the state entering the tile
//     comes from a lane-parallel decoupled look-back over per-channel status
//     words (one 64-bit word per channel and time block); time-block order
//     comes from a per-channel-block ticket;
//   * a wave addresses its rows through a wave-uniform row pointer plus a
//     32-bit lane offset (scalar-base global loads), and tiles that lie fully
//     inside the array run without any per-element predication;
//   * every input byte is read once and every output byte written once (the
//     backward kernel also reads one row above and one below each wave's
//     steps; those hit in cache).
//
// Kernels:
//   k_scan_fwd_tbd : h_t = a_t h_{t-1} + b_t
//   k_scan_bwd_tbd : reverse-time adjoint (see k_scan_bwd_bdt)
//   k_sru_fwd      : SRU layer, gates + cell-state scan + highway output fused
//                    (page "CUDA并行化RNN训练：从O(T)到O(log T)的工程实践与参数调优",
//                    SRU paragraph and checklist item 2: one kernel for every
//                    element-wise operation)
#include <stdlib.h>

#include "lrs_tbd.hpp"

namespace lrs {

// ---------------------------------------------------------------------------
// forward scan, [T, B, D]
// ---------------------------------------------------------------------------
template <typename IO, int NW, int L, int CPT, bool FULL, bool NT>
__device__ __forceinline__ void scan_fwd_tile(const IO* __restrict__ a,
                                              const IO* __restrict__ b,
                                              const float* __restrict__ h0, IO* __restrict__ h,
                                              int64_t T, int64_t C, int tb, int cb, bool multi,
                                              uint64_t* st, ColShared<NW, CPT>& s) {
  const ColPos q = col_pos<NW, L, CPT>(tb, cb, C);
  const int64_t cbase = (int64_t)cb * (kWave * CPT);
  float av[L][CPT], bv[L][CPT];
  const IO* ap = a + q.row0 * C + cbase;
  const IO* bp = b + q.row0 * C + cbase;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int nv = (FULL || q.row0 + i < T) ? q.nvc : 0;
    load_row<CPT, FULL, NT>(ap, q.off, nv, 1.0f, av[i]);
    load_row<CPT, FULL, NT>(bp, q.off, nv, 0.0f, bv[i]);
    ap += C;
    bp += C;
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
  float x0[CPT], x[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) x0[k] = (h0 && k < q.nvc) ? h0[q.c0 + k] : 0.0f;
  col_enter_state<NW, CPT>(A, B, multi, tb, x0, h0, cbase, clamp_valid(C - cbase, kWave * CPT),
                           st, s, x);
  IO* hp = h + q.row0 * C + cbase;
#pragma unroll
  for (int i = 0; i < L; ++i) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      x[k] = __builtin_fmaf(av[i][k], x[k], bv[i][k]);
      bv[i][k] = x[k];
    }
    const int nv = (FULL || q.row0 + i < T) ? q.nvc : 0;
    store_row<CPT, FULL, NT>(hp, q.off, nv, bv[i]);
    hp += C;
  }
}

template <typename IO, int NW, int L, int CPT, bool NT>
__global__ __launch_bounds__(NW* kWave) void k_scan_fwd_tbd(
    const IO* __restrict__ a, const IO* __restrict__ b, const float* __restrict__ h0,
    IO* __restrict__ h, int64_t T, int64_t C, int ncb, int ntb, int vec,
    uint64_t* __restrict__ status, unsigned* __restrict__ tickets) {
  constexpr int CW = kWave * CPT, TW = NW * L;
  __shared__ ColShared<NW, CPT> s;
  const bool multi = ntb > 1;
  const int cb = (int)(blockIdx.x % (unsigned)ncb);
  const int tb = col_ticket<NW, CPT>(multi, tickets, cb, s);
  uint64_t* st = status + (int64_t)cb * ntb * CW;
  const bool full = vec && ((int64_t)(tb + 1) * TW <= T) && ((int64_t)(cb + 1) * CW <= C);
  if (full)
    scan_fwd_tile<IO, NW, L, CPT, true, NT>(a, b, h0, h, T, C, tb, cb, multi, st, s);
  else
    scan_fwd_tile<IO, NW, L, CPT, false, NT>(a, b, h0, h, T, C, tb, cb, multi, st, s);
}

// ---------------------------------------------------------------------------
// backward scan, [T, B, D]: logical time block 0 is the last physical block,
// wave 0 takes the latest steps of the block, each thread runs time backwards.
// grad_b may alias grad_h (each element of g is read by the thread that
// writes the same element of grad_b, before it writes).
// ---------------------------------------------------------------------------
template <typename IO, int NW, int L, int CPT, bool FULL, bool NT>
__device__ __forceinline__ void scan_bwd_tile(const IO* __restrict__ a,
                                              const IO* __restrict__ h,
                                              const float* __restrict__ h0, const IO* g,
                                              IO* __restrict__ da, IO* db,
                                              float* __restrict__ dh0, int64_t T, int64_t C,
                                              int tb, int ntb, int cb, bool multi, uint64_t* st,
                                              ColShared<NW, CPT>& s) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int ptb = ntb - 1 - tb;
  const uint32_t off = (uint32_t)(lane * CPT);
  const int64_t cbase = (int64_t)cb * (kWave * CPT);
  const int64_t c0 = cbase + off;
  const int nvc = FULL ? CPT : clamp_valid(C - c0, CPT);
  const int64_t row0 = (int64_t)ptb * (NW * L) + (int64_t)(NW - 1 - wid) * L;

  float av[L + 1][CPT], hv[L][CPT], gv[L][CPT], hp[CPT];
  {
    const IO* ap = a + row0 * C + cbase;
    const IO* hpp = h + row0 * C + cbase;
    const IO* gp = g + row0 * C + cbase;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int nv = (FULL || row0 + i < T) ? nvc : 0;
      load_row<CPT, FULL, NT>(ap, off, nv, 1.0f, av[i]);
      load_row<CPT, FULL, NT>(hpp, off, nv, 0.0f, hv[i]);
      load_row<CPT, FULL, NT>(gp, off, nv, 0.0f, gv[i]);
      ap += C;
      hpp += C;
      gp += C;
    }
    // halo rows (wave-uniform branches): a at row0+L (0 exactly one past the
    // end, 1 beyond), h at row0-1 (h0 before the first step)
    const int64_t tn = row0 + L;
    if (tn < T) {
      load_row<CPT, FULL>(ap, off, nvc, 1.0f, av[L]);
    } else {
#pragma unroll
      for (int k = 0; k < CPT; ++k) av[L][k] = (tn == T) ? 0.0f : 1.0f;
    }
    if (row0 > 0 && row0 <= T) {
      load_row<CPT, FULL>(h + (row0 - 1) * C + cbase, off, nvc, 0.0f, hp);
    } else {
#pragma unroll
      for (int k = 0; k < CPT; ++k) hp[k] = (h0 && k < nvc) ? h0[c0 + k] : 0.0f;
    }
  }
  if (!FULL && row0 + L > T - 1) {  // alpha of the last real step is zero
#pragma unroll
    for (int i = 0; i < L; ++i)
      if (row0 + i + 1 == T) {
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
  float zero[CPT], x[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) zero[k] = 0.0f;
  col_enter_state<NW, CPT>(A, B, multi, tb, zero, nullptr, cbase,
                           clamp_valid(C - cbase, kWave * CPT), st, s, x);
  IO* dap = da + (row0 + L - 1) * C + cbase;
  IO* dbp = db + (row0 + L - 1) * C + cbase;
#pragma unroll
  for (int i = L - 1; i >= 0; --i) {
    float dav[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      x[k] = __builtin_fmaf(av[i + 1][k], x[k], gv[i][k]);
      dav[k] = x[k] * (i > 0 ? hv[i - 1][k] : hp[k]);
      gv[i][k] = x[k];
    }
    const int nv = (FULL || row0 + i < T) ? nvc : 0;
    store_row<CPT, FULL, NT>(dap, off, nv, dav);
    store_row<CPT, FULL, NT>(dbp, off, nv, gv[i]);
    dap -= C;
    dbp -= C;
  }
  if (dh0 && row0 == 0) {
#pragma unroll
    for (int k = 0; k < CPT; ++k)
      if (k < nvc) dh0[c0 + k] = av[0][k] * x[k];
  }
}

template <typename IO, int NW, int L, int CPT, bool NT>
__global__ __launch_bounds__(NW* kWave) void k_scan_bwd_tbd(
    const IO* __restrict__ a, const IO* __restrict__ h, const float* __restrict__ h0,
    const IO* g, IO* __restrict__ da, IO* db, float* __restrict__ dh0, int64_t T,
    int64_t C, int ncb, int ntb, int vec, uint64_t* __restrict__ status,
    unsigned* __restrict__ tickets) {
  constexpr int CW = kWave * CPT, TW = NW * L;
  __shared__ ColShared<NW, CPT> s;
  const bool multi = ntb > 1;
  const int cb = (int)(blockIdx.x % (unsigned)ncb);
  const int tb = col_ticket<NW, CPT>(multi, tickets, cb, s);
  uint64_t* st = status + (int64_t)cb * ntb * CW;
  const int ptb = ntb - 1 - tb;
  const bool full = vec && ((int64_t)(ptb + 1) * TW <= T) && ((int64_t)(cb + 1) * CW <= C);
  if (full)
    scan_bwd_tile<IO, NW, L, CPT, true, NT>(a, h, h0, g, da, db, dh0, T, C, tb, ntb, cb, multi, st,
                                        s);
  else
    scan_bwd_tile<IO, NW, L, CPT, false, NT>(a, h, h0, g, da, db, dh0, T, C, tb, ntb, cb, multi, st,
                                         s);
}

// ---------------------------------------------------------------------------
// fused SRU forward, [T, B, D]:
//   f = sigmoid(zf + bf[d]), r = sigmoid(zr + br[d]),
//   c_t = f c_{t-1} + (1 - f) zx,   h = r tanh(c) + (1 - r) zx
// Gates and state are fp32.  sigmoid(x) = 1/(1 + 2^(-x log2 e)) and
// tanh(c) = 1 - 2/(1 + 2^(2 c log2 e)), each one v_exp_f32 and one v_rcp_f32;
// the biases are pre-scaled by -log2 e so each gate input is a single FMA.
// ---------------------------------------------------------------------------

template <typename IO, int NW, int L, int CPT, bool FULL, bool NT>
__device__ __forceinline__ void sru_tile(const IO* __restrict__ zf, const IO* __restrict__ zr,
                                         const IO* __restrict__ zx,
                                         const float* __restrict__ bias_f,
                                         const float* __restrict__ bias_r,
                                         const float* __restrict__ c0p, IO* __restrict__ h,
                                         float* __restrict__ c_last, float* __restrict__ cs,
                                         int64_t T, int64_t C,
                                         int64_t D, int tb, int cb, bool multi, uint64_t* st,
                                         ColShared<NW, CPT>& s) {
  const ColPos q = col_pos<NW, L, CPT>(tb, cb, C);
  const int64_t cbase = (int64_t)cb * (kWave * CPT);
  // per-channel gate biases, pre-scaled by -log2(e)
  float nbf[CPT], nbr[CPT];
  {
    int64_t d = (q.nvc > 0) ? q.c0 % D : 0;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int64_t dk = (k < q.nvc) ? d : 0;
      nbf[k] = -kLog2e * bias_f[dk];
      nbr[k] = -kLog2e * bias_r[dk];
      d = (d + 1 == D) ? 0 : d + 1;
    }
  }
  float av[L][CPT], bv[L][CPT];
  IoRow<IO, CPT> rr[L], xr[L];
  {
    const IO* fp = zf + q.row0 * C + cbase;
    const IO* rp = zr + q.row0 * C + cbase;
    const IO* xp = zx + q.row0 * C + cbase;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int nv = (FULL || q.row0 + i < T) ? q.nvc : 0;
      IoRow<IO, CPT> fr;
      fr.template load<FULL, NT>(fp, q.off, nv);
      rr[i].template load<FULL, NT>(rp, q.off, nv);
      xr[i].template load<FULL, NT>(xp, q.off, nv);
      fp += C;
      rp += C;
      xp += C;
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        const float f = __builtin_amdgcn_rcpf(
            1.0f + __builtin_amdgcn_exp2f(__builtin_fmaf(fr.get(k), -kLog2e, nbf[k])));
        const float zxv = xr[i].get(k);
        if (FULL || k < nv) {
          av[i][k] = f;
          bv[i][k] = __builtin_fmaf(-f, zxv, zxv);  // (1 - f) * zx
        } else {
          av[i][k] = 1.0f;
          bv[i][k] = 0.0f;
        }
      }
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
  float x0[CPT], x[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) x0[k] = (c0p && k < q.nvc) ? c0p[q.c0 + k] : 0.0f;
  col_enter_state<NW, CPT>(A, B, multi, tb, x0, c0p, cbase, clamp_valid(C - cbase, kWave * CPT),
                           st, s, x);
  IO* hp = h + q.row0 * C + cbase;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    float out[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      x[k] = __builtin_fmaf(av[i][k], x[k], bv[i][k]);
      const float r = __builtin_amdgcn_rcpf(
          1.0f + __builtin_amdgcn_exp2f(__builtin_fmaf(rr[i].get(k), -kLog2e, nbr[k])));
      const float th = __builtin_fmaf(
          -2.0f, __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f((2.0f * kLog2e) * x[k])),
          1.0f);
      const float zxv = xr[i].get(k);
      out[k] = __builtin_fmaf(r, th - zxv, zxv);  // r tanh(c) + (1 - r) zx
    }
    const int nv = (FULL || q.row0 + i < T) ? q.nvc : 0;
    IoRow<IO, CPT>::template store<FULL, NT>(hp, q.off, nv, out);
    hp += C;
    if (cs) store_row<CPT, FULL, NT>(cs + (q.row0 + i) * C + cbase, q.off, nv, x);
    if (c_last && q.row0 + i == T - 1) {
#pragma unroll
      for (int k = 0; k < CPT; ++k)
        if (k < q.nvc) c_last[q.c0 + k] = x[k];
    }
  }
}

template <typename IO, int NW, int L, int CPT, bool NT>
__global__ __launch_bounds__(NW* kWave) void k_sru_fwd(
    const IO* __restrict__ zf, const IO* __restrict__ zr, const IO* __restrict__ zx,
    const float* __restrict__ bias_f, const float* __restrict__ bias_r,
    const float* __restrict__ c0p, IO* __restrict__ h, float* __restrict__ c_last,
    float* __restrict__ cs, int64_t T,
    int64_t C, int64_t D, int ncb, int ntb, int vec, uint64_t* __restrict__ status,
    unsigned* __restrict__ tickets) {
  constexpr int CW = kWave * CPT, TW = NW * L;
  __shared__ ColShared<NW, CPT> s;
  const bool multi = ntb > 1;
  const int cb = (int)(blockIdx.x % (unsigned)ncb);
  const int tb = col_ticket<NW, CPT>(multi, tickets, cb, s);
  uint64_t* st = status + (int64_t)cb * ntb * CW;
  const bool full = vec && ((int64_t)(tb + 1) * TW <= T) && ((int64_t)(cb + 1) * CW <= C);
  if (full)
    sru_tile<IO, NW, L, CPT, true, NT>(zf, zr, zx, bias_f, bias_r, c0p, h, c_last, cs, T, C, D, tb, cb,
                                   multi, st, s);
  else
    sru_tile<IO, NW, L, CPT, false, NT>(zf, zr, zx, bias_f, bias_r, c0p, h, c_last, cs, T, C, D, tb, cb,
                                    multi, st, s);
}

// ---------------------------------------------------------------------------
// Persistent SRU forward: one workgroup per channel block walks every time tile
// in order, carrying the per-channel state in LDS, and loads the next tile's
// rows while it processes the current one.  No look-back state and no reset
// kernel; used when the channel blocks alone fill the GPU (B*D large), where
// it streams about 10% faster than the look-back tiles at B=32 D=1024 T=2048
// (whose workgroups each load their whole tile before any store).
// ---------------------------------------------------------------------------
template <typename IO, int L, int CPT, bool FULL, bool NT>
__device__ __forceinline__ void sru_persist_load(const IO* __restrict__ zf,
                                                 const IO* __restrict__ zr,
                                                 const IO* __restrict__ zx, int64_t row0,
                                                 int64_t T, int64_t C, int64_t cbase,
                                                 uint32_t off, int nvc, IoRow<IO, CPT> (&fr)[L],
                                                 IoRow<IO, CPT> (&rr)[L],
                                                 IoRow<IO, CPT> (&xr)[L]) {
  const IO* fp = zf + row0 * C + cbase;
  const IO* rp = zr + row0 * C + cbase;
  const IO* xp = zx + row0 * C + cbase;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int nv = (FULL || row0 + i < T) ? nvc : 0;
    fr[i].template load<FULL, NT>(fp, off, nv);
    rr[i].template load<FULL, NT>(rp, off, nv);
    xr[i].template load<FULL, NT>(xp, off, nv);
    fp += C;
    rp += C;
    xp += C;
  }
}

// One tile of the persistent walk: gates of the current rows (fr, rr, xr),
// then the next tile's rows are loaded into the same arrays (PF: 0 none,
// 1 full rows, 2 predicated rows), then the waves' maps combine with the
// carried state, the outputs are written and the carry advances.  FULL: the
// current tile lies inside the arrays (no predication).
template <typename IO, int NW, int L, int CPT, bool FULL, int PF, bool SAVE, bool NT>
__device__ __forceinline__ void sru_persist_tile(
    const IO* __restrict__ zf, const IO* __restrict__ zr, const IO* __restrict__ zx,
    IO* __restrict__ h, float* __restrict__ cs, int64_t row0, int64_t T, int64_t C,
    int64_t cbase, uint32_t off, int nvc, const float (&nbf)[CPT], const float (&nbr)[CPT],
    IoRow<IO, CPT> (&fr)[L], IoRow<IO, CPT> (&rr)[L], IoRow<IO, CPT> (&xr)[L],
    PersistShared<NW, CPT>& s, int wid, int par) {
  constexpr int TW = NW * L;
  float av[L][CPT], bv[L][CPT];
  IoRow<IO, CPT> rcur[L], xcur[L];
#pragma unroll
  for (int i = 0; i < L; ++i) {
    rcur[i] = rr[i];
    xcur[i] = xr[i];
    const bool row_ok = FULL || row0 + i < T;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      if (FULL || (row_ok && k < nvc)) {
        const float f = fast_sigmoid(fr[i].get(k), nbf[k]);
        const float z = xr[i].get(k);
        av[i][k] = f;
        bv[i][k] = __builtin_fmaf(-f, z, z);  // (1 - f) * zx
      } else {  // identity past the end
        av[i][k] = 1.0f;
        bv[i][k] = 0.0f;
      }
    }
  }
  if (PF == 1)
    sru_persist_load<IO, L, CPT, true, NT>(zf, zr, zx, row0 + TW, T, C, cbase, off, nvc, fr, rr, xr);
  else if (PF == 2)
    sru_persist_load<IO, L, CPT, false, NT>(zf, zr, zx, row0 + TW, T, C, cbase, off, nvc, fr, rr,
                                            xr);
  float A[CPT], B[CPT], x[CPT];
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
  persist_enter<NW, CPT>(A, B, s, wid, off, x, par);
  IO* hp = h + row0 * C + cbase;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    float out[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      x[k] = __builtin_fmaf(av[i][k], x[k], bv[i][k]);
      const float r = fast_sigmoid(rcur[i].get(k), nbr[k]);
      const float zxv = xcur[i].get(k);
      out[k] = __builtin_fmaf(r, fast_tanh(x[k]) - zxv, zxv);  // r tanh(c) + (1 - r) zx
    }
    const int nv = (FULL || row0 + i < T) ? nvc : 0;
    IoRow<IO, CPT>::template store<FULL, NT>(hp, off, nv, out);
    if (SAVE) store_row<CPT, FULL, NT>(cs + (row0 + i) * C + cbase, off, nv, x);
    hp += C;
  }
  persist_advance<NW, CPT, SAVE>(x, s, wid, off, par);
}

template <typename IO, int NW, int L, int CPT, bool SAVE, bool NT>
__global__ __launch_bounds__(NW* kWave) void k_sru_fwd_persist(
    const IO* __restrict__ zf, const IO* __restrict__ zr, const IO* __restrict__ zx,
    const float* __restrict__ bias_f, const float* __restrict__ bias_r,
    const float* __restrict__ c0p, IO* __restrict__ h, float* __restrict__ c_last,
    float* __restrict__ cs, int64_t T, int64_t C, int64_t D, int vec) {
  constexpr int CW = kWave * CPT, TW = NW * L;
  __shared__ PersistShared<NW, CPT> s;
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t cbase = (int64_t)blockIdx.x * CW;
  const uint32_t off = (uint32_t)(lane * CPT);
  const int64_t c0i = cbase + off;
  const int nvc = clamp_valid(C - c0i, CPT);
  const bool cfull = vec && cbase + CW <= C;
  float nbf[CPT], nbr[CPT];
  {
    int64_t d = (nvc > 0) ? c0i % D : 0;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int64_t dk = (k < nvc) ? d : 0;
      nbf[k] = -kLog2e * bias_f[dk];
      nbr[k] = -kLog2e * bias_r[dk];
      d = (d + 1 == D) ? 0 : d + 1;
    }
  }
  for (int j = threadIdx.x; j < CW; j += NW * kWave)
    s.carry[0][j] = (c0p && cbase + j < C) ? c0p[cbase + j] : 0.0f;
  const int64_t ntb = (T + TW - 1) / TW, nfull = T / TW;
  const int64_t w0 = (int64_t)wid * L;
  IoRow<IO, CPT> fr[L], rr[L], xr[L];
#define LRS_TILE(FULLT, PFT, TB)                                                               \
  sru_persist_tile<IO, NW, L, CPT, FULLT, PFT, SAVE, NT>(zf, zr, zx, h, cs, (TB) * TW + w0, T, C, \
                                                         cbase, off, nvc, nbf, nbr, fr, rr, xr, s, wid, \
                                                         (int)((TB) & 1))
  if (cfull && nfull > 0) {
    // full tiles in a straight loop (each loads the next full tile), then the
    // last full tile and the ragged tail, if any
    sru_persist_load<IO, L, CPT, true, NT>(zf, zr, zx, w0, T, C, cbase, off, nvc, fr, rr, xr);
    for (int64_t tb = 0; tb + 1 < nfull; ++tb) LRS_TILE(true, 1, tb);
    if (ntb > nfull) {
      LRS_TILE(true, 2, nfull - 1);
      LRS_TILE(false, 0, nfull);
    } else {
      LRS_TILE(true, 0, nfull - 1);
    }
  } else {
    sru_persist_load<IO, L, CPT, false, NT>(zf, zr, zx, w0, T, C, cbase, off, nvc, fr, rr, xr);
    for (int64_t tb = 0; tb < ntb; ++tb) {
      if (tb + 1 < ntb) LRS_TILE(false, 2, tb);
      else LRS_TILE(false, 0, tb);
    }
  }
#undef LRS_TILE
  // rows past the end keep the state, so the final carry is c_T
  if (c_last) {
    __syncthreads();
    for (int j = threadIdx.x; j < CW; j += NW * kWave)
      if (cbase + j < C) c_last[cbase + j] = s.carry[ntb & 1][j];
  }
}

// ---------------------------------------------------------------------------
// SRU backward, [T, B, D] (reverse time, as k_scan_bwd_tbd: logical time block
// 0 is the last physical block, wave 0 takes its latest steps).  With the cell
// states c saved by the forward pass, the gradient of the cell state runs
//   gc_t = e_t + f_{t+1} gc_{t+1},   e_t = gh_t r_t (1 - tanh^2 c_t),
// from dL/dc_T after the last step (f beyond the sequence counts as 1), and
//   dzx = gh (1 - r) + gc (1 - f),   dzr = gh (tanh c - zx) r (1 - r),
//   dzf = gc (c_{t-1} - zx) f (1 - f),   dc0 = f_1 gc_1.
// r and tanh c are recomputed in the output pass instead of being kept.  Each
// tile writes its per-channel sums of dzf and dzr over its steps; a two-stage column sum
// adds them up per feature for the bias gradients, in a fixed order.
// ---------------------------------------------------------------------------

template <typename IO, int NW, int L, int CPT, bool FULL, bool NT>
__device__ __forceinline__ void sru_bwd_tile(
    const IO* __restrict__ zf, const IO* __restrict__ zr, const IO* __restrict__ zx,
    const float* __restrict__ bias_f, const float* __restrict__ bias_r,
    const float* __restrict__ c0p, const float* __restrict__ cs, const IO* __restrict__ gh,
    const float* __restrict__ gcl, IO* __restrict__ dzf, IO* __restrict__ dzr,
    IO* __restrict__ dzx, float* __restrict__ dc0, float* __restrict__ part, int64_t T,
    int64_t C, int64_t D, int tb, int ntb, int cb, bool multi, uint64_t* st,
    ColShared<NW, CPT>& s, float (&crow)[NW][kWave * CPT]) {
  constexpr int CW = kWave * CPT;
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int ptb = ntb - 1 - tb;
  const uint32_t off = (uint32_t)(lane * CPT);
  const int64_t cbase = (int64_t)cb * CW;
  const int64_t c0i = cbase + off;
  const int nvc = FULL ? CPT : clamp_valid(C - c0i, CPT);
  const int64_t row0 = (int64_t)ptb * (NW * L) + (int64_t)(NW - 1 - wid) * L;
  float nbf[CPT], nbr[CPT];
  {
    int64_t d = (nvc > 0) ? c0i % D : 0;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int64_t dk = (k < nvc) ? d : 0;
      nbf[k] = -kLog2e * bias_f[dk];
      nbr[k] = -kLog2e * bias_r[dk];
      d = (d + 1 == D) ? 0 : d + 1;
    }
  }
  // f and c at rows row0 .. row0+L-1 (f = 1 beyond the end of the sequence),
  // c just before the wave's first row
  float f[L][CPT], c[L][CPT], cp[CPT];
  IoRow<IO, CPT> rr[L], xr[L], gr[L];
  {
    const IO* fp = zf + row0 * C + cbase;
    const IO* rp = zr + row0 * C + cbase;
    const IO* xp = zx + row0 * C + cbase;
    const IO* gp = gh + row0 * C + cbase;
    const float* cq = cs + row0 * C + cbase;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int nv = (FULL || row0 + i < T) ? nvc : 0;
      IoRow<IO, CPT> fr;
      fr.template load<FULL, NT>(fp, off, nv);
      rr[i].template load<FULL, NT>(rp, off, nv);
      xr[i].template load<FULL, NT>(xp, off, nv);
      gr[i].template load<FULL, NT>(gp, off, nv);
      load_row<CPT, FULL, NT>(cq, off, nv, 0.0f, c[i]);
#pragma unroll
      for (int k = 0; k < CPT; ++k) f[i][k] = (FULL || k < nv) ? fast_sigmoid(fr.get(k), nbf[k]) : 1.0f;
      fp += C;
      rp += C;
      xp += C;
      gp += C;
      cq += C;
    }
    // c before the first row: the earlier wave's last row (shared through LDS
    // below), read from memory only by the wave at the tile's start
    if (wid == NW - 1) {
      if (row0 > 0 && row0 <= T) {
        load_row<CPT, FULL, false>(cs + (row0 - 1) * C + cbase, off, nvc, 0.0f, cp);
      } else {
#pragma unroll
        for (int k = 0; k < CPT; ++k) cp[k] = (c0p && k < nvc) ? c0p[c0i + k] : 0.0f;
      }
    }
#pragma unroll
    for (int k = 0; k < CPT; ++k) crow[wid][off + k] = c[L - 1][k];
  }
  // e_t with r_t and tanh c_t (rows and channels out of range have gh = 0)
  auto e_at = [&](int i, int k, float& r, float& th) {
    r = fast_sigmoid(rr[i].get(k), nbr[k]);
    th = fast_tanh(c[i][k]);
    const float gr_ = gr[i].get(k) * r;
    return __builtin_fmaf(-gr_ * th, th, gr_);
  };
  // The state passed between waves and tiles is y = f_t gc_t at the first row
  // t of the later wave (y = dL/dc_T past the end, where f = 1), so every
  // forget gate a wave needs is one of its own rows:
  //   gc_{L-1} = e_{L-1} + y_in,  gc_i = e_i + f_{i+1} gc_{i+1},  y_out = f_0 gc_0.
  float A[CPT], B[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    float r, th;
    A[k] = 1.0f;
    B[k] = e_at(L - 1, k, r, th);
#pragma unroll
    for (int i = L - 2; i >= 0; --i) {
      B[k] = __builtin_fmaf(f[i + 1][k], B[k], e_at(i, k, r, th));
      A[k] = A[k] * f[i + 1][k];
    }
    A[k] = A[k] * f[0][k];
    B[k] = B[k] * f[0][k];
  }
  float x0[CPT], x[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) x0[k] = (gcl && k < nvc) ? gcl[c0i + k] : 0.0f;
  col_enter_state<NW, CPT>(A, B, multi, tb, x0, gcl, cbase, clamp_valid(C - cbase, CW), st, s, x);
  if (wid < NW - 1) {  // past col_enter_state's barrier: every wave has written crow
#pragma unroll
    for (int k = 0; k < CPT; ++k) cp[k] = crow[wid + 1][off + k];
  }
  float pf[CPT], pr[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) { pf[k] = 0.0f; pr[k] = 0.0f; }
  IO* qf = dzf + (row0 + L - 1) * C + cbase;
  IO* qr = dzr + (row0 + L - 1) * C + cbase;
  IO* qx = dzx + (row0 + L - 1) * C + cbase;
#pragma unroll
  for (int i = L - 1; i >= 0; --i) {
    float of[CPT], orr[CPT], ox[CPT];
    const bool row_ok = FULL || row0 + i < T;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      float r, th;
      const float e = e_at(i, k, r, th);
      x[k] = (i == L - 1) ? x[k] + e : __builtin_fmaf(f[i + 1][k], x[k], e);  // gc_t
      const float g = gr[i].get(k), z = xr[i].get(k), fi = f[i][k];
      const float cprev = (i > 0) ? c[i - 1][k] : cp[k];
      ox[k] = __builtin_fmaf(g, 1.0f - r, x[k] * (1.0f - fi));
      orr[k] = g * (th - z) * (r * (1.0f - r));
      of[k] = x[k] * (cprev - z) * (fi * (1.0f - fi));
      if (FULL || (row_ok && k < nvc)) {
        pf[k] += of[k];
        pr[k] += orr[k];
      }
    }
    const int nv = row_ok ? nvc : 0;
    IoRow<IO, CPT>::template store<FULL, NT>(qf, off, nv, of);
    IoRow<IO, CPT>::template store<FULL, NT>(qr, off, nv, orr);
    IoRow<IO, CPT>::template store<FULL, NT>(qx, off, nv, ox);
    qf -= C;
    qr -= C;
    qx -= C;
  }
  if (dc0 && row0 == 0) {
#pragma unroll
    for (int k = 0; k < CPT; ++k)
      if (k < nvc) dc0[c0i + k] = f[0][k] * x[k];
  }
  // per-tile bias partials, waves added in a fixed order
  __syncthreads();  // every wave is past its last read of s.A / s.B
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    s.A[wid][off + k] = pf[k];
    s.B[wid][off + k] = pr[k];
  }
  __syncthreads();
  if (wid == 0) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      float sf = 0.0f, sr = 0.0f;
      for (int w = 0; w < NW; ++w) {
        sf += s.A[w][off + k];
        sr += s.B[w][off + k];
      }
      if (k < nvc) {
        part[(int64_t)tb * C + c0i + k] = sf;
        part[((int64_t)ntb + tb) * C + c0i + k] = sr;
      }
    }
  }
}

template <typename IO, int NW, int L, int CPT, bool NT>
__global__ __launch_bounds__(NW* kWave) void k_sru_bwd(
    const IO* __restrict__ zf, const IO* __restrict__ zr, const IO* __restrict__ zx,
    const float* __restrict__ bias_f, const float* __restrict__ bias_r,
    const float* __restrict__ c0p, const float* __restrict__ cs, const IO* __restrict__ gh,
    const float* __restrict__ gcl, IO* __restrict__ dzf, IO* __restrict__ dzr,
    IO* __restrict__ dzx, float* __restrict__ dc0, float* __restrict__ part, int64_t T,
    int64_t C, int64_t D, int ncb, int ntb, int vec, uint64_t* __restrict__ status,
    unsigned* __restrict__ tickets) {
  constexpr int CW = kWave * CPT, TW = NW * L;
  __shared__ ColShared<NW, CPT> s;
  __shared__ float crow[NW][CW];
  const bool multi = ntb > 1;
  const int cb = (int)(blockIdx.x % (unsigned)ncb);
  const int tb = col_ticket<NW, CPT>(multi, tickets, cb, s);
  uint64_t* st = status + (int64_t)cb * ntb * CW;
  const int ptb = ntb - 1 - tb;
  const bool full = vec && ((int64_t)(ptb + 1) * TW <= T) && ((int64_t)(cb + 1) * CW <= C);
  if (full)
    sru_bwd_tile<IO, NW, L, CPT, true, NT>(zf, zr, zx, bias_f, bias_r, c0p, cs, gh, gcl, dzf, dzr,
                                           dzx, dc0, part, T, C, D, tb, ntb, cb, multi, st, s,
                                           crow);
  else
    sru_bwd_tile<IO, NW, L, CPT, false, NT>(zf, zr, zx, bias_f, bias_r, c0p, cs, gh, gcl, dzf,
                                            dzr, dzx, dc0, part, T, C, D, tb, ntb, cb, multi, st,
                                            s, crow);
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

// Channel blocks needed for the persistent kernels: the device's compute
// units, or the caller's override (0 = always, a huge value = never).
int64_t persist_min_blocks(const Opts& o) {
  return o.persist_min_blocks >= 0 ? o.persist_min_blocks : device_cus();
}

int64_t col_status_words(const ColPlan& p) {
  return (p.ntb > 1 && !p.persist) ? p.ncb * p.ntb * kWave * p.cpt : 0;
}

// Tile shapes (waves along time x steps per lane x channels per lane).
namespace {
constexpr int kFwdNW = 8, kFwdL = 32, kFwdCPT = 1;
constexpr int kBwdNW = 8, kBwdL = 16, kBwdCPT = 1;
// bf16 I/O: two channels per lane (4-byte row accesses instead of 2-byte)
constexpr int kFwd16NW = 8, kFwd16L = 16, kFwd16CPT = 2;
constexpr int kBwd16NW = 8, kBwd16L = 8, kBwd16CPT = 2;
constexpr int kSruNW = 4, kSruL = 16, kSruCPT = 2;          // bf16 I/O
constexpr int kSruF32NW = 8, kSruF32L = 8, kSruF32CPT = 2;  // fp32 I/O
constexpr int kSruBwdNW = 4, kSruBwdL = 8, kSruBwdCPT = 2;  // backward, both I/O types
constexpr int kSruPNW = 8, kSruPL = 8, kSruPCPT = 2;        // persistent forward, both I/O types
}  // namespace

ColPlan plan_scan_fwd_tbd(int64_t C, int64_t T, int io) {
  ColPlan p = io == kIoBf16 ? plan_cols(C, T, kFwd16NW, kFwd16L, kFwd16CPT)
                            : plan_cols(C, T, kFwdNW, kFwdL, kFwdCPT);
  p.stream = 3 * C * T * io_bytes(io) >= kStreamFootprint;  // a, b, h
  return p;
}
ColPlan plan_scan_bwd_tbd(int64_t C, int64_t T, int io) {
  ColPlan p = io == kIoBf16 ? plan_cols(C, T, kBwd16NW, kBwd16L, kBwd16CPT)
                            : plan_cols(C, T, kBwdNW, kBwdL, kBwdCPT);
  p.stream = 5 * C * T * io_bytes(io) >= kStreamFootprint;  // a, h, g, grad_a, grad_b
  return p;
}
ColPlan plan_sru_bwd(int64_t C, int64_t T, int io_dtype) {
  ColPlan p = plan_cols(C, T, kSruBwdNW, kSruBwdL, kSruBwdCPT);
  // z_f, z_r, z_x, grad_h, the three gradients (io type) and the cell states
  p.stream = C * T * (7 * (io_dtype == 1 ? 2 : 4) + 4) >= kStreamFootprint;
  return p;
}
ColPlan plan_sru(int64_t C, int64_t T, int io_dtype, bool allow_persist, const Opts& o) {
  ColPlan p = io_dtype == 1 ? plan_cols(C, T, kSruNW, kSruL, kSruCPT)
                            : plan_cols(C, T, kSruF32NW, kSruF32L, kSruF32CPT);
  const int64_t ncb_p = (C + kWave * kSruPCPT - 1) / (kWave * kSruPCPT);
  if (allow_persist && ncb_p >= persist_min_blocks(o)) {  // the channel blocks alone fill the GPU
    p = plan_cols(C, T, kSruPNW, kSruPL, kSruPCPT);
    p.persist = true;
  }
  p.stream = 4 * C * T * (io_dtype == 1 ? 2 : 4) >= kStreamFootprint;  // z_f, z_r, z_x, h
  return p;
}

template <typename IO, int NW, int L, int CPT>
static void scan_fwd_tbd_io(const IO* a, const IO* b, const float* h0, IO* h, int64_t C, int64_t T,
                            const ColPlan& p, int vec, uint64_t* status, unsigned* tickets,
                            hipStream_t stream) {
  const uint64_t grid = (uint64_t)p.ncb * (uint64_t)p.ntb;
  if (p.stream)
    hipLaunchKernelGGL((k_scan_fwd_tbd<IO, NW, L, CPT, true>), dim3((unsigned)grid),
                       dim3(NW * kWave), 0, stream, a, b, h0, h, T, C, (int)p.ncb, (int)p.ntb,
                       vec, status, tickets);
  else
    hipLaunchKernelGGL((k_scan_fwd_tbd<IO, NW, L, CPT, false>), dim3((unsigned)grid),
                       dim3(NW * kWave), 0, stream, a, b, h0, h, T, C, (int)p.ncb, (int)p.ntb,
                       vec, status, tickets);
}

hipError_t launch_scan_fwd_tbd(const void* a, const void* b, const float* h0, void* h, int io,
                               int64_t C, int64_t T, const ColPlan& p, int vec, uint64_t* status,
                               unsigned* tickets, hipStream_t stream) {
  if (io == kIoBf16)
    scan_fwd_tbd_io<uint16_t, kFwd16NW, kFwd16L, kFwd16CPT>(
        (const uint16_t*)a, (const uint16_t*)b, h0, (uint16_t*)h, C, T, p, vec, status, tickets,
        stream);
  else
    scan_fwd_tbd_io<float, kFwdNW, kFwdL, kFwdCPT>((const float*)a, (const float*)b, h0, (float*)h,
                                                   C, T, p, vec, status, tickets, stream);
  return hipGetLastError();
}

template <typename IO, int NW, int L, int CPT>
static void scan_bwd_tbd_io(const IO* a, const IO* h, const float* h0, const IO* g, IO* da, IO* db,
                            float* dh0, int64_t C, int64_t T, const ColPlan& p, int vec,
                            uint64_t* status, unsigned* tickets, hipStream_t stream) {
  const uint64_t grid = (uint64_t)p.ncb * (uint64_t)p.ntb;
  if (p.stream)
    hipLaunchKernelGGL((k_scan_bwd_tbd<IO, NW, L, CPT, true>), dim3((unsigned)grid),
                       dim3(NW * kWave), 0, stream, a, h, h0, g, da, db, dh0, T, C, (int)p.ncb,
                       (int)p.ntb, vec, status, tickets);
  else
    hipLaunchKernelGGL((k_scan_bwd_tbd<IO, NW, L, CPT, false>), dim3((unsigned)grid),
                       dim3(NW * kWave), 0, stream, a, h, h0, g, da, db, dh0, T, C, (int)p.ncb,
                       (int)p.ntb, vec, status, tickets);
}

hipError_t launch_scan_bwd_tbd(const void* a, const void* h, const float* h0, const void* g,
                               void* da, void* db, float* dh0, int io, int64_t C, int64_t T,
                               const ColPlan& p, int vec, uint64_t* status, unsigned* tickets,
                               hipStream_t stream) {
  if (io == kIoBf16)
    scan_bwd_tbd_io<uint16_t, kBwd16NW, kBwd16L, kBwd16CPT>(
        (const uint16_t*)a, (const uint16_t*)h, h0, (const uint16_t*)g, (uint16_t*)da,
        (uint16_t*)db, dh0, C, T, p, vec, status, tickets, stream);
  else
    scan_bwd_tbd_io<float, kBwdNW, kBwdL, kBwdCPT>((const float*)a, (const float*)h, h0,
                                                   (const float*)g, (float*)da, (float*)db, dh0, C,
                                                   T, p, vec, status, tickets, stream);
  return hipGetLastError();
}

hipError_t launch_sru_fwd(const void* zf, const void* zr, const void* zx, const float* bias_f,
                          const float* bias_r, const float* c0, void* h, float* c_last,
                          float* c_states, int64_t T,
                          int64_t B, int64_t D, int io_dtype, const ColPlan& p, int vec,
                          uint64_t* status, unsigned* tickets, hipStream_t stream) {
  const uint64_t grid = (uint64_t)p.ncb * (uint64_t)p.ntb;
  const int64_t C = B * D;
  if (p.persist) {
#define LRS_SRUP(IO, SV, NTF)                                                                     \
  hipLaunchKernelGGL((k_sru_fwd_persist<IO, kSruPNW, kSruPL, kSruPCPT, SV, NTF>),                \
                     dim3((unsigned)p.ncb), dim3(kSruPNW * kWave), 0, stream, (const IO*)zf,       \
                     (const IO*)zr, (const IO*)zx, bias_f, bias_r, c0, (IO*)h, c_last, c_states, T, \
                     C, D, vec)
#define LRS_SRUP_SAVE(IO, NTF)                  \
  if (c_states) LRS_SRUP(IO, true, NTF);        \
  else LRS_SRUP(IO, false, NTF)
    if (io_dtype == 1) {
      if (p.stream) { LRS_SRUP_SAVE(uint16_t, true); }
      else { LRS_SRUP_SAVE(uint16_t, false); }
    } else {
      if (p.stream) { LRS_SRUP_SAVE(float, true); }
      else { LRS_SRUP_SAVE(float, false); }
    }
#undef LRS_SRUP_SAVE
#undef LRS_SRUP
    return hipGetLastError();
  }
#define LRS_SRU(IO, NW_, L_, CPT_, NTF)                                                          \
  hipLaunchKernelGGL((k_sru_fwd<IO, NW_, L_, CPT_, NTF>), dim3((unsigned)grid), dim3(NW_ * kWave), \
                     0, stream, (const IO*)zf, (const IO*)zr, (const IO*)zx, bias_f, bias_r, c0,  \
                     (IO*)h, c_last, c_states, T, C, D, (int)p.ncb, (int)p.ntb, vec, status, tickets)
  if (io_dtype == 1) {
    if (p.stream) LRS_SRU(uint16_t, kSruNW, kSruL, kSruCPT, true);
    else LRS_SRU(uint16_t, kSruNW, kSruL, kSruCPT, false);
  } else {
    if (p.stream) LRS_SRU(float, kSruF32NW, kSruF32L, kSruF32CPT, true);
    else LRS_SRU(float, kSruF32NW, kSruF32L, kSruF32CPT, false);
  }
#undef LRS_SRU
  return hipGetLastError();
}

hipError_t launch_sru_bwd(const void* zf, const void* zr, const void* zx, const float* bias_f,
                          const float* bias_r, const float* c0, const float* cs, const void* gh,
                          const float* gcl, void* dzf, void* dzr, void* dzx, float* dbf,
                          float* dbr, float* dc0, float* part, double* acc, int64_t T, int64_t B,
                          int64_t D, int io_dtype, const ColPlan& p, int vec, uint64_t* status,
                          unsigned* tickets, hipStream_t stream) {
  const uint64_t grid = (uint64_t)p.ncb * (uint64_t)p.ntb;
  const int64_t C = B * D;
#define LRS_SRUB(IO, NTF)                                                                         \
  hipLaunchKernelGGL((k_sru_bwd<IO, kSruBwdNW, kSruBwdL, kSruBwdCPT, NTF>), dim3((unsigned)grid), \
                     dim3(kSruBwdNW * kWave), 0, stream, (const IO*)zf, (const IO*)zr,             \
                     (const IO*)zx, bias_f, bias_r, c0, cs, (const IO*)gh, gcl, (IO*)dzf,          \
                     (IO*)dzr, (IO*)dzx, dc0, part, T, C, D, (int)p.ncb, (int)p.ntb, vec, status, \
                     tickets)
  if (io_dtype == 1) {
    if (p.stream) LRS_SRUB(uint16_t, true);
    else LRS_SRUB(uint16_t, false);
  } else {
    if (p.stream) LRS_SRUB(float, true);
    else LRS_SRUB(float, false);
  }
#undef LRS_SRUB
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // bias gradients: column sums over (time block, batch) rows of the partials
  return launch_col_sums(part, 2, p.ntb * B, D, acc, dbf, dbr, stream);
}

}  // namespace lrs
