// gated_cell.hip -- LSTM cell-state layer with gates computed from the inputs
// alone, [T, B, D] layout, forward and backward, each one fused kernel.
//
// Page "RNN CUDA内核优化：实现序列长度无关的恒定推理延迟", body: the LSTM cell
// state C_t = f_t*C_{t-1} + i_t*C~_t is a linear recurrence whose coefficient
// is the forget gate and whose input is i_t*C~_t, once the gates no longer
// read h_{t-1} (the model-change step of its deployment list).  With the
// pre-activations z_f, z_i, z_c, z_o made outside (input projection + bias):
//   f = sigmoid(z_f), i = sigmoid(z_i), g = tanh(z_c), o = sigmoid(z_o),
//   c_t = f_t c_{t-1} + i_t g_t,   h_t = o_t tanh(c_t).
// The tiles, look-back and row access are those of the SRU kernels
// (lrs_tbd.hpp): each gate activation is evaluated once per element, next to
// the load of its pre-activation, and the scan runs on (f, i g).
#include "lrs_tbd.hpp"

namespace lrs {

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
template <typename IO, int NW, int L, int CPT, bool FULL, bool NT>
__device__ __forceinline__ void lstm_tile(const IO* __restrict__ zf, const IO* __restrict__ zi,
                                          const IO* __restrict__ zc, const IO* __restrict__ zo,
                                          const float* __restrict__ c0p, IO* __restrict__ h,
                                          float* __restrict__ c_last, float* __restrict__ cs,
                                          int64_t T, int64_t C, int tb, int cb, bool multi,
                                          uint64_t* st, ColShared<NW, CPT>& s) {
  const ColPos q = col_pos<NW, L, CPT>(tb, cb, C);
  const int64_t cbase = (int64_t)cb * (kWave * CPT);
  float av[L][CPT], bv[L][CPT];
  IoRow<IO, CPT> orow[L];
  {
    const IO* fp = zf + q.row0 * C + cbase;
    const IO* ip = zi + q.row0 * C + cbase;
    const IO* gp = zc + q.row0 * C + cbase;
    const IO* op = zo + q.row0 * C + cbase;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int nv = (FULL || q.row0 + i < T) ? q.nvc : 0;
      IoRow<IO, CPT> fr, ir, gr;
      fr.template load<FULL, NT>(fp, q.off, nv);
      ir.template load<FULL, NT>(ip, q.off, nv);
      gr.template load<FULL, NT>(gp, q.off, nv);
      orow[i].template load<FULL, NT>(op, q.off, nv);
      fp += C;
      ip += C;
      gp += C;
      op += C;
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        if (FULL || k < nv) {
          av[i][k] = fast_sigmoid(fr.get(k), 0.0f);
          bv[i][k] = fast_sigmoid(ir.get(k), 0.0f) * fast_tanh(gr.get(k));
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
      out[k] = fast_sigmoid(orow[i].get(k), 0.0f) * fast_tanh(x[k]);
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
__global__ __launch_bounds__(NW* kWave) void k_lstm_fwd(
    const IO* __restrict__ zf, const IO* __restrict__ zi, const IO* __restrict__ zc,
    const IO* __restrict__ zo, const float* __restrict__ c0p, IO* __restrict__ h,
    float* __restrict__ c_last, float* __restrict__ cs, int64_t T, int64_t C, int ncb, int ntb,
    int vec, uint64_t* __restrict__ status, unsigned* __restrict__ tickets) {
  constexpr int CW = kWave * CPT, TW = NW * L;
  __shared__ ColShared<NW, CPT> s;
  const bool multi = ntb > 1;
  const int cb = (int)(blockIdx.x % (unsigned)ncb);
  const int tb = col_ticket<NW, CPT>(multi, tickets, cb, s);
  uint64_t* st = status + (int64_t)cb * ntb * CW;
  const bool full = vec && ((int64_t)(tb + 1) * TW <= T) && ((int64_t)(cb + 1) * CW <= C);
  if (full)
    lstm_tile<IO, NW, L, CPT, true, NT>(zf, zi, zc, zo, c0p, h, c_last, cs, T, C, tb, cb, multi,
                                        st, s);
  else
    lstm_tile<IO, NW, L, CPT, false, NT>(zf, zi, zc, zo, c0p, h, c_last, cs, T, C, tb, cb, multi,
                                         st, s);
}

// ---------------------------------------------------------------------------
// persistent forward: one workgroup per channel block visits every time tile
// in order, the state entering the tile carried in LDS (persist_enter /
// persist_advance), so there is no look-back state and no reset kernel; the
// next tile's rows are loaded into registers while the current one is
// processed.  Used when the channel blocks alone fill the GPU (B*D large),
// as for the SRU forward.
// ---------------------------------------------------------------------------
template <typename IO, int L, int CPT, bool FULL, bool NT>
__device__ __forceinline__ void lstm_persist_load(const IO* __restrict__ zf,
                                                  const IO* __restrict__ zi,
                                                  const IO* __restrict__ zc,
                                                  const IO* __restrict__ zo, int64_t row0,
                                                  int64_t T, int64_t C, int64_t cbase,
                                                  uint32_t off, int nvc, IoRow<IO, CPT> (&fr)[L],
                                                  IoRow<IO, CPT> (&ir)[L],
                                                  IoRow<IO, CPT> (&gr)[L],
                                                  IoRow<IO, CPT> (&orr)[L]) {
  const IO* fp = zf + row0 * C + cbase;
  const IO* ip = zi + row0 * C + cbase;
  const IO* gp = zc + row0 * C + cbase;
  const IO* op = zo + row0 * C + cbase;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int nv = (FULL || row0 + i < T) ? nvc : 0;
    fr[i].template load<FULL, NT>(fp, off, nv);
    ir[i].template load<FULL, NT>(ip, off, nv);
    gr[i].template load<FULL, NT>(gp, off, nv);
    orr[i].template load<FULL, NT>(op, off, nv);
    fp += C;
    ip += C;
    gp += C;
    op += C;
  }
}

// One tile of the walk: the gates of the current rows, then the next tile's
// rows into the same registers (PF: 0 none, 1 full rows, 2 predicated rows),
// then the waves' maps combine with the carried state and the outputs are
// written.  FULL: the current tile lies inside the arrays.
template <typename IO, int NW, int L, int CPT, bool FULL, int PF, bool SAVE, bool NT>
__device__ __forceinline__ void lstm_persist_tile(
    const IO* __restrict__ zf, const IO* __restrict__ zi, const IO* __restrict__ zc,
    const IO* __restrict__ zo, IO* __restrict__ h, float* __restrict__ cs, int64_t row0,
    int64_t T, int64_t C, int64_t cbase, uint32_t off, int nvc, IoRow<IO, CPT> (&fr)[L],
    IoRow<IO, CPT> (&ir)[L], IoRow<IO, CPT> (&gr)[L], IoRow<IO, CPT> (&orr)[L],
    PersistShared<NW, CPT>& s, int wid, int par) {
  constexpr int TW = NW * L;
  float av[L][CPT], bv[L][CPT];
  IoRow<IO, CPT> ocur[L];
#pragma unroll
  for (int i = 0; i < L; ++i) {
    ocur[i] = orr[i];
    const bool row_ok = FULL || row0 + i < T;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      if (FULL || (row_ok && k < nvc)) {
        av[i][k] = fast_sigmoid(fr[i].get(k), 0.0f);
        bv[i][k] = fast_sigmoid(ir[i].get(k), 0.0f) * fast_tanh(gr[i].get(k));
      } else {  // identity past the end
        av[i][k] = 1.0f;
        bv[i][k] = 0.0f;
      }
    }
  }
  if (PF == 1)
    lstm_persist_load<IO, L, CPT, true, NT>(zf, zi, zc, zo, row0 + TW, T, C, cbase, off, nvc, fr,
                                            ir, gr, orr);
  else if (PF == 2)
    lstm_persist_load<IO, L, CPT, false, NT>(zf, zi, zc, zo, row0 + TW, T, C, cbase, off, nvc, fr,
                                             ir, gr, orr);
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
      out[k] = fast_sigmoid(ocur[i].get(k), 0.0f) * fast_tanh(x[k]);
    }
    const int nv = (FULL || row0 + i < T) ? nvc : 0;
    IoRow<IO, CPT>::template store<FULL, NT>(hp, off, nv, out);
    if (SAVE) store_row<CPT, FULL, NT>(cs + (row0 + i) * C + cbase, off, nv, x);
    hp += C;
  }
  persist_advance<NW, CPT>(x, s, wid, off, par);
}

template <typename IO, int NW, int L, int CPT, bool SAVE, bool NT>
__global__ __launch_bounds__(NW* kWave) void k_lstm_fwd_persist(
    const IO* __restrict__ zf, const IO* __restrict__ zi, const IO* __restrict__ zc,
    const IO* __restrict__ zo, const float* __restrict__ c0p, IO* __restrict__ h,
    float* __restrict__ c_last, float* __restrict__ cs, int64_t T, int64_t C, int vec) {
  constexpr int CW = kWave * CPT, TW = NW * L;
  __shared__ PersistShared<NW, CPT> s;
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t cbase = (int64_t)blockIdx.x * CW;
  const uint32_t off = (uint32_t)(lane * CPT);
  const int nvc = clamp_valid(C - (cbase + off), CPT);
  const bool cfull = vec && cbase + CW <= C;
  for (int j = threadIdx.x; j < CW; j += NW * kWave)
    s.carry[0][j] = (c0p && cbase + j < C) ? c0p[cbase + j] : 0.0f;
  const int64_t ntb = (T + TW - 1) / TW, nfull = T / TW;
  const int64_t w0 = (int64_t)wid * L;
  IoRow<IO, CPT> fr[L], ir[L], gr[L], orr[L];
#define LRS_TILE(FULLT, PFT, TB)                                                                 \
  lstm_persist_tile<IO, NW, L, CPT, FULLT, PFT, SAVE, NT>(zf, zi, zc, zo, h, cs, (TB) * TW + w0, T, \
                                                          C, cbase, off, nvc, fr, ir, gr, orr, s, wid, \
                                                          (int)((TB) & 1))
  if (cfull && nfull > 0) {
    // full tiles in a straight loop (each loads the next full tile), then the
    // last full tile and the ragged tail, if any
    lstm_persist_load<IO, L, CPT, true, NT>(zf, zi, zc, zo, w0, T, C, cbase, off, nvc, fr, ir, gr,
                                            orr);
    for (int64_t tb = 0; tb + 1 < nfull; ++tb) LRS_TILE(true, 1, tb);
    if (ntb > nfull) {
      LRS_TILE(true, 2, nfull - 1);
      LRS_TILE(false, 0, nfull);
    } else {
      LRS_TILE(true, 0, nfull - 1);
    }
  } else {
    lstm_persist_load<IO, L, CPT, false, NT>(zf, zi, zc, zo, w0, T, C, cbase, off, nvc, fr, ir, gr,
                                             orr);
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
// backward (reverse time, as k_sru_bwd: logical time block 0 is the last
// physical block, wave 0 takes its latest steps).  With the cell states c
// saved by the forward pass, the cell-state gradient runs
//   gc_t = e_t + f_{t+1} gc_{t+1},   e_t = gh_t o_t (1 - tanh^2 c_t),
// from dL/dc_T after the last step (f beyond the sequence counts as 1), and
//   dz_o = gh tanh(c) o (1 - o)      (needs no gc: written in the first pass)
//   dz_f = gc c_{t-1} f (1 - f),  dz_i = gc g i (1 - i),  dz_c = gc i (1 - g^2),
//   dc0 = f_1 gc_1.
// Each gate is evaluated once per element: o and tanh c in the first pass
// (which folds e), i and g in the output pass; f is kept from the first pass.
// ---------------------------------------------------------------------------
template <typename IO, int NW, int L, int CPT, bool FULL, bool NT>
__device__ __forceinline__ void lstm_bwd_tile(
    const IO* __restrict__ zf, const IO* __restrict__ zi, const IO* __restrict__ zc,
    const IO* __restrict__ zo, const float* __restrict__ c0p, const float* __restrict__ cs,
    const IO* __restrict__ gh, const float* __restrict__ gcl, IO* __restrict__ dzf,
    IO* __restrict__ dzi, IO* __restrict__ dzc, IO* __restrict__ dzo, float* __restrict__ dc0,
    int64_t T, int64_t C, int tb, int ntb, int cb, bool multi, uint64_t* st,
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
  // f, c and e at rows row0 .. row0+L-1 (f = 1 beyond the end of the
  // sequence), c just before the wave's first row
  float f[L][CPT], c[L][CPT], cp[CPT], e[L][CPT];
  IoRow<IO, CPT> irow[L], grow[L];
  {
    const IO* fp = zf + row0 * C + cbase;
    const IO* ip = zi + row0 * C + cbase;
    const IO* gp = zc + row0 * C + cbase;
    const IO* op = zo + row0 * C + cbase;
    const IO* hp = gh + row0 * C + cbase;
    const float* cq = cs + row0 * C + cbase;
    IO* qo = dzo + row0 * C + cbase;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const bool row_ok = FULL || row0 + i < T;
      const int nv = row_ok ? nvc : 0;
      IoRow<IO, CPT> fr, orr, hr;
      fr.template load<FULL, NT>(fp, off, nv);
      irow[i].template load<FULL, NT>(ip, off, nv);
      grow[i].template load<FULL, NT>(gp, off, nv);
      orr.template load<FULL, NT>(op, off, nv);
      hr.template load<FULL, NT>(hp, off, nv);
      load_row<CPT, FULL, NT>(cq, off, nv, 0.0f, c[i]);
      float od[CPT];
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        const bool ok = FULL || k < nv;
        f[i][k] = ok ? fast_sigmoid(fr.get(k), 0.0f) : 1.0f;
        const float o = fast_sigmoid(orr.get(k), 0.0f);
        const float th = fast_tanh(c[i][k]);
        const float go = hr.get(k) * o;  // 0 out of range (gh row reads 0)
        e[i][k] = __builtin_fmaf(-go * th, th, go);
        od[k] = go * th * (1.0f - o);
      }
      IoRow<IO, CPT>::template store<FULL, NT>(qo, off, nv, od);
      fp += C;
      ip += C;
      gp += C;
      op += C;
      hp += C;
      cq += C;
      qo += C;
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
  // The state passed between waves and tiles is y = f_t gc_t at the first row
  // t of the later wave (y = dL/dc_T past the end, where f = 1), so every
  // forget gate a wave needs is one of its own rows:
  //   gc_{L-1} = e_{L-1} + y_in,  gc_i = e_i + f_{i+1} gc_{i+1},  y_out = f_0 gc_0.
  float A[CPT], B[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    A[k] = 1.0f;
    B[k] = e[L - 1][k];
#pragma unroll
    for (int i = L - 2; i >= 0; --i) {
      B[k] = __builtin_fmaf(f[i + 1][k], B[k], e[i][k]);
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
  IO* qf = dzf + (row0 + L - 1) * C + cbase;
  IO* qi = dzi + (row0 + L - 1) * C + cbase;
  IO* qc = dzc + (row0 + L - 1) * C + cbase;
#pragma unroll
  for (int i = L - 1; i >= 0; --i) {
    float of[CPT], oi[CPT], oc[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      x[k] = (i == L - 1) ? x[k] + e[i][k] : __builtin_fmaf(f[i + 1][k], x[k], e[i][k]);  // gc_t
      const float fi = f[i][k];
      const float ig = fast_sigmoid(irow[i].get(k), 0.0f);
      const float g = fast_tanh(grow[i].get(k));
      const float cprev = (i > 0) ? c[i - 1][k] : cp[k];
      of[k] = x[k] * cprev * (fi * (1.0f - fi));
      oi[k] = x[k] * g * (ig * (1.0f - ig));
      oc[k] = x[k] * ig * __builtin_fmaf(-g, g, 1.0f);
    }
    const int nv = (FULL || row0 + i < T) ? nvc : 0;
    IoRow<IO, CPT>::template store<FULL, NT>(qf, off, nv, of);
    IoRow<IO, CPT>::template store<FULL, NT>(qi, off, nv, oi);
    IoRow<IO, CPT>::template store<FULL, NT>(qc, off, nv, oc);
    qf -= C;
    qi -= C;
    qc -= C;
  }
  if (dc0 && row0 == 0) {
#pragma unroll
    for (int k = 0; k < CPT; ++k)
      if (k < nvc) dc0[c0i + k] = f[0][k] * x[k];
  }
}

template <typename IO, int NW, int L, int CPT, bool NT>
__global__ __launch_bounds__(NW* kWave) void k_lstm_bwd(
    const IO* __restrict__ zf, const IO* __restrict__ zi, const IO* __restrict__ zc,
    const IO* __restrict__ zo, const float* __restrict__ c0p, const float* __restrict__ cs,
    const IO* __restrict__ gh, const float* __restrict__ gcl, IO* __restrict__ dzf,
    IO* __restrict__ dzi, IO* __restrict__ dzc, IO* __restrict__ dzo, float* __restrict__ dc0,
    int64_t T, int64_t C, int ncb, int ntb, int vec, uint64_t* __restrict__ status,
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
    lstm_bwd_tile<IO, NW, L, CPT, true, NT>(zf, zi, zc, zo, c0p, cs, gh, gcl, dzf, dzi, dzc, dzo,
                                            dc0, T, C, tb, ntb, cb, multi, st, s, crow);
  else
    lstm_bwd_tile<IO, NW, L, CPT, false, NT>(zf, zi, zc, zo, c0p, cs, gh, gcl, dzf, dzi, dzc,
                                             dzo, dc0, T, C, tb, ntb, cb, multi, st, s, crow);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
namespace {
constexpr int kLstmNW = 4, kLstmL = 16, kLstmCPT = 2;          // forward, bf16 I/O
constexpr int kLstmF32NW = 8, kLstmF32L = 8, kLstmF32CPT = 2;  // forward, fp32 I/O
constexpr int kLstmBwdNW = 4, kLstmBwdL = 8, kLstmBwdCPT = 2;  // backward, both I/O types
constexpr int kLstmPNW = 8, kLstmPL = 8, kLstmPCPT = 2;        // persistent forward
}  // namespace

ColPlan plan_lstm(int64_t C, int64_t T, int io_dtype, bool save, bool allow_persist,
                  const Opts& o) {
  ColPlan p = io_dtype == 1 ? plan_cols(C, T, kLstmNW, kLstmL, kLstmCPT)
                            : plan_cols(C, T, kLstmF32NW, kLstmF32L, kLstmF32CPT);
  const int64_t ncb_p = (C + kWave * kLstmPCPT - 1) / (kWave * kLstmPCPT);
  if (allow_persist && ncb_p >= persist_min_blocks(o)) {  // the channel blocks alone fill the GPU
    p = plan_cols(C, T, kLstmPNW, kLstmPL, kLstmPCPT);
    p.persist = true;
  }
  // z_f, z_i, z_c, z_o, h (+ the cell states)
  p.stream = C * T * (5 * (io_dtype == 1 ? 2 : 4) + (save ? 4 : 0)) >= kStreamFootprint;
  return p;
}

ColPlan plan_lstm_bwd(int64_t C, int64_t T, int io_dtype) {
  ColPlan p = plan_cols(C, T, kLstmBwdNW, kLstmBwdL, kLstmBwdCPT);
  // four pre-activations, grad_h, four gradients (io type) and the cell states
  p.stream = C * T * (9 * (io_dtype == 1 ? 2 : 4) + 4) >= kStreamFootprint;
  return p;
}

hipError_t launch_lstm_fwd(const void* zf, const void* zi, const void* zc, const void* zo,
                           const float* c0, void* h, float* c_last, float* c_states, int64_t T,
                           int64_t C, int io_dtype, const ColPlan& p, int vec, uint64_t* status,
                           unsigned* tickets, hipStream_t stream) {
  const uint64_t grid = (uint64_t)p.ncb * (uint64_t)p.ntb;
  if (p.persist) {
#define LRS_LSTMP(IO, SV, NTF)                                                                   \
  hipLaunchKernelGGL((k_lstm_fwd_persist<IO, kLstmPNW, kLstmPL, kLstmPCPT, SV, NTF>),             \
                     dim3((unsigned)p.ncb), dim3(kLstmPNW * kWave), 0, stream, (const IO*)zf,      \
                     (const IO*)zi, (const IO*)zc, (const IO*)zo, c0, (IO*)h, c_last, c_states, T, \
                     C, vec)
#define LRS_LSTMP_SAVE(IO, NTF)                  \
  if (c_states) LRS_LSTMP(IO, true, NTF);        \
  else LRS_LSTMP(IO, false, NTF)
    if (io_dtype == 1) {
      if (p.stream) { LRS_LSTMP_SAVE(uint16_t, true); }
      else { LRS_LSTMP_SAVE(uint16_t, false); }
    } else {
      if (p.stream) { LRS_LSTMP_SAVE(float, true); }
      else { LRS_LSTMP_SAVE(float, false); }
    }
#undef LRS_LSTMP_SAVE
#undef LRS_LSTMP
    return hipGetLastError();
  }
#define LRS_LSTM(IO, NW_, L_, CPT_, NTF)                                                        \
  hipLaunchKernelGGL((k_lstm_fwd<IO, NW_, L_, CPT_, NTF>), dim3((unsigned)grid),               \
                     dim3(NW_ * kWave), 0, stream, (const IO*)zf, (const IO*)zi, (const IO*)zc, \
                     (const IO*)zo, c0, (IO*)h, c_last, c_states, T, C, (int)p.ncb, (int)p.ntb,  \
                     vec, status, tickets)
  if (io_dtype == 1) {
    if (p.stream) LRS_LSTM(uint16_t, kLstmNW, kLstmL, kLstmCPT, true);
    else LRS_LSTM(uint16_t, kLstmNW, kLstmL, kLstmCPT, false);
  } else {
    if (p.stream) LRS_LSTM(float, kLstmF32NW, kLstmF32L, kLstmF32CPT, true);
    else LRS_LSTM(float, kLstmF32NW, kLstmF32L, kLstmF32CPT, false);
  }
#undef LRS_LSTM
  return hipGetLastError();
}

hipError_t launch_lstm_bwd(const void* zf, const void* zi, const void* zc, const void* zo,
                           const float* c0, const float* cs, const void* gh, const float* gcl,
                           void* dzf, void* dzi, void* dzc, void* dzo, float* dc0, int64_t T,
                           int64_t C, int io_dtype, const ColPlan& p, int vec, uint64_t* status,
                           unsigned* tickets, hipStream_t stream) {
  const uint64_t grid = (uint64_t)p.ncb * (uint64_t)p.ntb;
#define LRS_LSTMB(IO, NTF)                                                                   \
  hipLaunchKernelGGL((k_lstm_bwd<IO, kLstmBwdNW, kLstmBwdL, kLstmBwdCPT, NTF>),             \
                     dim3((unsigned)grid), dim3(kLstmBwdNW * kWave), 0, stream, (const IO*)zf, \
                     (const IO*)zi, (const IO*)zc, (const IO*)zo, c0, cs, (const IO*)gh, gcl,  \
                     (IO*)dzf, (IO*)dzi, (IO*)dzc, (IO*)dzo, dc0, T, C, (int)p.ncb,            \
                     (int)p.ntb, vec, status, tickets)
  if (io_dtype == 1) {
    if (p.stream) LRS_LSTMB(uint16_t, true);
    else LRS_LSTMB(uint16_t, false);
  } else {
    if (p.stream) LRS_LSTMB(float, true);
    else LRS_LSTMB(float, false);
  }
#undef LRS_LSTMB
  return hipGetLastError();
}

}  // namespace lrs
