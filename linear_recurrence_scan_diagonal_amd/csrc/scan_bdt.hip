// scan_bdt.hip -- time-contiguous kernels: one channel is one row of T values
// ([B, D, T] layout, "stored contiguously along time" as the DEER page's
// engineering section recommends for the input, state and Jacobian arrays).
//
// Work decomposition (same for all three kernels):
//   * a workgroup of NW waves owns one chunk of CH = NW*R*256 consecutive steps
//     of one channel; each wave owns R "rows" of 256 consecutive steps and in
//     every row lane l owns 4 consecutive steps, so each row is one fully
//     coalesced 1 KiB access per array (16 bytes per lane);
//   * per row: each lane folds its 4 steps serially (FMA), the 64 lane maps are
//     scanned across the wave with DPP, the row maps are chained in registers,
//     and the wave maps are combined through LDS;
//   * a channel longer than one chunk is split into chunks (the page's
//     T = N*S sub-sequence split, one block per sub-sequence); the state
//     entering a chunk comes from a decoupled look-back over per-chunk status
//     words, and chunk order comes from a per-channel ticket so the wait always
//     terminates;
//   * every input byte is read once and every output byte written once; the
//     values a step needs from its neighbour (a_{t+1}, h_{t-1}) come from the
//     neighbouring lane through DPP, from the neighbouring row through a
//     readlane, and only at wave edges from memory (one scalar per wave).
//
// Kernels:
//   k_scan_fwd_bdt : h_t = a_t h_{t-1} + b_t
//   k_scan_bwd_bdt : reverse-time adjoint, lam_t = g_t + a_{t+1} lam_{t+1},
//                    da_t = lam_t h_{t-1}, db_t = lam_t, dh0 = a_1 lam_1
//   k_scan_fused_bdt: both of the above in one pass for channels that fit one
//                    workgroup (h kept in registers between the two scans)
//   k_deer_iter    : one fused DEER Newton iteration for h_t = tanh(w h_{t-1}+u_t)
#include <algorithm>

#include "lrs_device.hpp"
#include "lrs_internal.hpp"

namespace lrs {

template <int NW>
struct BlockShared {
  float wA[NW];
  float wB[NW];
  uint32_t wmax[NW];
  float carry;
  int chunk;
};

// Per-wave maps (uniform within each wave) combined in wave order: every
// thread gets the composition of the waves before its own (PA, PB) and of the
// whole block (TA, TB).
template <int NW>
__device__ __forceinline__ void block_combine(float WA, float WB, BlockShared<NW>& s, float& PA,
                                              float& PB, float& TA, float& TB) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  if (lane == 0) {
    s.wA[wid] = WA;
    s.wB[wid] = WB;
  }
  __syncthreads();
  PA = 1.0f; PB = 0.0f; TA = 1.0f; TB = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
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
// directly; otherwise wave 0 publishes this chunk's aggregate (or, for the
// last chunk of a 64-chunk group, its inclusive state once known), resolves
// the carry by the fixed-order group rule of lookback_group_wave and shares
// it through LDS.
template <int NW>
__device__ __forceinline__ float chunk_carry(bool multi, int c, float TA, float TB, float x0,
                                             uint64_t* st, BlockShared<NW>& s) {
  if (!multi) return x0;
  if (threadIdx.x < kWave) {
    const bool gend = group_end(c, kWaveGroup);
    if (!gend && threadIdx.x == 0) status_store(st + c, pack_agg(TA, TB));
    const float x_in = lookback_group_wave(st, c, 1, x0);
    if (threadIdx.x == 0) {
      if (gend) status_store(st + c, pack_inc(__builtin_fmaf(TA, x_in, TB)));
      s.carry = x_in;
    }
  }
  __syncthreads();
  return s.carry;
}

// Channel served by workgroup `blk` of a multi-chunk launch (C * nchunk
// workgroups).  Workgroups are dealt to channels in runs of kRun, so the
// resident workgroups sweep memory in long contiguous runs (one run per
// channel) rather than touching every channel at once, while at most kRun
// chunks of a channel are in flight (inside one look-back window).  Every
// channel receives exactly nchunk workgroups; the order of its chunks comes
// from the per-channel ticket.
constexpr int64_t kRun = 16;
__device__ __forceinline__ int64_t chunk_channel(uint64_t blk, int64_t C, int64_t nchunk) {
  const int64_t full = nchunk / kRun;            // complete rounds of kRun chunks per channel
  const int64_t head = full * kRun * C;          // workgroups in those rounds
  if ((int64_t)blk < head) return (int64_t)((blk % (uint64_t)(kRun * C)) / kRun);
  const int64_t rem = nchunk - full * kRun;      // 1 .. kRun-1 chunks left per channel
  return (int64_t)((blk - head) / rem);
}

template <int NW>
__device__ __forceinline__ int chunk_ticket(bool multi, unsigned* tickets, int64_t ch,
                                            BlockShared<NW>& s) {
  if (!multi) return 0;
  if (threadIdx.x == 0) s.chunk = (int)take_ticket(tickets + ch);
  __syncthreads();
  return s.chunk;
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return as_f32((uint32_t)__builtin_amdgcn_readlane((int)as_u32(v), lane));
}

// Value of the next lane (wave_shl:1); lane 63 receives `lane63`.
__device__ __forceinline__ float wave_shift_down(float x, float lane63) {
  return as_f32((uint32_t)__builtin_amdgcn_update_dpp((int)as_u32(lane63), (int)as_u32(x), 0x130,
                                                      0xf, 0xf, false));
}

// Chain the R row maps of a wave into the wave's map.
template <int R>
__device__ __forceinline__ void chain_rows(const float (&RA)[R], const float (&RB)[R], float& WA,
                                           float& WB) {
  WA = RA[0];
  WB = RB[0];
#pragma unroll
  for (int r = 1; r < R; ++r) {
    WB = __builtin_fmaf(RA[r], WB, RB[r]);
    WA = WA * RA[r];
  }
}

// ---------------------------------------------------------------------------
// forward scan
// ---------------------------------------------------------------------------
template <typename IO, int NW, int R, bool NTL, bool NTS, bool FULL>
__device__ __forceinline__ void scan_fwd_chunk(const IO* __restrict__ a,
                                               const IO* __restrict__ b,
                                               const float* __restrict__ h0,
                                               IO* __restrict__ h, int64_t T, int64_t ch, int c,
                                               bool multi, int vec, uint64_t* st,
                                               BlockShared<NW>& s) {
  constexpr int S = R * 256, CH = NW * S;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const int64_t base = (int64_t)c * CH + (int64_t)wid * S + 4 * lane;
  const IO* arow = a + ch * T;
  const IO* brow = b + ch * T;

  // A chunk of a long channel loads its rows a few at a time: each wave waits
  // for the loads of one fp32 row (two bf16 rows) before it issues the next,
  // so at most 2 KiB per wave are in flight.  At B=2, D=256, T=2^20 that
  // streams 2% faster (1064 against 1088 us) than issuing all rows at once;
  // single-chunk channels see no difference and issue all rows at once.
  constexpr int kRowsPerWait = sizeof(IO) == 2 ? 2 : 1;
  float4 a4[R], b4[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    a4[r] = ld4<FULL, NTL>(arow, base + r * 256, T, vec, 1.0f);
    b4[r] = ld4<FULL, NTL>(brow, base + r * 256, T, vec, 0.0f);
    if (multi && (r + 1) % kRowsPerWait == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  float Ai[R], Bi[R], RA[R], RB[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float A = a4[r].x, B = b4[r].x;
    B = __builtin_fmaf(a4[r].y, B, b4[r].y); A = A * a4[r].y;
    B = __builtin_fmaf(a4[r].z, B, b4[r].z); A = A * a4[r].z;
    B = __builtin_fmaf(a4[r].w, B, b4[r].w); A = A * a4[r].w;
    wave_scan(A, B);
    Ai[r] = A; Bi[r] = B;
    RA[r] = readlane_f(A, kWave - 1);
    RB[r] = readlane_f(B, kWave - 1);
  }
  float WA, WB, PA, PB, TA, TB;
  chain_rows<R>(RA, RB, WA, WB);
  block_combine<NW>(WA, WB, s, PA, PB, TA, TB);
  const float x0 = h0 ? h0[ch] : 0.0f;
  const float x_in = chunk_carry<NW>(multi, c, TA, TB, x0, st, s);

  float xr = __builtin_fmaf(PA, x_in, PB);  // state entering this wave's first row
  IO* hrow = h + ch * T;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float x = wave_shift_up(__builtin_fmaf(Ai[r], xr, Bi[r]), xr);  // entering this lane's group
    float4 o;
    x = __builtin_fmaf(a4[r].x, x, b4[r].x); o.x = x;
    x = __builtin_fmaf(a4[r].y, x, b4[r].y); o.y = x;
    x = __builtin_fmaf(a4[r].z, x, b4[r].z); o.z = x;
    x = __builtin_fmaf(a4[r].w, x, b4[r].w); o.w = x;
    st4<FULL, NTS>(hrow, base + r * 256, T, vec, o);
    xr = __builtin_fmaf(RA[r], xr, RB[r]);
  }
}

// MULTI: channels span several chunks (look-back compiled in); otherwise each
// channel is one chunk and the kernel carries no look-back code at all.
template <typename IO, int NW, int R, bool NTL = false, bool NTS = false, bool MULTI = false>
__global__ __launch_bounds__(NW* kWave) void k_scan_fwd_bdt(
    const IO* __restrict__ a, const IO* __restrict__ b, const float* __restrict__ h0,
    IO* __restrict__ h, int64_t T, int64_t C, int nchunk, int vec,
    uint64_t* __restrict__ status, unsigned* __restrict__ tickets) {
  constexpr int CH = NW * R * 256;
  __shared__ BlockShared<NW> s;
  constexpr bool multi = MULTI;
  const int64_t ch = multi ? chunk_channel(blockIdx.x, C, nchunk) : (int64_t)blockIdx.x;
  const int c = chunk_ticket<NW>(multi, tickets, ch, s);
  uint64_t* st = status + ch * nchunk;
  if (vec && (int64_t)(c + 1) * CH <= T)
    scan_fwd_chunk<IO, NW, R, NTL, NTS, true>(a, b, h0, h, T, ch, c, multi, vec, st, s);
  else
    scan_fwd_chunk<IO, NW, R, NTL, NTS, false>(a, b, h0, h, T, ch, c, multi, vec, st, s);
}

// ---------------------------------------------------------------------------
// backward (reverse-time) scan.  Scan order is descending time: logical chunk 0
// is the last physical chunk, logical wave w takes the w-th segment counted
// from the chunk's end, logical row r the r-th row counted from the segment's
// end, and lane l the l-th group counted from the row's end, so the forward
// combine applies unchanged.  grad_b may alias grad_h: each element of g is
// read by the thread that writes the same element of grad_b, before it writes.
// ---------------------------------------------------------------------------
template <typename IO, int NW, int R, bool NTL, bool NTS, bool FULL>
__device__ __forceinline__ void scan_bwd_chunk(const IO* __restrict__ a,
                                               const IO* __restrict__ h,
                                               const float* __restrict__ h0, const IO* g,
                                               IO* __restrict__ da, IO* db,
                                               float* __restrict__ dh0, int64_t T, int64_t ch,
                                               int c, int pc, bool multi, int vec, uint64_t* st,
                                               BlockShared<NW>& s) {
  constexpr int S = R * 256, CH = NW * S;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const int64_t wend = (int64_t)(pc + 1) * CH - (int64_t)wid * S;  // physical end of the segment
  const int64_t wbeg = wend - S;
  const IO* arow = a + ch * T;
  const IO* hrow = h + ch * T;
  const IO* grow = g + ch * T;

  // Step p has coefficient alpha_p = a_{p+1}.  Reading a as 0 at and past
  // index T makes every step past the end a reset to zero, so the state
  // entering the last real step is lam_{T+1} = 0 and alpha_{T-1} = 0 without
  // any per-element fix-up.
  const int64_t pb = wend - 256 + 4 * (kWave - 1 - lane);  // this lane's group in row 0
  float4 a4[R], h4[R], g4[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    a4[r] = ld4<FULL, NTL>(arow, pb - r * 256, T, vec, 0.0f);
    h4[r] = ld4<FULL, NTL>(hrow, pb - r * 256, T, vec, 0.0f);
    g4[r] = ld4<FULL, NTL>(grow, pb - r * 256, T, vec, 0.0f);
  }
  const float x0h = h0 ? h0[ch] : 0.0f;
  // wave-edge halos (uniform): a just past the segment, h just before it
  const float a_after = (wend < T) ? io_ld(arow, wend) : 0.0f;
  const float h_before = (wbeg > 0) ? ((wbeg - 1 < T) ? io_ld(hrow, wbeg - 1) : 0.0f) : x0h;

  float an[R], hp[R], Ai[R], Bi[R], RA[R], RB[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    // the group's last alpha is the first a of the next group (previous lane,
    // or lane 63 of the previous row, or the wave-edge halo)
    const float fa = (r > 0) ? readlane_f(a4[r - 1].x, kWave - 1) : a_after;
    an[r] = wave_shift_up(a4[r].x, fa);
    const float fh = (r < R - 1) ? readlane_f(h4[r + 1].w, 0) : h_before;
    hp[r] = wave_shift_down(h4[r].w, fh);  // h at the group's first step - 1
    float A = an[r], B = g4[r].w;
    B = __builtin_fmaf(a4[r].w, B, g4[r].z); A = A * a4[r].w;
    B = __builtin_fmaf(a4[r].z, B, g4[r].y); A = A * a4[r].z;
    B = __builtin_fmaf(a4[r].y, B, g4[r].x); A = A * a4[r].y;
    wave_scan(A, B);
    Ai[r] = A; Bi[r] = B;
    RA[r] = readlane_f(A, kWave - 1);
    RB[r] = readlane_f(B, kWave - 1);
  }
  float WA, WB, PA, PB, TA, TB;
  chain_rows<R>(RA, RB, WA, WB);
  block_combine<NW>(WA, WB, s, PA, PB, TA, TB);
  const float x_in = chunk_carry<NW>(multi, c, TA, TB, 0.0f, st, s);

  float xr = __builtin_fmaf(PA, x_in, PB);
  IO* darow = da + ch * T;
  IO* dbrow = db + ch * T;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float x = wave_shift_up(__builtin_fmaf(Ai[r], xr, Bi[r]), xr);  // lam past the group
    const float l3 = __builtin_fmaf(an[r], x, g4[r].w);
    const float l2 = __builtin_fmaf(a4[r].w, l3, g4[r].z);
    const float l1 = __builtin_fmaf(a4[r].z, l2, g4[r].y);
    const float l0 = __builtin_fmaf(a4[r].y, l1, g4[r].x);
    const int64_t p = pb - r * 256;
    st4<FULL, NTS>(darow, p, T, vec,
                     make_float4(l0 * hp[r], l1 * h4[r].x, l2 * h4[r].y, l3 * h4[r].z));
    st4<FULL, NTS>(dbrow, p, T, vec, make_float4(l0, l1, l2, l3));
    if (dh0 && p == 0) dh0[ch] = a4[r].x * l0;
    xr = __builtin_fmaf(RA[r], xr, RB[r]);
  }
}


template <typename IO, int NW, int R, bool NTL = false, bool NTS = false, bool MULTI = false>
__global__ __launch_bounds__(NW* kWave) void k_scan_bwd_bdt(
    const IO* __restrict__ a, const IO* __restrict__ h, const float* __restrict__ h0,
    const IO* g, IO* __restrict__ da, IO* db, float* __restrict__ dh0, int64_t T,
    int64_t C, int nchunk, int vec, uint64_t* __restrict__ status,
    unsigned* __restrict__ tickets) {
  constexpr int CH = NW * R * 256;
  __shared__ BlockShared<NW> s;
  constexpr bool multi = MULTI;
  const int64_t ch = multi ? chunk_channel(blockIdx.x, C, nchunk) : (int64_t)blockIdx.x;
  const int c = chunk_ticket<NW>(multi, tickets, ch, s);
  const int pc = nchunk - 1 - c;
  uint64_t* st = status + ch * nchunk;
  if (vec && (int64_t)(pc + 1) * CH <= T)
    scan_bwd_chunk<IO, NW, R, NTL, NTS, true>(a, h, h0, g, da, db, dh0, T, ch, c, pc, multi, vec,
                                              st, s);
  else
    scan_bwd_chunk<IO, NW, R, NTL, NTS, false>(a, h, h0, g, da, db, dh0, T, ch, c, pc, multi,
                                               vec, st, s);
}

// ---------------------------------------------------------------------------
// forward and backward scan in one pass, for channels that fit one workgroup.
// The forward runs as in k_scan_fwd_bdt and leaves h in registers; the
// backward then runs in the same lane mapping, scanning descending time: each
// lane folds its group from its last step down, the lane maps are scanned from
// lane 63 down to lane 0 (the wave reversed with ds_bpermute around the
// ascending DPP scan), rows are chained from the last one down and waves
// combine from the last one down.  h_{t-1} at a wave's first step is the state
// entering that wave, known from the forward combine; a_{t+1} past the last
// step reads as 0.  Reads a, b, g and writes h (optional), grad_a, grad_b:
// 24 bytes per element instead of the 32 of the two separate passes, or 20
// without h.  grad_b may alias g and h may alias b: each thread reads those
// elements before it writes the same elements.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float lane_reverse(float x, int lane) {
  return as_f32((uint32_t)__builtin_amdgcn_ds_bpermute((kWave - 1 - lane) << 2, (int)as_u32(x)));
}

// Inclusive scan from lane 63 down to lane 0 (lane 63's map applies first).
__device__ __forceinline__ void wave_scan_down(float& A, float& B, int lane) {
  A = lane_reverse(A, lane);
  B = lane_reverse(B, lane);
  wave_scan(A, B);
  A = lane_reverse(A, lane);
  B = lane_reverse(B, lane);
}

// Per-wave maps combined from the last wave down: every thread gets the
// composition of the waves after its own, the last one applied first.
template <int NW>
__device__ __forceinline__ void block_combine_down(float WA, float WB, BlockShared<NW>& s,
                                                   float& PA, float& PB) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  if (lane == 0) {
    s.wA[wid] = WA;
    s.wB[wid] = WB;
  }
  __syncthreads();
  PA = 1.0f;
  PB = 0.0f;
#pragma unroll
  for (int w = NW - 1; w >= 0; --w) {
    if (w > wid) {
      const float wa = s.wA[w], wb = s.wB[w];
      PB = __builtin_fmaf(wa, PB, wb);
      PA = PA * wa;
    }
  }
}

template <typename IO, int NW, int R, bool NTL, bool NTS, bool FULL>
__device__ __forceinline__ void scan_fused_chunk(const IO* __restrict__ a, const IO* b,
                                                 const float* __restrict__ h0, const IO* g,
                                                 IO* h, IO* __restrict__ da, IO* db,
                                                 float* __restrict__ dh0, int64_t T, int64_t ch,
                                                 int vec, BlockShared<NW>& s,
                                                 BlockShared<NW>& s2) {
  constexpr int S = R * 256;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const int64_t base = (int64_t)wid * S + 4 * lane;
  const IO* arow = a + ch * T;
  const IO* brow = b + ch * T;
  const IO* grow = g + ch * T;

  // a reads as 0 past the end: harmless for the forward (those steps are not
  // written) and the zero coefficient the backward needs after step T-1
  float4 a4[R], x4[R], g4[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    a4[r] = ld4<FULL, NTL>(arow, base + r * 256, T, vec, 0.0f);
    x4[r] = ld4<FULL, NTL>(brow, base + r * 256, T, vec, 0.0f);
    g4[r] = ld4<FULL, NTL>(grow, base + r * 256, T, vec, 0.0f);
  }
  // ---- forward: x4 turns from b into h
  float Ai[R], Bi[R], RA[R], RB[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float A = a4[r].x, B = x4[r].x;
    B = __builtin_fmaf(a4[r].y, B, x4[r].y); A = A * a4[r].y;
    B = __builtin_fmaf(a4[r].z, B, x4[r].z); A = A * a4[r].z;
    B = __builtin_fmaf(a4[r].w, B, x4[r].w); A = A * a4[r].w;
    wave_scan(A, B);
    Ai[r] = A; Bi[r] = B;
    RA[r] = readlane_f(A, kWave - 1);
    RB[r] = readlane_f(B, kWave - 1);
  }
  float WA, WB, PA, PB, TA, TB;
  chain_rows<R>(RA, RB, WA, WB);
  block_combine<NW>(WA, WB, s, PA, PB, TA, TB);
  const float x0 = h0 ? h0[ch] : 0.0f;
  const float h_before = __builtin_fmaf(PA, x0, PB);  // h entering this wave
  IO* hrow = h ? h + ch * T : nullptr;
  {
    float xr = h_before;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float x = wave_shift_up(__builtin_fmaf(Ai[r], xr, Bi[r]), xr);
      x = __builtin_fmaf(a4[r].x, x, x4[r].x); x4[r].x = x;
      x = __builtin_fmaf(a4[r].y, x, x4[r].y); x4[r].y = x;
      x = __builtin_fmaf(a4[r].z, x, x4[r].z); x4[r].z = x;
      x = __builtin_fmaf(a4[r].w, x, x4[r].w); x4[r].w = x;
      if (hrow) st4<FULL, NTS>(hrow, base + r * 256, T, vec, x4[r]);
      xr = __builtin_fmaf(RA[r], xr, RB[r]);
    }
  }
  // ---- backward: step p has coefficient a_{p+1}
  // a just past this wave's segment (the next wave's first step, 0 past T)
  const int64_t wend = base - 4 * lane + S;
  const float a_after = (wend < T) ? io_ld(arow, wend) : 0.0f;
  float an[R], hp[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float fa = (r < R - 1) ? readlane_f(a4[r + 1].x, 0) : a_after;
    an[r] = wave_shift_down(a4[r].x, fa);  // a after the group's last step
    const float fh = (r > 0) ? readlane_f(x4[r - 1].w, kWave - 1) : h_before;
    hp[r] = wave_shift_up(x4[r].w, fh);    // h before the group's first step
    float A = an[r], B = g4[r].w;
    B = __builtin_fmaf(a4[r].w, B, g4[r].z); A = A * a4[r].w;
    B = __builtin_fmaf(a4[r].z, B, g4[r].y); A = A * a4[r].z;
    B = __builtin_fmaf(a4[r].y, B, g4[r].x); A = A * a4[r].y;
    wave_scan_down(A, B, lane);
    Ai[r] = A; Bi[r] = B;
    RA[r] = readlane_f(A, 0);
    RB[r] = readlane_f(B, 0);
  }
  WA = RA[R - 1];
  WB = RB[R - 1];
#pragma unroll
  for (int r = R - 2; r >= 0; --r) {
    WB = __builtin_fmaf(RA[r], WB, RB[r]);
    WA = WA * RA[r];
  }
  block_combine_down<NW>(WA, WB, s2, PA, PB);
  float xr = PB;  // lam just past this wave's segment (lam past the channel is 0)
  IO* darow = da + ch * T;
  IO* dbrow = db + ch * T;
#pragma unroll
  for (int r = R - 1; r >= 0; --r) {
    const float x = wave_shift_down(__builtin_fmaf(Ai[r], xr, Bi[r]), xr);  // lam past the group
    const float l3 = __builtin_fmaf(an[r], x, g4[r].w);
    const float l2 = __builtin_fmaf(a4[r].w, l3, g4[r].z);
    const float l1 = __builtin_fmaf(a4[r].z, l2, g4[r].y);
    const float l0 = __builtin_fmaf(a4[r].y, l1, g4[r].x);
    const int64_t p = base + r * 256;
    st4<FULL, NTS>(darow, p, T, vec,
                   make_float4(l0 * hp[r], l1 * x4[r].x, l2 * x4[r].y, l3 * x4[r].z));
    st4<FULL, NTS>(dbrow, p, T, vec, make_float4(l0, l1, l2, l3));
    if (dh0 && p == 0) dh0[ch] = a4[r].x * l0;
    xr = __builtin_fmaf(RA[r], xr, RB[r]);
  }
}

template <typename IO, int NW, int R, bool NTL = false, bool NTS = false>
__global__ __launch_bounds__(NW* kWave) void k_scan_fused_bdt(
    const IO* __restrict__ a, const IO* b, const float* __restrict__ h0, const IO* g,
    IO* h, IO* __restrict__ da, IO* db, float* __restrict__ dh0, int64_t T, int vec) {
  constexpr int CH = NW * R * 256;
  __shared__ BlockShared<NW> s, s2;
  const int64_t ch = (int64_t)blockIdx.x;
  if (vec && (int64_t)CH <= T)
    scan_fused_chunk<IO, NW, R, NTL, NTS, true>(a, b, h0, g, h, da, db, dh0, T, ch, vec, s, s2);
  else
    scan_fused_chunk<IO, NW, R, NTL, NTS, false>(a, b, h0, g, h, da, db, dh0, T, ch, vec, s, s2);
}

// ---------------------------------------------------------------------------
// Short channels, packed: a workgroup takes k whole consecutive channels
// (k*T contiguous elements of the [B,D,T] arrays) and scans them as one
// sequence in which each channel's first step is a reset (coefficient 0,
// input a_1 h0 + b_1), so the single-chunk scan above yields every channel's
// own recurrence with fully coalesced rows, where the one-channel-per-
// workgroup kernels would leave most lanes idle.  The backward resets the
// other way: the coefficient after a channel's last step is 0, h before its
// first step is its h0, and grad_h0 is a_1 lam_1 of each channel.
// Positions inside the packed block are below 2^31 (k*T <= chunk size).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void set4(float4& v, int j, float x) {
  if (j == 0) v.x = x; else if (j == 1) v.y = x; else if (j == 2) v.z = x; else v.w = x;
}
__device__ __forceinline__ float get4(const float4& v, int j) {
  return j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w));
}

template <typename IO, int NW, int R>
__global__ __launch_bounds__(NW* kWave) void k_scan_fwd_packed(
    const IO* __restrict__ a, const IO* __restrict__ b, const float* __restrict__ h0,
    IO* __restrict__ h, int64_t T, int64_t C, int k, int vec) {
  constexpr int S = R * 256;
  __shared__ BlockShared<NW> s;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const int64_t c0 = (int64_t)blockIdx.x * k;
  const int64_t nch = (C - c0 < k) ? C - c0 : k;
  const int64_t len = nch * T;
  const IO* arow = a + c0 * T;
  const IO* brow = b + c0 * T;
  const uint32_t Tu = (uint32_t)T;
  const int64_t base = (int64_t)wid * S + 4 * lane;
  float4 a4[R], b4[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t p = base + r * 256;
    a4[r] = ld4<false, false>(arow, p, len, vec, 0.0f);
    b4[r] = ld4<false, false>(brow, p, len, vec, 0.0f);
    uint32_t m = (uint32_t)p % Tu, cl = (uint32_t)p / Tu;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (m == 0 && p + j < len) {  // channel start: reset, fold h0
        const float aj = get4(a4[r], j), bj = get4(b4[r], j);
        set4(b4[r], j, h0 ? __builtin_fmaf(aj, h0[c0 + cl], bj) : bj);
        set4(a4[r], j, 0.0f);
      }
      if (++m == Tu) { m = 0; ++cl; }
    }
  }
  float Ai[R], Bi[R], RA[R], RB[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float A = a4[r].x, B = b4[r].x;
    B = __builtin_fmaf(a4[r].y, B, b4[r].y); A = A * a4[r].y;
    B = __builtin_fmaf(a4[r].z, B, b4[r].z); A = A * a4[r].z;
    B = __builtin_fmaf(a4[r].w, B, b4[r].w); A = A * a4[r].w;
    wave_scan(A, B);
    Ai[r] = A; Bi[r] = B;
    RA[r] = readlane_f(A, kWave - 1);
    RB[r] = readlane_f(B, kWave - 1);
  }
  float WA, WB, PA, PB, TA, TB;
  chain_rows<R>(RA, RB, WA, WB);
  block_combine<NW>(WA, WB, s, PA, PB, TA, TB);
  float xr = PB;  // the block starts with a reset: no carry in
  IO* hrow = h + c0 * T;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float x = wave_shift_up(__builtin_fmaf(Ai[r], xr, Bi[r]), xr);
    float4 o;
    x = __builtin_fmaf(a4[r].x, x, b4[r].x); o.x = x;
    x = __builtin_fmaf(a4[r].y, x, b4[r].y); o.y = x;
    x = __builtin_fmaf(a4[r].z, x, b4[r].z); o.z = x;
    x = __builtin_fmaf(a4[r].w, x, b4[r].w); o.w = x;
    st4<false, false>(hrow, base + r * 256, len, vec, o);
    xr = __builtin_fmaf(RA[r], xr, RB[r]);
  }
}

template <typename IO, int NW, int R>
__global__ __launch_bounds__(NW* kWave) void k_scan_bwd_packed(
    const IO* __restrict__ a, const IO* __restrict__ h, const float* __restrict__ h0,
    const IO* g, IO* __restrict__ da, IO* db, float* __restrict__ dh0, int64_t T,
    int64_t C, int k, int vec) {
  constexpr int S = R * 256, CH = NW * S;
  __shared__ BlockShared<NW> s;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const int64_t c0 = (int64_t)blockIdx.x * k;
  const int64_t nch = (C - c0 < k) ? C - c0 : k;
  const int64_t len = nch * T;
  const IO* arow = a + c0 * T;
  const IO* hrow = h + c0 * T;
  const IO* grow = g + c0 * T;
  const uint32_t Tu = (uint32_t)T;
  const int64_t wend = (int64_t)CH - (int64_t)wid * S;  // end of this wave's segment
  const int64_t wbeg = wend - S;
  const int64_t pb = wend - 256 + 4 * (kWave - 1 - lane);  // this lane's group in row 0
  float4 a4[R], h4[R], g4[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t p = pb - r * 256;
    a4[r] = ld4<false, false>(arow, p, len, vec, 0.0f);
    h4[r] = ld4<false, false>(hrow, p, len, vec, 0.0f);
    g4[r] = ld4<false, false>(grow, p, len, vec, 0.0f);
    uint32_t m = (uint32_t)p % Tu;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (m == 0) set4(a4[r], j, 0.0f);  // no coefficient into a channel's first step
      if (++m == Tu) m = 0;
    }
  }
  const float a_after = (wend < len && (uint32_t)wend % Tu != 0) ? io_ld(arow, wend) : 0.0f;
  const float h_before = (wbeg > 0 && wbeg - 1 < len) ? io_ld(hrow, wbeg - 1) : 0.0f;
  float an[R], hp[R], Ai[R], Bi[R], RA[R], RB[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float fa = (r > 0) ? readlane_f(a4[r - 1].x, kWave - 1) : a_after;
    an[r] = wave_shift_up(a4[r].x, fa);
    const float fh = (r < R - 1) ? readlane_f(h4[r + 1].w, 0) : h_before;
    hp[r] = wave_shift_down(h4[r].w, fh);
    float A = an[r], B = g4[r].w;
    B = __builtin_fmaf(a4[r].w, B, g4[r].z); A = A * a4[r].w;
    B = __builtin_fmaf(a4[r].z, B, g4[r].y); A = A * a4[r].z;
    B = __builtin_fmaf(a4[r].y, B, g4[r].x); A = A * a4[r].y;
    wave_scan(A, B);
    Ai[r] = A; Bi[r] = B;
    RA[r] = readlane_f(A, kWave - 1);
    RB[r] = readlane_f(B, kWave - 1);
  }
  float WA, WB, PA, PB, TA, TB;
  chain_rows<R>(RA, RB, WA, WB);
  block_combine<NW>(WA, WB, s, PA, PB, TA, TB);
  float xr = PB;  // lam past the block is 0
  IO* darow = da + c0 * T;
  IO* dbrow = db + c0 * T;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float x = wave_shift_up(__builtin_fmaf(Ai[r], xr, Bi[r]), xr);
    float l[4];
    l[3] = __builtin_fmaf(an[r], x, g4[r].w);
    l[2] = __builtin_fmaf(a4[r].w, l[3], g4[r].z);
    l[1] = __builtin_fmaf(a4[r].z, l[2], g4[r].y);
    l[0] = __builtin_fmaf(a4[r].y, l[1], g4[r].x);
    const int64_t p = pb - r * 256;
    float hv[4] = {hp[r], h4[r].x, h4[r].y, h4[r].z};  // h before each step
    uint32_t m = (uint32_t)p % Tu, cl = (uint32_t)p / Tu;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (m == 0 && p + j < len) {  // a channel's first step: h before it is its h0
        const float x0 = h0 ? h0[c0 + cl] : 0.0f;
        hv[j] = x0;
        if (dh0) dh0[c0 + cl] = io_ld(arow, p + j) * l[j];
      }
      if (++m == Tu) { m = 0; ++cl; }
    }
    st4<false, false>(darow, p, len, vec,
                      make_float4(l[0] * hv[0], l[1] * hv[1], l[2] * hv[2], l[3] * hv[3]));
    st4<false, false>(dbrow, p, len, vec, make_float4(l[0], l[1], l[2], l[3]));
    xr = __builtin_fmaf(RA[r], xr, RB[r]);
  }
}

// ---------------------------------------------------------------------------
// Adjoint of the nonlinear RNN h_t = tanh(w h_{t-1} + u_t) at its solution h
// (the DEER solve's result): with s_t = 1 - h_t^2, the same reverse-time scan
// as k_scan_bwd_bdt with coefficient a_t = w s_t built from h on the fly,
//   lam_t = g_t + a_{t+1} lam_{t+1},   dL/du_t = s_t lam_t,   dL/dh0 = a_1 lam_1,
// and dL/dw[d] = sum over the batch and time of s_t lam_t h_{t-1}: each chunk
// writes its channel's partial sum (waves added in a fixed order), and a
// two-stage column sum over (chunk, batch) rows finishes it.  Reads h and g,
// writes dL/du: 12 bytes per element.
// ---------------------------------------------------------------------------
__device__ __forceinline__ double wave_sum_f64(double v) {
  // fixed butterfly order: every lane ends with the same, reproducible sum
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

template <int NW, int R, bool NT, bool FULL>
__device__ __forceinline__ void deer_bwd_chunk(const float* __restrict__ w,
                                               const float* __restrict__ h,
                                               const float* __restrict__ h0,
                                               const float* __restrict__ g,
                                               float* __restrict__ du, float* __restrict__ dh0,
                                               float* __restrict__ part, int64_t T, int64_t C,
                                               int64_t D, int64_t ch, int c, int pc, bool multi,
                                               int vec, uint64_t* st, BlockShared<NW>& s) {
  constexpr int S = R * 256, CH = NW * S;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const int64_t wend = (int64_t)(pc + 1) * CH - (int64_t)wid * S;  // physical end of the segment
  const int64_t wbeg = wend - S;
  const float wd = w[ch % D];
  const float* hrow = h + ch * T;
  const float* grow = g + ch * T;
  // a_p = w (1 - h_p^2) for p < T and 0 at and past T (no step after the end)
  auto coef = [&](float hv, int64_t p) {
    return (FULL || p < T) ? wd * __builtin_fmaf(-hv, hv, 1.0f) : 0.0f;
  };
  const int64_t pb = wend - 256 + 4 * (kWave - 1 - lane);  // this lane's group in row 0
  float4 h4[R], g4[R], a4[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    h4[r] = ld4<FULL, NT>(hrow, pb - r * 256, T, vec, 0.0f);
    g4[r] = ld4<FULL, NT>(grow, pb - r * 256, T, vec, 0.0f);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t p = pb - r * 256;
    a4[r] = make_float4(coef(h4[r].x, p), coef(h4[r].y, p + 1), coef(h4[r].z, p + 2),
                        coef(h4[r].w, p + 3));
  }
  const float x0h = h0 ? h0[ch] : 0.0f;
  // wave-edge halos (uniform): coefficient just past the segment, h just before it
  const float a_after = (wend < T) ? coef(hrow[wend], wend) : 0.0f;
  const float h_before = (wbeg > 0) ? ((wbeg - 1 < T) ? hrow[wbeg - 1] : 0.0f) : x0h;

  float an[R], hp[R], Ai[R], Bi[R], RA[R], RB[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float fa = (r > 0) ? readlane_f(a4[r - 1].x, kWave - 1) : a_after;
    an[r] = wave_shift_up(a4[r].x, fa);
    const float fh = (r < R - 1) ? readlane_f(h4[r + 1].w, 0) : h_before;
    hp[r] = wave_shift_down(h4[r].w, fh);  // h at the group's first step - 1
    float A = an[r], B = g4[r].w;
    B = __builtin_fmaf(a4[r].w, B, g4[r].z); A = A * a4[r].w;
    B = __builtin_fmaf(a4[r].z, B, g4[r].y); A = A * a4[r].z;
    B = __builtin_fmaf(a4[r].y, B, g4[r].x); A = A * a4[r].y;
    wave_scan(A, B);
    Ai[r] = A; Bi[r] = B;
    RA[r] = readlane_f(A, kWave - 1);
    RB[r] = readlane_f(B, kWave - 1);
  }
  float WA, WB, PA, PB, TA, TB;
  chain_rows<R>(RA, RB, WA, WB);
  block_combine<NW>(WA, WB, s, PA, PB, TA, TB);
  const float x_in = chunk_carry<NW>(multi, c, TA, TB, 0.0f, st, s);

  float xr = __builtin_fmaf(PA, x_in, PB);
  float* durow = du + ch * T;
  // this lane's part of sum s_t lam_t h_{t-1}, in fp64: a chunk adds up to
  // 16384 terms before the per-feature sum over the batch
  double acc = 0.0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float x = wave_shift_up(__builtin_fmaf(Ai[r], xr, Bi[r]), xr);  // lam past the group
    const float l3 = __builtin_fmaf(an[r], x, g4[r].w);
    const float l2 = __builtin_fmaf(a4[r].w, l3, g4[r].z);
    const float l1 = __builtin_fmaf(a4[r].z, l2, g4[r].y);
    const float l0 = __builtin_fmaf(a4[r].y, l1, g4[r].x);
    const float u0 = __builtin_fmaf(-h4[r].x, h4[r].x, 1.0f) * l0;
    const float u1 = __builtin_fmaf(-h4[r].y, h4[r].y, 1.0f) * l1;
    const float u2 = __builtin_fmaf(-h4[r].z, h4[r].z, 1.0f) * l2;
    const float u3 = __builtin_fmaf(-h4[r].w, h4[r].w, 1.0f) * l3;
    const int64_t p = pb - r * 256;
    st4<FULL, NT>(durow, p, T, vec, make_float4(u0, u1, u2, u3));
    // steps at or past T have lam = 0, so they add nothing
    acc += (double)(u0 * hp[r]) + (double)(u1 * h4[r].x) + (double)(u2 * h4[r].y) +
           (double)(u3 * h4[r].z);
    if (dh0 && p == 0) dh0[ch] = a4[r].x * l0;
    xr = __builtin_fmaf(RA[r], xr, RB[r]);
  }
  // per-chunk partial of dL/dw: lanes by a fixed butterfly, waves in order
  acc = wave_sum_f64(acc);
  __shared__ double wsum[NW];
  if (lane == 0) wsum[wid] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
#pragma unroll
    for (int i = 0; i < NW; ++i) t += wsum[i];
    part[(int64_t)c * C + ch] = (float)t;
  }
}

template <int NW, int R, bool NT = false, bool MULTI = false>
__global__ __launch_bounds__(NW* kWave) void k_deer_bwd(
    const float* __restrict__ w, const float* __restrict__ h, const float* __restrict__ h0,
    const float* __restrict__ g, float* __restrict__ du, float* __restrict__ dh0,
    float* __restrict__ part, int64_t T, int64_t C, int64_t D, int nchunk, int vec,
    uint64_t* __restrict__ status, unsigned* __restrict__ tickets) {
  constexpr int CH = NW * R * 256;
  __shared__ BlockShared<NW> s;
  constexpr bool multi = MULTI;
  const int64_t ch = multi ? chunk_channel(blockIdx.x, C, nchunk) : (int64_t)blockIdx.x;
  const int c = chunk_ticket<NW>(multi, tickets, ch, s);
  const int pc = nchunk - 1 - c;
  uint64_t* st = status + ch * nchunk;
  if (vec && (int64_t)(pc + 1) * CH <= T)
    deer_bwd_chunk<NW, R, NT, true>(w, h, h0, g, du, dh0, part, T, C, D, ch, c, pc, multi, vec,
                                    st, s);
  else
    deer_bwd_chunk<NW, R, NT, false>(w, h, h0, g, du, dh0, part, T, C, D, ch, c, pc, multi, vec,
                                     st, s);
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
// One chunk (chunk index c of the channel) of a DEER iteration.  x_start is
// the state entering the chunk when the caller knows it (multi == false);
// returns the state leaving the chunk and folds |y' - y| into dmax.
template <int NW, int R, bool FULL, bool NT>
__device__ __forceinline__ float deer_chunk(const float* __restrict__ w, const float* __restrict__ u,
                                            const float* __restrict__ y,
                                            const float* __restrict__ h0, float* __restrict__ yn,
                                            int64_t T, int64_t D, int64_t ch, int c, bool multi,
                                            float x_start, int vec, uint64_t* st,
                                            uint32_t& dmax, BlockShared<NW>& s) {
  constexpr int S = R * 256, CH = NW * S;
  // tanh(v) = 1 - 2 / (1 + 2^(v * 2 log2 e)); the scale is folded into w and u
  constexpr float k2l2e = 2.0f * 1.4426950408889634f;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const int64_t wbeg = (int64_t)c * CH + (int64_t)wid * S;
  const int64_t base = wbeg + 4 * lane;
  const float wd = w[ch % D];
  const float ws = wd * k2l2e;
  const float x0 = h0 ? h0[ch] : 0.0f;
  const float* urow = u + ch * T;
  const float* yrow = y ? y + ch * T : nullptr;

  float4 u4[R], y4[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    u4[r] = ld4<FULL, NT>(urow, base + r * 256, T, vec, 0.0f);
    y4[r] = yrow ? ld4<FULL, NT>(yrow, base + r * 256, T, vec, 0.0f)
                 : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // y just before the wave's segment (h0 at the start of the sequence)
  const float y_before = (wbeg > 0) ? ((yrow && wbeg - 1 < T) ? yrow[wbeg - 1] : 0.0f) : x0;

  // J = w (1 - z^2) and rhs = z - J y_{t-1} (z = tanh(w y_{t-1} + u_t)) are
  // kept for the output pass, which applies y'_t = J y'_{t-1} + rhs in lane
  // order from the scanned state.
  float Jv[R][4], rv[R][4], yf[R], Ai[R], Bi[R], RA[R], RB[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float fy = (r > 0) ? readlane_f(y4[r - 1].w, kWave - 1) : y_before;
    yf[r] = wave_shift_up(y4[r].w, fy);
    const float yp[4] = {yf[r], y4[r].x, y4[r].y, y4[r].z};
    const float uv[4] = {u4[r].x, u4[r].y, u4[r].z, u4[r].w};
    float J[4], rh[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(ws, yp[j], k2l2e * uv[j]));
      const float z = __builtin_fmaf(-2.0f, __builtin_amdgcn_rcpf(1.0f + e), 1.0f);
      J[j] = __builtin_fmaf(-wd * z, z, wd);    // w (1 - z^2)
      rh[j] = __builtin_fmaf(-J[j], yp[j], z);  // z - J y_{t-1}
    }
    if (!FULL) {
      const int64_t p = base + r * 256;
      if (p + 4 > T) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (p + j >= T) { J[j] = 1.0f; rh[j] = 0.0f; }
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) { Jv[r][j] = J[j]; rv[r][j] = rh[j]; }
    float A = J[0], B = rh[0];
#pragma unroll
    for (int j = 1; j < 4; ++j) {
      B = __builtin_fmaf(J[j], B, rh[j]);
      A = A * J[j];
    }
    wave_scan(A, B);
    Ai[r] = A; Bi[r] = B;
    RA[r] = readlane_f(A, kWave - 1);
    RB[r] = readlane_f(B, kWave - 1);
  }
  float WA, WB, PA, PB, TA, TB;
  chain_rows<R>(RA, RB, WA, WB);
  block_combine<NW>(WA, WB, s, PA, PB, TA, TB);
  const float x_in = multi ? chunk_carry<NW>(true, c, TA, TB, x0, st, s) : x_start;

  float xr = __builtin_fmaf(PA, x_in, PB);
  float* ynrow = yn + ch * T;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float x = wave_shift_up(__builtin_fmaf(Ai[r], xr, Bi[r]), xr);
    const int64_t p = base + r * 256;
    const float yo[4] = {y4[r].x, y4[r].y, y4[r].z, y4[r].w};
    float o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x = __builtin_fmaf(Jv[r][j], x, rv[r][j]);
      o[j] = x;
      const uint32_t d = as_u32(fabsf(x - yo[j]));
      if (FULL || p + j < T) dmax = d > dmax ? d : dmax;
    }
    st4<FULL, NT>(ynrow, p, T, vec, make_float4(o[0], o[1], o[2], o[3]));
    xr = __builtin_fmaf(RA[r], xr, RB[r]);
  }
  return __builtin_fmaf(TA, x_in, TB);
}

// The update norm of an iteration is accumulated in kDeltaSlots words on
// separate cache lines (workgroup b uses slot b % kDeltaSlots), so thousands of
// workgroups do not serialise on one atomic address.  Three such sets rotate:
// iteration i accumulates into set i % 3, reads the norm of iteration i - 1
// from set (i - 1) % 3, and its workgroup 0 clears set (i + 1) % 3 for the
// next iteration and stores the folded norm of iteration i - 1 in out[i - 1].
__device__ __forceinline__ uint32_t* delta_set(uint32_t* delta_bits, int iter) {
  return delta_bits + (iter % 3) * (kDeltaSlots * kDeltaStride);
}

// Fold a workgroup's max |y' - y| into its slot of the iteration.
template <int NW>
__device__ __forceinline__ void deer_publish_delta(uint32_t dmax, uint32_t* __restrict__ delta_bits,
                                                   int iter, BlockShared<NW>& s) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  dmax = wave_max_u32(dmax);
  if (lane == 0) s.wmax[wid] = dmax;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) m = s.wmax[i] > m ? s.wmax[i] : m;
    uint32_t* slot = delta_set(delta_bits, iter) + (blockIdx.x % kDeltaSlots) * kDeltaStride;
    __hip_atomic_fetch_max(slot, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Bookkeeping at the start of iteration iter > 0: every workgroup folds the
// previous iteration's slots (completed by the previous kernel, so plain loads
// see them) and gets the norm through LDS; workgroup 0 also records it and
// clears the set the next iteration accumulates into.
template <int NW>
__device__ __forceinline__ float deer_prev_delta(uint32_t* __restrict__ delta_bits,
                                                 uint32_t* __restrict__ delta_out, int iter,
                                                 BlockShared<NW>& s) {
  static_assert(kDeltaSlots == kWave, "one slot per lane");
  if (threadIdx.x < kWave) {
    uint32_t v = delta_set(delta_bits, iter - 1)[threadIdx.x * kDeltaStride];
    v = wave_max_u32(v);
    if (blockIdx.x == 0) {
      delta_set(delta_bits, iter + 1)[threadIdx.x * kDeltaStride] = 0u;
      if (threadIdx.x == 0) delta_out[iter - 1] = v;
    }
    if (threadIdx.x == 0) s.wmax[0] = v;
  }
  __syncthreads();
  const float d = as_f32(s.wmax[0]);
  __syncthreads();  // s.wmax is reused by deer_publish_delta
  return d;
}

// End of a solve (one wave): fold the last iteration's slots into
// out[k_max - 1] and write the solve record rec = {iterations performed,
// converged, last norm non-finite}.  An iteration counts as performed unless
// the one before it met the stop rule (it then exits on entry), so the count
// is one past the first norm below eps, or k_max.
__global__ __launch_bounds__(kWave) void k_deer_finish(const uint32_t* __restrict__ delta_bits,
                                                       uint32_t* __restrict__ out,
                                                       int* __restrict__ rec, int k_max,
                                                       float eps) {
  const int lane = threadIdx.x;
  const int last = k_max - 1;
  uint32_t v = delta_bits[(last % 3) * (kDeltaSlots * kDeltaStride) + lane * kDeltaStride];
  v = wave_max_u32(v);
  int first = k_max;  // first index with norm < eps
  for (int i0 = 0; i0 < k_max; i0 += kWave) {
    const int i = i0 + lane;
    const float d = (i < last) ? as_f32(out[i]) : as_f32(v);
    const uint64_t hit = __ballot(i < k_max && d < eps);
    if (hit) {
      first = i0 + (int)__builtin_ctzll(hit);
      break;
    }
  }
  if (lane == 0) {
    out[last] = v;
    const int iters = first < k_max ? first + 1 : k_max;
    const float d = (iters - 1 < last) ? as_f32(out[iters - 1]) : as_f32(v);
    rec[0] = iters;
    rec[1] = d < eps ? 1 : 0;
    rec[2] = (d - d != 0.0f) ? 1 : 0;  // NaN or infinite
  }
}

// Leave the solve's last iterate in h: it sits in p0 or p1 according to the
// parity of the iteration count; copy it unless that buffer is h.
__global__ __launch_bounds__(256) void k_deer_select(const float* __restrict__ p0,
                                                     const float* __restrict__ p1,
                                                     float* __restrict__ h, int64_t n,
                                                     const int* __restrict__ rec) {
  const float* src = ((rec[0] - 1) & 1) ? p1 : p0;
  if (src == h) return;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if ((((uintptr_t)src | (uintptr_t)h) & 15) == 0) {
    const int64_t n4 = n / 4;
    for (int64_t i = tid; i < n4; i += stride)
      reinterpret_cast<float4*>(h)[i] = reinterpret_cast<const float4*>(src)[i];
    for (int64_t i = n4 * 4 + tid; i < n; i += stride) h[i] = src[i];
  } else {
    for (int64_t i = tid; i < n; i += stride) h[i] = src[i];
  }
}

// MULTI: a channel spans several workgroups (look-back).  Otherwise one
// workgroup owns the whole channel and walks it as SUB sequential sub-chunks
// of NW*R*256 steps, carrying the state between them in registers (fewer
// registers than one tile of SUB times the rows, and no look-back).
//
// Per-sequence stopping (seq_slots != nullptr): every sequence (batch entry,
// D consecutive channels) keeps its own norm; a workgroup exits when its
// sequence's norm of the previous iteration (folded into seq_delta by
// k_deer_seq_book before this launch) met the stop rule, and folds its update
// into its sequence's slots instead of the global ones.
template <int NW, int R, bool MULTI = false, int SUB = 1, bool NT = false>
__global__ __launch_bounds__(NW* kWave) void k_deer_iter(
    const float* __restrict__ w, const float* __restrict__ u, const float* __restrict__ y,
    const float* __restrict__ h0, float* __restrict__ yn, int64_t T, int64_t C, int64_t D,
    int nchunk, int vec, uint64_t* __restrict__ status, unsigned* __restrict__ tickets,
    uint32_t* __restrict__ delta_bits, uint32_t* __restrict__ delta_out, int iter, float eps,
    uint32_t* __restrict__ seq_slots, const uint32_t* __restrict__ seq_delta, int k_max) {
  constexpr int CH = NW * R * 256;
  __shared__ BlockShared<NW> s;
  const int64_t ch0 = MULTI ? chunk_channel(blockIdx.x, C, nchunk) : (int64_t)blockIdx.x;
  const int64_t seq = ch0 / D;
  if (seq_slots) {
    if (iter > 0 && as_f32(seq_delta[seq * k_max + iter - 1]) < eps) return;
  } else if (iter > 0 && deer_prev_delta<NW>(delta_bits, delta_out, iter, s) < eps) {
    return;  // stop rule of the previous iteration (uniform across the whole grid)
  }
  uint32_t dmax = 0;
  if (MULTI) {
    const int64_t ch = ch0;
    const int c = chunk_ticket<NW>(true, tickets, ch, s);
    uint64_t* st = status + ch * nchunk;
    if (vec && (int64_t)(c + 1) * CH <= T)
      deer_chunk<NW, R, true, NT>(w, u, y, h0, yn, T, D, ch, c, true, 0.0f, vec, st, dmax, s);
    else
      deer_chunk<NW, R, false, NT>(w, u, y, h0, yn, T, D, ch, c, true, 0.0f, vec, st, dmax, s);
  } else {
    const int64_t ch = blockIdx.x;
    float x = h0 ? h0[ch] : 0.0f;
#pragma unroll 1
    for (int c = 0; c < SUB && (int64_t)c * CH < T; ++c) {
      if (c > 0) __syncthreads();  // LDS of the previous sub-chunk fully read
      if (vec && (int64_t)(c + 1) * CH <= T)
        x = deer_chunk<NW, R, true, NT>(w, u, y, h0, yn, T, D, ch, c, false, x, vec, nullptr, dmax, s);
      else
        x = deer_chunk<NW, R, false, NT>(w, u, y, h0, yn, T, D, ch, c, false, x, vec, nullptr, dmax, s);
    }
  }
  if (seq_slots) {
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    dmax = wave_max_u32(dmax);
    if (lane == 0) s.wmax[wid] = dmax;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < NW; ++i) m = s.wmax[i] > m ? s.wmax[i] : m;
      const int64_t nseq = C / D;
      uint32_t* slot = seq_slots + (int64_t)(iter % 3) * nseq * kSeqSlots * kDeltaStride +
                       (seq * kSeqSlots + (int64_t)(blockIdx.x % kSeqSlots)) * kDeltaStride;
      __hip_atomic_fetch_max(slot, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else {
    deer_publish_delta<NW>(dmax, delta_bits, iter, s);
  }
}

// ---------------------------------------------------------------------------
// DEER solve with the Newton iterations fused into one walk over each channel
// (channels that one workgroup walks as sequential sub-chunks).  For every
// sub-chunk the workgroup loads u, and the starting iterate if there is one,
// once, then computes iterates 1..m in order, each from the previous one held
// in registers.  Iteration k's scan state entering a sub-chunk comes from the
// previous sub-chunk (LDS slot xc[k]); it is also y_k at the step before the
// sub-chunk, which iteration k+1 needs, and inside a sub-chunk y_{k-1} at the
// step before a wave's first step is iteration k-1's state entering that wave
// (from the block combine).  Only the last iterate is stored: 8 bytes per
// element for the whole solve instead of 8 + 12 (m - 1).  The arithmetic of
// each iteration is that of k_deer_iter, and iteration k's max |y_k - y_{k-1}|
// is folded into slot set k - 1.  The global stop rule is known only after the
// pass, so the pass runs m = k_max iterations; when the rule stops the solve
// earlier (rec[0] < k_max, written by k_deer_fused_finish), a second launch
// with `redo` set recomputes exactly rec[0] iterations into h (any other redo
// launch returns at once).
// ---------------------------------------------------------------------------
template <int NW>
struct FusedShared {
  float2 wm[2][NW];                    // the waves' maps (A, B), by iteration parity
  float y0w[NW];                       // starting iterate at each wave's last step
  float xc[kDeerFuseMax + 1];          // iteration k's state entering the sub-chunk
  uint32_t dlane[kDeerFuseMax][NW * kWave];  // per-thread max |y_k - y_{k-1}|
  uint32_t dmax[kDeerFuseMax][NW];           // per-wave max, folded after the walk
};

// Applies the waves' maps in wave order to xin, the state entering the
// sub-chunk: returns the state entering this wave (wid is uniform, so the
// loop picks it up when it reaches it) and leaves the state after the last
// wave in xend.
template <int NW>
__device__ __forceinline__ float fused_combine(float WA, float WB, FusedShared<NW>& s, int par,
                                               float xin, float& xend) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if (lane == 0) s.wm[par][wid] = make_float2(WA, WB);
  __syncthreads();
  float x = xin, xr = xin;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (w == wid) xr = x;
    const float2 m = s.wm[par][w];
    x = __builtin_fmaf(m.x, x, m.y);
  }
  xend = x;
  return xr;
}

// One Newton iteration k of a sub-chunk of the fused solve: y_k (yout) from
// y_{k-1} (yin, held in registers); ent is y_{k-1} at the step before this
// wave's first step on entry and y_k there on exit.  max |y_k - y_{k-1}| over
// the thread's steps is folded into its slot of s.dlane[k - 1] with the NaN-propagating
// maximum (v_maximum3_f32), so a non-finite step still reads as the largest
// update: the bit pattern of a non-negative float or a NaN orders as unsigned.
template <int NW, int R, int E, bool FULL>
__device__ __forceinline__ void deer_fused_iter(int k, const float (&us)[R][E],
                                                const float (&yin)[R][E], float (&yout)[R][E],
                                                int64_t base, int64_t T, float ws, float wd,
                                                float& ent, int& par, FusedShared<NW>& s) {
  constexpr int RS = kWave * E;
  const float xin = s.xc[k];
  // J = w (1 - z^2) and rhs = z - J y_{t-1} per step, kept for the output pass
  float Jv[R][E], rv[R][E], Ai[R], Bi[R], RA[R], RB[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float fy = (r > 0) ? readlane_f(yin[r - 1][E - 1], kWave - 1) : ent;
    const float yf = wave_shift_up(yin[r][E - 1], fy);  // y_{t-1} at the lane's first step
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const float yp = j == 0 ? yf : yin[r][j - 1];
      const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(ws, yp, us[r][j]));
      const float z = __builtin_fmaf(-2.0f, __builtin_amdgcn_rcpf(1.0f + e), 1.0f);
      Jv[r][j] = __builtin_fmaf(-wd * z, z, wd);    // w (1 - z^2)
      rv[r][j] = __builtin_fmaf(-Jv[r][j], yp, z);  // z - J y_{t-1}
    }
    if (!FULL) {
      const int64_t p = base + r * RS;
#pragma unroll
      for (int j = 0; j < E; ++j)
        if (p + j >= T) { Jv[r][j] = 1.0f; rv[r][j] = 0.0f; }
    }
    float A = Jv[r][0], B = rv[r][0];
#pragma unroll
    for (int j = 1; j < E; ++j) {
      B = __builtin_fmaf(Jv[r][j], B, rv[r][j]);
      A = A * Jv[r][j];
    }
    wave_scan(A, B);
    Ai[r] = A; Bi[r] = B;
    RA[r] = readlane_f(A, kWave - 1);
    RB[r] = readlane_f(B, kWave - 1);
  }
  float WA, WB, xend;
  chain_rows<R>(RA, RB, WA, WB);
  // y_k at the step before this wave's first step
  float xr = fused_combine<NW>(WA, WB, s, par, xin, xend);
  par ^= 1;
  if (threadIdx.x == 0) s.xc[k] = xend;  // every thread read xin above
  ent = xr;
  float dmf = 0.0f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float x = wave_shift_up(__builtin_fmaf(Ai[r], xr, Bi[r]), xr);
    const int64_t p = base + r * RS;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      x = __builtin_fmaf(Jv[r][j], x, rv[r][j]);
      const float d = __builtin_elementwise_maximum(dmf, fabsf(x - yin[r][j]));
      dmf = (FULL || p + j < T) ? d : dmf;
      yout[r][j] = x;
    }
    xr = __builtin_fmaf(RA[r], xr, RB[r]);
  }
  // each thread folds into a slot of its own; the wave and block maxima are
  // taken once, after the last sub-chunk
  __hip_atomic_fetch_max(&s.dlane[k - 1][threadIdx.x], as_u32(dmf), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_WORKGROUP);
}

// One sub-chunk (index c) of the fused solve: iterations 1..m.  Each lane
// takes E consecutive steps (4 or 8) of each of the wave's R rows of 64 E
// steps.  y0last: the starting iterate at the previous sub-chunk's last step
// (updated for the next one); par: LDS parity of the wave maps (alternates per
// iteration).  Iterates alternate between two register sets, so each
// iteration writes its result in place of the one before the previous.
template <int NW, int R, int E, bool FULL, bool NT>
__device__ __forceinline__ void deer_fused_sub(const float* __restrict__ urow,
                                               const float* __restrict__ y0row,
                                               float* __restrict__ orow, int64_t T, int c,
                                               int vec, int m, float wd, float x0,
                                               float& y0last, int& par, FusedShared<NW>& s) {
  static_assert(E == 4 || E == 8, "4 or 8 steps per lane");
  constexpr int RS = kWave * E, S = R * RS, CH = NW * S;
  constexpr float k2l2e = 2.0f * 1.4426950408889634f;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const int64_t base = (int64_t)c * CH + (int64_t)wid * S + E * lane;
  const float ws = wd * k2l2e;
  float us[R][E], ya[R][E], yb[R][E];  // us: u scaled by 2 log2(e)
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int q = 0; q < E; q += 4) {
      const float4 u4 = ld4<FULL, NT>(urow, base + r * RS + q, T, vec, 0.0f);
      const float4 y4 = y0row ? ld4<FULL, NT>(y0row, base + r * RS + q, T, vec, 0.0f)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
      us[r][q] = k2l2e * u4.x; us[r][q + 1] = k2l2e * u4.y;
      us[r][q + 2] = k2l2e * u4.z; us[r][q + 3] = k2l2e * u4.w;
      ya[r][q] = y4.x; ya[r][q + 1] = y4.y; ya[r][q + 2] = y4.z; ya[r][q + 3] = y4.w;
    }
  }
  // starting iterate at the step before this wave's first step
  float ent;
  if (y0row) {
    if (lane == kWave - 1) s.y0w[wid] = ya[R - 1][E - 1];
    __syncthreads();
    ent = wid > 0 ? s.y0w[wid - 1] : (c == 0 ? x0 : y0last);
    y0last = s.y0w[NW - 1];  // read before any later write: the next writes follow a barrier
  } else {
    ent = (c == 0 && wid == 0) ? x0 : 0.0f;
    if (c > 0) __syncthreads();  // the previous sub-chunk's last carry write (m = 1) is seen
  }
  int k = 1;
#pragma unroll 1
  for (; k + 1 <= m; k += 2) {
    deer_fused_iter<NW, R, E, FULL>(k, us, ya, yb, base, T, ws, wd, ent, par, s);
    deer_fused_iter<NW, R, E, FULL>(k + 1, us, yb, ya, base, T, ws, wd, ent, par, s);
  }
  if (k <= m) {  // odd count: the last iterate goes to yb
    deer_fused_iter<NW, R, E, FULL>(k, us, ya, yb, base, T, ws, wd, ent, par, s);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < E; ++j) ya[r][j] = yb[r][j];
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int q = 0; q < E; q += 4)
      st4<FULL, NT>(orow, base + r * RS + q, T, vec,
                    make_float4(ya[r][q], ya[r][q + 1], ya[r][q + 2], ya[r][q + 3]));
}

// sets: k_max slot sets of kDeltaSlots words, kDeltaStride apart (redo: unused).
// Per-sequence stopping (seq != 0): the norms go to seq_delta[b * k_max + k]
// of the channel's sequence b (batch entry) and the redo reads that
// sequence's record rec[4 b] (as written by k_deer_seq_finish).
template <int NW, int R, int E, bool NT>
__device__ __forceinline__ void deer_fused_body(
    const float* __restrict__ w, const float* __restrict__ u, const float* __restrict__ y0,
    const float* __restrict__ h0, float* __restrict__ out, int64_t T, int64_t D, int vec,
    int k_max, uint32_t* __restrict__ sets, const int* __restrict__ rec, bool redo, bool seq,
    FusedShared<NW>& s) {
  constexpr int CH = NW * R * kWave * E;
  const int64_t ch = blockIdx.x;
  int m = k_max;
  if (redo) {
    m = seq ? rec[4 * (ch / D)] : rec[0];
    if (m < 1 || m >= k_max) return;  // the pass already holds the answer
  }
  const float wd = w[ch % D];
  const float x0 = h0 ? h0[ch] : 0.0f;
  if (threadIdx.x <= (unsigned)m) s.xc[threadIdx.x] = x0;  // every iteration starts from h0
#pragma unroll
  for (int i = 0; i < kDeerFuseMax; ++i) s.dlane[i][threadIdx.x] = 0u;
  __syncthreads();
  const float* urow = u + ch * T;
  const float* y0row = y0 ? y0 + ch * T : nullptr;
  float* orow = out + ch * T;
  const int64_t nsub = (T + CH - 1) / CH;
  float y0last = x0;
  int par = 0;
#pragma unroll 1
  for (int64_t c = 0; c < nsub; ++c) {
    if (vec && (c + 1) * CH <= T)
      deer_fused_sub<NW, R, E, true, NT>(urow, y0row, orow, T, (int)c, vec, m, wd, x0, y0last, par,
                                         s);
    else
      deer_fused_sub<NW, R, E, false, NT>(urow, y0row, orow, T, (int)c, vec, m, wd, x0, y0last,
                                          par, s);
  }
  if (redo) return;
  __syncthreads();
  {
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
#pragma unroll 1
    for (int k = 0; k < m; ++k) {
      const uint32_t v = wave_max_u32(s.dlane[k][threadIdx.x]);
      if (lane == 0) s.dmax[k][wid] = v;
    }
  }
  __syncthreads();
  if (threadIdx.x < (unsigned)m) {
    const int k = threadIdx.x;
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) v = s.dmax[k][i] > v ? s.dmax[k][i] : v;
    uint32_t* slot = seq ? sets + (ch / D) * k_max + k
                         : sets + (int64_t)k * (kDeltaSlots * kDeltaStride) +
                               (blockIdx.x % kDeltaSlots) * kDeltaStride;
    __hip_atomic_fetch_max(slot, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The pass over all k_max iterations.
template <int NW, int R, int E, bool NT>
__global__ __launch_bounds__(NW* kWave) void k_deer_fused(
    const float* __restrict__ w, const float* __restrict__ u, const float* __restrict__ y0,
    const float* __restrict__ h0, float* __restrict__ out, int64_t T, int64_t D, int vec,
    int k_max, uint32_t* __restrict__ sets, int seq) {
  __shared__ FusedShared<NW> s;
  deer_fused_body<NW, R, E, NT>(w, u, y0, h0, out, T, D, vec, k_max, sets, nullptr, false,
                                seq != 0, s);
}

// The recompute with the iteration count the stop rule gave (rec[0], or the
// sequence's rec[4 b]); returns at once when that count is k_max (the pass
// already holds the answer).
template <int NW, int R, int E, bool NT>
__global__ __launch_bounds__(NW* kWave) void k_deer_redo(
    const float* __restrict__ w, const float* __restrict__ u, const float* __restrict__ y0,
    const float* __restrict__ h0, float* __restrict__ out, int64_t T, int64_t D, int vec,
    int k_max, const int* __restrict__ rec, int seq) {
  __shared__ FusedShared<NW> s;
  deer_fused_body<NW, R, E, NT>(w, u, y0, h0, out, T, D, vec, k_max, nullptr, rec, true,
                                seq != 0, s);
}

// Per-sequence form of k_deer_fused_select (blockIdx.y = sequence of n floats):
// copy the pass's result for the sequences that ran to k_max.
__global__ __launch_bounds__(256) void k_deer_fused_seq_select(const float* __restrict__ src,
                                                               float* __restrict__ h, int64_t n,
                                                               const int* __restrict__ seq_rec,
                                                               int k_max) {
  const int64_t b = blockIdx.y;
  if (src == h || seq_rec[4 * b] != k_max) return;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    h[b * n + i] = src[b * n + i];
}

// After the fused pass (one wave): fold iteration k's slots into out[k], write
// the solve record as k_deer_finish does, and zero the norms of the
// iterations past the stop (the record reports only those performed).
__global__ __launch_bounds__(kWave) void k_deer_fused_finish(const uint32_t* __restrict__ sets,
                                                             uint32_t* __restrict__ out,
                                                             int* __restrict__ rec, int k_max,
                                                             float eps) {
  const int lane = threadIdx.x;
  int first = k_max;
  for (int k = 0; k < k_max; ++k) {
    const uint32_t v = wave_max_u32(sets[(int64_t)k * (kDeltaSlots * kDeltaStride) +
                                         lane * kDeltaStride]);
    if (lane == 0) out[k] = v;
    if (first == k_max && as_f32(v) < eps) first = k;
  }
  if (lane == 0) {
    const int iters = first < k_max ? first + 1 : k_max;
    const float d = as_f32(out[iters - 1]);
    for (int k = iters; k < k_max; ++k) out[k] = 0u;
    rec[0] = iters;
    rec[1] = d < eps ? 1 : 0;
    rec[2] = (d - d != 0.0f) ? 1 : 0;  // NaN or infinite
  }
}

// The fused pass wrote k_max iterations into src; leave them in h unless the
// redo launch already wrote the (earlier) answer there.
__global__ __launch_bounds__(256) void k_deer_fused_select(const float* __restrict__ src,
                                                           float* __restrict__ h, int64_t n,
                                                           const int* __restrict__ rec,
                                                           int k_max) {
  if (src == h || rec[0] != k_max) return;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    h[i] = src[i];
}

// Per-sequence bookkeeping before iteration iter (and once after the last):
// fold each sequence's slots of iteration iter - 1 into seq_delta[seq][iter - 1]
// and clear its slots of the set iteration iter + 1 will use.
__global__ __launch_bounds__(256) void k_deer_seq_book(uint32_t* __restrict__ seq_slots,
                                                       uint32_t* __restrict__ seq_delta,
                                                       int64_t nseq, int k_max, int iter) {
  const int64_t set = nseq * kSeqSlots * kDeltaStride;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nseq;
       b += (int64_t)gridDim.x * blockDim.x) {
    uint32_t v = 0;
    for (int k = 0; k < kSeqSlots; ++k) {
      const uint32_t x = seq_slots[(int64_t)((iter - 1) % 3) * set + (b * kSeqSlots + k) * kDeltaStride];
      v = x > v ? x : v;
      seq_slots[(int64_t)((iter + 1) % 3) * set + (b * kSeqSlots + k) * kDeltaStride] = 0u;
    }
    seq_delta[b * k_max + iter - 1] = v;
  }
}

// Per-sequence record {iterations, converged, non-finite, 0}: the iteration
// count is one past the first norm below eps, or k_max.
__global__ __launch_bounds__(256) void k_deer_seq_finish(const uint32_t* __restrict__ seq_delta,
                                                         int* __restrict__ seq_rec, int64_t nseq,
                                                         int k_max, float eps) {
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nseq;
       b += (int64_t)gridDim.x * blockDim.x) {
    int iters = k_max;
    for (int i = 0; i < k_max; ++i)
      if (as_f32(seq_delta[b * k_max + i]) < eps) { iters = i + 1; break; }
    const float d = as_f32(seq_delta[b * k_max + iters - 1]);
    seq_rec[4 * b + 0] = iters;
    seq_rec[4 * b + 1] = d < eps ? 1 : 0;
    seq_rec[4 * b + 2] = (d - d != 0.0f) ? 1 : 0;
    seq_rec[4 * b + 3] = 0;
  }
}

// Leave each sequence's last iterate in h (blockIdx.y = sequence of n floats).
__global__ __launch_bounds__(256) void k_deer_seq_select(const float* __restrict__ p0,
                                                         const float* __restrict__ p1,
                                                         float* __restrict__ h, int64_t n,
                                                         const int* __restrict__ seq_rec) {
  const int64_t b = blockIdx.y;
  const float* src = (((seq_rec[4 * b] - 1) & 1) ? p1 : p0) + b * n;
  float* dst = h + b * n;
  if (src == dst) return;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = src[i];
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
// Chunk shapes (waves x rows of 256 steps).  A channel that fits one chunk
// takes the smallest single-chunk shape that covers it (up to 8x4, 8192
// steps); a longer channel is split into chunks of the multi-chunk shape and
// uses the look-back.  Tile choices come from measured sweeps on MI355X: for
// long scans the chunk must be large enough to amortise the wait on its
// predecessors (8x4 forward, 16x4 backward: about 4 points of HBM bandwidth
// over 8x2 at 2^20 steps), but a 16-wave chunk holding a whole channel is slow
// (DEER backward at 8192 steps: 214 us as one 16x4 chunk, 125 us as 8x4); the
// DEER iteration keeps 8x2 chunks.
namespace {
struct Shape { int nw, r; };
constexpr Shape kScanSingle[] = {{1, 1}, {2, 1}, {4, 1}, {8, 1}, {8, 2}, {8, 4}};
constexpr Shape kScanFwdMulti = {8, 4};
constexpr Shape kScanBwdMulti = {16, 4};
// bf16 arrays (B=2, D=256, T=2^20): forward chunks of 8 x 8 rows with a wait
// every two rows, 582-594 us against 612-629 us for 8 x 4 (and 680 us for
// 8 x 8 waiting every row, 795-806 us for 16 x 4); the backward keeps 16 x 4
// (8 x 8: the same time, 16 x 2: 24% slower)
constexpr Shape kScanFwdMulti16 = {8, 8};
constexpr Shape kScanBwdMulti16 = {16, 4};
template <typename IO> constexpr Shape fwd_multi() { return sizeof(IO) == 2 ? kScanFwdMulti16 : kScanFwdMulti; }
template <typename IO> constexpr Shape bwd_multi() { return sizeof(IO) == 2 ? kScanBwdMulti16 : kScanBwdMulti; }
constexpr Shape kDeerSingle[] = {{1, 1}, {2, 1}, {4, 1}, {8, 1}, {8, 2}};
constexpr Shape kDeerMulti = {8, 2};
// sub-chunk shape of the fused solve for channels of more than 2048 steps
// (waves x rows).  With 4 steps per lane, measured at B=16 D=512 T=8192
// (solve time): 4x4 300 us, 1x4 301, 2x4 302, 2x2 306, 4x2 309-319, 4x1 331,
// 8x2 342, 8x1 364, 16x1 534.  The pass is bound by VALU issue; 8 steps per
// lane on 4x2 (the same 4096-step sub-chunk) halves the wave-scan work per
// step: 309 instead of 355 VALU per wave and iteration, 0.23 instead of
// 0.25 ms per solve.
constexpr Shape kDeerFused = {4, 2};  // with 8 steps per lane
// a DEER channel of up to kDeerSub chunks of the largest single shape stays in
// one workgroup, walked as sequential sub-chunks
constexpr int kDeerSub = 2;
template <size_t N>
RowPlan pick(int64_t T, const Shape (&single)[N], Shape multi) {
  RowPlan p;
  for (size_t i = 0; i < N; ++i) {
    const int64_t chunk = (int64_t)single[i].nw * single[i].r * 256;
    if (chunk >= T) {
      p.nw = single[i].nw;
      p.r = single[i].r;
      p.nchunk = 1;
      return p;
    }
  }
  // a multi-chunk shape larger than the channel would run it as one chunk of
  // 16 waves, which measured far slower than two chunks of the largest
  // single shape; those take over until the channel spans two multi chunks
  Shape m = multi;
  if ((int64_t)m.nw * m.r * 256 >= T) m = single[N - 1];
  p.nw = m.nw;
  p.r = m.r;
  p.nchunk = (T + p.chunk() - 1) / p.chunk();
  return p;
}
}  // namespace

// Short channels.  Measured on 2^24 elements (bench.py --crossover): the
// packed kernels (k whole channels per 2048-step workgroup) run at 76-82% of
// peak forward and 62-69% backward for every T up to 2048, against 3-43% /
// 4-53% for one channel per workgroup below T = 128 (T = 64: 31 vs 58 us
// forward, 63 vs 79 us backward; at T = 128 both forms are within 4%); the
// sequential kernels (one lane per channel) only beat them at T <= 4.  The
// caller's options may move both limits (e.g. 0 = never).
constexpr int64_t kSerialFwdMaxT = 4;
constexpr int64_t kSerialBwdMaxT = 4;
constexpr int64_t kPackedMaxT = 64;
constexpr int64_t kPackedSteps = 2048;  // 8 waves x 1 row of 256 steps

static int64_t limit_or(int64_t v, int64_t dflt) { return v >= 0 ? v : dflt; }

// Channels per packed workgroup: as many as fit, a multiple that keeps every
// block 16-byte aligned (k*T divisible by 4); 0 if none fits.
static int packed_channels(int64_t T) {
  if (T < 1 || T > kPackedSteps) return 0;
  int64_t k = kPackedSteps / T;
  const int64_t q = (T % 4 == 0) ? 1 : (T % 2 == 0 ? 2 : 4);
  k -= k % q;
  return (int)k;
}

static void plan_short(RowPlan& p, int64_t T, int64_t serial_max, int64_t packed_max) {
  p.serial = T <= serial_max;
  if (!p.serial && T <= packed_max) p.packed = packed_channels(T);
  if (p.serial || p.packed) {
    p.nchunk = 1;
    p.nw = 8;
    p.r = 1;
  }
}

RowPlan plan_scan_fwd_rows(int64_t C, int64_t T, const Opts& o, int io) {
  RowPlan p = pick(T, kScanSingle, io == kIoBf16 ? kScanFwdMulti16 : kScanFwdMulti);
  p.stream = 3 * C * T * io_bytes(io) >= kStreamFootprint;  // a, b, h
  plan_short(p, T, limit_or(o.serial_fwd_max_t, kSerialFwdMaxT),
             limit_or(o.packed_max_t, kPackedMaxT));
  return p;
}

RowPlan plan_scan_bwd_rows(int64_t C, int64_t T, const Opts& o, int io) {
  RowPlan p = pick(T, kScanSingle, io == kIoBf16 ? kScanBwdMulti16 : kScanBwdMulti);
  p.stream = 5 * C * T * io_bytes(io) >= kStreamFootprint;  // a, h, g, grad_a, grad_b
  plan_short(p, T, limit_or(o.serial_bwd_max_t, kSerialBwdMaxT),
             limit_or(o.packed_max_t, kPackedMaxT));
  return p;
}

RowPlan plan_deer_bwd_rows(int64_t C, int64_t T) {
  RowPlan p = pick(T, kScanSingle, kScanBwdMulti);
  p.stream = 3 * C * T * 4 >= kStreamFootprint;  // h, g, grad_u
  return p;
}

// Fused forward + backward: single-chunk shapes only (nchunk > 1 = not fusable).
RowPlan plan_scan_fused_rows(int64_t C, int64_t T, int io) {
  RowPlan p = pick(T, kScanSingle, kScanFwdMulti);
  p.stream = 6 * C * T * io_bytes(io) >= kStreamFootprint;  // a, b, g, h, grad_a, grad_b
  return p;
}

RowPlan plan_deer_rows(int64_t C, int64_t T) {
  RowPlan p = pick(T, kDeerSingle, kDeerMulti);
  p.stream = 3 * C * T * 4 >= kStreamFootprint;  // u, y, y'

  p.sub = 1;
  if (p.nchunk > 1 && p.nchunk <= kDeerSub) {  // one workgroup walks the channel
    p.sub = (int)p.nchunk;
    p.nchunk = 1;
  }
  return p;
}

// Dispatch on the (waves, rows) shape and the streaming flag.
#define LRS_SHAPE_CASE(NW_, R_, ...) \
  if (p.nw == NW_ && p.r == R_) { constexpr int NW = NW_, RR = R_; __VA_ARGS__; return hipGetLastError(); }

template <typename IO>
static hipError_t scan_fwd_bdt_io(const IO* a, const IO* b, const float* h0, IO* h, int64_t C,
                                  int64_t T, const RowPlan& p, int vec, uint64_t* status,
                                  unsigned* tickets, hipStream_t stream) {
  const dim3 grid((unsigned)((uint64_t)C * (uint64_t)p.nchunk));
#define LRS_FWD(NTF, M) hipLaunchKernelGGL((k_scan_fwd_bdt<IO, NW, RR, NTF, NTF, M>), grid, dim3(NW * kWave), \
                                           0, stream, a, b, h0, h, T, C, (int)p.nchunk, vec, status, \
                                           tickets)
  constexpr Shape M = fwd_multi<IO>();
  if (p.nchunk > 1) {  // the multi shape, or 8x4 chunks for channels under two of them
    if (p.stream) {
      LRS_SHAPE_CASE(M.nw, M.r, LRS_FWD(true, true))
      LRS_SHAPE_CASE(8, 4, LRS_FWD(true, true))
    } else {
      LRS_SHAPE_CASE(M.nw, M.r, LRS_FWD(false, true))
      LRS_SHAPE_CASE(8, 4, LRS_FWD(false, true))
    }
  } else if (p.stream) {
    LRS_SHAPE_CASE(1, 1, LRS_FWD(true, false))
    LRS_SHAPE_CASE(2, 1, LRS_FWD(true, false))
    LRS_SHAPE_CASE(4, 1, LRS_FWD(true, false))
    LRS_SHAPE_CASE(8, 1, LRS_FWD(true, false))
    LRS_SHAPE_CASE(8, 2, LRS_FWD(true, false))
    LRS_SHAPE_CASE(8, 4, LRS_FWD(true, false))
  } else {
    LRS_SHAPE_CASE(1, 1, LRS_FWD(false, false))
    LRS_SHAPE_CASE(2, 1, LRS_FWD(false, false))
    LRS_SHAPE_CASE(4, 1, LRS_FWD(false, false))
    LRS_SHAPE_CASE(8, 1, LRS_FWD(false, false))
    LRS_SHAPE_CASE(8, 2, LRS_FWD(false, false))
    LRS_SHAPE_CASE(8, 4, LRS_FWD(false, false))
  }
#undef LRS_FWD
  return hipErrorInvalidValue;
}

hipError_t launch_scan_fwd_bdt(const void* a, const void* b, const float* h0, void* h, int io,
                               int64_t C, int64_t T, const RowPlan& p, int vec,
                               uint64_t* status, unsigned* tickets, hipStream_t stream) {
  if (p.serial) return launch_scan_fwd_serial(a, b, h0, h, io, C, T, vec, stream);
  if (p.packed) return launch_scan_fwd_packed(a, b, h0, h, io, C, T, p.packed, vec, stream);
  if (io == kIoBf16)
    return scan_fwd_bdt_io((const uint16_t*)a, (const uint16_t*)b, h0, (uint16_t*)h, C, T, p, vec,
                           status, tickets, stream);
  return scan_fwd_bdt_io((const float*)a, (const float*)b, h0, (float*)h, C, T, p, vec, status,
                         tickets, stream);
}

template <typename IO>
static hipError_t scan_bwd_bdt_io(const IO* a, const IO* h, const float* h0, const IO* g, IO* da,
                                  IO* db, float* dh0, int64_t C, int64_t T, const RowPlan& p,
                                  int vec, uint64_t* status, unsigned* tickets,
                                  hipStream_t stream) {
  const dim3 grid((unsigned)((uint64_t)C * (uint64_t)p.nchunk));
#define LRS_BWD(NTF, M) hipLaunchKernelGGL((k_scan_bwd_bdt<IO, NW, RR, NTF, NTF, M>), grid, dim3(NW * kWave), \
                                           0, stream, a, h, h0, g, da, db, dh0, T, C, (int)p.nchunk, \
                                           vec, status, tickets)
  constexpr Shape M = bwd_multi<IO>();
  if (p.nchunk > 1) {  // the multi shape, or 8x4 chunks for channels under two of them
    if (p.stream) {
      LRS_SHAPE_CASE(M.nw, M.r, LRS_BWD(true, true))
      LRS_SHAPE_CASE(8, 4, LRS_BWD(true, true))
    } else {
      LRS_SHAPE_CASE(M.nw, M.r, LRS_BWD(false, true))
      LRS_SHAPE_CASE(8, 4, LRS_BWD(false, true))
    }
  } else if (p.stream) {
    LRS_SHAPE_CASE(1, 1, LRS_BWD(true, false))
    LRS_SHAPE_CASE(2, 1, LRS_BWD(true, false))
    LRS_SHAPE_CASE(4, 1, LRS_BWD(true, false))
    LRS_SHAPE_CASE(8, 1, LRS_BWD(true, false))
    LRS_SHAPE_CASE(8, 2, LRS_BWD(true, false))
    LRS_SHAPE_CASE(8, 4, LRS_BWD(true, false))
  } else {
    LRS_SHAPE_CASE(1, 1, LRS_BWD(false, false))
    LRS_SHAPE_CASE(2, 1, LRS_BWD(false, false))
    LRS_SHAPE_CASE(4, 1, LRS_BWD(false, false))
    LRS_SHAPE_CASE(8, 1, LRS_BWD(false, false))
    LRS_SHAPE_CASE(8, 2, LRS_BWD(false, false))
    LRS_SHAPE_CASE(8, 4, LRS_BWD(false, false))
  }
#undef LRS_BWD
  return hipErrorInvalidValue;
}

hipError_t launch_scan_bwd_bdt(const void* a, const void* h, const float* h0, const void* g,
                               void* da, void* db, float* dh0, int io, int64_t C, int64_t T,
                               const RowPlan& p, int vec, uint64_t* status, unsigned* tickets,
                               hipStream_t stream) {
  if (p.serial) return launch_scan_bwd_serial(a, h, h0, g, da, db, dh0, io, C, T, vec, stream);
  if (p.packed)
    return launch_scan_bwd_packed(a, h, h0, g, da, db, dh0, io, C, T, p.packed, vec, stream);
  if (io == kIoBf16)
    return scan_bwd_bdt_io((const uint16_t*)a, (const uint16_t*)h, h0, (const uint16_t*)g,
                           (uint16_t*)da, (uint16_t*)db, dh0, C, T, p, vec, status, tickets,
                           stream);
  return scan_bwd_bdt_io((const float*)a, (const float*)h, h0, (const float*)g, (float*)da,
                         (float*)db, dh0, C, T, p, vec, status, tickets, stream);
}

hipError_t launch_scan_fwd_packed(const void* a, const void* b, const float* h0, void* h, int io,
                                  int64_t C, int64_t T, int k, int vec, hipStream_t stream) {
  const dim3 grid((unsigned)((C + k - 1) / k));
  if (io == kIoBf16)
    hipLaunchKernelGGL((k_scan_fwd_packed<uint16_t, 8, 1>), grid, dim3(8 * kWave), 0, stream,
                       (const uint16_t*)a, (const uint16_t*)b, h0, (uint16_t*)h, T, C, k, vec);
  else
    hipLaunchKernelGGL((k_scan_fwd_packed<float, 8, 1>), grid, dim3(8 * kWave), 0, stream,
                       (const float*)a, (const float*)b, h0, (float*)h, T, C, k, vec);
  return hipGetLastError();
}

hipError_t launch_scan_bwd_packed(const void* a, const void* h, const float* h0, const void* g,
                                  void* da, void* db, float* dh0, int io, int64_t C, int64_t T,
                                  int k, int vec, hipStream_t stream) {
  const dim3 grid((unsigned)((C + k - 1) / k));
  if (io == kIoBf16)
    hipLaunchKernelGGL((k_scan_bwd_packed<uint16_t, 8, 1>), grid, dim3(8 * kWave), 0, stream,
                       (const uint16_t*)a, (const uint16_t*)h, h0, (const uint16_t*)g,
                       (uint16_t*)da, (uint16_t*)db, dh0, T, C, k, vec);
  else
    hipLaunchKernelGGL((k_scan_bwd_packed<float, 8, 1>), grid, dim3(8 * kWave), 0, stream,
                       (const float*)a, (const float*)h, h0, (const float*)g, (float*)da,
                       (float*)db, dh0, T, C, k, vec);
  return hipGetLastError();
}

template <typename IO>
static hipError_t scan_fused_bdt_io(const IO* a, const IO* b, const float* h0, const IO* g, IO* h,
                                    IO* da, IO* db, float* dh0, int64_t C, int64_t T,
                                    const RowPlan& p, int vec, hipStream_t stream) {
  const dim3 grid((unsigned)C);
  // nontemporal loads always (cold and warm calls measured no slower, warm
  // B=8 D=512 T=4096 calls 19% faster); nontemporal stores only for calls far
  // larger than the caches (steady-state 74% vs 70% of peak at 1.5 GiB)
#define LRS_FUSED(NTF) hipLaunchKernelGGL((k_scan_fused_bdt<IO, NW, RR, true, NTF>), grid, \
                                          dim3(NW * kWave), 0, stream, a, b, h0, g, h, da, db, dh0, T, vec)
  if (p.stream) {
    LRS_SHAPE_CASE(1, 1, LRS_FUSED(true))
    LRS_SHAPE_CASE(2, 1, LRS_FUSED(true))
    LRS_SHAPE_CASE(4, 1, LRS_FUSED(true))
    LRS_SHAPE_CASE(8, 1, LRS_FUSED(true))
    LRS_SHAPE_CASE(8, 2, LRS_FUSED(true))
    LRS_SHAPE_CASE(8, 4, LRS_FUSED(true))
  } else {
    LRS_SHAPE_CASE(1, 1, LRS_FUSED(false))
    LRS_SHAPE_CASE(2, 1, LRS_FUSED(false))
    LRS_SHAPE_CASE(4, 1, LRS_FUSED(false))
    LRS_SHAPE_CASE(8, 1, LRS_FUSED(false))
    LRS_SHAPE_CASE(8, 2, LRS_FUSED(false))
    LRS_SHAPE_CASE(8, 4, LRS_FUSED(false))
  }
#undef LRS_FUSED
  return hipErrorInvalidValue;
}

hipError_t launch_scan_fused_bdt(const void* a, const void* b, const float* h0, const void* g,
                                 void* h, void* da, void* db, float* dh0, int io, int64_t C,
                                 int64_t T, const RowPlan& p, int vec, hipStream_t stream) {
  if (p.nchunk != 1) return hipErrorInvalidValue;
  if (io == kIoBf16)
    return scan_fused_bdt_io((const uint16_t*)a, (const uint16_t*)b, h0, (const uint16_t*)g,
                             (uint16_t*)h, (uint16_t*)da, (uint16_t*)db, dh0, C, T, p, vec,
                             stream);
  return scan_fused_bdt_io((const float*)a, (const float*)b, h0, (const float*)g, (float*)h,
                           (float*)da, (float*)db, dh0, C, T, p, vec, stream);
}

hipError_t launch_deer_bwd(const float* w, const float* h, const float* h0, const float* g,
                           float* du, float* dw, float* dh0, float* part, double* acc, int64_t B,
                           int64_t D, int64_t T, const RowPlan& p, int vec, uint64_t* status,
                           unsigned* tickets, hipStream_t stream) {
  const int64_t C = B * D;
  const dim3 grid((unsigned)((uint64_t)C * (uint64_t)p.nchunk));
  hipError_t e = hipErrorInvalidValue;
#define LRS_DB(NTF, M) hipLaunchKernelGGL((k_deer_bwd<NW, RR, NTF, M>), grid, dim3(NW * kWave), 0, \
                                          stream, w, h, h0, g, du, dh0, part, T, C, D,         \
                                          (int)p.nchunk, vec, status, tickets)
#define LRS_DB_CASE(NW_, R_, ...) \
  if (p.nw == NW_ && p.r == R_) { constexpr int NW = NW_, RR = R_; __VA_ARGS__; e = hipGetLastError(); }
  if (p.nchunk > 1) {
    if (p.stream) {
      LRS_DB_CASE(kScanBwdMulti.nw, kScanBwdMulti.r, LRS_DB(true, true))
      else LRS_DB_CASE(8, 4, LRS_DB(true, true))
    } else {
      LRS_DB_CASE(kScanBwdMulti.nw, kScanBwdMulti.r, LRS_DB(false, true))
      else LRS_DB_CASE(8, 4, LRS_DB(false, true))
    }
  } else if (p.stream) {
    LRS_DB_CASE(1, 1, LRS_DB(true, false)) else LRS_DB_CASE(2, 1, LRS_DB(true, false))
    else LRS_DB_CASE(4, 1, LRS_DB(true, false)) else LRS_DB_CASE(8, 1, LRS_DB(true, false))
    else LRS_DB_CASE(8, 2, LRS_DB(true, false))
    else LRS_DB_CASE(8, 4, LRS_DB(true, false))
  } else {
    LRS_DB_CASE(1, 1, LRS_DB(false, false)) else LRS_DB_CASE(2, 1, LRS_DB(false, false))
    else LRS_DB_CASE(4, 1, LRS_DB(false, false)) else LRS_DB_CASE(8, 1, LRS_DB(false, false))
    else LRS_DB_CASE(8, 2, LRS_DB(false, false))
    else LRS_DB_CASE(8, 4, LRS_DB(false, false))
  }
#undef LRS_DB_CASE
#undef LRS_DB
  if (e != hipSuccess) return e;
  return launch_col_sums(part, 1, p.nchunk * B, D, acc, dw, nullptr, stream);
}

hipError_t launch_deer_finish(const uint32_t* delta_bits, uint32_t* delta_out, int* rec,
                              int k_max, float eps, hipStream_t stream) {
  hipLaunchKernelGGL(k_deer_finish, dim3(1), dim3(kWave), 0, stream, delta_bits, delta_out, rec,
                     k_max, eps);
  return hipGetLastError();
}

hipError_t launch_deer_select(const float* p0, const float* p1, float* h, int64_t n,
                              const int* rec, hipStream_t stream) {
  int64_t blocks = (n / 4 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(k_deer_select, dim3((unsigned)blocks), dim3(256), 0, stream, p0, p1, h, n,
                     rec);
  return hipGetLastError();
}

hipError_t launch_deer_iter(const float* w, const float* u, const float* y, const float* h0,
                            float* yn, int64_t C, int64_t D, int64_t T, const RowPlan& p, int vec,
                            uint64_t* status, unsigned* tickets, uint32_t* delta_bits,
                            uint32_t* delta_out, int iter, float eps, hipStream_t stream,
                            uint32_t* seq_slots, const uint32_t* seq_delta, int k_max) {
  const dim3 grid((unsigned)((uint64_t)C * (uint64_t)p.nchunk));
#define LRS_DEER(M, SB, NTF) hipLaunchKernelGGL((k_deer_iter<NW, RR, M, SB, NTF>), grid, dim3(NW * kWave), \
                                                0, stream, w, u, y, h0, yn, T, C, D, (int)p.nchunk, \
                                                vec, status, tickets, delta_bits, delta_out, iter, eps, \
                                                seq_slots, seq_delta, k_max)
  // the first iteration from y = 0 reads u only and is slightly faster with
  // the default policy
  const bool nt = p.stream && y != nullptr;
  if (p.nchunk > 1) {
    if (nt) { LRS_SHAPE_CASE(kDeerMulti.nw, kDeerMulti.r, LRS_DEER(true, 1, true)) }
    else { LRS_SHAPE_CASE(kDeerMulti.nw, kDeerMulti.r, LRS_DEER(true, 1, false)) }
  } else if (p.sub == 2) {
    if (nt) { LRS_SHAPE_CASE(8, 2, LRS_DEER(false, 2, true)) }
    else { LRS_SHAPE_CASE(8, 2, LRS_DEER(false, 2, false)) }
  } else if (nt) {
    LRS_SHAPE_CASE(1, 1, LRS_DEER(false, 1, true))
    LRS_SHAPE_CASE(2, 1, LRS_DEER(false, 1, true))
    LRS_SHAPE_CASE(4, 1, LRS_DEER(false, 1, true))
    LRS_SHAPE_CASE(8, 1, LRS_DEER(false, 1, true))
    LRS_SHAPE_CASE(8, 2, LRS_DEER(false, 1, true))
  } else {
    LRS_SHAPE_CASE(1, 1, LRS_DEER(false, 1, false))
    LRS_SHAPE_CASE(2, 1, LRS_DEER(false, 1, false))
    LRS_SHAPE_CASE(4, 1, LRS_DEER(false, 1, false))
    LRS_SHAPE_CASE(8, 1, LRS_DEER(false, 1, false))
    LRS_SHAPE_CASE(8, 2, LRS_DEER(false, 1, false))
  }
#undef LRS_DEER
  return hipErrorInvalidValue;
}

// Fused solve (see k_deer_fused): the pass, the finish, the redo and the select.
hipError_t launch_deer_fused(const float* w, const float* u, const float* y0, const float* h0,
                             float* out, float* h, int64_t C, int64_t D, int64_t T,
                             const RowPlan& plan, int vec, int k_max, float eps, uint32_t* sets,
                             uint32_t* delta_out, int* rec, hipStream_t stream,
                             uint32_t* seq_delta, int* seq_rec) {
  const dim3 grid((unsigned)C);
  if (seq_rec) rec = seq_rec;  // the redo reads the per-sequence records
  // channels of more than 2048 steps take the fused shape (4 waves of 2 rows
  // of 8 steps per lane, walking the channel as 4096-step sub-chunks); those
  // of 513 to 2048 steps one sub-chunk of 2 rows of 8 steps per lane on 2
  // waves or 1 (2048 or 1024 steps); shorter ones keep the plan's smallest
  // covering shape with 4 steps per lane
  RowPlan p = plan;
  const int e8 = T > 2048 ? 4 : T > 1024 ? 2 : T > 512 ? 1 : 0;  // waves of the 8-step shape
#define LRS_FUSED_DEER(E, NTF, OUT, REDO)                                                         \
  if (REDO)                                                                                        \
    hipLaunchKernelGGL((k_deer_redo<NW, RR, E, NTF>), grid, dim3(NW * kWave), 0, stream, w, u, y0, \
                       h0, OUT, T, D, vec, k_max, rec, seq_rec ? 1 : 0);                           \
  else                                                                                             \
    hipLaunchKernelGGL((k_deer_fused<NW, RR, E, NTF>), grid, dim3(NW * kWave), 0, stream, w, u,   \
                       y0, h0, OUT, T, D, vec, k_max, seq_rec ? seq_delta : sets,                  \
                       seq_rec ? 1 : 0)
#define LRS_FUSED_E8(NW_, NTF, OUT, REDO)                                           \
  if (e8 == NW_) {                                                                 \
    constexpr int NW = NW_, RR = kDeerFused.r;                                     \
    LRS_FUSED_DEER(8, NTF, OUT, REDO);                                             \
    return hipGetLastError();                                                      \
  }
#define LRS_FUSED_WIDE(NTF, OUT, REDO)                                             \
  {                                                                                \
    LRS_FUSED_E8(kDeerFused.nw, NTF, OUT, REDO)                                    \
    LRS_FUSED_E8(2, NTF, OUT, REDO)                                                \
    LRS_FUSED_E8(1, NTF, OUT, REDO)                                                \
  }
#define LRS_FUSED_SHAPES(OUT, REDO)                                 \
  if (p.stream) {                                                   \
    if (e8) LRS_FUSED_WIDE(true, OUT, REDO)                         \
    LRS_SHAPE_CASE(1, 1, LRS_FUSED_DEER(4, true, OUT, REDO))        \
    LRS_SHAPE_CASE(2, 1, LRS_FUSED_DEER(4, true, OUT, REDO))        \
    LRS_SHAPE_CASE(4, 1, LRS_FUSED_DEER(4, true, OUT, REDO))        \
    LRS_SHAPE_CASE(8, 1, LRS_FUSED_DEER(4, true, OUT, REDO))        \
    LRS_SHAPE_CASE(8, 2, LRS_FUSED_DEER(4, true, OUT, REDO))        \
    LRS_SHAPE_CASE(4, 4, LRS_FUSED_DEER(4, true, OUT, REDO))        \
  } else {                                                          \
    if (e8) LRS_FUSED_WIDE(false, OUT, REDO)                        \
    LRS_SHAPE_CASE(1, 1, LRS_FUSED_DEER(4, false, OUT, REDO))       \
    LRS_SHAPE_CASE(2, 1, LRS_FUSED_DEER(4, false, OUT, REDO))       \
    LRS_SHAPE_CASE(4, 1, LRS_FUSED_DEER(4, false, OUT, REDO))       \
    LRS_SHAPE_CASE(8, 1, LRS_FUSED_DEER(4, false, OUT, REDO))       \
    LRS_SHAPE_CASE(8, 2, LRS_FUSED_DEER(4, false, OUT, REDO))       \
    LRS_SHAPE_CASE(4, 4, LRS_FUSED_DEER(4, false, OUT, REDO))       \
  }                                                                 \
  return hipErrorInvalidValue;
  auto pass = [&]() -> hipError_t { LRS_FUSED_SHAPES(out, 0) };
  auto redo = [&]() -> hipError_t { LRS_FUSED_SHAPES(h, 1) };
#undef LRS_FUSED_SHAPES
#undef LRS_FUSED_WIDE
#undef LRS_FUSED_E8
#undef LRS_FUSED_DEER
  hipError_t e = pass();
  if (e != hipSuccess) return e;
  if (seq_rec) {  // per-sequence stopping
    const int64_t nseq = C / D;
    if ((e = launch_deer_seq_finish(seq_delta, seq_rec, nseq, k_max, eps, stream)) != hipSuccess)
      return e;
    e = redo();
    if (e != hipSuccess || out == h) return e;
    const int64_t n = D * T;
    const dim3 sgrid((unsigned)std::min<int64_t>((n + 255) / 256, 1024), (unsigned)nseq);
    hipLaunchKernelGGL(k_deer_fused_seq_select, sgrid, dim3(256), 0, stream, out, h, n, seq_rec,
                       k_max);
    return hipGetLastError();
  }
  if ((e = launch_deer_fused_finish(sets, delta_out, rec, k_max, eps, stream)) != hipSuccess)
    return e;
  e = redo();
  if (e != hipSuccess) return e;
  return launch_deer_fused_select(out, h, C * T, rec, k_max, stream);
}

hipError_t launch_deer_fused_finish(const uint32_t* sets, uint32_t* delta_out, int* rec,
                                    int k_max, float eps, hipStream_t stream) {
  hipLaunchKernelGGL(k_deer_fused_finish, dim3(1), dim3(kWave), 0, stream, sets, delta_out, rec,
                     k_max, eps);
  return hipGetLastError();
}

hipError_t launch_deer_fused_select(const float* src, float* h, int64_t n, const int* rec,
                                    int k_max, hipStream_t stream) {
  if (src == h) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(k_deer_fused_select, dim3((unsigned)blocks), dim3(256), 0, stream, src, h, n,
                     rec, k_max);
  return hipGetLastError();
}

hipError_t launch_deer_seq_book(uint32_t* seq_slots, uint32_t* seq_delta, int64_t nseq, int k_max,
                                int iter, hipStream_t stream) {
  const unsigned blocks = (unsigned)((nseq + 255) / 256 < 1024 ? (nseq + 255) / 256 : 1024);
  hipLaunchKernelGGL(k_deer_seq_book, dim3(blocks), dim3(256), 0, stream, seq_slots, seq_delta,
                     nseq, k_max, iter);
  return hipGetLastError();
}

hipError_t launch_deer_seq_finish(const uint32_t* seq_delta, int* seq_rec, int64_t nseq,
                                  int k_max, float eps, hipStream_t stream) {
  const unsigned blocks = (unsigned)((nseq + 255) / 256 < 1024 ? (nseq + 255) / 256 : 1024);
  hipLaunchKernelGGL(k_deer_seq_finish, dim3(blocks), dim3(256), 0, stream, seq_delta, seq_rec,
                     nseq, k_max, eps);
  return hipGetLastError();
}

hipError_t launch_deer_seq_select(const float* p0, const float* p1, float* h, int64_t nseq,
                                  int64_t n, const int* seq_rec, hipStream_t stream) {
  int64_t bx = (n + 255) / 256;
  if (bx > 1024) bx = 1024;
  if (bx < 1) bx = 1;
  hipLaunchKernelGGL(k_deer_seq_select, dim3((unsigned)bx, (unsigned)nseq), dim3(256), 0, stream,
                     p0, p1, h, n, seq_rec);
  return hipGetLastError();
}
#undef LRS_SHAPE_CASE

// ---------------------------------------------------------------------------
// Sequential tanh RNN: h_t = tanh(w_d h_{t-1} + u_t) evaluated one step after
// another, as the recurrence is written, with one lane per channel.  This is
// the O(T)-depth loop whose result the DEER solve reaches by Newton
// iterations, kept as a reference point for it.  A workgroup is one wave of 64
// channels.  Each lane holds kSeqTile = 128 consecutive steps of its own
// channel in registers (two such sets, 256 VGPRs): it loads the next 128 while
// it steps through the current ones and stores each result group as soon as
// it is known.  Tiles of 64 steps ran 272 us against 227 us at B=16, D=512,
// T=8192: each tile start still waits for the memory operations before it.  With BUF the accesses go
// through buffer resources that cover the wave's rows: a load out of range
// reads zero and a store out of range is dropped, so no access sits under a
// branch and the wave waits only for the loads of the tile it starts (a load
// or store under a branch would make the wait conservative: the wave would
// stall at every tile for all its memory operations).  VEC: 16-byte accesses
// (T % 4 == 0, 16-byte aligned arrays).  tanh is evaluated as in the DEER
// kernels, 1 - 2 / (1 + exp(2 p)).
// ---------------------------------------------------------------------------
constexpr int kSeqTile = 128;
constexpr int kBufferFlags = 0x00020000;  // raw buffer, 32-bit data format (gfx9)
typedef int SeqI32x4 __attribute__((ext_vector_type(4)));
typedef float SeqF32x4 __attribute__((ext_vector_type(4)));
// The raw buffer load and store intrinsics of the AMDGPU backend, declared by
// their LLVM names (rsrc: the 128-bit buffer resource, voffset per lane).
__device__ SeqF32x4 seq_buf_load4(SeqI32x4 rsrc, uint32_t voffset, int soffset, int aux) __asm(
    "llvm.amdgcn.raw.buffer.load.v4f32");
__device__ float seq_buf_load1(SeqI32x4 rsrc, uint32_t voffset, int soffset, int aux) __asm(
    "llvm.amdgcn.raw.buffer.load.f32");
__device__ void seq_buf_store4(SeqF32x4 v, SeqI32x4 rsrc, uint32_t voffset, int soffset,
                               int aux) __asm("llvm.amdgcn.raw.buffer.store.v4f32");
__device__ void seq_buf_store1(float v, SeqI32x4 rsrc, uint32_t voffset, int soffset,
                               int aux) __asm("llvm.amdgcn.raw.buffer.store.f32");

// Buffer resource over `bytes` bytes from p (stride 0: offsets are bytes; an
// access at or past `bytes` is out of range).
__device__ __forceinline__ SeqI32x4 seq_buf_rsrc(const void* p, int bytes) {
  const uint64_t a = (uint64_t)p;
  SeqI32x4 r;
  r.x = (int)(uint32_t)a;
  r.y = (int)((a >> 32) & 0xFFFFu);
  r.z = bytes;
  r.w = kBufferFlags;
  return r;
}

struct SeqRows {
  const float* urow;  // this lane's channel (channel 0 for a lane past C)
  float* hrow;
  SeqI32x4 ru, rh;    // BUF: the wave's rows of u and h
  uint32_t lane_off;  // BUF: byte offset of this lane's row
};

template <bool VEC, bool BUF>
__device__ __forceinline__ void rnn_seq_load(float (&v)[kSeqTile], const SeqRows& r, int64_t t0,
                                             int64_t T) {
#pragma unroll
  for (int q = 0; q < kSeqTile; q += 4) {
    if (BUF) {
      // past T the offsets run into the next row or out of range: read, unused
      const uint32_t off = r.lane_off + (uint32_t)(t0 + q) * 4u;
      if (VEC) {
        const SeqF32x4 b = seq_buf_load4(r.ru, off, 0, 0);
        v[q] = b.x; v[q + 1] = b.y; v[q + 2] = b.z; v[q + 3] = b.w;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          v[q + j] = seq_buf_load1(r.ru, off + 4u * j, 0, 0);
      }
    } else if (VEC) {
      // T % 4 == 0: a group of 4 steps is either wholly inside or wholly past
      // T; groups past T re-read the row's last group, unused
      const float4 f =
          *reinterpret_cast<const float4*>(r.urow + (t0 + q < T ? t0 + q : T - 4));
      v[q] = f.x; v[q + 1] = f.y; v[q + 2] = f.z; v[q + 3] = f.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[q + j] = r.urow[t0 + q + j < T ? t0 + q + j : T - 1];
    }
  }
}

// Steps through one tile (v: u on entry, h on exit) and stores the steps
// before T of a lane inside the channel range.
template <bool VEC, bool BUF>
__device__ __forceinline__ void rnn_seq_tile(float (&v)[kSeqTile], const SeqRows& r, int64_t t0,
                                             int64_t T, bool valid, float ws, float& x) {
  constexpr float k2l2e = 2.0f * 1.4426950408889634f;
#pragma unroll
  for (int q = 0; q < kSeqTile; q += 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(ws, x, k2l2e * v[q + j]));
      x = __builtin_fmaf(-2.0f, __builtin_amdgcn_rcpf(1.0f + e), 1.0f);
      v[q + j] = x;
    }
    if (BUF) {
      // a step past T gets an offset past every row, so its store is dropped
      const uint32_t off = r.lane_off + (uint32_t)(t0 + q) * 4u;
      if (VEC) {
        const uint32_t o = t0 + q < T ? off : 0xFFFFFFF0u;
        SeqF32x4 o4;
        o4.x = v[q]; o4.y = v[q + 1]; o4.z = v[q + 2]; o4.w = v[q + 3];
        seq_buf_store4(o4, r.rh, o, 0, 0);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          seq_buf_store1(v[q + j], r.rh, t0 + q + j < T ? off + 4u * j : 0xFFFFFFF0u, 0, 0);
      }
    } else if (VEC) {
      if (valid && t0 + q < T)
        *reinterpret_cast<float4*>(r.hrow + t0 + q) =
            make_float4(v[q], v[q + 1], v[q + 2], v[q + 3]);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (valid && t0 + q + j < T) r.hrow[t0 + q + j] = v[q + j];
    }
  }
}

// BUF requires the wave's rows of u and of h to span fewer than 2^31 bytes.
template <bool VEC, bool BUF>
__global__ __launch_bounds__(kWave) void k_rnn_seq(const float* __restrict__ w,
                                                   const float* __restrict__ u,
                                                   const float* __restrict__ h0,
                                                   float* __restrict__ h, int64_t T, int64_t C,
                                                   int64_t D) {
  constexpr float k2l2e = 2.0f * 1.4426950408889634f;
  const int64_t ch0 = (int64_t)blockIdx.x * kWave;
  const int64_t ch = ch0 + threadIdx.x;
  const bool valid = ch < C;
  const int64_t nch = C - ch0 < kWave ? C - ch0 : kWave;
  SeqRows r;
  r.urow = u + (valid ? ch : 0) * T;
  r.hrow = h + (valid ? ch : 0) * T;
  if (BUF) {
    const int bytes = (int)(nch * T * 4);
    r.ru = seq_buf_rsrc(u + ch0 * T, bytes);
    r.rh = seq_buf_rsrc(h + ch0 * T, bytes);
    // a lane past C starts past the wave's rows: its loads read zero and its
    // stores are dropped
    r.lane_off = valid ? (uint32_t)(threadIdx.x * T * 4) : 0x80000000u;
  }
  const float ws = valid ? w[ch % D] * k2l2e : 0.0f;
  float x = (valid && h0) ? h0[ch] : 0.0f;
  const int64_t ntile = (T + kSeqTile - 1) / kSeqTile;
  float va[kSeqTile], vb[kSeqTile];
  rnn_seq_load<VEC, BUF>(va, r, 0, T);
  // Tiles in pairs, so the two register sets swap roles without copies.  The
  // next tile is loaded unconditionally, also past the last one (its values
  // are never used): a load under a branch would make the wait before the
  // current tile conservative, stalling every tile on the next one's loads.
#pragma unroll 1
  for (int64_t k = 0; k < ntile; k += 2) {
    const int64_t t0 = k * kSeqTile;
    rnn_seq_load<VEC, BUF>(vb, r, t0 + kSeqTile, T);
    rnn_seq_tile<VEC, BUF>(va, r, t0, T, valid, ws, x);
    if (k + 1 >= ntile) break;
    rnn_seq_load<VEC, BUF>(va, r, t0 + 2 * kSeqTile, T);
    rnn_seq_tile<VEC, BUF>(vb, r, t0 + kSeqTile, T, valid, ws, x);
  }
}

hipError_t launch_rnn_seq(const float* w, const float* u, const float* h0, float* h, int64_t C,
                          int64_t D, int64_t T, int vec, hipStream_t stream) {
  const dim3 grid((unsigned)((C + kWave - 1) / kWave));
  // a wave's rows (64 T floats), and the offsets of the loads up to two tiles
  // past T, in a 31-bit byte range
  const bool buf = (int64_t)kWave * (T + 3 * kSeqTile) * 4 < ((int64_t)1 << 31);
#define LRS_SEQ(V, F) \
  hipLaunchKernelGGL((k_rnn_seq<V, F>), grid, dim3(kWave), 0, stream, w, u, h0, h, T, C, D)
  if (vec && buf) LRS_SEQ(true, true);
  else if (buf) LRS_SEQ(false, true);
  else if (vec) LRS_SEQ(true, false);
  else LRS_SEQ(false, false);
#undef LRS_SEQ
  return hipGetLastError();
}

}  // namespace lrs
