// lrs_tbd.hpp -- device building blocks of the feature-contiguous ([T, B, D])
// kernels: row loads and stores in fp32 and bf16 (default or nontemporal
// cache policy), the per-tile geometry, the block combine plus lane-parallel
// look-back that yields each channel's entering state, the time-block ticket,
// the LDS carry of persistent walks and the gate activations.  Included by
// scan_tbd.hip, gated_cell.hip and sru_deer.hip.
#pragma once

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

// ---- CPT-wide row access ------------------------------------------------
// `p` is a wave-uniform row pointer, `off` the lane's element offset.  FULL
// rows are in range and aligned; otherwise `nvalid` channels are in range
// (0 for a row past the end) and the rest read as `fill` / are not written.
// NT selects the nontemporal (streaming) cache policy for FULL rows.

template <bool NT, typename V>
__device__ __forceinline__ V ldv(const V* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT, typename V>
__device__ __forceinline__ void stv(V* p, V v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

template <int CPT, bool FULL, bool NT = false>
__device__ __forceinline__ void load_row(const float* __restrict__ p, uint32_t off, int nvalid,
                                         float fill, float (&v)[CPT]) {
  if (FULL) {
    if constexpr (CPT == 4) {
      const f32x4_t x = ldv<NT>(reinterpret_cast<const f32x4_t*>(p + off));
      v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    } else if constexpr (CPT == 2) {
      const f32x2_t x = ldv<NT>(reinterpret_cast<const f32x2_t*>(p + off));
      v[0] = x.x; v[1] = x.y;
    } else {
#pragma unroll
      for (int k = 0; k < CPT; ++k) v[k] = ldv<NT>(p + off + k);
    }
  } else {
#pragma unroll
    for (int k = 0; k < CPT; ++k) v[k] = (k < nvalid) ? p[off + k] : fill;
  }
}

template <int CPT, bool FULL, bool NT = false>
__device__ __forceinline__ void store_row(float* __restrict__ p, uint32_t off, int nvalid,
                                          const float (&v)[CPT]) {
  if (FULL) {
    if constexpr (CPT == 4) {
      stv<NT>(reinterpret_cast<f32x4_t*>(p + off), f32x4_t{v[0], v[1], v[2], v[3]});
    } else if constexpr (CPT == 2) {
      stv<NT>(reinterpret_cast<f32x2_t*>(p + off), f32x2_t{v[0], v[1]});
    } else {
#pragma unroll
      for (int k = 0; k < CPT; ++k) stv<NT>(p + off + k, v[k]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < CPT; ++k)
      if (k < nvalid) p[off + k] = v[k];
  }
}

// bf16 rows widened to fp32 values, with the fp32 rows' fill semantics (the
// scan kernels take either element type through these overloads).
template <int CPT, bool FULL, bool NT = false>
__device__ __forceinline__ void load_row(const uint16_t* __restrict__ p, uint32_t off, int nvalid,
                                         float fill, float (&v)[CPT]) {
  if (FULL) {
    if constexpr (CPT == 4) {
      const u32x2_t x = ldv<NT>(reinterpret_cast<const u32x2_t*>(p + off));
      v[0] = bf16_lo(x.x); v[1] = bf16_hi(x.x); v[2] = bf16_lo(x.y); v[3] = bf16_hi(x.y);
    } else if constexpr (CPT == 2) {
      const uint32_t x = ldv<NT>(reinterpret_cast<const uint32_t*>(p + off));
      v[0] = bf16_lo(x); v[1] = bf16_hi(x);
    } else {
#pragma unroll
      for (int k = 0; k < CPT; ++k) v[k] = bf16_lo((uint32_t)ldv<NT>(p + off + k));
    }
  } else {
#pragma unroll
    for (int k = 0; k < CPT; ++k) v[k] = (k < nvalid) ? io_ld(p, off + k) : fill;
  }
}

template <int CPT, bool FULL, bool NT = false>
__device__ __forceinline__ void store_row(uint16_t* __restrict__ p, uint32_t off, int nvalid,
                                          const float (&v)[CPT]) {
  if (FULL) {
    if constexpr (CPT == 4) {
      stv<NT>(reinterpret_cast<u32x2_t*>(p + off),
              u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])});
    } else if constexpr (CPT == 2) {
      stv<NT>(reinterpret_cast<uint32_t*>(p + off), pack_bf16x2(v[0], v[1]));
    } else {
#pragma unroll
      for (int k = 0; k < CPT; ++k)
        stv<NT>(p + off + k, (uint16_t)(pack_bf16x2(v[k], 0.0f) & 0xFFFFu));
    }
  } else {
#pragma unroll
    for (int k = 0; k < CPT; ++k)
      if (k < nvalid) io_st(p, off + k, v[k]);
  }
}

// bf16 rows are kept as packed pairs (CPT/2 words) and widened on use.
template <int CPT, bool FULL, bool NT = false>
__device__ __forceinline__ void load_row_bf16(const uint16_t* __restrict__ p, uint32_t off,
                                              int nvalid, uint32_t (&w)[CPT / 2]) {
  static_assert(CPT % 2 == 0, "bf16 rows hold an even number of channels");
  if (FULL) {
    if constexpr (CPT == 2) {
      w[0] = ldv<NT>(reinterpret_cast<const uint32_t*>(p + off));
    } else if constexpr (CPT == 4) {
      const u32x2_t x = ldv<NT>(reinterpret_cast<const u32x2_t*>(p + off));
      w[0] = x.x; w[1] = x.y;
    } else {
      static_assert(CPT == 8, "bf16 rows of 2, 4 or 8 channels");
      const u32x4_t x = ldv<NT>(reinterpret_cast<const u32x4_t*>(p + off));
      w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < CPT / 2; ++k) {
      const uint32_t lo = (2 * k < nvalid) ? p[off + 2 * k] : 0u;
      const uint32_t hi = (2 * k + 1 < nvalid) ? p[off + 2 * k + 1] : 0u;
      w[k] = lo | (hi << 16);
    }
  }
}

template <int CPT>
__device__ __forceinline__ float bf16_get(const uint32_t (&w)[CPT / 2], int k) {
  return (k & 1) ? bf16_hi(w[k >> 1]) : bf16_lo(w[k >> 1]);
}

template <int CPT, bool FULL, bool NT = false>
__device__ __forceinline__ void store_row_bf16(uint16_t* __restrict__ p, uint32_t off, int nvalid,
                                               const float (&v)[CPT]) {
  uint32_t w[CPT / 2];
#pragma unroll
  for (int k = 0; k < CPT / 2; ++k) w[k] = pack_bf16x2(v[2 * k], v[2 * k + 1]);
  if (FULL) {
    if constexpr (CPT == 2) {
      stv<NT>(reinterpret_cast<uint32_t*>(p + off), w[0]);
    } else if constexpr (CPT == 4) {
      stv<NT>(reinterpret_cast<u32x2_t*>(p + off), u32x2_t{w[0], w[1]});
    } else {
      stv<NT>(reinterpret_cast<u32x4_t*>(p + off), u32x4_t{w[0], w[1], w[2], w[3]});
    }
  } else {
#pragma unroll
    for (int k = 0; k < CPT; ++k)
      if (k < nvalid) p[off + k] = (uint16_t)(w[k / 2] >> (16 * (k & 1)));
  }
}

// ---- block-level pieces ----------------------------------------------------

// Look-back group (time blocks) of the feature-contiguous kernels: a block
// reads at most this many status words per channel.
constexpr int kColGroup = 8;

// Per channel, the state entering this wave's first step.  Each wave publishes
// its per-channel maps in LDS; the last CPT waves compose them into the block's
// per-channel maps, run the look-back (multi-block) and share the carries; every
// wave then composes the maps of the waves before it (wave order = scan order).
// st points at this channel block's status row for time block 0; time blocks
// are CW words apart.
template <int NW, int CPT>
__device__ __forceinline__ void col_enter_state(const float (&A)[CPT], const float (&B)[CPT],
                                                bool multi, int tb, const float (&x0)[CPT],
                                                const float* x0p, int64_t cbase, int cvalid,
                                                uint64_t* st, ColShared<NW, CPT>& s,
                                                float (&x)[CPT]) {
  constexpr int CW = kWave * CPT;
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int j0 = lane * CPT;
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    s.A[wid][j0 + k] = A[k];
    s.B[wid][j0 + k] = B[k];
  }
  __syncthreads();
  float carry[CPT];
  if (multi) {
    static_assert(NW >= CPT, "one look-back wave per channel of a lane");
    if (wid >= NW - CPT) {
      // wave NW-CPT+k resolves channels 64k .. 64k+63 of the tile, one per
      // lane: the look-back's registers stay off the other waves' paths, and
      // each wave's status words are contiguous (whole cache lines)
      const int j = (wid - (NW - CPT)) * kWave + lane;
      float TA = 1.0f, TB = 0.0f;
      for (int w = 0; w < NW; ++w) {
        const float wa = s.A[w][j], wb = s.B[w][j];
        TB = __builtin_fmaf(wa, TB, wb);
        TA = TA * wa;
      }
      float x_in = 0.0f;
      if (j < cvalid) {
        const bool gend = group_end(tb, kColGroup);
        if (!gend) status_store(st + (int64_t)tb * CW + j, pack_agg(TA, TB));
        const float xs = x0p ? x0p[cbase + j] : 0.0f;
        x_in = lookback_group_lane<kColGroup>(st + j, CW, tb, xs);
        if (gend) status_store(st + (int64_t)tb * CW + j, pack_inc(__builtin_fmaf(TA, x_in, TB)));
      }
      s.carry[j] = x_in;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < CPT; ++k) carry[k] = s.carry[j0 + k];
  } else {
#pragma unroll
    for (int k = 0; k < CPT; ++k) carry[k] = x0[k];
  }
  float PA[CPT], PB[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) { PA[k] = 1.0f; PB[k] = 0.0f; }
  for (int w = 0; w < wid; ++w) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const float wa = s.A[w][j0 + k], wb = s.B[w][j0 + k];
      PB[k] = __builtin_fmaf(wa, PB[k], wb);
      PA[k] = PA[k] * wa;
    }
  }
#pragma unroll
  for (int k = 0; k < CPT; ++k) x[k] = __builtin_fmaf(PA[k], carry[k], PB[k]);
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

// ---- persistent walks ------------------------------------------------------
// One workgroup per channel block visits every time tile in order and keeps
// the per-channel state entering the current tile in LDS (`carry`), so no
// look-back state is needed.  The wave maps and the carry alternate between
// two buffers by tile parity (tile tb uses buffer tb & 1), which leaves one
// barrier per tile: a buffer is written again only two tiles later, after
// every wave has passed the barrier of the tile in between.
template <int NW, int CPT>
struct PersistShared {
  float A[2][NW][kWave * CPT];
  float B[2][NW][kWave * CPT];
  float carry[2][kWave * CPT];  // carry[0]: the state entering tile 0
};

// Publish this wave's per-channel maps (A, B) and return in x the state
// entering this wave's first step: the maps of the earlier waves of the tile,
// in order, applied to the carry.  par: the tile's parity.
template <int NW, int CPT>
__device__ __forceinline__ void persist_enter(const float (&A)[CPT], const float (&B)[CPT],
                                              PersistShared<NW, CPT>& s, int wid, uint32_t off,
                                              float (&x)[CPT], int par) {
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    s.A[par][wid][off + k] = A[k];
    s.B[par][wid][off + k] = B[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    float PA = 1.0f, PB = 0.0f;
    for (int w = 0; w < wid; ++w) {
      PB = __builtin_fmaf(s.A[par][w][off + k], PB, s.B[par][w][off + k]);
      PA = PA * s.A[par][w][off + k];
    }
    x[k] = __builtin_fmaf(PA, s.carry[par][off + k], PB);
  }
}

// The last wave stores its final state (the state after the tile) as the
// next tile's carry, in the other buffer: that buffer was last read in the
// previous tile, which every wave finished before this tile's barrier.
// SYNC adds a barrier at the end of the tile, not needed for correctness: it
// keeps the waves' loads of the next tile behind every wave's stores of this
// one, which the SRU forward with saved cell states runs faster with.
template <int NW, int CPT, bool SYNC = false>
__device__ __forceinline__ void persist_advance(const float (&x)[CPT], PersistShared<NW, CPT>& s,
                                                int wid, uint32_t off, int par) {
  if (SYNC) __syncthreads();
  if (wid == NW - 1) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) s.carry[par ^ 1][off + k] = x[k];
  }
}

// Geometry of one thread inside its workgroup tile.
struct ColPos {
  int64_t row0;   // first time step of this wave (wave-uniform)
  int64_t c0;     // first channel of this lane
  uint32_t off;   // lane's element offset inside a row of the tile
  int nvc;        // channels of this lane inside [0, C)
};

template <int NW, int L, int CPT>
__device__ __forceinline__ ColPos col_pos(int tb, int cb, int64_t C) {
  ColPos q;
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  q.row0 = (int64_t)tb * (NW * L) + (int64_t)wid * L;
  q.off = (uint32_t)(lane * CPT);
  q.c0 = (int64_t)cb * (kWave * CPT) + q.off;
  q.nvc = clamp_valid(C - q.c0, CPT);
  return q;
}

// ---- gate activations and typed rows ---------------------------------------
// sigmoid(x) = 1/(1 + 2^(-x log2 e)) and tanh(c) = 1 - 2/(1 + 2^(2 c log2 e)),
// each one v_exp_f32 and one v_rcp_f32.
constexpr float kLog2e = 1.4426950408889634f;

template <typename IO, int CPT>
struct IoRow;

// One channel per lane: a single bf16, widened on use.
template <>
struct IoRow<uint16_t, 1> {
  uint32_t w;
  template <bool FULL, bool NT>
  __device__ __forceinline__ void load(const uint16_t* p, uint32_t off, int nv) {
    w = (FULL || nv > 0) ? (uint32_t)p[off] : 0u;
  }
  __device__ __forceinline__ float get(int) const { return bf16_lo(w); }
  template <bool FULL, bool NT>
  static __device__ __forceinline__ void store(uint16_t* p, uint32_t off, int nv,
                                               const float (&x)[1]) {
    if (FULL || nv > 0) p[off] = (uint16_t)(pack_bf16x2(x[0], 0.0f) & 0xFFFFu);
  }
};

template <int CPT>
struct IoRow<uint16_t, CPT> {
  uint32_t w[CPT / 2];
  template <bool FULL, bool NT>
  __device__ __forceinline__ void load(const uint16_t* p, uint32_t off, int nv) {
    load_row_bf16<CPT, FULL, NT>(p, off, nv, w);
  }
  __device__ __forceinline__ float get(int k) const { return bf16_get<CPT>(w, k); }
  template <bool FULL, bool NT>
  static __device__ __forceinline__ void store(uint16_t* p, uint32_t off, int nv,
                                               const float (&x)[CPT]) {
    store_row_bf16<CPT, FULL, NT>(p, off, nv, x);
  }
};

template <int CPT>
struct IoRow<float, CPT> {
  float v[CPT];
  template <bool FULL, bool NT>
  __device__ __forceinline__ void load(const float* p, uint32_t off, int nv) {
    load_row<CPT, FULL, NT>(p, off, nv, 0.0f, v);
  }
  __device__ __forceinline__ float get(int k) const { return v[k]; }
  template <bool FULL, bool NT>
  static __device__ __forceinline__ void store(float* p, uint32_t off, int nv,
                                               const float (&x)[CPT]) {
    store_row<CPT, FULL, NT>(p, off, nv, x);
  }
};

__device__ __forceinline__ float fast_sigmoid(float z, float nb) {
  // nb = -log2(e) * bias
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(__builtin_fmaf(z, -kLog2e, nb)));
}
__device__ __forceinline__ float fast_tanh(float v) {
  return __builtin_fmaf(-2.0f, __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f((2.0f * kLog2e) * v)),
                        1.0f);
}

}  // namespace lrs
