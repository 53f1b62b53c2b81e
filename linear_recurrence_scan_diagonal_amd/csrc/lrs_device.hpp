// lrs_device.hpp -- device building blocks for the diagonal linear-recurrence
// scan on gfx950 (CDNA4, wave64).
//
// The recurrence h_t = a_t*h_{t-1} + b_t is a composition of affine maps
// x -> a*x + b.  Composition is associative, which is what lets the sequence be
// evaluated as a parallel prefix scan (page "CUDA并行化RNN训练：从O(T)到O(log T)
// 的工程实践与参数调优", body, parallel-scan paragraph: treat the step as an
// associative operation and divide and conquer; page "RNN CUDA内核优化：实现序列
// 长度无关的恒定推理延迟", body: the cell-state update is a linear recurrence with
// time-varying coefficients, a prefix-scan problem).
//
// Levels used by every kernel in this library:
//   1. lane fold     : each lane folds a few consecutive steps serially (FMA);
//   2. wave64 scan   : 6 DPP steps (row_shr 1,2,4,8; row_bcast 15,31);
//   3. block scan    : per-wave aggregates combined through LDS;
//   4. chunk carry   : decoupled look-back over per-chunk status words in HBM,
//                      so a channel longer than one workgroup's chunk is still
//                      a single pass over memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lrs {

constexpr int kWave = 64;

__device__ __forceinline__ float as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u32(float f) { return __builtin_bit_cast(uint32_t, f); }

// ---- I/O element types ------------------------------------------------------
// Arrays are fp32 or bf16 (stored as uint16_t bit patterns); arithmetic and
// carried state are always fp32.  bf16 values widen exactly; results round to
// bf16 nearest-even with gfx950's v_cvt_pk_bf16_f32.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return as_f32(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return as_f32(w & 0xFFFF0000u); }

// Round a pair of fp32 to bf16 (nearest-even), packed low | high << 16.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  const bf16x2_t b = __builtin_convertvector(f, bf16x2_t);
  return __builtin_bit_cast(uint32_t, b);
}

// One element of an fp32 or bf16 array, widened to fp32 / rounded from fp32.
__device__ __forceinline__ float io_ld(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float io_ld(const uint16_t* p, int64_t i) {
  return as_f32((uint32_t)p[i] << 16);
}
__device__ __forceinline__ void io_st(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void io_st(uint16_t* p, int64_t i, float v) {
  p[i] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
}

// One Hillis-Steele step across lanes: lane i combines with the lane that the
// DPP control selects (an earlier lane in scan order):
//   (A_e, B_e) o (A, B) = (A_e*A, A*B_e + B).
// Written as two DPP-modified VALU ops (the earlier lane's value is read
// through DPP as src0).  With bound control off, a lane whose source lies
// outside the selected rows, or outside the row mask, is not written and so
// keeps (A, B): the result of combining with the identity (1, 0).  Each valid
// lane computes exactly fma(B_e, A, B) and A_e*A.  The leading s_nop gives the
// two wait states that a DPP read of a VGPR written by the preceding VALU op
// requires (the compiler does not look inside the asm for that hazard).
#define LRS_DPP_STEP(CTRL)                                                     \
  asm("s_nop 1\n\t"                                                          \
      "v_fmac_f32_dpp %1, %1, %0 " CTRL "\n\t"                               \
      "v_mul_f32_dpp %0, %0, %0 " CTRL                                        \
      : "+v"(A), "+v"(B))

// Inclusive scan of (A, B) over the 64 lanes of a wave, lane order = scan order
// (called with all 64 lanes active).
__device__ __forceinline__ void wave_scan(float& A, float& B) {
  LRS_DPP_STEP("row_shr:1 row_mask:0xf bank_mask:0xf");
  LRS_DPP_STEP("row_shr:2 row_mask:0xf bank_mask:0xf");
  LRS_DPP_STEP("row_shr:4 row_mask:0xf bank_mask:0xf");
  LRS_DPP_STEP("row_shr:8 row_mask:0xf bank_mask:0xf");
  LRS_DPP_STEP("row_bcast:15 row_mask:0xa bank_mask:0xf");  // into rows 1 and 3
  LRS_DPP_STEP("row_bcast:31 row_mask:0xc bank_mask:0xf");  // into rows 2 and 3
  // The compiler does not count the asm above as a VALU write of A and B, so
  // a DPP read of them that it places next would miss its wait states.
  asm("s_nop 1" : "+v"(A), "+v"(B));
}
#undef LRS_DPP_STEP

// Value of the previous lane (wave_shr:1); lane 0 receives `lane0`.
__device__ __forceinline__ float wave_shift_up(float x, float lane0) {
  return as_f32((uint32_t)__builtin_amdgcn_update_dpp((int)as_u32(lane0), (int)as_u32(x),
                                                      0x138, 0xf, 0xf, false));
}

// Maximum of a 32-bit unsigned value over the 64 lanes of a wave.
// Called with all 64 lanes active.
// Six DPP max steps leave the maximum over the wave in lane 63 (lanes whose
// source is out of range keep their value, and max is idempotent); it is then
// broadcast from there.  s_nop: the DPP read-after-VALU-write wait states.
#define LRS_DPP_MAX(CTRL) asm("s_nop 1\n\tv_max_u32_dpp %0, %0, %0 " CTRL : "+v"(v))
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  LRS_DPP_MAX("row_shr:1 row_mask:0xf bank_mask:0xf");
  LRS_DPP_MAX("row_shr:2 row_mask:0xf bank_mask:0xf");
  LRS_DPP_MAX("row_shr:4 row_mask:0xf bank_mask:0xf");
  LRS_DPP_MAX("row_shr:8 row_mask:0xf bank_mask:0xf");
  LRS_DPP_MAX("row_bcast:15 row_mask:0xa bank_mask:0xf");
  LRS_DPP_MAX("row_bcast:31 row_mask:0xc bank_mask:0xf");
  asm("s_nop 1" : "+v"(v));  // wait states for a DPP read of v (see wave_scan)
  return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}
#undef LRS_DPP_MAX

// ---------------------------------------------------------------------------
// Look-back status words.  One 64-bit word per (channel, chunk), written and
// read with relaxed agent-scope atomics (coherent across the XCDs' L2s), so the
// payload travels in the same word as its state and no fences are needed.
//   0xFFFFFFFF'FFFFFFFF        not ready (the reset value)
//   lo = A bits, hi = B bits   aggregate (A, B) of this chunk alone
//   lo = 0xFFFFFFFE, hi = x    inclusive: the state at the end of the chunk
// A is canonicalised so that neither marker can occur as a real A: any NaN is
// replaced by the default quiet NaN 0x7FC00000.
// ---------------------------------------------------------------------------
constexpr uint64_t kStatusEmpty = ~0ull;
constexpr uint32_t kIncTag = 0xFFFFFFFEu;

__device__ __forceinline__ uint64_t pack_agg(float A, float B) {
  uint32_t a = (A != A) ? 0x7FC00000u : as_u32(A);
  return (uint64_t)a | ((uint64_t)as_u32(B) << 32);
}
__device__ __forceinline__ uint64_t pack_inc(float x) {
  return (uint64_t)kIncTag | ((uint64_t)as_u32(x) << 32);
}
__device__ __forceinline__ void status_store(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t status_load(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Carry rule.  The chunks of a channel are taken G at a time ("groups").
// With g0 = c - c % G the first chunk of chunk c's group, the state entering
// chunk c is
//     x_in(c) = M_{c-1}( ... M_{g0}( x_end(g0 - 1) ) ... )
// where M_k is chunk k's aggregate map and x_end(g0 - 1) the state at the end
// of the previous group (the channel's initial state for the first group).
// Every chunk except the last one of a group publishes its aggregate as soon
// as it has it; the last chunk of a group publishes nothing but its inclusive
// state, once its own x_in is known.  Every reader therefore combines the
// same words in the same order, whatever had been published when it looked:
// the association order, and so every rounding, is fixed by the launch shape
// alone and results are bitwise reproducible from run to run.  A reader waits
// for at most G words (the G-1 aggregates before it in its group and one
// inclusive state).  Chunk indices come from a per-channel ticket, so every
// chunk waited on is resident or finished and the wait terminates.
//
// Safety net: a predecessor publishes within microseconds of starting, so a
// wait of kSpinLimit polls (~0.1 s) can only mean corrupted status words; the
// carry then becomes NaN, which poisons the outputs of this channel instead
// of hanging the device.
constexpr uint32_t kSpinLimit = 1u << 22;

__device__ __forceinline__ bool group_end(int c, int G) { return c % G == G - 1; }

// Wave-wide form, run by all 64 lanes of one wave, groups of 64 chunks: lane
// l < j loads the aggregate of chunk g0 + l, lane 63 the inclusive state at
// the end of the previous group; a poll re-loads only the words still
// unpublished.  The aggregates are composed by the wave scan (identity maps
// in the unused lanes, which leave every value unchanged) and the composite
// of the first j applied to the previous group's end state.  st points at
// chunk 0 of the channel, consecutive chunks `stride` words apart; x0 is the
// channel's initial state.  Returns x_in(c), uniform across the wave.
constexpr int kWaveGroup = kWave;
__device__ __forceinline__ float lookback_group_wave(const uint64_t* st, int c, int64_t stride,
                                                     float x0) {
  const int lane = threadIdx.x & (kWave - 1);
  const int g0 = c - c % kWaveGroup;
  const int j = c - g0;  // 0 .. 63 aggregates to compose
  int idx = -1;
  if (lane < j) idx = g0 + lane;
  else if (lane == kWave - 1 && g0 > 0) idx = g0 - 1;
  uint64_t v = kStatusEmpty;
  uint32_t spins = 0;
  while (true) {
    if (idx >= 0 && v == kStatusEmpty) v = status_load(st + (int64_t)idx * stride);
    if (__ballot(idx >= 0 && v == kStatusEmpty) == 0) break;
    if (++spins > kSpinLimit) return __builtin_nanf("");
    __builtin_amdgcn_s_sleep(1);
  }
  float xs = x0;
  if (g0 > 0) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, kWave - 1);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), kWave - 1);
    xs = (lo == kIncTag) ? as_f32(hi) : __builtin_nanf("");
  }
  if (j == 0) return xs;
  float A = 1.0f, B = 0.0f;
  if (lane < j) {
    A = as_f32((uint32_t)v);
    B = as_f32((uint32_t)(v >> 32));
  }
  wave_scan(A, B);
  const float PA = as_f32((uint32_t)__builtin_amdgcn_readlane((int)as_u32(A), j - 1));
  const float PB = as_f32((uint32_t)__builtin_amdgcn_readlane((int)as_u32(B), j - 1));
  return __builtin_fmaf(PA, xs, PB);
}

// Lane-parallel form for the feature-contiguous kernels: each lane resolves
// one channel of its own, groups of G blocks.  The lane loads every word it
// needs at once (v[i], i < j: aggregate of block g0 + i; v[G-1]: inclusive
// state of block g0 - 1), re-polls only the missing ones, then applies the
// aggregates in ascending block order to the previous group's end state.
// st points at block 0 of the lane's channel, consecutive blocks `stride`
// words apart; x0 is the channel's initial state.
template <int G>
__device__ __forceinline__ float lookback_group_lane(const uint64_t* st, int64_t stride, int c,
                                                     float x0) {
  const int g0 = c - c % G;
  const int j = c - g0;
  if (j == 0 && g0 == 0) return x0;
  uint64_t v[G];
#pragma unroll
  for (int i = 0; i < G; ++i) v[i] = kStatusEmpty;
  uint32_t spins = 0;
  while (true) {
#pragma unroll
    for (int i = 0; i < G - 1; ++i)
      if (i < j && v[i] == kStatusEmpty) v[i] = status_load(st + (int64_t)(g0 + i) * stride);
    if (g0 > 0 && v[G - 1] == kStatusEmpty) v[G - 1] = status_load(st + (int64_t)(g0 - 1) * stride);
    bool missing = g0 > 0 && v[G - 1] == kStatusEmpty;
#pragma unroll
    for (int i = 0; i < G - 1; ++i) missing |= (i < j && v[i] == kStatusEmpty);
    if (!missing) break;
    if (++spins > kSpinLimit) return __builtin_nanf("");
    __builtin_amdgcn_s_sleep(1);
  }
  float x = x0;
  if (g0 > 0)
    x = ((uint32_t)v[G - 1] == kIncTag) ? as_f32((uint32_t)(v[G - 1] >> 32)) : __builtin_nanf("");
#pragma unroll
  for (int i = 0; i < G - 1; ++i)
    if (i < j) x = __builtin_fmaf(as_f32((uint32_t)v[i]), x, as_f32((uint32_t)(v[i] >> 32)));
  return x;
}

__device__ __forceinline__ unsigned take_ticket(unsigned* counter) {
  return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Group loads/stores: the 4 consecutive floats starting at element p of a row
// of length T.  In-range groups use one 16-byte access when `vec` is true (row
// starts and base pointers 16-byte aligned, p a multiple of 4); the ragged
// tail is predicated element by element, out-of-range elements read as `fill`
// and are not written.
// ---------------------------------------------------------------------------
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// NT selects the nontemporal (streaming) cache policy for the 16-byte access.
template <bool NT = false>
__device__ __forceinline__ float4 load_group(const float* __restrict__ row, int64_t p, int64_t T,
                                             bool vec, float fill) {
  if (vec && p + 4 <= T) {
    if (NT) {
      const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(row + p));
      return make_float4(v.x, v.y, v.z, v.w);
    }
    return *reinterpret_cast<const float4*>(row + p);
  }
  float4 v;
  v.x = (p < T) ? row[p] : fill;
  v.y = (p + 1 < T) ? row[p + 1] : fill;
  v.z = (p + 2 < T) ? row[p + 2] : fill;
  v.w = (p + 3 < T) ? row[p + 3] : fill;
  return v;
}

// Full-range variants: the whole group is in range and aligned (no checks).
template <bool NT = false>
__device__ __forceinline__ float4 load_group_full(const float* __restrict__ row, int64_t p) {
  if (NT) {
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(row + p));
    return make_float4(v.x, v.y, v.z, v.w);
  }
  return *reinterpret_cast<const float4*>(row + p);
}

template <bool NT = false>
__device__ __forceinline__ void store_group_full(float* __restrict__ row, int64_t p, float4 v) {
  if (NT) {
    const f32x4_t x = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4_t*>(row + p));
  } else {
    *reinterpret_cast<float4*>(row + p) = v;
  }
}

template <bool NT = false>
__device__ __forceinline__ void store_group(float* __restrict__ row, int64_t p, int64_t T,
                                            bool vec, float4 v) {
  if (vec && p + 4 <= T) {
    if (NT) {
      const f32x4_t x = {v.x, v.y, v.z, v.w};
      __builtin_nontemporal_store(x, reinterpret_cast<f32x4_t*>(row + p));
    } else {
      *reinterpret_cast<float4*>(row + p) = v;
    }
    return;
  }
  if (p < T) row[p] = v.x;
  if (p + 1 < T) row[p + 1] = v.y;
  if (p + 2 < T) row[p + 2] = v.z;
  if (p + 3 < T) row[p + 3] = v.w;
}

// bf16 groups: the 4 consecutive elements starting at p as one 8-byte access
// (`vec`: row starts and base pointers 8-byte aligned, p a multiple of 4).
template <bool NT = false>
__device__ __forceinline__ float4 load_group_full(const uint16_t* __restrict__ row, int64_t p) {
  const u32x2_t* q = reinterpret_cast<const u32x2_t*>(row + p);
  const u32x2_t w = NT ? __builtin_nontemporal_load(q) : *q;
  return make_float4(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y));
}

template <bool NT = false>
__device__ __forceinline__ float4 load_group(const uint16_t* __restrict__ row, int64_t p, int64_t T,
                                             bool vec, float fill) {
  if (vec && p + 4 <= T) return load_group_full<NT>(row, p);
  float4 v;
  v.x = (p < T) ? io_ld(row, p) : fill;
  v.y = (p + 1 < T) ? io_ld(row, p + 1) : fill;
  v.z = (p + 2 < T) ? io_ld(row, p + 2) : fill;
  v.w = (p + 3 < T) ? io_ld(row, p + 3) : fill;
  return v;
}

template <bool NT = false>
__device__ __forceinline__ void store_group_full(uint16_t* __restrict__ row, int64_t p, float4 v) {
  const u32x2_t w = {pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
  u32x2_t* q = reinterpret_cast<u32x2_t*>(row + p);
  if (NT) __builtin_nontemporal_store(w, q);
  else *q = w;
}

template <bool NT = false>
__device__ __forceinline__ void store_group(uint16_t* __restrict__ row, int64_t p, int64_t T,
                                            bool vec, float4 v) {
  if (vec && p + 4 <= T) {
    store_group_full<NT>(row, p, v);
    return;
  }
  if (p < T) io_st(row, p, v.x);
  if (p + 1 < T) io_st(row, p + 1, v.y);
  if (p + 2 < T) io_st(row, p + 2, v.z);
  if (p + 3 < T) io_st(row, p + 3, v.w);
}

// FULL selects the unchecked access; otherwise the checked one above (either
// element type; IO = float or uint16_t for bf16).
template <bool FULL, bool NT, typename IO>
__device__ __forceinline__ float4 ld4(const IO* __restrict__ row, int64_t p, int64_t T, bool vec,
                                      float fill) {
  return FULL ? load_group_full<NT>(row, p) : load_group<NT>(row, p, T, vec, fill);
}
template <bool FULL, bool NT, typename IO>
__device__ __forceinline__ void st4(IO* __restrict__ row, int64_t p, int64_t T, bool vec,
                                    float4 v) {
  if (FULL) store_group_full<NT>(row, p, v);
  else store_group<NT>(row, p, T, vec, v);
}

// tanh from its definition through exp: tanh(x) = 1 - 2/(exp(2x) + 1).
// Saturates correctly at both ends (exp overflow -> 1, underflow -> -1);
// absolute error a few fp32 ulps of 1.
__device__ __forceinline__ float tanh_fast(float x) {
  const float e = __expf(2.0f * x);
  return 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
}

// logistic sigmoid 1/(1 + exp(-x))
__device__ __forceinline__ float sigmoid_fast(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

}  // namespace lrs
