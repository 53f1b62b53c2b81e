// lrs_internal.hpp -- host-side plumbing shared by the kernel files and the
// C ABI implementation (launch plans and launchers).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lrs {

// A call whose arrays (all it reads and writes) total at least this many bytes,
// twice the memory-side cache, streams them with nontemporal loads and stores:
// none of its data can still be cached for the next call, and keeping it out of
// the caches measured 8-12% faster.  Smaller calls keep the default policy, so
// that e.g. a backward pass finds part of the forward pass's data in cache.
constexpr int64_t kStreamFootprint = (int64_t)512 << 20;

// Plan overrides of one call (the C ABI's lrs_options); a negative field
// keeps the measured default.
struct Opts {
  int64_t serial_fwd_max_t = -1;    // one lane per channel for T <= this ([B,D,T] forward)
  int64_t serial_bwd_max_t = -1;    // the same for the backward
  int64_t packed_max_t = -1;        // whole channels packed per workgroup for T <= this
  int64_t persist_min_blocks = -1;  // [T,B,D] layers: persistent walk from this many blocks
  int deer_fuse = -1;               // 0: one launch per Newton iteration
};

// Time-contiguous kernels: chunks of nw waves x r rows x 256 steps, nchunk
// chunks per channel.
struct RowPlan {
  int nw = 8;
  int r = 2;
  int64_t nchunk = 1;
  bool stream = false;  // nontemporal loads and stores (arrays far larger than the caches)
  int sub = 1;          // sequential sub-chunks per workgroup (single-workgroup channels)
  bool serial = false;  // short channels: one lane walks each channel (scan_serial.hip)
  int packed = 0;       // short channels: k whole channels per 8-wave, 2048-step workgroup
  int threads() const { return nw * 64; }
  int64_t chunk() const { return (int64_t)nw * r * 256; }
};
// Element type of the scan arrays (the C ABI's LRS_F32 / LRS_BF16); state and
// arithmetic are fp32 either way.
constexpr int kIoF32 = 0, kIoBf16 = 1;
constexpr int64_t io_bytes(int io) { return io == kIoBf16 ? 2 : 4; }
RowPlan plan_scan_fwd_rows(int64_t C, int64_t T, const Opts& o = Opts(), int io = kIoF32);
RowPlan plan_scan_bwd_rows(int64_t C, int64_t T, const Opts& o = Opts(), int io = kIoF32);
RowPlan plan_deer_rows(int64_t C, int64_t T);
RowPlan plan_scan_fused_rows(int64_t C, int64_t T, int io = kIoF32);
RowPlan plan_deer_bwd_rows(int64_t C, int64_t T);

// Feature-contiguous kernels: blocks of 64*cpt channels x nw*l steps.
struct ColPlan {
  int nw = 8, l = 8, cpt = 4;
  int64_t ncb = 1, ntb = 1;
  bool stream = false;   // nontemporal loads and stores (see kStreamFootprint)
  bool persist = false;  // one workgroup per channel block walks all time tiles (no look-back)
};
// Compute units of the current device (cached per device).
int device_cus();
// Channel blocks from which the [T,B,D] layer kernels run persistent
// (device_cus(), or the caller's override).
int64_t persist_min_blocks(const Opts& o = Opts());
ColPlan plan_cols(int64_t C, int64_t T, int nw, int l, int cpt);
ColPlan plan_scan_fwd_tbd(int64_t C, int64_t T, int io = kIoF32);
ColPlan plan_scan_bwd_tbd(int64_t C, int64_t T, int io = kIoF32);
// allow_persist = false: the look-back tile plan (workspace queries size for it).
ColPlan plan_sru(int64_t C, int64_t T, int io_dtype, bool allow_persist = true,
                 const Opts& o = Opts());
int64_t col_status_words(const ColPlan& p);

// Resets look-back state: status words to "not ready", tickets and the
// optional 32-bit words `zero` to 0.  Plain stores from a kernel, so the call
// is safe inside captured graphs.
hipError_t launch_reset(uint64_t* status, int64_t nstatus, unsigned* tickets, int64_t ntickets,
                        uint32_t* zero, int64_t nzero, hipStream_t stream);

// Scan launchers: a, b, h, g, da, db are arrays of element type `io` (kIoF32
// or kIoBf16); h0 and dh0 are fp32.  `vec`: rows and base pointers allow
// 4-element accesses (T % 4 == 0, pointers aligned to 4 elements).
hipError_t launch_scan_fwd_bdt(const void* a, const void* b, const float* h0, void* h, int io,
                               int64_t C, int64_t T, const RowPlan& p, int vec, uint64_t* status,
                               unsigned* tickets, hipStream_t stream);
hipError_t launch_scan_bwd_bdt(const void* a, const void* h, const float* h0, const void* g,
                               void* da, void* db, float* dh0, int io, int64_t C, int64_t T,
                               const RowPlan& p, int vec, uint64_t* status, unsigned* tickets,
                               hipStream_t stream);
// Sequential per-channel scans (one lane per channel) for short channels.
hipError_t launch_scan_fwd_serial(const void* a, const void* b, const float* h0, void* h, int io,
                                  int64_t C, int64_t T, int vec, hipStream_t stream);
hipError_t launch_scan_bwd_serial(const void* a, const void* h, const float* h0, const void* g,
                                  void* da, void* db, float* dh0, int io, int64_t C, int64_t T,
                                  int vec, hipStream_t stream);
// Packed short channels (plan.packed = channels per workgroup).
hipError_t launch_scan_fwd_packed(const void* a, const void* b, const float* h0, void* h, int io,
                                  int64_t C, int64_t T, int k, int vec, hipStream_t stream);
hipError_t launch_scan_bwd_packed(const void* a, const void* h, const float* h0, const void* g,
                                  void* da, void* db, float* dh0, int io, int64_t C, int64_t T,
                                  int k, int vec, hipStream_t stream);
// Forward and backward scan in one pass; the plan must be single-chunk.
hipError_t launch_scan_fused_bdt(const void* a, const void* b, const float* h0, const void* g,
                                 void* h, void* da, void* db, float* dh0, int io, int64_t C,
                                 int64_t T, const RowPlan& p, int vec, hipStream_t stream);
// DEER update norms: three rotating sets of kDeltaSlots words, kDeltaStride
// words apart (one cache line per slot).
constexpr int kDeltaSlots = 64;
constexpr int kDeltaStride = 32;
constexpr int64_t kDeltaSetWords = 3 * kDeltaSlots * kDeltaStride;
// Solve record written by the finish kernel: iterations, converged, non-finite.
constexpr int kDeerRecordWords = 4;
hipError_t launch_deer_finish(const uint32_t* delta_bits, uint32_t* delta_out, int* rec,
                              int k_max, float eps, hipStream_t stream);
hipError_t launch_deer_select(const float* p0, const float* p1, float* h, int64_t n,
                              const int* rec, hipStream_t stream);
// Adjoint of the nonlinear RNN at its solution: the reverse scan kernel, then
// dL/dw from `part` (nchunk * B * D floats) via launch_col_sums.
hipError_t launch_deer_bwd(const float* w, const float* h, const float* h0, const float* g,
                           float* du, float* dw, float* dh0, float* part, double* acc, int64_t B,
                           int64_t D, int64_t T, const RowPlan& p, int vec, uint64_t* status,
                           unsigned* tickets, hipStream_t stream);
// Sequential tanh RNN (one lane per channel, ceil(C / 64) one-wave workgroups;
// vec: T % 4 == 0 and u, h 16-byte aligned).
hipError_t launch_rnn_seq(const float* w, const float* u, const float* h0, float* h, int64_t C,
                          int64_t D, int64_t T, int vec, hipStream_t stream);
// One Newton iteration.  seq_slots != nullptr: per-sequence stopping (norm
// slots kSeqSlots per sequence per set, three sets; seq_delta[seq * k_max + i]
// holds sequence seq's norm of iteration i once k_deer_seq_book folded it).
constexpr int kSeqSlots = 4;
hipError_t launch_deer_iter(const float* w, const float* u, const float* y, const float* h0,
                            float* yn, int64_t C, int64_t D, int64_t T, const RowPlan& p, int vec,
                            uint64_t* status, unsigned* tickets, uint32_t* delta_bits,
                            uint32_t* delta_out, int iter, float eps, hipStream_t stream,
                            uint32_t* seq_slots = nullptr, const uint32_t* seq_delta = nullptr,
                            int k_max = 0);
// DEER with the Newton iterations fused into one walk over each channel
// (single-workgroup channels, k_max <= kDeerFuseMax): the pass over all k_max
// iterations into `out` (h, or a buffer when h holds the starting iterate),
// the finish kernel writing the record and norms, the redo launch when the stop
// rule fired earlier, and the copy into h.  `sets` holds k_max slot sets of
// kDeltaSlots * kDeltaStride words, cleared beforehand.  Per-sequence
// stopping: seq_delta (B * k_max norms, cleared) and seq_rec (4 words per
// sequence) replace sets, delta_out and rec.
constexpr int kDeerFuseMax = 8;
hipError_t launch_deer_fused(const float* w, const float* u, const float* y0, const float* h0,
                             float* out, float* h, int64_t C, int64_t D, int64_t T,
                             const RowPlan& p, int vec, int k_max, float eps, uint32_t* sets,
                             uint32_t* delta_out, int* rec, hipStream_t stream,
                             uint32_t* seq_delta = nullptr, int* seq_rec = nullptr);
// Pieces shared by the fused solves: the record from the norm sets, and the
// copy of the pass's result into h unless a redo wrote h.
hipError_t launch_deer_fused_finish(const uint32_t* sets, uint32_t* delta_out, int* rec,
                                    int k_max, float eps, hipStream_t stream);
hipError_t launch_deer_fused_select(const float* src, float* h, int64_t n, const int* rec,
                                    int k_max, hipStream_t stream);
hipError_t launch_deer_seq_book(uint32_t* seq_slots, uint32_t* seq_delta, int64_t nseq, int k_max,
                                int iter, hipStream_t stream);
hipError_t launch_deer_seq_finish(const uint32_t* seq_delta, int* seq_rec, int64_t nseq,
                                  int k_max, float eps, hipStream_t stream);
hipError_t launch_deer_seq_select(const float* p0, const float* p1, float* h, int64_t nseq,
                                  int64_t n, const int* seq_rec, hipStream_t stream);

hipError_t launch_scan_fwd_tbd(const void* a, const void* b, const float* h0, void* h, int io,
                               int64_t C, int64_t T, const ColPlan& p, int vec, uint64_t* status,
                               unsigned* tickets, hipStream_t stream);
hipError_t launch_scan_bwd_tbd(const void* a, const void* h, const float* h0, const void* g,
                               void* da, void* db, float* dh0, int io, int64_t C, int64_t T,
                               const ColPlan& p, int vec, uint64_t* status, unsigned* tickets,
                               hipStream_t stream);
hipError_t launch_sru_fwd(const void* zf, const void* zr, const void* zx, const float* bias_f,
                          const float* bias_r, const float* c0, void* h, float* c_last,
                          float* c_states, int64_t T, int64_t B, int64_t D, int io_dtype,
                          const ColPlan& p, int vec, uint64_t* status, unsigned* tickets,
                          hipStream_t stream);
ColPlan plan_sru_bwd(int64_t C, int64_t T, int io_dtype);
// Per-feature parameter gradients: column sums of nmat consecutive [R, D]
// matrices of partial sums (R = partials per feature), accumulated in fp64 in a
// fixed order into out0 (and out1 for nmat = 2).  `acc` holds
// nmat * col_sum_blocks(R) * D doubles.
int64_t col_sum_blocks(int64_t R);
hipError_t launch_col_sums(const float* part, int nmat, int64_t R, int64_t D, double* acc,
                           float* out0, float* out1, hipStream_t stream);

// Launches the SRU backward kernel and the bias-gradient reduction; `part`
// holds 2 * ntb * B * D floats of per-tile partial sums.
hipError_t launch_sru_bwd(const void* zf, const void* zr, const void* zx, const float* bias_f,
                          const float* bias_r, const float* c0, const float* cs, const void* gh,
                          const float* gcl, void* dzf, void* dzr, void* dzx, float* dbf,
                          float* dbr, float* dc0, float* part, double* acc, int64_t T, int64_t B,
                          int64_t D, int io_dtype, const ColPlan& p, int vec, uint64_t* status,
                          unsigned* tickets, hipStream_t stream);

// LSTM cell-state layer with input-only gates (gated_cell.hip).  `save`: the
// forward also writes the cell states.
// allow_persist = false: the look-back tile plan (workspace queries size for it).
ColPlan plan_lstm(int64_t C, int64_t T, int io_dtype, bool save, bool allow_persist = true,
                  const Opts& o = Opts());
ColPlan plan_lstm_bwd(int64_t C, int64_t T, int io_dtype);
hipError_t launch_lstm_fwd(const void* zf, const void* zi, const void* zc, const void* zo,
                           const float* c0, void* h, float* c_last, float* c_states, int64_t T,
                           int64_t C, int io_dtype, const ColPlan& p, int vec, uint64_t* status,
                           unsigned* tickets, hipStream_t stream);
hipError_t launch_lstm_bwd(const void* zf, const void* zi, const void* zc, const void* zo,
                           const float* c0, const float* cs, const void* gh, const float* gcl,
                           void* dzf, void* dzi, void* dzc, void* dzo, float* dc0, int64_t T,
                           int64_t C, int io_dtype, const ColPlan& p, int vec, uint64_t* status,
                           unsigned* tickets, hipStream_t stream);

// SRU with v_f * c_{t-1} in the forget gate, by DEER (sru_deer.hip).
ColPlan plan_sru_deer(int64_t C, int64_t T, int io_dtype, bool allow_persist = true,
                      const Opts& o = Opts());
hipError_t launch_sru_deer_iter(const void* zf, const void* zx, const float* bias_f,
                                const float* v_f, const float* c0, const float* y, float* yn,
                                int64_t T, int64_t C, int64_t D, int io_dtype, const ColPlan& p,
                                int vec, uint64_t* status, unsigned* tickets,
                                uint32_t* delta_bits, uint32_t* delta_out, int iter, float eps,
                                hipStream_t stream);
// SRU-by-DEER with the iterations fused into the persistent walk (plan.persist,
// k_max <= kDeerFuseMax): pass into `out`, finish, redo into c_states, select.
hipError_t launch_sru_deer_fused(const void* zf, const void* zx, const float* bias_f,
                                 const float* v_f, const float* c0, const float* c_init,
                                 float* out, float* c_states, int64_t T, int64_t C, int64_t D,
                                 int io_dtype, const ColPlan& p, int vec, int k_max, float eps,
                                 uint32_t* sets, uint32_t* delta_out, int* rec,
                                 hipStream_t stream);
hipError_t launch_sru_deer_out(const void* zr, const void* zx, const float* bias_r,
                               const float* c, void* h, float* c_last, int64_t N, int64_t C,
                               int64_t D, int io_dtype, int vec, hipStream_t stream);

}  // namespace lrs
