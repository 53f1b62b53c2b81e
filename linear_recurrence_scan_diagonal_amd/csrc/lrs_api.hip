// lrs_api.hip -- the C ABI declared in include/lrs.h: argument validation,
// workspace carving and launch-plan choice.  All device work is enqueued on
// the caller's stream; nothing here allocates device memory.
#include <math.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/lrs.h"
#include "lrs_internal.hpp"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  return !__builtin_mul_overflow(a, b, out);
}

// B*D*T without overflow, and small enough that byte offsets fit in int64.
bool shape_ok(int64_t B, int64_t D, int64_t T, int64_t* C, int64_t* N) {
  if (B < 0 || D < 0 || T < 0) return false;
  if (!mul_ok(B, D, C) || !mul_ok(*C, T, N)) return false;
  return *N <= ((int64_t)1 << 60);
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool overlap(const void* p, size_t pn, const void* q, size_t qn) {
  if (!p || !q || pn == 0 || qn == 0) return false;
  const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
  return a < b + qn && b < a + pn;
}

struct Carve {
  char* base;
  size_t used = 0;
  explicit Carve(void* ws) : base((char*)ws) {}
  template <typename T>
  T* take(int64_t n) {
    if (n <= 0) return nullptr;
    T* p = (T*)(base + used);
    used = align_up(used + (size_t)n * sizeof(T));
    return p;
  }
};

// Bytes to carve `nstatus` 64-bit words + `ntickets` counters (+ slack so the
// caller's pointer need not be aligned).
size_t lookback_bytes(int64_t nstatus, int64_t ntickets) {
  if (nstatus <= 0) return 0;
  return kAlign + align_up((size_t)nstatus * 8) + align_up((size_t)ntickets * 4);
}

void* align_ptr(void* p) { return (void*)(((uintptr_t)p + kAlign - 1) & ~(uintptr_t)(kAlign - 1)); }

int hip_status(hipError_t e) { return e == hipSuccess ? LRS_OK : LRS_ERR_HIP; }

// Launch-size guard: HIP grids are limited to 2^32-1 work-items per dimension.
bool grid_ok(int64_t blocks, int threads) { return blocks > 0 && blocks * threads < (1ll << 32); }

// Launch guard of a [B,D,T] scan plan (sequential: 256 channels per
// workgroup; packed: p.packed channels per workgroup; else one per chunk).
bool rows_grid_ok(const lrs::RowPlan& p, int64_t C) {
  if (p.serial) return grid_ok((C + 255) / 256, 256);
  if (p.packed) return grid_ok((C + p.packed - 1) / p.packed, p.threads());
  return grid_ok(C * p.nchunk, p.threads());
}

int scan_ws_needs(int64_t C, int64_t T, int layout, int dtype, size_t* bytes) {
  if (layout == LRS_LAYOUT_BDT) {
    const lrs::RowPlan f = lrs::plan_scan_fwd_rows(C, T, lrs::Opts(), dtype),
                       b = lrs::plan_scan_bwd_rows(C, T, lrs::Opts(), dtype);
    const size_t bf = f.nchunk > 1 ? lookback_bytes(C * f.nchunk, C) : 0;
    const size_t bb = b.nchunk > 1 ? lookback_bytes(C * b.nchunk, C) : 0;
    *bytes = bf > bb ? bf : bb;
  } else {
    const lrs::ColPlan f = lrs::plan_scan_fwd_tbd(C, T, dtype), b = lrs::plan_scan_bwd_tbd(C, T, dtype);
    const size_t bf = lookback_bytes(lrs::col_status_words(f), f.ncb);
    const size_t bb = lookback_bytes(lrs::col_status_words(b), b.ncb);
    *bytes = bf > bb ? bf : bb;
  }
  return LRS_OK;
}

}  // namespace

// Fill dst[0..n) with src[0..n) or with zero (small per-channel outputs of
// empty-time problems).
namespace lrs {
__global__ void k_copy_or_zero(float* __restrict__ dst, const float* __restrict__ src, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.0f;
}
hipError_t launch_copy_or_zero(float* dst, const float* src, int64_t n, hipStream_t s) {
  if (n <= 0 || !dst) return hipSuccess;
  hipLaunchKernelGGL(k_copy_or_zero, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dst, src,
                     n);
  return hipGetLastError();
}
}  // namespace lrs

// Device array behind lrs_scan_fwd_bwd_noalloc: the look-back status words
// and tickets of its calls live here instead of in a caller's workspace.
// Each GPU the library runs on holds its own copy until the process ends.  In
// host code the array's name is not a device address: the address is looked
// up once per device with hipGetSymbolAddress (that device current) and kept
// in scratch_dev[], and only that pointer is handed to kernels.
static __device__ __align__(256) unsigned char scratch[LRS_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_dev[kMaxDevices];

// Device address of the current device's copy of `scratch`.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LRS_ERR_HIP;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LRS_ERR_HIP;
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return LRS_OK;
}
}  // namespace

extern "C" {

const char* lrs_status_string(int status) {
  switch (status) {
    case LRS_OK: return "LRS_OK";
    case LRS_ERR_INVALID_ARG: return "LRS_ERR_INVALID_ARG: invalid argument";
    case LRS_ERR_UNSUPPORTED: return "LRS_ERR_UNSUPPORTED: not supported by this build";
    case LRS_ERR_WORKSPACE: return "LRS_ERR_WORKSPACE: workspace missing or too small";
    case LRS_ERR_HIP: return "LRS_ERR_HIP: HIP runtime or launch failure";
    case LRS_ERR_NONFINITE: return "LRS_ERR_NONFINITE: non-finite DEER update";
    default: return "LRS_ERR_UNKNOWN";
  }
}

int lrs_version(void) { return 100; }

// ------------------------------------------------------------------- scan

size_t lrs_scan_workspace_bytes(int64_t B, int64_t D, int64_t T, int layout, int dtype) {
  int64_t C, N;
  if (!shape_ok(B, D, T, &C, &N) || (layout != LRS_LAYOUT_BDT && layout != LRS_LAYOUT_TBD) ||
      (dtype != LRS_F32 && dtype != LRS_BF16))
    return 0;
  if (N == 0) return 0;
  size_t bytes = 0;
  scan_ws_needs(C, T, layout, dtype, &bytes);
  return bytes;
}

static int scan_common_checks(int64_t B, int64_t D, int64_t T, int layout, int dtype,
                              int64_t* C, int64_t* N) {
  if (!shape_ok(B, D, T, C, N)) return LRS_ERR_INVALID_ARG;
  if (layout != LRS_LAYOUT_BDT && layout != LRS_LAYOUT_TBD) return LRS_ERR_INVALID_ARG;
  if (dtype != LRS_F32 && dtype != LRS_BF16) return LRS_ERR_INVALID_ARG;
  return LRS_OK;
}

static int scan_fwd_impl(const void* a, const void* b, const float* h0, void* h, int64_t B, int64_t D,
                 int64_t T, int layout, int dtype, void* workspace, size_t workspace_bytes,
                 void* stream,
    const lrs::Opts& opt) {
  int64_t C, N;
  int rc = scan_common_checks(B, D, T, layout, dtype, &C, &N);
  if (rc != LRS_OK) return rc;
  if (N == 0) return LRS_OK;
  if (!a || !b || !h) return LRS_ERR_INVALID_ARG;
  const size_t es = (size_t)lrs::io_bytes(dtype);
  if (!aligned(a, es) || !aligned(b, es) || !aligned(h, es) || (h0 && !aligned(h0, 4)))
    return LRS_ERR_INVALID_ARG;
  const size_t nbytes = (size_t)N * es;
  if (overlap(h, nbytes, a, nbytes) || overlap(h, nbytes, b, nbytes) ||
      overlap(h, nbytes, h0, (size_t)C * 4))
    return LRS_ERR_INVALID_ARG;
  size_t need = 0;
  scan_ws_needs(C, T, layout, dtype, &need);
  if (need && (!workspace || workspace_bytes < need)) return LRS_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  // 4-element groups: 16-byte (fp32) or 8-byte (bf16) accesses
  const bool al16 = aligned(a, 4 * es) && aligned(b, 4 * es) && aligned(h, 4 * es);

  if (layout == LRS_LAYOUT_BDT) {
    const lrs::RowPlan p = lrs::plan_scan_fwd_rows(C, T, opt, dtype);
    if (!rows_grid_ok(p, C)) return LRS_ERR_UNSUPPORTED;
    uint64_t* status = nullptr;
    unsigned* tickets = nullptr;
    if (p.nchunk > 1) {
      Carve cv(align_ptr(workspace));
      status = cv.take<uint64_t>(C * p.nchunk);
      tickets = cv.take<unsigned>(C);
      rc = hip_status(lrs::launch_reset(status, C * p.nchunk, tickets, C, nullptr, 0, s));
      if (rc != LRS_OK) return rc;
    }
    // packed blocks start group-aligned whatever T is
    const int vec = al16 && (p.packed || T % 4 == 0);
    return hip_status(lrs::launch_scan_fwd_bdt(a, b, h0, h, dtype, C, T, p, vec, status, tickets,
                                               s));
  }
  const lrs::ColPlan p = lrs::plan_scan_fwd_tbd(C, T, dtype);
  if (!grid_ok(p.ncb * p.ntb, p.nw * 64)) return LRS_ERR_UNSUPPORTED;
  uint64_t* status = nullptr;
  unsigned* tickets = nullptr;
  const int64_t nst = lrs::col_status_words(p);
  if (nst > 0) {
    Carve cv(align_ptr(workspace));
    status = cv.take<uint64_t>(nst);
    tickets = cv.take<unsigned>(p.ncb);
    rc = hip_status(lrs::launch_reset(status, nst, tickets, p.ncb, nullptr, 0, s));
    if (rc != LRS_OK) return rc;
  }
  const int vec = al16 && (C % p.cpt == 0);
  return hip_status(lrs::launch_scan_fwd_tbd(a, b, h0, h, dtype, C, T, p, vec, status, tickets, s));
}

static int scan_bwd_impl(const void* a, const void* h, const float* h0, const void* grad_h, void* grad_a,
                 void* grad_b, float* grad_h0, int64_t B, int64_t D, int64_t T, int layout,
                 int dtype, void* workspace, size_t workspace_bytes, void* stream,
    const lrs::Opts& opt) {
  int64_t C, N;
  int rc = scan_common_checks(B, D, T, layout, dtype, &C, &N);
  if (rc != LRS_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  if (N == 0) {
    // no time steps: nothing depends on h0, so its gradient is zero
    if (T == 0 && C > 0 && grad_h0) return hip_status(lrs::launch_copy_or_zero(grad_h0, nullptr, C, s));
    return LRS_OK;
  }
  if (!a || !h || !grad_h || !grad_a || !grad_b) return LRS_ERR_INVALID_ARG;
  const size_t es = (size_t)lrs::io_bytes(dtype);
  if (!aligned(a, es) || !aligned(h, es) || !aligned(grad_h, es) || !aligned(grad_a, es) ||
      !aligned(grad_b, es) || (h0 && !aligned(h0, 4)) || (grad_h0 && !aligned(grad_h0, 4)))
    return LRS_ERR_INVALID_ARG;
  const size_t nb = (size_t)N * es, cb = (size_t)C * 4;
  // outputs must not overlap inputs, except grad_b == grad_h exactly
  const void* ins[4] = {a, h, h0, grad_h};
  const size_t insz[4] = {nb, nb, cb, nb};
  for (int i = 0; i < 4; ++i) {
    if (overlap(grad_a, nb, ins[i], insz[i])) return LRS_ERR_INVALID_ARG;
    if (i != 3 && overlap(grad_b, nb, ins[i], insz[i])) return LRS_ERR_INVALID_ARG;
    if (overlap(grad_h0, cb, ins[i], insz[i])) return LRS_ERR_INVALID_ARG;
  }
  if (grad_b != grad_h && overlap(grad_b, nb, grad_h, nb)) return LRS_ERR_INVALID_ARG;
  if (overlap(grad_a, nb, grad_b, nb) || overlap(grad_h0, cb, grad_a, nb) ||
      overlap(grad_h0, cb, grad_b, nb))
    return LRS_ERR_INVALID_ARG;
  size_t need = 0;
  scan_ws_needs(C, T, layout, dtype, &need);
  if (need && (!workspace || workspace_bytes < need)) return LRS_ERR_WORKSPACE;
  const bool al16 = aligned(a, 4 * es) && aligned(h, 4 * es) && aligned(grad_h, 4 * es) &&
                    aligned(grad_a, 4 * es) && aligned(grad_b, 4 * es);

  if (layout == LRS_LAYOUT_BDT) {
    const lrs::RowPlan p = lrs::plan_scan_bwd_rows(C, T, opt, dtype);
    if (!rows_grid_ok(p, C)) return LRS_ERR_UNSUPPORTED;
    uint64_t* status = nullptr;
    unsigned* tickets = nullptr;
    if (p.nchunk > 1) {
      Carve cv(align_ptr(workspace));
      status = cv.take<uint64_t>(C * p.nchunk);
      tickets = cv.take<unsigned>(C);
      rc = hip_status(lrs::launch_reset(status, C * p.nchunk, tickets, C, nullptr, 0, s));
      if (rc != LRS_OK) return rc;
    }
    const int vec = al16 && (p.packed || T % 4 == 0);
    return hip_status(lrs::launch_scan_bwd_bdt(a, h, h0, grad_h, grad_a, grad_b, grad_h0, dtype, C,
                                               T, p, vec, status, tickets, s));
  }
  const lrs::ColPlan p = lrs::plan_scan_bwd_tbd(C, T, dtype);
  if (!grid_ok(p.ncb * p.ntb, p.nw * 64)) return LRS_ERR_UNSUPPORTED;
  uint64_t* status = nullptr;
  unsigned* tickets = nullptr;
  const int64_t nst = lrs::col_status_words(p);
  if (nst > 0) {
    Carve cv(align_ptr(workspace));
    status = cv.take<uint64_t>(nst);
    tickets = cv.take<unsigned>(p.ncb);
    rc = hip_status(lrs::launch_reset(status, nst, tickets, p.ncb, nullptr, 0, s));
    if (rc != LRS_OK) return rc;
  }
  const int vec = al16 && (C % p.cpt == 0);
  return hip_status(lrs::launch_scan_bwd_tbd(a, h, h0, grad_h, grad_a, grad_b, grad_h0, dtype, C, T,
                                             p, vec, status, tickets, s));
}

static int scan_fwd_bwd_impl(const void* a, const void* b, const float* h0, const void* grad_h, void* h,
                     void* grad_a, void* grad_b, float* grad_h0, int64_t B, int64_t D, int64_t T,
                     int layout, int dtype, void* workspace, size_t workspace_bytes,
                     void* stream,
    const lrs::Opts& opt) {
  int64_t C, N;
  int rc = scan_common_checks(B, D, T, layout, dtype, &C, &N);
  if (rc != LRS_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  if (N == 0) {
    if (T == 0 && C > 0 && grad_h0) return hip_status(lrs::launch_copy_or_zero(grad_h0, nullptr, C, s));
    return LRS_OK;
  }
  if (!a || !b || !grad_h || !grad_a || !grad_b) return LRS_ERR_INVALID_ARG;
  const size_t es = (size_t)lrs::io_bytes(dtype);
  if (!aligned(a, es) || !aligned(b, es) || !aligned(grad_h, es) || !aligned(grad_a, es) ||
      !aligned(grad_b, es) || (h && !aligned(h, es)) || (h0 && !aligned(h0, 4)) ||
      (grad_h0 && !aligned(grad_h0, 4)))
    return LRS_ERR_INVALID_ARG;
  const size_t nb = (size_t)N * es, cb = (size_t)C * 4;
  // outputs must not overlap inputs or each other, except grad_b == grad_h exactly
  const void* ins[4] = {a, b, h0, grad_h};
  const size_t insz[4] = {nb, nb, cb, nb};
  const void* outs[4] = {h, grad_a, grad_b, grad_h0};
  const size_t outsz[4] = {nb, nb, nb, cb};
  for (int o = 0; o < 4; ++o) {
    for (int i = 0; i < 4; ++i) {
      if (o == 2 && i == 3 && grad_b == grad_h) continue;
      if (overlap(outs[o], outsz[o], ins[i], insz[i])) return LRS_ERR_INVALID_ARG;
    }
    for (int o2 = o + 1; o2 < 4; ++o2)
      if (overlap(outs[o], outsz[o], outs[o2], outsz[o2])) return LRS_ERR_INVALID_ARG;
  }
  const lrs::RowPlan p = lrs::plan_scan_fused_rows(C, T, dtype);
  // short channels run the sequential or packed passes when h is wanted anyway
  // (the one-kernel form gives each channel a mostly idle workgroup)
  const lrs::RowPlan pf = lrs::plan_scan_fwd_rows(C, T, opt, dtype);
  const bool short_pair = h && (pf.serial || pf.packed);
  if (layout == LRS_LAYOUT_BDT && p.nchunk == 1 && !short_pair) {
    if (!grid_ok(C, p.threads())) return LRS_ERR_UNSUPPORTED;
    const bool al16 = aligned(a, 4 * es) && aligned(b, 4 * es) && aligned(grad_h, 4 * es) &&
                      aligned(grad_a, 4 * es) && aligned(grad_b, 4 * es) &&
                      (!h || aligned(h, 4 * es));
    const int vec = al16 && (T % 4 == 0);
    return hip_status(lrs::launch_scan_fused_bdt(a, b, h0, grad_h, h, grad_a, grad_b, grad_h0, dtype,
                                                 C, T, p, vec, s));
  }
  // the two passes, h stored between them (both validated before the first launch)
  if (!h) return LRS_ERR_UNSUPPORTED;
  size_t need = 0;
  scan_ws_needs(C, T, layout, dtype, &need);
  if (need && (!workspace || workspace_bytes < need)) return LRS_ERR_WORKSPACE;
  rc = scan_fwd_impl(a, b, h0, h, B, D, T, layout, dtype, workspace, workspace_bytes, stream, opt);
  if (rc != LRS_OK) return rc;
  return scan_bwd_impl(a, h, h0, grad_h, grad_a, grad_b, grad_h0, B, D, T, layout, dtype,
                       workspace, workspace_bytes, stream, opt);
}

// -------------------------------------------------------------------- SRU

size_t lrs_sru_workspace_bytes(int64_t T, int64_t B, int64_t D) {
  int64_t C, N;
  if (!shape_ok(B, D, T, &C, &N) || N == 0) return 0;
  size_t b1 = 0, b2 = 0;
  {
    const lrs::ColPlan p = lrs::plan_sru(C, T, LRS_BF16, false);
    b1 = lookback_bytes(lrs::col_status_words(p), p.ncb);
  }
  {
    const lrs::ColPlan p = lrs::plan_sru(C, T, LRS_F32, false);
    b2 = lookback_bytes(lrs::col_status_words(p), p.ncb);
  }
  return b1 > b2 ? b1 : b2;
}

static int sru_fwd_impl(const void* z_f, const void* z_r, const void* z_x, const float* bias_f,
                const float* bias_r, const float* c0, void* h, float* c_last, float* c_states,
                int64_t T, int64_t B, int64_t D, int io_dtype, void* workspace,
                size_t workspace_bytes, void* stream,
    const lrs::Opts& opt) {
  int64_t C, N;
  if (!shape_ok(B, D, T, &C, &N)) return LRS_ERR_INVALID_ARG;
  if (io_dtype != LRS_F32 && io_dtype != LRS_BF16) return LRS_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (N == 0) {
    if (T == 0 && C > 0 && c_last) return hip_status(lrs::launch_copy_or_zero(c_last, c0, C, s));
    return LRS_OK;
  }
  if (!z_f || !z_r || !z_x || !bias_f || !bias_r || !h) return LRS_ERR_INVALID_ARG;
  const size_t es = io_dtype == LRS_BF16 ? 2 : 4;
  if (!aligned(z_f, es) || !aligned(z_r, es) || !aligned(z_x, es) || !aligned(h, es) ||
      !aligned(bias_f, 4) || !aligned(bias_r, 4) || (c0 && !aligned(c0, 4)) ||
      (c_last && !aligned(c_last, 4)) || (c_states && !aligned(c_states, 4)))
    return LRS_ERR_INVALID_ARG;
  const size_t nb = (size_t)N * es, cb = (size_t)C * 4, db = (size_t)D * 4, sb = (size_t)N * 4;
  const void* ins[6] = {z_f, z_r, z_x, bias_f, bias_r, c0};
  const size_t insz[6] = {nb, nb, nb, db, db, cb};
  for (int i = 0; i < 6; ++i)
    if (overlap(h, nb, ins[i], insz[i]) || overlap(c_last, cb, ins[i], insz[i]) ||
        overlap(c_states, sb, ins[i], insz[i]))
      return LRS_ERR_INVALID_ARG;
  if (overlap(h, nb, c_last, cb) || overlap(h, nb, c_states, sb) ||
      overlap(c_last, cb, c_states, sb))
    return LRS_ERR_INVALID_ARG;
  const lrs::ColPlan p = lrs::plan_sru(C, T, io_dtype, true, opt);
  if (!grid_ok(p.ncb * p.ntb, p.nw * 64)) return LRS_ERR_UNSUPPORTED;
  const int64_t nst = lrs::col_status_words(p);
  const size_t need = lookback_bytes(nst, p.ncb);
  if (need && (!workspace || workspace_bytes < need)) return LRS_ERR_WORKSPACE;
  uint64_t* status = nullptr;
  unsigned* tickets = nullptr;
  if (nst > 0) {
    Carve cv(align_ptr(workspace));
    status = cv.take<uint64_t>(nst);
    tickets = cv.take<unsigned>(p.ncb);
    const int rc = hip_status(lrs::launch_reset(status, nst, tickets, p.ncb, nullptr, 0, s));
    if (rc != LRS_OK) return rc;
  }
  const size_t rowbytes = (size_t)p.cpt * es;
  const int vec = aligned(z_f, rowbytes) && aligned(z_r, rowbytes) && aligned(z_x, rowbytes) &&
                  aligned(h, rowbytes) && (!c_states || aligned(c_states, (size_t)p.cpt * 4)) &&
                  (C % p.cpt == 0);
  return hip_status(lrs::launch_sru_fwd(z_f, z_r, z_x, bias_f, bias_r, c0, h, c_last, c_states, T,
                                        B, D, io_dtype, p, vec, status, tickets, s));
}

// SRU backward: look-back state, 2 * ntb * C floats of per-tile bias partials
// and the fp64 stage of their reduction.
static size_t sru_bwd_ws(const lrs::ColPlan& p, int64_t B, int64_t D) {
  const int64_t C = B * D;
  return lookback_bytes(lrs::col_status_words(p), p.ncb) +
         align_up((size_t)(2 * p.ntb * C) * 4) +
         align_up((size_t)(2 * lrs::col_sum_blocks(p.ntb * B) * D) * 8);
}

size_t lrs_sru_bwd_workspace_bytes(int64_t T, int64_t B, int64_t D) {
  int64_t C, N;
  if (!shape_ok(B, D, T, &C, &N) || N == 0) return 0;
  const size_t b1 = sru_bwd_ws(lrs::plan_sru_bwd(C, T, LRS_BF16), B, D);
  const size_t b2 = sru_bwd_ws(lrs::plan_sru_bwd(C, T, LRS_F32), B, D);
  return kAlign + (b1 > b2 ? b1 : b2);
}

int lrs_sru_bwd(const void* z_f, const void* z_r, const void* z_x, const float* bias_f,
                const float* bias_r, const float* c0, const float* c_states, const void* grad_h,
                const float* grad_c_last, void* grad_zf, void* grad_zr, void* grad_zx,
                float* grad_bias_f, float* grad_bias_r, float* grad_c0, int64_t T, int64_t B,
                int64_t D, int io_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  int64_t C, N;
  if (!shape_ok(B, D, T, &C, &N)) return LRS_ERR_INVALID_ARG;
  if (io_dtype != LRS_F32 && io_dtype != LRS_BF16) return LRS_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (N == 0) {
    // no steps: the bias gradients are empty sums; dL/dc0 = dL/dc_T
    int rc = LRS_OK;
    if (D > 0 && grad_bias_f) rc = hip_status(lrs::launch_copy_or_zero(grad_bias_f, nullptr, D, s));
    if (rc == LRS_OK && D > 0 && grad_bias_r)
      rc = hip_status(lrs::launch_copy_or_zero(grad_bias_r, nullptr, D, s));
    if (rc == LRS_OK && T == 0 && C > 0 && grad_c0)
      rc = hip_status(lrs::launch_copy_or_zero(grad_c0, grad_c_last, C, s));
    return rc;
  }
  if (!z_f || !z_r || !z_x || !bias_f || !bias_r || !c_states || !grad_h || !grad_zf ||
      !grad_zr || !grad_zx || !grad_bias_f || !grad_bias_r)
    return LRS_ERR_INVALID_ARG;
  const size_t es = io_dtype == LRS_BF16 ? 2 : 4;
  const void* io[7] = {z_f, z_r, z_x, grad_h, grad_zf, grad_zr, grad_zx};
  for (int i = 0; i < 7; ++i)
    if (!aligned(io[i], es)) return LRS_ERR_INVALID_ARG;
  if (!aligned(bias_f, 4) || !aligned(bias_r, 4) || !aligned(c_states, 4) ||
      (c0 && !aligned(c0, 4)) || (grad_c_last && !aligned(grad_c_last, 4)) ||
      !aligned(grad_bias_f, 4) || !aligned(grad_bias_r, 4) || (grad_c0 && !aligned(grad_c0, 4)))
    return LRS_ERR_INVALID_ARG;
  const size_t nb = (size_t)N * es, cb = (size_t)C * 4, db = (size_t)D * 4, sb = (size_t)N * 4;
  const void* ins[8] = {z_f, z_r, z_x, grad_h, c_states, bias_f, bias_r, c0};
  const size_t insz[8] = {nb, nb, nb, nb, sb, db, db, cb};
  const void* outs[6] = {grad_zf, grad_zr, grad_zx, grad_bias_f, grad_bias_r, grad_c0};
  const size_t outsz[6] = {nb, nb, nb, db, db, cb};
  for (int o = 0; o < 6; ++o) {
    for (int i = 0; i < 8; ++i)
      if (overlap(outs[o], outsz[o], ins[i], insz[i])) return LRS_ERR_INVALID_ARG;
    if (overlap(outs[o], outsz[o], grad_c_last, cb)) return LRS_ERR_INVALID_ARG;
    for (int o2 = o + 1; o2 < 6; ++o2)
      if (overlap(outs[o], outsz[o], outs[o2], outsz[o2])) return LRS_ERR_INVALID_ARG;
  }
  const lrs::ColPlan p = lrs::plan_sru_bwd(C, T, io_dtype);
  if (!grid_ok(p.ncb * p.ntb, p.nw * 64)) return LRS_ERR_UNSUPPORTED;
  const size_t need = lrs_sru_bwd_workspace_bytes(T, B, D);
  if (!workspace || workspace_bytes < need) return LRS_ERR_WORKSPACE;
  Carve cv(align_ptr(workspace));
  float* part = cv.take<float>(2 * p.ntb * C);
  double* acc = cv.take<double>(2 * lrs::col_sum_blocks(p.ntb * B) * D);
  uint64_t* status = nullptr;
  unsigned* tickets = nullptr;
  const int64_t nst = lrs::col_status_words(p);
  if (nst > 0) {
    status = cv.take<uint64_t>(nst);
    tickets = cv.take<unsigned>(p.ncb);
    const int rc = hip_status(lrs::launch_reset(status, nst, tickets, p.ncb, nullptr, 0, s));
    if (rc != LRS_OK) return rc;
  }
  const size_t rowbytes = (size_t)p.cpt * es;
  int vec = (C % p.cpt == 0) && aligned(c_states, (size_t)p.cpt * 4);
  for (int i = 0; i < 7; ++i) vec = vec && aligned(io[i], rowbytes);
  return hip_status(lrs::launch_sru_bwd(z_f, z_r, z_x, bias_f, bias_r, c0, c_states, grad_h,
                                        grad_c_last, grad_zf, grad_zr, grad_zx, grad_bias_f,
                                        grad_bias_r, grad_c0, part, acc, T, B, D, io_dtype, p,
                                        vec, status, tickets, s));
}

// ------------------------------------------------------------------- LSTM

size_t lrs_lstm_workspace_bytes(int64_t T, int64_t B, int64_t D) {
  int64_t C, N;
  if (!shape_ok(B, D, T, &C, &N) || N == 0) return 0;
  size_t need = 0;
  for (int io = 0; io < 2; ++io) {
    const lrs::ColPlan ps[3] = {lrs::plan_lstm(C, T, io, false, false),
                                lrs::plan_lstm(C, T, io, true, false),
                                lrs::plan_lstm_bwd(C, T, io)};
    for (const lrs::ColPlan& p : ps) {
      const size_t b = lookback_bytes(lrs::col_status_words(p), p.ncb);
      need = b > need ? b : need;
    }
  }
  return need;
}

// Carves and resets the look-back state of a [T,B,D] plan.
static int col_lookback(const lrs::ColPlan& p, void* workspace, size_t workspace_bytes,
                        hipStream_t s, uint64_t** status, unsigned** tickets) {
  *status = nullptr;
  *tickets = nullptr;
  const int64_t nst = lrs::col_status_words(p);
  const size_t need = lookback_bytes(nst, p.ncb);
  if (need && (!workspace || workspace_bytes < need)) return LRS_ERR_WORKSPACE;
  if (nst == 0) return LRS_OK;
  Carve cv(align_ptr(workspace));
  *status = cv.take<uint64_t>(nst);
  *tickets = cv.take<unsigned>(p.ncb);
  return hip_status(lrs::launch_reset(*status, nst, *tickets, p.ncb, nullptr, 0, s));
}

static int lstm_fwd_impl(const void* z_f, const void* z_i, const void* z_c, const void* z_o,
                         const float* c0, void* h, float* c_last, float* c_states, int64_t T,
                         int64_t B, int64_t D, int io_dtype, void* workspace,
                         size_t workspace_bytes, void* stream, const lrs::Opts& opt) {
  int64_t C, N;
  if (!shape_ok(B, D, T, &C, &N)) return LRS_ERR_INVALID_ARG;
  if (io_dtype != LRS_F32 && io_dtype != LRS_BF16) return LRS_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (N == 0) {
    if (T == 0 && C > 0 && c_last) return hip_status(lrs::launch_copy_or_zero(c_last, c0, C, s));
    return LRS_OK;
  }
  if (!z_f || !z_i || !z_c || !z_o || !h) return LRS_ERR_INVALID_ARG;
  const size_t es = io_dtype == LRS_BF16 ? 2 : 4;
  if (!aligned(z_f, es) || !aligned(z_i, es) || !aligned(z_c, es) || !aligned(z_o, es) ||
      !aligned(h, es) || (c0 && !aligned(c0, 4)) || (c_last && !aligned(c_last, 4)) ||
      (c_states && !aligned(c_states, 4)))
    return LRS_ERR_INVALID_ARG;
  const size_t nb = (size_t)N * es, cb = (size_t)C * 4, sb = (size_t)N * 4;
  const void* ins[5] = {z_f, z_i, z_c, z_o, c0};
  const size_t insz[5] = {nb, nb, nb, nb, cb};
  for (int i = 0; i < 5; ++i)
    if (overlap(h, nb, ins[i], insz[i]) || overlap(c_last, cb, ins[i], insz[i]) ||
        overlap(c_states, sb, ins[i], insz[i]))
      return LRS_ERR_INVALID_ARG;
  if (overlap(h, nb, c_last, cb) || overlap(h, nb, c_states, sb) ||
      overlap(c_last, cb, c_states, sb))
    return LRS_ERR_INVALID_ARG;
  const lrs::ColPlan p = lrs::plan_lstm(C, T, io_dtype, c_states != nullptr, true, opt);
  if (!grid_ok(p.persist ? p.ncb : p.ncb * p.ntb, p.nw * 64)) return LRS_ERR_UNSUPPORTED;
  uint64_t* status;
  unsigned* tickets;
  const int rc = col_lookback(p, workspace, workspace_bytes, s, &status, &tickets);
  if (rc != LRS_OK) return rc;
  const size_t rowbytes = (size_t)p.cpt * es;
  const int vec = aligned(z_f, rowbytes) && aligned(z_i, rowbytes) && aligned(z_c, rowbytes) &&
                  aligned(z_o, rowbytes) && aligned(h, rowbytes) &&
                  (!c_states || aligned(c_states, (size_t)p.cpt * 4)) && (C % p.cpt == 0);
  return hip_status(lrs::launch_lstm_fwd(z_f, z_i, z_c, z_o, c0, h, c_last, c_states, T, C,
                                         io_dtype, p, vec, status, tickets, s));
}

int lrs_lstm_bwd(const void* z_f, const void* z_i, const void* z_c, const void* z_o,
                 const float* c0, const float* c_states, const void* grad_h,
                 const float* grad_c_last, void* grad_zf, void* grad_zi, void* grad_zc,
                 void* grad_zo, float* grad_c0, int64_t T, int64_t B, int64_t D, int io_dtype,
                 void* workspace, size_t workspace_bytes, void* stream) {
  int64_t C, N;
  if (!shape_ok(B, D, T, &C, &N)) return LRS_ERR_INVALID_ARG;
  if (io_dtype != LRS_F32 && io_dtype != LRS_BF16) return LRS_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (N == 0) {
    // no steps: dL/dc0 = dL/dc_T
    if (T == 0 && C > 0 && grad_c0)
      return hip_status(lrs::launch_copy_or_zero(grad_c0, grad_c_last, C, s));
    return LRS_OK;
  }
  if (!z_f || !z_i || !z_c || !z_o || !c_states || !grad_h || !grad_zf || !grad_zi ||
      !grad_zc || !grad_zo)
    return LRS_ERR_INVALID_ARG;
  const size_t es = io_dtype == LRS_BF16 ? 2 : 4;
  const void* io[9] = {z_f, z_i, z_c, z_o, grad_h, grad_zf, grad_zi, grad_zc, grad_zo};
  for (int i = 0; i < 9; ++i)
    if (!aligned(io[i], es)) return LRS_ERR_INVALID_ARG;
  if (!aligned(c_states, 4) || (c0 && !aligned(c0, 4)) ||
      (grad_c_last && !aligned(grad_c_last, 4)) || (grad_c0 && !aligned(grad_c0, 4)))
    return LRS_ERR_INVALID_ARG;
  const size_t nb = (size_t)N * es, cb = (size_t)C * 4, sb = (size_t)N * 4;
  const void* ins[8] = {z_f, z_i, z_c, z_o, grad_h, c_states, c0, grad_c_last};
  const size_t insz[8] = {nb, nb, nb, nb, nb, sb, cb, cb};
  const void* outs[5] = {grad_zf, grad_zi, grad_zc, grad_zo, grad_c0};
  const size_t outsz[5] = {nb, nb, nb, nb, cb};
  for (int o = 0; o < 5; ++o) {
    for (int i = 0; i < 8; ++i)
      if (overlap(outs[o], outsz[o], ins[i], insz[i])) return LRS_ERR_INVALID_ARG;
    for (int o2 = o + 1; o2 < 5; ++o2)
      if (overlap(outs[o], outsz[o], outs[o2], outsz[o2])) return LRS_ERR_INVALID_ARG;
  }
  const lrs::ColPlan p = lrs::plan_lstm_bwd(C, T, io_dtype);
  if (!grid_ok(p.ncb * p.ntb, p.nw * 64)) return LRS_ERR_UNSUPPORTED;
  uint64_t* status;
  unsigned* tickets;
  const int rc = col_lookback(p, workspace, workspace_bytes, s, &status, &tickets);
  if (rc != LRS_OK) return rc;
  const size_t rowbytes = (size_t)p.cpt * es;
  int vec = (C % p.cpt == 0) && aligned(c_states, (size_t)p.cpt * 4);
  for (int i = 0; i < 9; ++i) vec = vec && aligned(io[i], rowbytes);
  return hip_status(lrs::launch_lstm_bwd(z_f, z_i, z_c, z_o, c0, c_states, grad_h, grad_c_last,
                                         grad_zf, grad_zi, grad_zc, grad_zo, grad_c0, T, C,
                                         io_dtype, p, vec, status, tickets, s));
}

// ------------------------------------------------------------------- DEER

static lrs::RowPlan deer_plan(int64_t C, int64_t T) { return lrs::plan_deer_rows(C, T); }

// The workspace starts with the norm slot sets, the solve record and the
// per-iteration norms (cleared together at the start of a solve).
static size_t deer_record_bytes(int k_max) {
  return align_up(((size_t)lrs::kDeltaSetWords + lrs::kDeerRecordWords + (size_t)k_max) * 4);
}

struct DeerRecord {
  uint32_t* delta_bits;  // slot sets
  int* rec;              // {iterations, converged, non-finite, unused}
  uint32_t* delta_out;   // k_max norms
};

static DeerRecord carve_deer_record(Carve& cv, int k_max) {
  DeerRecord r;
  r.delta_bits = cv.take<uint32_t>(lrs::kDeltaSetWords + lrs::kDeerRecordWords + k_max);
  r.rec = reinterpret_cast<int*>(r.delta_bits + lrs::kDeltaSetWords);
  r.delta_out = r.delta_bits + lrs::kDeltaSetWords + lrs::kDeerRecordWords;
  return r;
}

// Read a finished solve's record and norms to the host (waits for the stream).
static int read_deer_record(const DeerRecord& r, int k_max, int* iters_out, float* deltas_out,
                            int* converged_out, hipStream_t s) {
  std::vector<uint32_t> buf((size_t)lrs::kDeerRecordWords + (size_t)k_max);
  if (hipMemcpyAsync(buf.data(), r.rec, sizeof(uint32_t) * buf.size(), hipMemcpyDeviceToHost,
                     s) != hipSuccess)
    return LRS_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return LRS_ERR_HIP;
  const int iters = (int)buf[0];
  if (iters < 1 || iters > k_max) return LRS_ERR_HIP;  // no finished solve in this workspace
  if (iters_out) *iters_out = iters;
  if (converged_out) *converged_out = (int)buf[1];
  if (deltas_out) {
    for (int i = 0; i < k_max; ++i) {
      float d = 0.0f;
      if (i < iters) memcpy(&d, &buf[(size_t)lrs::kDeerRecordWords + i], 4);
      deltas_out[i] = d;
    }
  }
  return buf[2] ? LRS_ERR_NONFINITE : LRS_OK;
}

// The fused solve (all Newton iterations in one walk over each channel, one
// workgroup per channel) needs k_max <= kDeerFuseMax: one norm slot set per
// iteration.  By default it runs where one workgroup walks the channel in any
// case (T <= 8192), and for longer channels when there are at least as many
// channels as compute units.  It moves 8 bytes per element for the whole solve
// against 56 for one launch per iteration: per 5-iteration solve, 0.35 ms
// against 1.35 ms at 8192 channels of 16384 steps and 50 us against 122 us at
// 256 channels of 32768.  With fewer channels each walk is a long serial
// chain on a mostly idle device, and the per-iteration launches, which spread
// every channel over many workgroups, take over.  deer_fuse = 0 in the
// caller's options never fuses; deer_fuse > 0 fuses whenever k_max allows.
static bool deer_use_fused(const lrs::RowPlan& p, int64_t C, int k_max, const lrs::Opts& opt) {
  if (k_max > lrs::kDeerFuseMax || opt.deer_fuse == 0) return false;
  if (opt.deer_fuse > 0) return true;
  return p.nchunk == 1 || C >= (int64_t)lrs::device_cus();
}

// deer_fuse = 0 in the caller's options runs the SRU-by-DEER iterations one
// launch each even where its fused walk applies.
static bool deer_fuse_enabled(const lrs::Opts& opt) { return opt.deer_fuse != 0; }

static size_t deer_fused_set_words(int k_max) {
  return (size_t)k_max * lrs::kDeltaSlots * lrs::kDeltaStride;
}

size_t lrs_deer_workspace_bytes(int64_t B, int64_t D, int64_t T, int k_max) {
  int64_t C, N;
  if (!shape_ok(B, D, T, &C, &N) || k_max < 1) return 0;
  if (N == 0) return 0;
  const lrs::RowPlan p = deer_plan(C, T);
  size_t bytes = kAlign + deer_record_bytes(k_max) + align_up((size_t)N * 4);
  if (p.nchunk > 1) bytes += align_up((size_t)(C * p.nchunk) * 8) + align_up((size_t)C * 4);
  // the fused solve's norm sets, whichever plan the call takes
  if (k_max <= lrs::kDeerFuseMax) bytes += align_up(deer_fused_set_words(k_max) * 4);
  return bytes;
}

static int deer_solve_impl(const float* w, const float* u, const float* h0, const float* h_init, float* h,
                   int64_t B, int64_t D, int64_t T, float eps, int k_max, int* iters_out,
                   float* deltas_out, int* converged_out, void* workspace,
                   size_t workspace_bytes, void* stream,
    const lrs::Opts& opt) {
  int64_t C, N;
  if (!shape_ok(B, D, T, &C, &N) || k_max < 1 || k_max > 1000000) return LRS_ERR_INVALID_ARG;
  if (N == 0) {
    if (iters_out) *iters_out = 0;
    if (converged_out) *converged_out = 1;
    if (deltas_out) memset(deltas_out, 0, sizeof(float) * (size_t)k_max);
    return LRS_OK;
  }
  if (!w || !u || !h) return LRS_ERR_INVALID_ARG;
  if (!aligned(w, 4) || !aligned(u, 4) || !aligned(h, 4) || (h0 && !aligned(h0, 4)) ||
      (h_init && !aligned(h_init, 4)))
    return LRS_ERR_INVALID_ARG;
  const size_t nb = (size_t)N * 4, cb = (size_t)C * 4;
  if (overlap(h, nb, w, (size_t)D * 4) || overlap(h, nb, u, nb) || overlap(h, nb, h0, cb))
    return LRS_ERR_INVALID_ARG;
  if (h_init && h_init != h && overlap(h, nb, h_init, nb)) return LRS_ERR_INVALID_ARG;
  const size_t need = lrs_deer_workspace_bytes(B, D, T, k_max);
  if (!workspace || workspace_bytes < need) return LRS_ERR_WORKSPACE;
  const lrs::RowPlan p = deer_plan(C, T);
  if (!grid_ok(C * p.nchunk, p.threads())) return LRS_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;

  Carve cv(align_ptr(workspace));
  const DeerRecord r = carve_deer_record(cv, k_max);
  uint32_t* delta_bits = r.delta_bits;
  uint32_t* delta_out = r.delta_out;
  float* ybuf = cv.take<float>(N);
  uint64_t* status = nullptr;
  unsigned* tickets = nullptr;
  if (p.nchunk > 1) {
    status = cv.take<uint64_t>(C * p.nchunk);
    tickets = cv.take<unsigned>(C);
  }
  if (overlap(ybuf, nb, u, nb) || overlap(ybuf, nb, h, nb) || overlap(ybuf, nb, h_init, nb))
    return LRS_ERR_INVALID_ARG;
  const int vec = aligned(u, 16) && aligned(h, 16) && aligned(ybuf, 16) &&
                  (!h_init || aligned(h_init, 16)) && (T % 4 == 0);

  if (deer_use_fused(p, C, k_max, opt)) {
    uint32_t* sets = cv.take<uint32_t>((int64_t)deer_fused_set_words(k_max));
    // the pass must not overwrite a starting iterate held in h: a redo may need it
    float* out = (h_init == h) ? ybuf : h;
    int rc = hip_status(lrs::launch_reset(nullptr, 0, nullptr, 0, sets,
                                          (int64_t)deer_fused_set_words(k_max), s));
    if (rc != LRS_OK) return rc;
    rc = hip_status(lrs::launch_deer_fused(w, u, h_init, h0, out, h, C, D, T, p, vec, k_max, eps,
                                           sets, delta_out, r.rec, s));
    if (rc != LRS_OK) return rc;
    if (!iters_out && !deltas_out && !converged_out) return LRS_OK;  // asynchronous form
    return read_deer_record(r, k_max, iters_out, deltas_out, converged_out, s);
  }

  // ping-pong: iteration i writes P[i % 2]; if the starting iterate lives in h,
  // iteration 0 must not write h, so the roles swap
  float* P[2] = {h, ybuf};
  if (h_init == h) { P[0] = ybuf; P[1] = h; }
  int rc = hip_status(lrs::launch_reset(status, p.nchunk > 1 ? C * p.nchunk : 0, tickets,
                                        p.nchunk > 1 ? C : 0, delta_bits,
                                        lrs::kDeltaSetWords + lrs::kDeerRecordWords + k_max, s));
  if (rc != LRS_OK) return rc;
  for (int i = 0; i < k_max; ++i) {
    if (i > 0 && p.nchunk > 1) {
      rc = hip_status(lrs::launch_reset(status, C * p.nchunk, tickets, C, nullptr, 0, s));
      if (rc != LRS_OK) return rc;
    }
    const float* y = (i == 0) ? h_init : P[(i - 1) & 1];
    rc = hip_status(lrs::launch_deer_iter(w, u, y, h0, P[i & 1], C, D, T, p, vec, status,
                                          tickets, delta_bits, delta_out, i, eps, s));
    if (rc != LRS_OK) return rc;
  }
  rc = hip_status(lrs::launch_deer_finish(delta_bits, delta_out, r.rec, k_max, eps, s));
  if (rc != LRS_OK) return rc;
  rc = hip_status(lrs::launch_deer_select(P[0], P[1], h, N, r.rec, s));
  if (rc != LRS_OK) return rc;
  if (!iters_out && !deltas_out && !converged_out) return LRS_OK;  // asynchronous form
  return read_deer_record(r, k_max, iters_out, deltas_out, converged_out, s);
}

// ------------------------------------------- DEER, per-sequence stopping

// Workspace: per-sequence norm slots (three sets), norms and records, the
// second iterate buffer and the look-back state.
size_t lrs_deer_seq_workspace_bytes(int64_t B, int64_t D, int64_t T, int k_max) {
  int64_t C, N;
  if (!shape_ok(B, D, T, &C, &N) || N == 0 || k_max < 1 || k_max > 1000000) return 0;
  const lrs::RowPlan p = deer_plan(C, T);
  size_t bytes = kAlign + align_up((size_t)(3 * B * lrs::kSeqSlots * lrs::kDeltaStride) * 4) +
                 align_up((size_t)(B * k_max) * 4) + align_up((size_t)(B * 4) * 4) +
                 align_up((size_t)N * 4);
  if (p.nchunk > 1) bytes += align_up((size_t)(C * p.nchunk) * 8) + align_up((size_t)C * 4);
  return bytes;
}

static int deer_solve_seq_impl(const float* w, const float* u, const float* h0, const float* h_init,
                       float* h, int64_t B, int64_t D, int64_t T, float eps, int k_max,
                       int* iters_out, int* converged_out, void* workspace,
                       size_t workspace_bytes, void* stream,
    const lrs::Opts& opt) {
  int64_t C, N;
  if (!shape_ok(B, D, T, &C, &N) || k_max < 1 || k_max > 1000000) return LRS_ERR_INVALID_ARG;
  if (N == 0) {
    for (int64_t b = 0; b < B; ++b) {
      if (iters_out) iters_out[b] = 0;
      if (converged_out) converged_out[b] = 1;
    }
    return LRS_OK;
  }
  if (B > 65535) return LRS_ERR_UNSUPPORTED;
  if (!w || !u || !h) return LRS_ERR_INVALID_ARG;
  if (!aligned(w, 4) || !aligned(u, 4) || !aligned(h, 4) || (h0 && !aligned(h0, 4)) ||
      (h_init && !aligned(h_init, 4)))
    return LRS_ERR_INVALID_ARG;
  const size_t nb = (size_t)N * 4, cb = (size_t)C * 4;
  if (overlap(h, nb, w, (size_t)D * 4) || overlap(h, nb, u, nb) || overlap(h, nb, h0, cb))
    return LRS_ERR_INVALID_ARG;
  if (h_init && h_init != h && overlap(h, nb, h_init, nb)) return LRS_ERR_INVALID_ARG;
  const size_t need = lrs_deer_seq_workspace_bytes(B, D, T, k_max);
  if (!workspace || workspace_bytes < need) return LRS_ERR_WORKSPACE;
  const lrs::RowPlan p = deer_plan(C, T);
  if (!grid_ok(C * p.nchunk, p.threads())) return LRS_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;

  Carve cv(align_ptr(workspace));
  const int64_t nslots = 3 * B * lrs::kSeqSlots * lrs::kDeltaStride;
  uint32_t* seq_slots = cv.take<uint32_t>(nslots);
  uint32_t* seq_delta = cv.take<uint32_t>(B * k_max);
  int* seq_rec = cv.take<int>(B * 4);
  float* ybuf = cv.take<float>(N);
  uint64_t* status = nullptr;
  unsigned* tickets = nullptr;
  if (p.nchunk > 1) {
    status = cv.take<uint64_t>(C * p.nchunk);
    tickets = cv.take<unsigned>(C);
  }
  if (overlap(ybuf, nb, u, nb) || overlap(ybuf, nb, h, nb) || overlap(ybuf, nb, h_init, nb))
    return LRS_ERR_INVALID_ARG;
  float* P[2] = {h, ybuf};
  if (h_init == h) { P[0] = ybuf; P[1] = h; }
  const int vec = aligned(u, 16) && aligned(h, 16) && aligned(ybuf, 16) &&
                  (!h_init || aligned(h_init, 16)) && (T % 4 == 0);
  // slots, norms and records are contiguous: one reset clears them all
  int rc = hip_status(lrs::launch_reset(status, p.nchunk > 1 ? C * p.nchunk : 0, tickets,
                                        p.nchunk > 1 ? C : 0, seq_slots,
                                        (int64_t)((char*)(seq_rec + B * 4) - (char*)seq_slots) / 4,
                                        s));
  if (rc != LRS_OK) return rc;
  if (deer_use_fused(p, C, k_max, opt)) {
    // all iterations in one pass, each sequence's norms folded into seq_delta
    float* out = (h_init == h) ? ybuf : h;
    rc = hip_status(lrs::launch_deer_fused(w, u, h_init, h0, out, h, C, D, T, p, vec, k_max, eps,
                                           nullptr, nullptr, nullptr, s, seq_delta, seq_rec));
    if (rc != LRS_OK) return rc;
  } else {
    for (int i = 0; i < k_max; ++i) {
      if (i > 0) {
        rc = hip_status(lrs::launch_deer_seq_book(seq_slots, seq_delta, B, k_max, i, s));
        if (rc == LRS_OK && p.nchunk > 1)
          rc = hip_status(lrs::launch_reset(status, C * p.nchunk, tickets, C, nullptr, 0, s));
        if (rc != LRS_OK) return rc;
      }
      const float* y = (i == 0) ? h_init : P[(i - 1) & 1];
      rc = hip_status(lrs::launch_deer_iter(w, u, y, h0, P[i & 1], C, D, T, p, vec, status, tickets,
                                            nullptr, nullptr, i, eps, s, seq_slots, seq_delta,
                                            k_max));
      if (rc != LRS_OK) return rc;
    }
    rc = hip_status(lrs::launch_deer_seq_book(seq_slots, seq_delta, B, k_max, k_max, s));
    if (rc == LRS_OK) rc = hip_status(lrs::launch_deer_seq_finish(seq_delta, seq_rec, B, k_max, eps, s));
    if (rc == LRS_OK) rc = hip_status(lrs::launch_deer_seq_select(P[0], P[1], h, B, D * T, seq_rec, s));
    if (rc != LRS_OK) return rc;
  }
  if (!iters_out && !converged_out) return LRS_OK;  // asynchronous form
  std::vector<int> rec((size_t)B * 4);
  if (hipMemcpyAsync(rec.data(), seq_rec, sizeof(int) * rec.size(), hipMemcpyDeviceToHost, s) !=
      hipSuccess)
    return LRS_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return LRS_ERR_HIP;
  int nonfinite = 0;
  for (int64_t b = 0; b < B; ++b) {
    if (iters_out) iters_out[b] = rec[4 * b];
    if (converged_out) converged_out[b] = rec[4 * b + 1];
    nonfinite |= rec[4 * b + 2];
  }
  return nonfinite ? LRS_ERR_NONFINITE : LRS_OK;
}

// ------------------------------------------------------- SRU by DEER

// Workspace: the solve record (first, so lrs_deer_stats reads it), a second
// cell-state buffer and the look-back state of the [T,B,D] tile (sized for the
// look-back tile plan; the persistent one needs none).
size_t lrs_sru_deer_workspace_bytes(int64_t T, int64_t B, int64_t D, int k_max) {
  int64_t C, N;
  if (!shape_ok(B, D, T, &C, &N) || N == 0 || k_max < 1 || k_max > 1000000) return 0;
  size_t need = 0;
  for (int io = 0; io < 2; ++io) {
    const lrs::ColPlan p = lrs::plan_sru_deer(C, T, io, false);
    const size_t b = lookback_bytes(lrs::col_status_words(p), p.ncb);
    need = b > need ? b : need;
  }
  // norm slot sets of the fused solve (used when the persistent plan applies)
  if (k_max <= lrs::kDeerFuseMax) need += align_up(deer_fused_set_words(k_max) * 4);
  return kAlign + deer_record_bytes(k_max) + align_up((size_t)N * 4) + need;
}

static int sru_deer_fwd_impl(const void* z_f, const void* z_r, const void* z_x, const float* bias_f,
                     const float* bias_r, const float* v_f, const float* c0, const float* c_init,
                     void* h, float* c_states, float* c_last, int64_t T, int64_t B, int64_t D,
                     int io_dtype, float eps, int k_max, int* iters_out, float* deltas_out,
                     int* converged_out, void* workspace, size_t workspace_bytes, void* stream,
    const lrs::Opts& opt) {
  int64_t C, N;
  if (!shape_ok(B, D, T, &C, &N) || k_max < 1 || k_max > 1000000) return LRS_ERR_INVALID_ARG;
  if (io_dtype != LRS_F32 && io_dtype != LRS_BF16) return LRS_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (N == 0) {
    if (iters_out) *iters_out = 0;
    if (converged_out) *converged_out = 1;
    if (deltas_out) memset(deltas_out, 0, sizeof(float) * (size_t)k_max);
    if (T == 0 && C > 0 && c_last) return hip_status(lrs::launch_copy_or_zero(c_last, c0, C, s));
    return LRS_OK;
  }
  if (!z_f || !z_r || !z_x || !bias_f || !bias_r || !v_f || !h || !c_states)
    return LRS_ERR_INVALID_ARG;
  const size_t es = io_dtype == LRS_BF16 ? 2 : 4;
  if (!aligned(z_f, es) || !aligned(z_r, es) || !aligned(z_x, es) || !aligned(h, es) ||
      !aligned(bias_f, 4) || !aligned(bias_r, 4) || !aligned(v_f, 4) || !aligned(c_states, 4) ||
      (c0 && !aligned(c0, 4)) || (c_init && !aligned(c_init, 4)) ||
      (c_last && !aligned(c_last, 4)))
    return LRS_ERR_INVALID_ARG;
  const size_t nb = (size_t)N * es, cb = (size_t)C * 4, db = (size_t)D * 4, sb = (size_t)N * 4;
  const void* ins[7] = {z_f, z_r, z_x, bias_f, bias_r, v_f, c0};
  const size_t insz[7] = {nb, nb, nb, db, db, db, cb};
  const void* outs[3] = {h, c_states, c_last};
  const size_t outsz[3] = {nb, sb, cb};
  for (int o = 0; o < 3; ++o) {
    for (int i = 0; i < 7; ++i)
      if (overlap(outs[o], outsz[o], ins[i], insz[i])) return LRS_ERR_INVALID_ARG;
    if (!(o == 1 && c_init == c_states) && overlap(outs[o], outsz[o], c_init, sb))
      return LRS_ERR_INVALID_ARG;
    for (int o2 = o + 1; o2 < 3; ++o2)
      if (overlap(outs[o], outsz[o], outs[o2], outsz[o2])) return LRS_ERR_INVALID_ARG;
  }
  const size_t need = lrs_sru_deer_workspace_bytes(T, B, D, k_max);
  if (!workspace || workspace_bytes < need) return LRS_ERR_WORKSPACE;
  const lrs::ColPlan p = lrs::plan_sru_deer(C, T, io_dtype, true, opt);
  if (!grid_ok(p.persist ? p.ncb : p.ncb * p.ntb, p.nw * 64)) return LRS_ERR_UNSUPPORTED;

  Carve cv(align_ptr(workspace));
  const DeerRecord r = carve_deer_record(cv, k_max);
  float* ybuf = cv.take<float>(N);
  const int64_t nst = lrs::col_status_words(p);
  uint64_t* status = nullptr;
  unsigned* tickets = nullptr;
  if (nst > 0) {
    status = cv.take<uint64_t>(nst);
    tickets = cv.take<unsigned>(p.ncb);
  }
  const void* all[10] = {z_f, z_r, z_x, bias_f, bias_r, v_f, c0, c_init, h, c_states};
  const size_t allsz[10] = {nb, nb, nb, db, db, db, cb, sb, nb, sb};
  for (int i = 0; i < 10; ++i)
    if (overlap(ybuf, sb, all[i], allsz[i])) return LRS_ERR_INVALID_ARG;

  // ping-pong as in lrs_deer_solve: iteration i writes P[i % 2]; a start in
  // c_states itself swaps the roles so that iteration 0 does not overwrite it
  float* P[2] = {c_states, ybuf};
  if (c_init == c_states) { P[0] = ybuf; P[1] = c_states; }
  const size_t rowbytes = (size_t)p.cpt * es;
  const int vec = aligned(z_f, rowbytes) && aligned(z_x, rowbytes) &&
                  aligned(c_states, (size_t)p.cpt * 4) && aligned(ybuf, (size_t)p.cpt * 4) &&
                  (!c_init || aligned(c_init, (size_t)p.cpt * 4)) && (C % p.cpt == 0);
  const int vec4 = (C % 4 == 0) && aligned(z_r, 4 * es) && aligned(z_x, 4 * es) &&
                   aligned(h, 4 * es) && aligned(c_states, 16);

  if (p.persist && k_max <= lrs::kDeerFuseMax && deer_fuse_enabled(opt)) {
    // all iterations in one walk (see lrs_deer_solve); the pass must not
    // overwrite a starting iterate held in c_states: a redo may need it.
    // The walk holds one channel per lane (one workgroup per 64 channels), so
    // its grid is checked on its own, and the element alignment checked
    // above is all its full tiles need (vec = 1).
    if (!grid_ok((C + 63) / 64, p.nw * 64)) return LRS_ERR_UNSUPPORTED;
    uint32_t* sets = cv.take<uint32_t>((int64_t)deer_fused_set_words(k_max));
    float* out = (c_init == c_states) ? ybuf : c_states;
    int rc = hip_status(lrs::launch_reset(nullptr, 0, nullptr, 0, sets,
                                          (int64_t)deer_fused_set_words(k_max), s));
    if (rc != LRS_OK) return rc;
    rc = hip_status(lrs::launch_sru_deer_fused(z_f, z_x, bias_f, v_f, c0, c_init, out, c_states,
                                               T, C, D, io_dtype, p, 1, k_max, eps, sets,
                                               r.delta_out, r.rec, s));
    if (rc != LRS_OK) return rc;
    rc = hip_status(lrs::launch_sru_deer_out(z_r, z_x, bias_r, c_states, h, c_last, N, C, D,
                                             io_dtype, vec4, s));
    if (rc != LRS_OK) return rc;
    if (!iters_out && !deltas_out && !converged_out) return LRS_OK;  // asynchronous form
    return read_deer_record(r, k_max, iters_out, deltas_out, converged_out, s);
  }

  int rc = hip_status(lrs::launch_reset(status, nst, tickets, nst > 0 ? p.ncb : 0, r.delta_bits,
                                        lrs::kDeltaSetWords + lrs::kDeerRecordWords + k_max, s));
  if (rc != LRS_OK) return rc;
  for (int i = 0; i < k_max; ++i) {
    if (i > 0 && nst > 0) {
      rc = hip_status(lrs::launch_reset(status, nst, tickets, p.ncb, nullptr, 0, s));
      if (rc != LRS_OK) return rc;
    }
    const float* y = (i == 0) ? c_init : P[(i - 1) & 1];
    rc = hip_status(lrs::launch_sru_deer_iter(z_f, z_x, bias_f, v_f, c0, y, P[i & 1], T, C, D,
                                              io_dtype, p, vec, status, tickets, r.delta_bits,
                                              r.delta_out, i, eps, s));
    if (rc != LRS_OK) return rc;
  }
  rc = hip_status(lrs::launch_deer_finish(r.delta_bits, r.delta_out, r.rec, k_max, eps, s));
  if (rc != LRS_OK) return rc;
  rc = hip_status(lrs::launch_deer_select(P[0], P[1], c_states, N, r.rec, s));
  if (rc != LRS_OK) return rc;
  rc = hip_status(lrs::launch_sru_deer_out(z_r, z_x, bias_r, c_states, h, c_last, N, C, D,
                                           io_dtype, vec4, s));
  if (rc != LRS_OK) return rc;
  if (!iters_out && !deltas_out && !converged_out) return LRS_OK;  // asynchronous form
  return read_deer_record(r, k_max, iters_out, deltas_out, converged_out, s);
}

// Sequential tanh RNN: no workspace, one launch.
int lrs_rnn_seq(const float* w, const float* u, const float* h0, float* h, int64_t B, int64_t D,
                int64_t T, void* stream) {
  int64_t C, N;
  if (!shape_ok(B, D, T, &C, &N)) return LRS_ERR_INVALID_ARG;
  if (N == 0) return LRS_OK;
  if (!w || !u || !h) return LRS_ERR_INVALID_ARG;
  if (!aligned(w, 4) || !aligned(u, 4) || !aligned(h, 4) || (h0 && !aligned(h0, 4)))
    return LRS_ERR_INVALID_ARG;
  const size_t nb = (size_t)N * 4;
  if (overlap(h, nb, u, nb) || overlap(h, nb, w, (size_t)D * 4) ||
      overlap(h, nb, h0, (size_t)C * 4))
    return LRS_ERR_INVALID_ARG;
  if (!grid_ok((C + 63) / 64, 64)) return LRS_ERR_UNSUPPORTED;
  const int vec = aligned(u, 16) && aligned(h, 16) && T % 4 == 0;
  return hip_status(lrs::launch_rnn_seq(w, u, h0, h, C, D, T, vec, (hipStream_t)stream));
}

// DEER backward: look-back state, nchunk * C floats of dL/dw partials and the
// fp64 stage of their reduction.
size_t lrs_deer_bwd_workspace_bytes(int64_t B, int64_t D, int64_t T) {
  int64_t C, N;
  if (!shape_ok(B, D, T, &C, &N) || N == 0) return 0;
  const lrs::RowPlan p = lrs::plan_deer_bwd_rows(C, T);
  size_t bytes = kAlign + align_up((size_t)(p.nchunk * C) * 4) +
                 align_up((size_t)(lrs::col_sum_blocks(p.nchunk * B) * D) * 8);
  if (p.nchunk > 1) bytes += lookback_bytes(C * p.nchunk, C);
  return bytes;
}

int lrs_deer_bwd(const float* w, const float* h0, const float* h, const float* grad_h,
                 float* grad_u, float* grad_w, float* grad_h0, int64_t B, int64_t D, int64_t T,
                 void* workspace, size_t workspace_bytes, void* stream) {
  int64_t C, N;
  if (!shape_ok(B, D, T, &C, &N)) return LRS_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (N == 0) {
    // no steps: dL/dw is an empty sum and nothing depends on h0
    int rc = LRS_OK;
    if (D > 0 && grad_w) rc = hip_status(lrs::launch_copy_or_zero(grad_w, nullptr, D, s));
    if (rc == LRS_OK && T == 0 && C > 0 && grad_h0)
      rc = hip_status(lrs::launch_copy_or_zero(grad_h0, nullptr, C, s));
    return rc;
  }
  if (!w || !h || !grad_h || !grad_u || !grad_w) return LRS_ERR_INVALID_ARG;
  if (!aligned(w, 4) || !aligned(h, 4) || !aligned(grad_h, 4) || !aligned(grad_u, 4) ||
      !aligned(grad_w, 4) || (h0 && !aligned(h0, 4)) || (grad_h0 && !aligned(grad_h0, 4)))
    return LRS_ERR_INVALID_ARG;
  const size_t nb = (size_t)N * 4, cb = (size_t)C * 4, db = (size_t)D * 4;
  const void* ins[4] = {w, h0, h, grad_h};
  const size_t insz[4] = {db, cb, nb, nb};
  const void* outs[3] = {grad_u, grad_w, grad_h0};
  const size_t outsz[3] = {nb, db, cb};
  for (int o = 0; o < 3; ++o) {
    for (int i = 0; i < 4; ++i)
      if (overlap(outs[o], outsz[o], ins[i], insz[i])) return LRS_ERR_INVALID_ARG;
    for (int o2 = o + 1; o2 < 3; ++o2)
      if (overlap(outs[o], outsz[o], outs[o2], outsz[o2])) return LRS_ERR_INVALID_ARG;
  }
  const lrs::RowPlan p = lrs::plan_deer_bwd_rows(C, T);
  if (!grid_ok(C * p.nchunk, p.threads())) return LRS_ERR_UNSUPPORTED;
  const size_t need = lrs_deer_bwd_workspace_bytes(B, D, T);
  if (!workspace || workspace_bytes < need) return LRS_ERR_WORKSPACE;
  Carve cv(align_ptr(workspace));
  float* part = cv.take<float>(p.nchunk * C);
  double* acc = cv.take<double>(lrs::col_sum_blocks(p.nchunk * B) * D);
  uint64_t* status = nullptr;
  unsigned* tickets = nullptr;
  if (p.nchunk > 1) {
    status = cv.take<uint64_t>(C * p.nchunk);
    tickets = cv.take<unsigned>(C);
    const int rc = hip_status(lrs::launch_reset(status, C * p.nchunk, tickets, C, nullptr, 0, s));
    if (rc != LRS_OK) return rc;
  }
  const int vec = aligned(h, 16) && aligned(grad_h, 16) && aligned(grad_u, 16) && (T % 4 == 0);
  return hip_status(lrs::launch_deer_bwd(w, h, h0, grad_h, grad_u, grad_w, grad_h0, part, acc, B,
                                         D, T, p, vec, status, tickets, s));
}

int lrs_deer_stats(const void* workspace, size_t workspace_bytes, int k_max, int* iters_out,
                   float* deltas_out, int* converged_out, void* stream) {
  if (k_max < 1 || k_max > 1000000) return LRS_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < kAlign + deer_record_bytes(k_max)) return LRS_ERR_WORKSPACE;
  Carve cv(align_ptr(const_cast<void*>(workspace)));
  const DeerRecord r = carve_deer_record(cv, k_max);
  return read_deer_record(r, k_max, iters_out, deltas_out, converged_out, (hipStream_t)stream);
}


// ------------------------------------------------- plan overrides

void lrs_options_default(lrs_options* opt) {
  if (!opt) return;
  opt->serial_fwd_max_t = -1;
  opt->serial_bwd_max_t = -1;
  opt->packed_max_t = -1;
  opt->persist_min_blocks = -1;
  opt->deer_fuse = -1;
  opt->reserved = 0;
}

static lrs::Opts to_opts(const lrs_options* o) {
  lrs::Opts r;
  if (o) {
    r.serial_fwd_max_t = o->serial_fwd_max_t;
    r.serial_bwd_max_t = o->serial_bwd_max_t;
    r.packed_max_t = o->packed_max_t;
    r.persist_min_blocks = o->persist_min_blocks;
    r.deer_fuse = o->deer_fuse;
  }
  return r;
}

int lrs_scan_fwd(const void* a, const void* b, const float* h0, void* h, int64_t B, int64_t D,
                 int64_t T, int layout, int dtype, void* workspace, size_t workspace_bytes,
                 void* stream) {
  return scan_fwd_impl(a, b, h0, h, B, D, T, layout, dtype, workspace, workspace_bytes, stream, lrs::Opts());
}
int lrs_scan_fwd_ex(const void* a, const void* b, const float* h0, void* h, int64_t B, int64_t D,
                 int64_t T, int layout, int dtype, void* workspace, size_t workspace_bytes,
                 void* stream,
    const lrs_options* options) {
  return scan_fwd_impl(a, b, h0, h, B, D, T, layout, dtype, workspace, workspace_bytes, stream, to_opts(options));
}

int lrs_scan_bwd(const void* a, const void* h, const float* h0, const void* grad_h, void* grad_a,
                 void* grad_b, float* grad_h0, int64_t B, int64_t D, int64_t T, int layout,
                 int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return scan_bwd_impl(a, h, h0, grad_h, grad_a, grad_b, grad_h0, B, D, T, layout, dtype, workspace, workspace_bytes, stream, lrs::Opts());
}
int lrs_scan_bwd_ex(const void* a, const void* h, const float* h0, const void* grad_h, void* grad_a,
                 void* grad_b, float* grad_h0, int64_t B, int64_t D, int64_t T, int layout,
                 int dtype, void* workspace, size_t workspace_bytes, void* stream,
    const lrs_options* options) {
  return scan_bwd_impl(a, h, h0, grad_h, grad_a, grad_b, grad_h0, B, D, T, layout, dtype, workspace, workspace_bytes, stream, to_opts(options));
}

int lrs_scan_fwd_bwd(const void* a, const void* b, const float* h0, const void* grad_h, void* h,
                     void* grad_a, void* grad_b, float* grad_h0, int64_t B, int64_t D, int64_t T,
                     int layout, int dtype, void* workspace, size_t workspace_bytes,
                     void* stream) {
  return scan_fwd_bwd_impl(a, b, h0, grad_h, h, grad_a, grad_b, grad_h0, B, D, T, layout, dtype, workspace, workspace_bytes, stream, lrs::Opts());
}
int lrs_scan_fwd_bwd_ex(const void* a, const void* b, const float* h0, const void* grad_h, void* h,
                     void* grad_a, void* grad_b, float* grad_h0, int64_t B, int64_t D, int64_t T,
                     int layout, int dtype, void* workspace, size_t workspace_bytes,
                     void* stream,
    const lrs_options* options) {
  return scan_fwd_bwd_impl(a, b, h0, grad_h, h, grad_a, grad_b, grad_h0, B, D, T, layout, dtype, workspace, workspace_bytes, stream, to_opts(options));
}

int lrs_sru_fwd(const void* z_f, const void* z_r, const void* z_x, const float* bias_f,
                const float* bias_r, const float* c0, void* h, float* c_last, float* c_states,
                int64_t T, int64_t B, int64_t D, int io_dtype, void* workspace,
                size_t workspace_bytes, void* stream) {
  return sru_fwd_impl(z_f, z_r, z_x, bias_f, bias_r, c0, h, c_last, c_states, T, B, D, io_dtype, workspace, workspace_bytes, stream, lrs::Opts());
}
int lrs_sru_fwd_ex(const void* z_f, const void* z_r, const void* z_x, const float* bias_f,
                const float* bias_r, const float* c0, void* h, float* c_last, float* c_states,
                int64_t T, int64_t B, int64_t D, int io_dtype, void* workspace,
                size_t workspace_bytes, void* stream,
    const lrs_options* options) {
  return sru_fwd_impl(z_f, z_r, z_x, bias_f, bias_r, c0, h, c_last, c_states, T, B, D, io_dtype, workspace, workspace_bytes, stream, to_opts(options));
}

int lrs_sru_deer_fwd(const void* z_f, const void* z_r, const void* z_x, const float* bias_f,
                     const float* bias_r, const float* v_f, const float* c0, const float* c_init,
                     void* h, float* c_states, float* c_last, int64_t T, int64_t B, int64_t D,
                     int io_dtype, float eps, int k_max, int* iters_out, float* deltas_out,
                     int* converged_out, void* workspace, size_t workspace_bytes, void* stream) {
  return sru_deer_fwd_impl(z_f, z_r, z_x, bias_f, bias_r, v_f, c0, c_init, h, c_states, c_last, T, B, D, io_dtype, eps, k_max, iters_out, deltas_out, converged_out, workspace, workspace_bytes, stream, lrs::Opts());
}
int lrs_sru_deer_fwd_ex(const void* z_f, const void* z_r, const void* z_x, const float* bias_f,
                     const float* bias_r, const float* v_f, const float* c0, const float* c_init,
                     void* h, float* c_states, float* c_last, int64_t T, int64_t B, int64_t D,
                     int io_dtype, float eps, int k_max, int* iters_out, float* deltas_out,
                     int* converged_out, void* workspace, size_t workspace_bytes, void* stream,
    const lrs_options* options) {
  return sru_deer_fwd_impl(z_f, z_r, z_x, bias_f, bias_r, v_f, c0, c_init, h, c_states, c_last, T, B, D, io_dtype, eps, k_max, iters_out, deltas_out, converged_out, workspace, workspace_bytes, stream, to_opts(options));
}

int lrs_deer_solve(const float* w, const float* u, const float* h0, const float* h_init, float* h,
                   int64_t B, int64_t D, int64_t T, float eps, int k_max, int* iters_out,
                   float* deltas_out, int* converged_out, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return deer_solve_impl(w, u, h0, h_init, h, B, D, T, eps, k_max, iters_out, deltas_out, converged_out, workspace, workspace_bytes, stream, lrs::Opts());
}
int lrs_deer_solve_ex(const float* w, const float* u, const float* h0, const float* h_init, float* h,
                   int64_t B, int64_t D, int64_t T, float eps, int k_max, int* iters_out,
                   float* deltas_out, int* converged_out, void* workspace,
                   size_t workspace_bytes, void* stream,
    const lrs_options* options) {
  return deer_solve_impl(w, u, h0, h_init, h, B, D, T, eps, k_max, iters_out, deltas_out, converged_out, workspace, workspace_bytes, stream, to_opts(options));
}

int lrs_deer_solve_seq(const float* w, const float* u, const float* h0, const float* h_init,
                       float* h, int64_t B, int64_t D, int64_t T, float eps, int k_max,
                       int* iters_out, int* converged_out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return deer_solve_seq_impl(w, u, h0, h_init, h, B, D, T, eps, k_max, iters_out, converged_out, workspace, workspace_bytes, stream, lrs::Opts());
}
int lrs_deer_solve_seq_ex(const float* w, const float* u, const float* h0, const float* h_init,
                       float* h, int64_t B, int64_t D, int64_t T, float eps, int k_max,
                       int* iters_out, int* converged_out, void* workspace,
                       size_t workspace_bytes, void* stream,
    const lrs_options* options) {
  return deer_solve_seq_impl(w, u, h0, h_init, h, B, D, T, eps, k_max, iters_out, converged_out, workspace, workspace_bytes, stream, to_opts(options));
}

int lrs_lstm_fwd(const void* z_f, const void* z_i, const void* z_c, const void* z_o,
                 const float* c0, void* h, float* c_last, float* c_states, int64_t T, int64_t B,
                 int64_t D, int io_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return lstm_fwd_impl(z_f, z_i, z_c, z_o, c0, h, c_last, c_states, T, B, D, io_dtype, workspace,
                       workspace_bytes, stream, lrs::Opts());
}
int lrs_lstm_fwd_ex(const void* z_f, const void* z_i, const void* z_c, const void* z_o,
                    const float* c0, void* h, float* c_last, float* c_states, int64_t T,
                    int64_t B, int64_t D, int io_dtype, void* workspace, size_t workspace_bytes,
                    void* stream, const lrs_options* options) {
  return lstm_fwd_impl(z_f, z_i, z_c, z_o, c0, h, c_last, c_states, T, B, D, io_dtype, workspace,
                       workspace_bytes, stream, to_opts(options));
}

// ------------------------------------------------- DEER tolerance schedule

float lrs_deer_eps_schedule(int64_t step, int64_t total_steps, float early, float late) {
  if (!(early > 0.0f) || !(late > 0.0f) || !isfinite(early) || !isfinite(late)) return NAN;
  if (total_steps <= 1) return late;
  double frac = (double)step / (double)(total_steps - 1);
  frac = frac < 0.0 ? 0.0 : (frac > 1.0 ? 1.0 : frac);
  return (float)((double)early * pow((double)late / (double)early, frac));
}

// ------------------------------------------------- allocation-free form

int lrs_scan_fwd_bwd_noalloc(const void* a, const void* b, const float* h0, const void* grad_h,
                             void* h, void* grad_a, void* grad_b, float* grad_h0, int64_t B,
                             int64_t D, int64_t T, int layout, int dtype, void* stream) {
  // the workspace this shape needs (0 for one that needs none, or an invalid
  // one, which the common path then rejects)
  const size_t need = lrs_scan_workspace_bytes(B, D, T, layout, dtype);
  if (need > (size_t)LRS_STATIC_SCRATCH_BYTES) return LRS_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    const int rc = scratch_address(&ws);
    if (rc != LRS_OK) return rc;
  }
  // the look-back state is cleared by a reset kernel at the start of every
  // pass that uses it, so whatever an earlier call left there is harmless
  return scan_fwd_bwd_impl(a, b, h0, grad_h, h, grad_a, grad_b, grad_h0, B, D, T, layout, dtype,
                           ws, need > 0 ? (size_t)LRS_STATIC_SCRATCH_BYTES : 0, stream,
                           lrs::Opts());
}

}  // extern "C"
