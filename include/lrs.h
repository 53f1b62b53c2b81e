/*
 * lrs.h -- C ABI of liblrs.so: the diagonal linear-recurrence scan
 * h_t = a_t (.) h_{t-1} + b_t on AMD MI355X (gfx950), with its reverse-time
 * backward pass, fused SRU and LSTM cell-state layers and a DEER Newton solver
 * built on it.
 *
 * Sources (four blog pages on one subject; cited by title and section):
 *  [P1] "CUDA并行化RNN训练：从O(T)到O(log T)的工程实践与参数调优", body:
 *       SRU paragraph (gates that do not wait for h_{t-1}, highway through the
 *       reset gate), parallel-scan paragraph (associative step, forward and
 *       backward passes both as log-depth scans), checklist item 2 (fuse all
 *       element-wise work into one kernel).
 *  [P2] "RNN CUDA内核优化：实现序列长度无关的恒定推理延迟", body: the cell state
 *       C_t = f_t*C_{t-1} + i_t*C~_t is a linear recurrence with time-varying
 *       coefficients, i.e. a prefix-scan problem; the deployment list's first
 *       step (change the model so the recurrent part is linear).
 *  [P4] DEER page "cuda-parallel-rnn-training-logt-optimization": section
 *       "核心原理" (Newton in function space; the inverse operator is a linear
 *       recurrence with an initial condition, solved by a parallel prefix scan)
 *       and section "工程实现" (stop when ||y(i+1) - y(i)|| < eps or after K_max
 *       iterations; example eps = 1e-5, K_max = 5).
 *
 * Conventions for every entry point
 *  - A channel is one (batch b, feature d) pair; C = B*D channels.  The time
 *    axis has T steps, stored at index 0..T-1 for t = 1..T.  h0 is the state at
 *    t = 0; it is an input and is not part of the output.
 *  - Layouts: LRS_LAYOUT_BDT = [B, D, T] (time contiguous, element (b,d,t) at
 *    (b*D + d)*T + t); LRS_LAYOUT_TBD = [T, B, D] (feature contiguous, element
 *    at (t*B + b)*D + d).  Per-channel arrays (h0, grad_h0, c0, c_last) are
 *    [B, D] in both layouts; per-feature arrays (bias_f, bias_r, w) are [D].
 *  - Every tensor pointer is a DEVICE pointer owned by the caller; the library
 *    never allocates, frees or retains memory.  Scratch space comes from the
 *    caller's `workspace`, sized by the matching *_workspace_bytes query (a
 *    size of 0 means no workspace is needed and `workspace` may be NULL).
 *    Pointers must be aligned to their element size; 16-byte alignment of all
 *    arrays (and T % 4 == 0 for [B,D,T] fp32) enables the widest accesses.
 *  - `stream` is a hipStream_t passed as an opaque pointer (NULL = the null
 *    stream).  Scan, SRU and LSTM calls only enqueue work and return; DEER does the
 *    same when it is given no host outputs, and otherwise reads its solve
 *    record back to the host and returns after the solve.
 *  - Errors are return codes (lrs_status); nothing is thrown and nothing
 *    aborts.  Arguments are validated before any launch, so an error other
 *    than LRS_ERR_HIP leaves all outputs untouched.  An empty problem
 *    (B*D*T == 0) is valid and does nothing.
 *  - Output arrays must not overlap input arrays unless a function says so.
 *  - Calls that share a workspace must be ordered (same stream or synchronised).
 *  - Plans.  [B,D,T] scans of short channels pack whole channels into each
 *    workgroup (T <= 64) or, for the shortest (T <= 4), run one lane per
 *    channel; the limits are measured crossovers.  The SRU and LSTM forward and the
 *    SRU-by-DEER iterations switch to persistent kernels (one workgroup per
 *    128 channels walks every time tile, no cross-workgroup look-back and no
 *    reset between iterations) when the 128-channel blocks are at least as
 *    many as the device's compute units; with the persistent plan and
 *    k_max <= 8, the SRU-by-DEER solve runs all its Newton iterations in that
 *    one walk, and DEER solves do the same with one workgroup per channel when
 *    the channels have at most 8192 steps or number at least the device's
 *    compute units.
 *    The entry points with the suffix _ex take an lrs_options argument that
 *    moves these choices explicitly (for comparing kernel families on the
 *    same inputs, or measuring crossovers); the library keeps no global or
 *    environment-driven state.  Every plan gives the same results within
 *    fp32 rounding, and the workspace queries cover every plan.
 *  - Reproducibility.  A channel longer than one workgroup's chunk (time
 *    block) is split into chunks whose states are combined by a fixed rule:
 *    chunks are grouped (64 per group for [B,D,T] scans, 8 for [T,B,D]
 *    kernels), the state entering a chunk is the previous group's end state
 *    carried through the aggregates of the chunks before it in its group, in
 *    ascending order, and only the last chunk of a group publishes an end
 *    state.  The association order of every result therefore depends on the
 *    launch shape alone (shape, layout, dtype and options), not on timing:
 *    repeated calls with the same arguments give the same bits.
 *  - Look-back time-out.  A workgroup that waits on a predecessor's status
 *    word gives up after about 2^22 polls (only corrupted or foreign
 *    workspace contents can cause that) and then writes NaN for the channels
 *    it serves instead of hanging; the call still returns LRS_OK, so a NaN
 *    in outputs whose inputs are finite signals such a time-out.  Calls that
 *    share a workspace concurrently (not ordered on one stream) are the usual
 *    cause, and are not allowed.
 */
#ifndef LRS_H
#define LRS_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define LRS_API __attribute__((visibility("default")))
#else
#define LRS_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define LRS_OK 0
#define LRS_ERR_INVALID_ARG 1 /* null/misaligned pointer, negative or overflowing size, bad enum */
#define LRS_ERR_UNSUPPORTED 2 /* valid request this build does not implement (e.g. dtype) */
#define LRS_ERR_WORKSPACE 3   /* workspace smaller than the query returned, or NULL */
#define LRS_ERR_HIP 4         /* a HIP runtime call or kernel launch failed */
#define LRS_ERR_NONFINITE 5   /* DEER: the last iteration's update was NaN or infinite */

/* Layouts (see conventions above). */
#define LRS_LAYOUT_BDT 0
#define LRS_LAYOUT_TBD 1

/* Element types of I/O tensors; the recurrence state is always fp32. */
#define LRS_F32 0
#define LRS_BF16 1

/* Human-readable name of a return code (static string, never NULL). */
LRS_API const char *lrs_status_string(int status);

/* Library ABI version (major*100 + minor). */
LRS_API int lrs_version(void);

/* ------------------------------------------------------ plan options --- */

/* Explicit plan choices for the _ex entry points.  A negative field keeps the
 * library's measured default; lrs_options_default sets every field so.
 * Passing NULL options, or the defaults, selects exactly the plan of the
 * entry point without the suffix. */
typedef struct lrs_options {
  int64_t serial_fwd_max_t;   /* [B,D,T] forward scan: one lane per channel for
                                 T <= this (default 4; 0 = never) */
  int64_t serial_bwd_max_t;   /* [B,D,T] backward scan: the same (default 4) */
  int64_t packed_max_t;       /* [B,D,T] scans: whole channels packed into each
                                 2048-step workgroup for T <= this (default 64) */
  int64_t persist_min_blocks; /* SRU forward, SRU by DEER, LSTM forward: persistent walk when
                                 the 128-channel blocks number at least this
                                 (default: the device's compute units; 0 =
                                 always, a huge value = never) */
  int32_t deer_fuse;          /* DEER and SRU-by-DEER solves: 0 = one launch per
                                 Newton iteration; > 0 = all iterations in one
                                 pass whenever k_max <= 8 (SRU by DEER: on the
                                 persistent plan); otherwise (default) one pass
                                 where it applies: k_max <= 8 and channels of
                                 at most 8192 steps or at least as many
                                 channels as compute units (SRU by DEER: the
                                 persistent plan) */
  int32_t reserved;           /* set to 0 */
} lrs_options;

/* Fill *options with the defaults (every field -1, reserved 0); NULL is a no-op. */
LRS_API void lrs_options_default(lrs_options *options);

/* ---------------------------------------------------------------- scan --- */

/* Workspace bytes needed by lrs_scan_fwd / lrs_scan_bwd for this shape, layout
 * and element type (look-back status words when a channel spans more than one
 * workgroup).  Returns 0 for an invalid shape. */
LRS_API size_t lrs_scan_workspace_bytes(int64_t B, int64_t D, int64_t T, int layout, int dtype);

/* Forward scan ([P1] parallel-scan paragraph; [P2] cell-state paragraph):
 *   h_t = a_t * h_{t-1} + b_t  for t = 1..T, every channel independently.
 * a, b, h : [B,D,T] or [T,B,D] per `layout`, element type `dtype`: LRS_F32, or
 *           LRS_BF16 (bf16 bit patterns, aligned to 2 bytes).
 * h0      : [B,D] fp32, or NULL for a zero initial state.
 * h must not overlap a, b or h0.  Arithmetic and the carried state are fp32
 * with fused multiply-add whatever `dtype` is; bf16 inputs widen exactly and
 * each h_t is rounded to bf16 (nearest-even) only when stored.  The
 * association order of the scan is fixed by the launch shape (see
 * Reproducibility above), so repeated calls give the same bits. */
LRS_API int lrs_scan_fwd(const void *a, const void *b, const float *h0, void *h, int64_t B, int64_t D,
                 int64_t T, int layout, int dtype, void *workspace, size_t workspace_bytes,
                 void *stream);
/* lrs_scan_fwd with explicit plan options (NULL = the defaults). */
LRS_API int lrs_scan_fwd_ex(const void *a, const void *b, const float *h0, void *h, int64_t B,
                            int64_t D, int64_t T, int layout, int dtype, void *workspace,
                            size_t workspace_bytes, void *stream, const lrs_options *options);

/* Backward scan: reverse-time adjoint of lrs_scan_fwd for a loss L whose
 * gradient with respect to h is grad_h ([P1]: the backward pass is also a
 * log-depth scan).  With lam_{T+1} = 0:
 *   lam_t = grad_h_t + a_{t+1} * lam_{t+1}
 *   grad_b_t = lam_t,  grad_a_t = lam_t * h_{t-1} (h0 at t = 1),
 *   grad_h0 = a_1 * lam_1.
 * h is the forward output; h0 as in lrs_scan_fwd (NULL = zero).
 * grad_h, grad_a, grad_b: same shape/layout/dtype as a (bf16 outputs are
 * rounded from fp32 values).  grad_h0: [B,D] fp32 or NULL.
 * grad_b may be the same buffer as grad_h (lam overwrites the incoming
 * gradient); no other overlap is allowed. */
LRS_API int lrs_scan_bwd(const void *a, const void *h, const float *h0, const void *grad_h, void *grad_a,
                 void *grad_b, float *grad_h0, int64_t B, int64_t D, int64_t T, int layout,
                 int dtype, void *workspace, size_t workspace_bytes, void *stream);
/* lrs_scan_bwd with explicit plan options (NULL = the defaults). */
LRS_API int lrs_scan_bwd_ex(const void *a, const void *h, const float *h0, const void *grad_h,
                            void *grad_a, void *grad_b, float *grad_h0, int64_t B, int64_t D,
                            int64_t T, int layout, int dtype, void *workspace,
                            size_t workspace_bytes, void *stream, const lrs_options *options);

/* Forward and backward scan in one call: the results of lrs_scan_fwd followed
 * by lrs_scan_bwd on the same inputs ([P1] parallel-scan paragraph: both
 * passes are scans).  For [B,D,T] channels of at most 8192 steps, one kernel
 * does both with h kept on chip, reading a, b, grad_h and writing h, grad_a,
 * grad_b (24 bytes per element instead of 32); h may then be NULL (the
 * backward with the forward recomputed, 20 bytes per element).  Other shapes
 * and layouts run the two passes and need h.
 * Arrays as for lrs_scan_fwd / lrs_scan_bwd; workspace as lrs_scan_workspace_bytes.
 * grad_b may be the same buffer as grad_h; no other output may overlap an
 * input or another output.  Returns LRS_ERR_UNSUPPORTED when h is NULL and
 * the shape needs the two passes. */
LRS_API int lrs_scan_fwd_bwd(const void *a, const void *b, const float *h0, const void *grad_h,
                             void *h, void *grad_a, void *grad_b, float *grad_h0, int64_t B,
                             int64_t D, int64_t T, int layout, int dtype, void *workspace,
                             size_t workspace_bytes, void *stream);
/* lrs_scan_fwd_bwd with explicit plan options (NULL = the defaults). */
LRS_API int lrs_scan_fwd_bwd_ex(const void *a, const void *b, const float *h0,
                                const void *grad_h, void *h, void *grad_a, void *grad_b,
                                float *grad_h0, int64_t B, int64_t D, int64_t T, int layout,
                                int dtype, void *workspace, size_t workspace_bytes, void *stream,
                                const lrs_options *options);

/* Bytes of the fixed device array that lrs_scan_fwd_bwd_noalloc uses in place
 * of a workspace (one copy per GPU). */
#define LRS_STATIC_SCRATCH_BYTES (8u << 20)

/* lrs_scan_fwd_bwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The look-back state lives in a fixed
 * array of LRS_STATIC_SCRATCH_BYTES (8 MiB) inside the library, one copy per
 * GPU, allocated when the library's device code is loaded and held until the
 * process ends; the call itself allocates and frees nothing.  Inputs, outputs
 * and their rules are those of lrs_scan_fwd_bwd (h may not be NULL where that
 * function needs it), and the results are bit for bit the same.
 * Limit: shapes whose lrs_scan_workspace_bytes exceeds LRS_STATIC_SCRATCH_BYTES
 * return LRS_ERR_WORKSPACE before any launch ([B,D,T]: up to about one
 * million look-back chunks, e.g. 4096 channels of 2^20 steps; [T,B,D]: B*D*T
 * up to about 2^27).  The array belongs to the current device, and `stream` must be
 * a stream of that device.  Every call on one GPU shares the array: calls
 * that may overlap in time on one GPU (different streams, or different host
 * threads, without ordering between them) race on it and give wrong results,
 * so they must be ordered.  The first call on each device looks up the
 * array's address (hipGetSymbolAddress); make it outside graph capture. */
LRS_API int lrs_scan_fwd_bwd_noalloc(const void *a, const void *b, const float *h0,
                                     const void *grad_h, void *h, void *grad_a, void *grad_b,
                                     float *grad_h0, int64_t B, int64_t D, int64_t T, int layout,
                                     int dtype, void *stream);

/* ----------------------------------------------------------------- SRU --- */

/* Workspace bytes needed by lrs_sru_fwd for this shape (0 for an invalid one). */
LRS_API size_t lrs_sru_workspace_bytes(int64_t T, int64_t B, int64_t D);

/* Fused SRU layer forward ([P1] SRU paragraph and checklist item 2), with the
 * input projections already applied (pre-activations z_*) and no recurrent
 * term in the forget gate, so the cell state is a linear recurrence:
 *   f_t = sigmoid(z_f,t + bias_f),  r_t = sigmoid(z_r,t + bias_r)
 *   c_t = f_t * c_{t-1} + (1 - f_t) * z_x,t
 *   h_t = r_t * tanh(c_t) + (1 - r_t) * z_x,t
 * z_f, z_r, z_x, h : [T,B,D], element type io_dtype (LRS_BF16 or LRS_F32).
 * bias_f, bias_r   : [D] fp32.   c0: [B,D] fp32 or NULL (zero).
 * c_last           : [B,D] fp32 output (c_T) or NULL.
 * c_states         : [T,B,D] fp32 output (every c_t, as lrs_sru_bwd needs
 *                    them) or NULL.
 * Gates, state and activations are computed in fp32; h is rounded to io_dtype
 * (nearest-even).  No output may overlap an input or another output. */
LRS_API int lrs_sru_fwd(const void *z_f, const void *z_r, const void *z_x, const float *bias_f,
                const float *bias_r, const float *c0, void *h, float *c_last, float *c_states,
                int64_t T, int64_t B, int64_t D, int io_dtype, void *workspace,
                size_t workspace_bytes, void *stream);
/* lrs_sru_fwd with explicit plan options (NULL = the defaults). */
LRS_API int lrs_sru_fwd_ex(const void *z_f, const void *z_r, const void *z_x,
                           const float *bias_f, const float *bias_r, const float *c0, void *h,
                           float *c_last, float *c_states, int64_t T, int64_t B, int64_t D,
                           int io_dtype, void *workspace, size_t workspace_bytes, void *stream,
                           const lrs_options *options);

/* Workspace bytes needed by lrs_sru_bwd for this shape (0 for an invalid one). */
LRS_API size_t lrs_sru_bwd_workspace_bytes(int64_t T, int64_t B, int64_t D);

/* SRU layer backward ([P1] SRU paragraph and parallel-scan paragraph: the
 * backward pass is also a scan; the formulas are the chain rule of
 * lrs_sru_fwd).  Given the upstream gradients gh_t = dL/dh_t and dL/dc_T, the
 * gradient of the cell state runs backwards in time,
 *   gc_t = gh_t r_t (1 - tanh^2 c_t) + f_{t+1} gc_{t+1}   (gc_T adds dL/dc_T),
 * and
 *   dL/dz_x = gh (1 - r) + gc (1 - f),  dL/dz_r = gh (tanh c - z_x) r (1 - r),
 *   dL/dz_f = gc (c_{t-1} - z_x) f (1 - f),  dL/dc0 = f_1 gc_1,
 *   dL/dbias_f[d], dL/dbias_r[d] = sums of dL/dz_f, dL/dz_r over batch and time.
 * z_f, z_r, z_x, grad_h, grad_z*: [T,B,D], element type io_dtype.
 * bias_f, bias_r: [D] fp32.   c0: [B,D] fp32 or NULL (zero).
 * c_states   : [T,B,D] fp32, the cell states lrs_sru_fwd wrote for the same
 *              inputs.
 * grad_c_last: [B,D] fp32 (dL/dc_T) or NULL (zero).
 * grad_bias_f, grad_bias_r: [D] fp32 outputs (overwritten; the sums are taken
 *              in a fixed order, so results do not depend on scheduling).
 * grad_c0    : [B,D] fp32 output or NULL.
 * No output may overlap an input or another output. */
LRS_API int lrs_sru_bwd(const void *z_f, const void *z_r, const void *z_x, const float *bias_f,
                const float *bias_r, const float *c0, const float *c_states,
                const void *grad_h, const float *grad_c_last, void *grad_zf, void *grad_zr,
                void *grad_zx, float *grad_bias_f, float *grad_bias_r, float *grad_c0,
                int64_t T, int64_t B, int64_t D, int io_dtype, void *workspace,
                size_t workspace_bytes, void *stream);

/* ------------------------------------------------------- SRU by DEER --- */

/* Workspace bytes needed by lrs_sru_deer_fwd (0 for an invalid or empty shape). */
LRS_API size_t lrs_sru_deer_workspace_bytes(int64_t T, int64_t B, int64_t D, int k_max);

/* SRU layer whose forget gate also reads the previous cell state ([P1] SRU
 * paragraph, f_t = sigmoid(W_f x_t + v_f (.) c_{t-1} + b_f)), solved by DEER
 * ([P4] core principle: Newton's method on the whole sequence, the linear
 * inverse operator a recurrence solved by the parallel scan; engineering
 * section: stop when ||c' - c||_inf < eps or after k_max iterations):
 *   f_t = sigmoid(z_f,t + bias_f + v_f * c_{t-1}),  r_t = sigmoid(z_r,t + bias_r)
 *   c_t = f_t * c_{t-1} + (1 - f_t) * z_x,t,        h_t = r_t tanh(c_t) + (1 - r_t) z_x,t
 * Each iteration linearises the cell map around the current iterate (diagonal
 * Jacobian J_t = f + (c_{t-1} - z_x) f (1 - f) v_f) and solves the resulting
 * linear recurrence with the [T,B,D] scan; with v_f = 0 the first iteration
 * is already lrs_sru_fwd's cell state.
 * z_f, z_r, z_x, h: [T,B,D] in io_dtype.  bias_f, bias_r, v_f: [D] fp32.
 * c0: [B,D] fp32 or NULL (zero).  c_init: starting iterate [T,B,D] fp32 or NULL
 * (zero); it may be c_states itself (warm start in place).
 * c_states: [T,B,D] fp32 output, the last iterate (the cell states, as
 * lrs_sru_bwd takes them for the v_f = 0 layer).  c_last: [B,D] or NULL.
 * iters_out, deltas_out (k_max floats), converged_out: host outputs as for
 * lrs_deer_solve; with all three NULL the call only enqueues work and
 * lrs_deer_stats reads the record from the workspace afterwards.
 * Returns LRS_ERR_NONFINITE if the last update was NaN or infinite. */
LRS_API int lrs_sru_deer_fwd(const void *z_f, const void *z_r, const void *z_x,
                             const float *bias_f, const float *bias_r, const float *v_f,
                             const float *c0, const float *c_init, void *h, float *c_states,
                             float *c_last, int64_t T, int64_t B, int64_t D, int io_dtype,
                             float eps, int k_max, int *iters_out, float *deltas_out,
                             int *converged_out, void *workspace, size_t workspace_bytes,
                             void *stream);
/* lrs_sru_deer_fwd with explicit plan options (NULL = the defaults). */
LRS_API int lrs_sru_deer_fwd_ex(const void *z_f, const void *z_r, const void *z_x,
                                const float *bias_f, const float *bias_r, const float *v_f,
                                const float *c0, const float *c_init, void *h, float *c_states,
                                float *c_last, int64_t T, int64_t B, int64_t D, int io_dtype,
                                float eps, int k_max, int *iters_out, float *deltas_out,
                                int *converged_out, void *workspace, size_t workspace_bytes,
                                void *stream, const lrs_options *options);

/* ---------------------------------------------------------------- LSTM --- */

/* Workspace bytes needed by lrs_lstm_fwd and lrs_lstm_bwd for this shape, in
 * either I/O type (0 for an invalid or empty shape). */
LRS_API size_t lrs_lstm_workspace_bytes(int64_t T, int64_t B, int64_t D);

/* Fused LSTM cell-state layer forward with every gate computed from the
 * inputs alone ([P2] cell-state paragraph: C_t = f_t*C_{t-1} + i_t*C~_t is a
 * linear recurrence once the gates do not read h_{t-1}, as its deployment
 * list's model-change step asks; [P1] checklist item 2: one kernel for all
 * element-wise work).  With the pre-activations z_* (input projection plus
 * bias, made by the caller):
 *   f = sigmoid(z_f), i = sigmoid(z_i), g = tanh(z_c), o = sigmoid(z_o)
 *   c_t = f_t * c_{t-1} + i_t * g_t,   h_t = o_t * tanh(c_t)
 * z_f, z_i, z_c, z_o, h : [T,B,D], element type io_dtype (LRS_BF16 or LRS_F32).
 * c0       : [B,D] fp32 or NULL (zero).
 * c_last   : [B,D] fp32 output (c_T) or NULL.
 * c_states : [T,B,D] fp32 output (every c_t, as lrs_lstm_bwd needs them) or NULL.
 * Gates, state and activations are fp32; h is rounded to io_dtype
 * (nearest-even).  No output may overlap an input or another output. */
LRS_API int lrs_lstm_fwd(const void *z_f, const void *z_i, const void *z_c, const void *z_o,
                         const float *c0, void *h, float *c_last, float *c_states, int64_t T,
                         int64_t B, int64_t D, int io_dtype, void *workspace,
                         size_t workspace_bytes, void *stream);
/* lrs_lstm_fwd with explicit plan options (NULL = the defaults). */
LRS_API int lrs_lstm_fwd_ex(const void *z_f, const void *z_i, const void *z_c, const void *z_o,
                            const float *c0, void *h, float *c_last, float *c_states, int64_t T,
                            int64_t B, int64_t D, int io_dtype, void *workspace,
                            size_t workspace_bytes, void *stream, const lrs_options *options);

/* LSTM cell-state layer backward (the chain rule of lrs_lstm_fwd; the
 * cell-state gradient is a reverse-time linear recurrence, [P1] parallel-scan
 * paragraph).  Given gh_t = dL/dh_t and dL/dc_T:
 *   gc_t = gh_t o_t (1 - tanh^2 c_t) + f_{t+1} gc_{t+1}   (gc_T adds dL/dc_T),
 *   dL/dz_o = gh tanh(c) o (1 - o),   dL/dz_f = gc c_{t-1} f (1 - f),
 *   dL/dz_i = gc g i (1 - i),         dL/dz_c = gc i (1 - g^2),
 *   dL/dc0 = f_1 gc_1.
 * z_*, grad_h, grad_z*: [T,B,D], element type io_dtype.  c0: [B,D] fp32 or NULL.
 * c_states   : [T,B,D] fp32, the cell states lrs_lstm_fwd wrote for the same
 *              inputs and c0.
 * grad_c_last: [B,D] fp32 (dL/dc_T) or NULL (zero).
 * grad_c0    : [B,D] fp32 output or NULL.
 * The biases live inside the pre-activations, so their gradients are the
 * callers' sums of grad_z* over batch and time.
 * No output may overlap an input or another output. */
LRS_API int lrs_lstm_bwd(const void *z_f, const void *z_i, const void *z_c, const void *z_o,
                         const float *c0, const float *c_states, const void *grad_h,
                         const float *grad_c_last, void *grad_zf, void *grad_zi, void *grad_zc,
                         void *grad_zo, float *grad_c0, int64_t T, int64_t B, int64_t D,
                         int io_dtype, void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------- DEER --- */

/* Workspace bytes needed by lrs_deer_solve (a second iterate buffer of
 * B*D*T floats, the per-iteration update norms and look-back status). */
LRS_API size_t lrs_deer_workspace_bytes(int64_t B, int64_t D, int64_t T, int k_max);

/* DEER Newton solve ([P4] core principle and engineering sections) of the
 * element-wise nonlinear RNN  h_t = tanh(w_d * h_{t-1} + u_t),  [B,D,T] fp32.
 * Iteration i (1-based) maps the iterate y to y' by
 *   z_t = tanh(w y_{t-1} + u_t),  J_t = w (1 - z_t^2),
 *   y'_t = J_t * y'_{t-1} + (z_t - J_t * y_{t-1}),   y'_0 = y_0 = h0,
 * solving the linear recurrence with the parallel scan, and records
 * delta_i = max over all B*D*T entries of |y' - y|.  It stops after the first
 * iteration with delta_i < eps, or after k_max iterations.
 * w       : [D] fp32 (one weight per feature, shared across the batch).
 * u       : [B,D,T] fp32.       h0: [B,D] fp32 or NULL (zero).
 * h_init  : [B,D,T] starting iterate, or NULL for zero (may equal h).
 * h       : [B,D,T] output, the last iterate.
 * iters_out (host, may be NULL): iterations performed (1..k_max).
 * deltas_out (host, may be NULL): k_max floats; entries 0..iters-1 receive
 *   delta_1..delta_iters, the rest 0.
 * converged_out (host, may be NULL): 1 if the last delta < eps, else 0.
 * An iteration whose predecessor met the stop rule exits immediately on the
 * device, so all k_max iterations are enqueued without host involvement; a
 * final device step leaves the last iterate in h and records the iteration
 * count, convergence flag and norms in the workspace.
 * If any of iters_out, deltas_out, converged_out is given, the call then
 * reads that record back (one device-to-host copy; waits for the stream) and
 * returns LRS_ERR_NONFINITE, with all outputs written, when the last delta is
 * NaN or infinite.  If all three are NULL the call is asynchronous: it returns
 * LRS_OK once everything is enqueued (and may be captured in a HIP graph);
 * lrs_deer_stats reads the record later.
 * When k_max <= 8 and the channels have at most 8192 steps or number at
 * least the device's compute units, all iterations run in one pass over each
 * channel, one workgroup per channel (u read once, the last iterate
 * written once; the norms of every iteration are kept), and when the stop rule
 * ends the solve before k_max a second pass recomputes exactly that many
 * iterations (an early stop thus costs k_max plus that many iterations of
 * work: a caller that expects one, as after a warm start, saves time by
 * passing the count it expects as k_max); the record, the iteration count and the result (within fp32
 * rounding) are those of the one-launch-per-iteration path, which
 * lrs_deer_solve_ex with options->deer_fuse = 0 selects.  Solves that share a
 * workspace must be ordered. */
LRS_API int lrs_deer_solve(const float *w, const float *u, const float *h0, const float *h_init, float *h,
                   int64_t B, int64_t D, int64_t T, float eps, int k_max, int *iters_out,
                   float *deltas_out, int *converged_out, void *workspace,
                   size_t workspace_bytes, void *stream);
/* lrs_deer_solve with explicit plan options (NULL = the defaults). */
LRS_API int lrs_deer_solve_ex(const float *w, const float *u, const float *h0,
                              const float *h_init, float *h, int64_t B, int64_t D, int64_t T,
                              float eps, int k_max, int *iters_out, float *deltas_out,
                              int *converged_out, void *workspace, size_t workspace_bytes,
                              void *stream, const lrs_options *options);

/* Workspace bytes needed by lrs_deer_solve_seq (0 for an invalid or empty shape). */
LRS_API size_t lrs_deer_seq_workspace_bytes(int64_t B, int64_t D, int64_t T, int k_max);

/* lrs_deer_solve with per-sequence stopping ([P4] engineering section's stop
 * rule applied to each sequence on its own): sequence b (its D channels)
 * keeps its own norm delta_b = max over its D*T entries of |y' - y| and stops
 * iterating once delta_b < eps, while the others go on, up to k_max.  Each
 * sequence's result is its last iterate, exactly what lrs_deer_solve returns
 * for that sequence alone.  iters_out[b], converged_out[b] (host arrays of B
 * ints, each may be NULL) receive the per-sequence iteration counts and
 * convergence flags; with both NULL the call only enqueues work.  Other
 * arguments as for lrs_deer_solve.  B is limited to 65535.  Returns
 * LRS_ERR_NONFINITE when some sequence's last update was NaN or infinite.
 * Under the same conditions as lrs_deer_solve all iterations run in one pass that keeps each
 * sequence's norms per iteration; sequences whose stop rule fired before
 * k_max are recomputed to their own count in a second pass. */
LRS_API int lrs_deer_solve_seq(const float *w, const float *u, const float *h0,
                               const float *h_init, float *h, int64_t B, int64_t D, int64_t T,
                               float eps, int k_max, int *iters_out, int *converged_out,
                               void *workspace, size_t workspace_bytes, void *stream);
/* lrs_deer_solve_seq with explicit plan options (NULL = the defaults). */
LRS_API int lrs_deer_solve_seq_ex(const float *w, const float *u, const float *h0,
                                  const float *h_init, float *h, int64_t B, int64_t D,
                                  int64_t T, float eps, int k_max, int *iters_out,
                                  int *converged_out, void *workspace, size_t workspace_bytes,
                                  void *stream, const lrs_options *options);

/* Record of the most recent lrs_deer_solve or lrs_sru_deer_fwd that used this
 * workspace with this k_max (same meaning of iters_out, deltas_out, converged_out as there; each
 * may be NULL).  Waits for `stream`, on which that solve must have been
 * enqueued.  Returns LRS_ERR_NONFINITE when that solve's last delta was NaN or
 * infinite, LRS_ERR_WORKSPACE for a workspace too small for k_max, and
 * LRS_ERR_HIP if the workspace holds no finished solve record. */
LRS_API int lrs_deer_stats(const void *workspace, size_t workspace_bytes, int k_max,
                   int *iters_out, float *deltas_out, int *converged_out, void *stream);

/* Newton tolerance for training step `step` of `total_steps` ([P4]
 * engineering section: relax the stop tolerance early in training, tighten it
 * late): log-linear interpolation from `early` at step 0 to `late` at step
 * total_steps - 1,
 *   eps(step) = early * (late / early)^(step / (total_steps - 1)),
 * with step clamped to [0, total_steps - 1]; total_steps <= 1 gives `late`.
 * Computed in double precision and rounded once to float.  Returns NaN when
 * early or late is not a positive finite number. */
LRS_API float lrs_deer_eps_schedule(int64_t step, int64_t total_steps, float early, float late);

/* Workspace bytes needed by lrs_deer_bwd (0 for an invalid or empty shape). */
LRS_API size_t lrs_deer_bwd_workspace_bytes(int64_t B, int64_t D, int64_t T);

/* Backward of the nonlinear RNN h_t = tanh(w_d * h_{t-1} + u_t) at its
 * solution h (the result of lrs_deer_solve; [P4] core principle: the solve
 * returns the sequential solution, so its derivative is that of the
 * recurrence), computed as a reverse-time scan ([P1] parallel-scan paragraph:
 * the backward pass is also a log-depth scan).  With s_t = 1 - h_t^2 and
 * g_t = dL/dh_t:
 *   lam_T = g_T,  lam_t = g_t + w s_{t+1} lam_{t+1},
 *   dL/du_t = s_t lam_t,  dL/dh0 = w s_1 lam_1,
 *   dL/dw[d] = sum over batch and time of s_t lam_t h_{t-1}   (h_0 = h0).
 * w: [D] fp32.  h0: [B,D] fp32 or NULL (zero).  h, grad_h: [B,D,T] fp32.
 * grad_u: [B,D,T] output.  grad_w: [D] output (overwritten; summed in a fixed
 * order, so results do not depend on scheduling).  grad_h0: [B,D] or NULL.
 * No output may overlap an input or another output.  If the solve stopped at
 * K_max before convergence, this is the derivative at the returned iterate. */
LRS_API int lrs_deer_bwd(const float *w, const float *h0, const float *h, const float *grad_h,
                 float *grad_u, float *grad_w, float *grad_h0, int64_t B, int64_t D, int64_t T,
                 void *workspace, size_t workspace_bytes, void *stream);

/* The same recurrence h_t = tanh(w_d * h_{t-1} + u_t) evaluated step after
 * step, one lane per channel: the O(T)-depth loop that DEER replaces by a few
 * Newton iterations of log-depth scans ([P4] core principle: the solve's fixed
 * point is this sequential solution).  A reference point for lrs_deer_solve:
 * its time is T dependent steps whatever the number of channels.
 * w: [D] fp32.  u: [B,D,T] fp32.  h0: [B,D] fp32 or NULL (zero).
 * h: [B,D,T] fp32 output; it must not overlap u, w or h0.  No workspace. */
LRS_API int lrs_rnn_seq(const float *w, const float *u, const float *h0, float *h, int64_t B,
                        int64_t D, int64_t T, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LRS_H */
