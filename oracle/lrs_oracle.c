/*
 * lrs_oracle.c -- plain, sequential fp64 reference for the diagonal linear
 * recurrence, its reverse-time adjoint, the SRU and LSTM cell-state layers and
 * the DEER Newton solve of an element-wise nonlinear RNN.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, helper or constant
 * with the HIP kernels.
 *
 * Every loop below is the textbook definition written out one time step at a
 * time, in double precision, with no blocking, reordering or fusion.  The
 * callers hand in the exact values the device path sees (fp32 or bf16 values
 * widened exactly to double).  The only parallelism is an optional OpenMP loop
 * over independent channels, which does not change any arithmetic.
 *
 * Sources (four blog pages on one subject, cited by title and section):
 *  [P1] "CUDA并行化RNN训练：从O(T)到O(log T)的工程实践与参数调优"
 *       (CUDA-parallel RNN training, O(T) to O(log T)), body: the SRU
 *       paragraph and the parallel-scan paragraph.
 *  [P2] "RNN CUDA内核优化：实现序列长度无关的恒定推理延迟"
 *       (RNN CUDA kernel optimisation, constant latency), body: the paragraph
 *       on the LSTM cell state C_t = f_t*C_{t-1} + i_t*C~_t as a linear
 *       recurrence with time-varying coefficients.
 *  [P4] DEER page "cuda-parallel-rnn-training-logt-optimization", sections
 *       "核心原理" (core principle: Newton in function space, the linear inverse
 *       operator as a recurrence with an initial condition) and "工程实现"
 *       (engineering: stop when ||y(i+1)-y(i)|| < eps or i reaches K_max).
 *
 * Conventions shared with the tests: a channel is one (batch, feature) pair;
 * the time axis has T steps stored at index 0..T-1 for t = 1..T; h0 is the
 * state at t = 0 and is not part of the output.  Layout of the scan and DEER
 * arrays is channel-major [C, T] (time contiguous); the SRU and LSTM arrays
 * are [T, B, D] (feature contiguous), as the SRU workload states them.
 *
 * Parity status: every function here is pinned by tests in tests/ against
 * closed forms, exact rational brute force, adjoint identities, finite
 * differences or the Newton invariants (see tests/test_oracle_*.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL 1
#define ORACLE_ENOMEM 2

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* Forward recurrence h_t = a_t * h_{t-1} + b_t  ([P1] parallel-scan paragraph;
 * [P2] cell-state paragraph).  h0 may be NULL (zero initial state). */
int lrs_oracle_scan_fwd(const double *a, const double *b, const double *h0,
                        double *h, int64_t C, int64_t T, int nthreads)
{
    if (C < 0 || T < 0 || (C * T > 0 && (!a || !b || !h))) return ORACLE_EINVAL;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t c = 0; c < C; ++c) {
        const double *ac = a + c * T, *bc = b + c * T;
        double *hc = h + c * T;
        double state = h0 ? h0[c] : 0.0;
        for (int64_t t = 0; t < T; ++t) {
            state = ac[t] * state + bc[t];
            hc[t] = state;
        }
    }
    return ORACLE_OK;
}

/* Reverse-time adjoint of the forward recurrence for the loss
 * L = sum_t <g_t, h_t>, g = dL/dh given per step.  [P1] states that the
 * backward pass is also a scan; the formulas are the chain rule:
 *   lam_T = g_T,  lam_t = g_t + a_{t+1} * lam_{t+1}
 *   dL/db_t = lam_t,  dL/da_t = lam_t * h_{t-1} (h_0 at t = 1),
 *   dL/dh_0 = a_1 * lam_1.
 * h is the forward output (steps 1..T); h0 may be NULL (zero); dh0 may be NULL. */
int lrs_oracle_scan_bwd(const double *a, const double *h, const double *h0,
                        const double *g, double *da, double *db, double *dh0,
                        int64_t C, int64_t T, int nthreads)
{
    if (C < 0 || T < 0 || (C * T > 0 && (!a || !h || !g || !da || !db)))
        return ORACLE_EINVAL;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t c = 0; c < C; ++c) {
        const double *ac = a + c * T, *hc = h + c * T, *gc = g + c * T;
        double *dac = da + c * T, *dbc = db + c * T;
        double lam = 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            double next = (t + 1 < T) ? ac[t + 1] * lam : 0.0;
            lam = gc[t] + next;
            double hprev = (t > 0) ? hc[t - 1] : (h0 ? h0[c] : 0.0);
            dbc[t] = lam;
            dac[t] = lam * hprev;
        }
        if (dh0) dh0[c] = (T > 0) ? ac[0] * lam : 0.0;
    }
    return ORACLE_OK;
}

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* SRU layer forward with precomputed pre-activations ([P1] SRU paragraph: a
 * forget gate that does not wait for h_{t-1}, and a highway connection through
 * the reset gate r).  The recurrent term v_f*c_{t-1} is absent, as in the
 * workload this oracle serves, so the cell state is a linear recurrence:
 *   f_t = sigma(zf_t + bf),  r_t = sigma(zr_t + br)
 *   c_t = f_t * c_{t-1} + (1 - f_t) * zx_t
 *   h_t = r_t * tanh(c_t) + (1 - r_t) * zx_t
 * Arrays are [T, B, D]; bf, br are [D]; c0 is [B, D] or NULL (zero);
 * c_last is [B, D] or NULL. */
int lrs_oracle_sru_fwd(const double *zf, const double *zr, const double *zx,
                       const double *bf, const double *br, const double *c0,
                       double *h, double *c_last, int64_t T, int64_t B,
                       int64_t D, int nthreads)
{
    if (T < 0 || B < 0 || D < 0) return ORACLE_EINVAL;
    if (T * B * D > 0 && (!zf || !zr || !zx || !bf || !br || !h)) return ORACLE_EINVAL;
    set_threads(nthreads);
    const int64_t C = B * D;
#pragma omp parallel for schedule(static)
    for (int64_t ch = 0; ch < C; ++ch) {
        const int64_t d = ch % D;
        double c = c0 ? c0[ch] : 0.0;
        for (int64_t t = 0; t < T; ++t) {
            const int64_t i = t * C + ch;
            double f = sigmoid(zf[i] + bf[d]);
            double r = sigmoid(zr[i] + br[d]);
            c = f * c + (1.0 - f) * zx[i];
            h[i] = r * tanh(c) + (1.0 - r) * zx[i];
        }
        if (c_last) c_last[ch] = c;
    }
    return ORACLE_OK;
}

/* Reverse-mode derivative of the SRU layer above ([P1] SRU paragraph; the
 * page states that the backward pass is also a scan, the formulas are the
 * chain rule applied to the forward definition).  With the upstream gradient
 * gh_t = dL/dh_t and gcl = dL/dc_T (NULL = 0), the total gradient of the cell
 * state runs backwards in time:
 *   gc_t = gh_t r_t (1 - tanh^2 c_t) + f_{t+1} gc_{t+1},   gc_T starts from gcl,
 * and the inputs' gradients are
 *   dzx_t = gh_t (1 - r_t) + gc_t (1 - f_t)
 *   dzr_t = gh_t (tanh c_t - zx_t) r_t (1 - r_t)
 *   dzf_t = gc_t (c_{t-1} - zx_t) f_t (1 - f_t)
 *   dc0   = f_1 gc_1,   dbf[d] = sum over b, t of dzf,   dbr[d] = sum of dzr.
 * The cell states are recomputed by the forward loop of each channel first.
 * Arrays as for lrs_oracle_sru_fwd; dzf, dzr, dzx are [T, B, D]; dbf, dbr
 * are [D]; dc0 is [B, D] or NULL. */
int lrs_oracle_sru_bwd(const double *zf, const double *zr, const double *zx,
                       const double *bf, const double *br, const double *c0,
                       const double *gh, const double *gcl, double *dzf,
                       double *dzr, double *dzx, double *dbf, double *dbr,
                       double *dc0, int64_t T, int64_t B, int64_t D, int nthreads)
{
    if (T < 0 || B < 0 || D < 0) return ORACLE_EINVAL;
    if (T * B * D > 0 && (!zf || !zr || !zx || !bf || !br || !gh || !dzf || !dzr || !dzx ||
                          !dbf || !dbr))
        return ORACLE_EINVAL;
    set_threads(nthreads);
    const int64_t C = B * D;
    double *sf = calloc((size_t)(C > 0 ? C : 1), sizeof(double));
    double *sr = calloc((size_t)(C > 0 ? C : 1), sizeof(double));
    if (!sf || !sr) { free(sf); free(sr); return ORACLE_ENOMEM; }
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t ch = 0; ch < C; ++ch) {
        const int64_t d = ch % D;
        double *c = malloc((size_t)(T > 0 ? T : 1) * sizeof(double));
        if (!c) { fail = 1; continue; }
        /* forward: cell states c_1..c_T */
        double state = c0 ? c0[ch] : 0.0;
        for (int64_t t = 0; t < T; ++t) {
            const int64_t i = t * C + ch;
            const double f = sigmoid(zf[i] + bf[d]);
            state = f * state + (1.0 - f) * zx[i];
            c[t] = state;
        }
        /* reverse: carry = f_{t+1} gc_{t+1} (gcl at the end of the sequence) */
        double carry = gcl ? gcl[ch] : 0.0;
        double acc_f = 0.0, acc_r = 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            const int64_t i = t * C + ch;
            const double f = sigmoid(zf[i] + bf[d]);
            const double r = sigmoid(zr[i] + br[d]);
            const double th = tanh(c[t]);
            const double gc = gh[i] * r * (1.0 - th * th) + carry;
            const double cprev = t > 0 ? c[t - 1] : (c0 ? c0[ch] : 0.0);
            dzx[i] = gh[i] * (1.0 - r) + gc * (1.0 - f);
            dzr[i] = gh[i] * (th - zx[i]) * r * (1.0 - r);
            dzf[i] = gc * (cprev - zx[i]) * f * (1.0 - f);
            acc_f += dzf[i];
            acc_r += dzr[i];
            carry = f * gc;
        }
        if (dc0) dc0[ch] = carry;
        sf[ch] = acc_f;
        sr[ch] = acc_r;
        free(c);
    }
    if (!fail) {
        for (int64_t d = 0; d < D; ++d) { dbf[d] = 0.0; dbr[d] = 0.0; }
        for (int64_t ch = 0; ch < C; ++ch) {  /* fixed order: deterministic sums */
            dbf[ch % D] += sf[ch];
            dbr[ch % D] += sr[ch];
        }
    }
    free(sf);
    free(sr);
    return fail ? ORACLE_ENOMEM : ORACLE_OK;
}

/* LSTM cell-state layer with every gate computed from the inputs alone
 * ([P2] the LSTM cell state C_t = f_t*C_{t-1} + i_t*C~_t read as a linear
 * recurrence with coefficient f_t and input i_t*C~_t; the model-change step
 * of its deployment list asks for gates that do not depend on h_{t-1}).
 * The pre-activations (input projections plus biases, made outside) are
 * z_f, z_i, z_c, z_o, all [T, B, D]:
 *   f = sigmoid(z_f), i = sigmoid(z_i), g = tanh(z_c), o = sigmoid(z_o),
 *   c_t = f_t c_{t-1} + i_t g_t,   h_t = o_t tanh(c_t).
 * c0 [B, D] (NULL = 0); h [T, B, D]; c_last [B, D] or NULL. */
int lrs_oracle_lstm_fwd(const double *zf, const double *zi, const double *zc,
                        const double *zo, const double *c0, double *h, double *c_last,
                        int64_t T, int64_t B, int64_t D, int nthreads)
{
    if (T < 0 || B < 0 || D < 0) return ORACLE_EINVAL;
    if (T * B * D > 0 && (!zf || !zi || !zc || !zo || !h)) return ORACLE_EINVAL;
    set_threads(nthreads);
    const int64_t C = B * D;
#pragma omp parallel for schedule(static)
    for (int64_t ch = 0; ch < C; ++ch) {
        double c = c0 ? c0[ch] : 0.0;
        for (int64_t t = 0; t < T; ++t) {
            const int64_t k = t * C + ch;
            const double f = sigmoid(zf[k]), i = sigmoid(zi[k]);
            const double g = tanh(zc[k]), o = sigmoid(zo[k]);
            c = f * c + i * g;
            h[k] = o * tanh(c);
        }
        if (c_last) c_last[ch] = c;
    }
    return ORACLE_OK;
}

/* Reverse-mode derivative of the LSTM cell-state layer above (the chain rule
 * of its definition; the cell-state gradient is again a reverse-time linear
 * recurrence, [P1] parallel-scan paragraph).  With gh_t = dL/dh_t and
 * gcl = dL/dc_T (NULL = 0):
 *   gc_t = gh_t o_t (1 - tanh^2 c_t) + f_{t+1} gc_{t+1},   gc_T starts from gcl,
 *   dz_o = gh_t tanh(c_t) o_t (1 - o_t),   dz_f = gc_t c_{t-1} f_t (1 - f_t),
 *   dz_i = gc_t g_t i_t (1 - i_t),         dz_c = gc_t i_t (1 - g_t^2),
 *   dc0  = f_1 gc_1.
 * The cell states are recomputed by each channel's forward loop first.
 * dzf, dzi, dzc, dzo are [T, B, D]; dc0 is [B, D] or NULL. */
int lrs_oracle_lstm_bwd(const double *zf, const double *zi, const double *zc,
                        const double *zo, const double *c0, const double *gh,
                        const double *gcl, double *dzf, double *dzi, double *dzc,
                        double *dzo, double *dc0, int64_t T, int64_t B, int64_t D,
                        int nthreads)
{
    if (T < 0 || B < 0 || D < 0) return ORACLE_EINVAL;
    if (T * B * D > 0 && (!zf || !zi || !zc || !zo || !gh || !dzf || !dzi || !dzc || !dzo))
        return ORACLE_EINVAL;
    set_threads(nthreads);
    const int64_t C = B * D;
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t ch = 0; ch < C; ++ch) {
        double *c = malloc((size_t)(T > 0 ? T : 1) * sizeof(double));
        if (!c) { fail = 1; continue; }
        double state = c0 ? c0[ch] : 0.0;
        for (int64_t t = 0; t < T; ++t) {
            const int64_t k = t * C + ch;
            state = sigmoid(zf[k]) * state + sigmoid(zi[k]) * tanh(zc[k]);
            c[t] = state;
        }
        /* reverse: carry = f_{t+1} gc_{t+1} (gcl at the end of the sequence) */
        double carry = gcl ? gcl[ch] : 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            const int64_t k = t * C + ch;
            const double f = sigmoid(zf[k]), i = sigmoid(zi[k]);
            const double g = tanh(zc[k]), o = sigmoid(zo[k]);
            const double th = tanh(c[t]);
            const double gc = gh[k] * o * (1.0 - th * th) + carry;
            const double cprev = t > 0 ? c[t - 1] : (c0 ? c0[ch] : 0.0);
            dzo[k] = gh[k] * th * o * (1.0 - o);
            dzf[k] = gc * cprev * f * (1.0 - f);
            dzi[k] = gc * g * i * (1.0 - i);
            dzc[k] = gc * i * (1.0 - g * g);
            carry = f * gc;
        }
        if (dc0) dc0[ch] = carry;
        free(c);
    }
    return fail ? ORACLE_ENOMEM : ORACLE_OK;
}

/* SRU layer with the forget gate reading the previous cell state ([P1] SRU
 * paragraph: f_t = sigmoid(W_f x_t + v_f (.) c_{t-1} + b_f)); the reset gate
 * and the highway output are as in lrs_oracle_sru_fwd.  With v_f != 0 the
 * cell recurrence is element-wise nonlinear:
 *   f_t = sigmoid(zf_t + bf[d] + vf[d] * c_{t-1})
 *   c_t = f_t * c_{t-1} + (1 - f_t) * zx_t,   h_t = r_t tanh(c_t) + (1 - r_t) zx_t.
 * This is the plain sequential loop (the ground truth for the Newton solve
 * below).  Arrays [T, B, D]; bf, br, vf [D]; c0 [B, D] or NULL; c [T, B, D]
 * receives every cell state, h the outputs (either may be NULL). */
int lrs_oracle_sru_nl_seq(const double *zf, const double *zr, const double *zx,
                          const double *bf, const double *br, const double *vf,
                          const double *c0, double *c, double *h, int64_t T, int64_t B,
                          int64_t D, int nthreads)
{
    if (T < 0 || B < 0 || D < 0) return ORACLE_EINVAL;
    if (T * B * D > 0 && (!zf || !zr || !zx || !bf || !br || !vf)) return ORACLE_EINVAL;
    set_threads(nthreads);
    const int64_t C = B * D;
#pragma omp parallel for schedule(static)
    for (int64_t ch = 0; ch < C; ++ch) {
        const int64_t d = ch % D;
        double state = c0 ? c0[ch] : 0.0;
        for (int64_t t = 0; t < T; ++t) {
            const int64_t i = t * C + ch;
            const double f = sigmoid(zf[i] + bf[d] + vf[d] * state);
            state = f * state + (1.0 - f) * zx[i];
            if (c) c[i] = state;
            if (h) {
                const double r = sigmoid(zr[i] + br[d]);
                h[i] = r * tanh(state) + (1.0 - r) * zx[i];
            }
        }
    }
    return ORACLE_OK;
}

/* The same layer's cell states by DEER ([P4] core principle: Newton's method
 * on the whole sequence, the inverse operator a linear recurrence with an
 * initial condition; engineering section: stop when the update's norm is
 * below eps or after k_max iterations).  With F(c_{t-1}) = f (c_{t-1} - zx) + zx
 * the cell map and its derivative (diagonal Jacobian)
 *   J_t = f + (c_{t-1} - zx) f (1 - f) vf[d],
 * one iteration from the iterate y (y_{-1} = c0 fixed) solves
 *   y'_t = J_t y'_{t-1} + (F(y_{t-1}) - J_t y_{t-1})
 * sequentially, with f and J evaluated at y_{t-1}.  delta_i = max over all
 * entries of |y' - y|; stop at delta_i < eps or i == k_max.  c_init is the
 * starting iterate (NULL: zero).  c receives the last iterate; h, if not NULL,
 * the layer output computed from it.  deltas (length >= k_max) gets
 * delta_1..delta_iters and *iters the iteration count. */
int lrs_oracle_sru_deer(const double *zf, const double *zr, const double *zx,
                        const double *bf, const double *br, const double *vf,
                        const double *c0, const double *c_init, double *c, double *h,
                        int64_t T, int64_t B, int64_t D, double eps, int k_max, int *iters,
                        double *deltas, int nthreads)
{
    if (T < 0 || B < 0 || D < 0 || k_max < 1 || !iters) return ORACLE_EINVAL;
    const int64_t C = B * D, N = C * T;
    if (N > 0 && (!zf || !zr || !zx || !bf || !br || !vf || !c)) return ORACLE_EINVAL;
    set_threads(nthreads);
    double *y = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
    double *yn = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
    if (!y || !yn) { free(y); free(yn); return ORACLE_ENOMEM; }
    if (c_init && N > 0) memcpy(y, c_init, (size_t)N * sizeof(double));
    else memset(y, 0, (size_t)(N > 0 ? N : 1) * sizeof(double));
    int done = 0;
    for (int i = 1; i <= k_max; ++i) {
        double delta = 0.0;
        int saw_nan = 0;
#pragma omp parallel for schedule(static) reduction(max : delta) reduction(| : saw_nan)
        for (int64_t ch = 0; ch < C; ++ch) {
            const int64_t d = ch % D;
            const double start = c0 ? c0[ch] : 0.0;
            double state = start; /* y'_{-1} */
            for (int64_t t = 0; t < T; ++t) {
                const int64_t k = t * C + ch;
                const double yprev = t > 0 ? y[k - C] : start;
                const double f = sigmoid(zf[k] + bf[d] + vf[d] * yprev);
                const double F = f * (yprev - zx[k]) + zx[k];
                const double J = f + (yprev - zx[k]) * f * (1.0 - f) * vf[d];
                state = J * state + (F - J * yprev);
                yn[k] = state;
                const double diff = fabs(state - y[k]);
                if (diff != diff) saw_nan = 1;
                else if (diff > delta) delta = diff;
            }
        }
        if (saw_nan) delta = NAN;
        double *tmp = y; y = yn; yn = tmp;
        if (deltas) deltas[i - 1] = delta;
        done = i;
        if (delta < eps) break;
    }
    if (N > 0) memcpy(c, y, (size_t)N * sizeof(double));
    if (h) {
#pragma omp parallel for schedule(static)
        for (int64_t k = 0; k < N; ++k) {
            const int64_t d = k % D;
            const double r = sigmoid(zr[k] + br[d]);
            h[k] = r * tanh(y[k]) + (1.0 - r) * zx[k];
        }
    }
    *iters = done;
    free(y);
    free(yn);
    return ORACLE_OK;
}

/* Adjoint of the nonlinear RNN h_t = tanh(w_d h_{t-1} + u_t) at a solution h
 * (the DEER solve's result, [P4] core principle; the backward pass as a
 * reverse-time scan, [P1] parallel-scan paragraph).  With s_t = 1 - h_t^2 and
 * the upstream gradient g_t = dL/dh_t:
 *   lam_T = g_T,   lam_t = g_t + w s_{t+1} lam_{t+1},
 *   dL/du_t = s_t lam_t,   dL/dh0 = w s_1 lam_1,
 *   dL/dw[d] = sum over b, t of s_t lam_t h_{t-1}   (h_0 = h0).
 * u is not needed: at the solution, tanh(w h_{t-1} + u_t) = h_t.
 * h, g, du are [B, D, T]; w is [D]; h0, dh0 are [B, D] or NULL. */
int lrs_oracle_deer_bwd(const double *w, const double *h0, const double *h,
                        const double *g, double *du, double *dw, double *dh0,
                        int64_t B, int64_t D, int64_t T, int nthreads)
{
    if (B < 0 || D < 0 || T < 0) return ORACLE_EINVAL;
    if (B * D * T > 0 && (!w || !h || !g || !du || !dw)) return ORACLE_EINVAL;
    set_threads(nthreads);
    const int64_t C = B * D;
    double *part = calloc((size_t)(C > 0 ? C : 1), sizeof(double));
    if (!part) return ORACLE_ENOMEM;
#pragma omp parallel for schedule(static)
    for (int64_t ch = 0; ch < C; ++ch) {
        const double wd = w[ch % D];
        const double *hc = h + ch * T, *gc = g + ch * T;
        double *duc = du + ch * T;
        double lam_next = 0.0, s_next = 0.0, acc = 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            const double s = 1.0 - hc[t] * hc[t];
            const double lam = gc[t] + (t + 1 < T ? wd * s_next * lam_next : 0.0);
            const double hprev = t > 0 ? hc[t - 1] : (h0 ? h0[ch] : 0.0);
            duc[t] = s * lam;
            acc += s * lam * hprev;
            lam_next = lam;
            s_next = s;
        }
        if (dh0) dh0[ch] = T > 0 ? wd * s_next * lam_next : 0.0;
        part[ch] = acc;
    }
    for (int64_t d = 0; d < D; ++d) dw[d] = 0.0;
    for (int64_t ch = 0; ch < C; ++ch) dw[ch % D] += part[ch];  /* fixed order */
    free(part);
    return ORACLE_OK;
}

/* Plain sequential nonlinear RNN h_t = tanh(w_d * h_{t-1} + u_t): the ground
 * truth that the DEER iteration converges to ([P4] core principle).
 * u, h are [B, D, T]; w is [D]; h0 is [B, D] or NULL. */
int lrs_oracle_rnn_seq(const double *w, const double *u, const double *h0,
                       double *h, int64_t B, int64_t D, int64_t T, int nthreads)
{
    if (B < 0 || D < 0 || T < 0) return ORACLE_EINVAL;
    if (B * D * T > 0 && (!w || !u || !h)) return ORACLE_EINVAL;
    set_threads(nthreads);
    const int64_t C = B * D;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ch = 0; ch < C; ++ch) {
        const double wd = w[ch % D];
        const double *uc = u + ch * T;
        double *hc = h + ch * T;
        double state = h0 ? h0[ch] : 0.0;
        for (int64_t t = 0; t < T; ++t) {
            state = tanh(wd * state + uc[t]);
            hc[t] = state;
        }
    }
    return ORACLE_OK;
}

/* DEER: solve the nonlinear recurrence as a root-finding problem by Newton's
 * method in function space ([P4] core principle, three steps per iteration:
 * evaluate f and its Jacobian, multiply by the Jacobian, apply the linear
 * inverse operator, which for an RNN is a linear recurrence with an initial
 * condition).  For the element-wise cell f(h_{t-1}, u_t) = tanh(w h_{t-1}+u_t)
 * the Jacobian is diagonal, so one iteration from the iterate y reads
 *   z_t   = tanh(w * y_{t-1} + u_t)
 *   J_t   = w * (1 - z_t^2)
 *   rhs_t = z_t - J_t * y_{t-1}
 *   y'_t  = J_t * y'_{t-1} + rhs_t,   y'_0 = y_0 = h0
 * and the linear recurrence is solved here sequentially.  Stop rule ([P4]
 * engineering section): after iteration i (1-based) compute
 * delta_i = max over all B*D*T entries of |y' - y|; stop when delta_i < eps
 * or i == k_max.  h_init is the starting iterate (NULL: zero); the result is
 * the last iterate.  deltas (length >= k_max) receives delta_1..delta_iters;
 * *iters receives the number of iterations performed. */
int lrs_oracle_deer(const double *w, const double *u, const double *h0,
                    const double *h_init, double *h, int64_t B, int64_t D,
                    int64_t T, double eps, int k_max, int *iters,
                    double *deltas, int nthreads)
{
    if (B < 0 || D < 0 || T < 0 || k_max < 1 || !iters) return ORACLE_EINVAL;
    const int64_t C = B * D, N = C * T;
    if (N > 0 && (!w || !u || !h)) return ORACLE_EINVAL;
    set_threads(nthreads);
    double *y = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
    double *yn = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
    if (!y || !yn) { free(y); free(yn); return ORACLE_ENOMEM; }
    if (h_init && N > 0) memcpy(y, h_init, (size_t)N * sizeof(double));
    else memset(y, 0, (size_t)(N > 0 ? N : 1) * sizeof(double));

    int done = 0;
    for (int i = 1; i <= k_max; ++i) {
        double delta = 0.0;
        int saw_nan = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(max : delta) reduction(| : saw_nan)
        for (int64_t ch = 0; ch < C; ++ch) {
            const double wd = w[ch % D];
            const double y0 = h0 ? h0[ch] : 0.0;
            const double *uc = u + ch * T, *yc = y + ch * T;
            double *ync = yn + ch * T;
            double state = y0; /* y'_0 */
            for (int64_t t = 0; t < T; ++t) {
                double yprev = (t > 0) ? yc[t - 1] : y0;
                double z = tanh(wd * yprev + uc[t]);
                double J = wd * (1.0 - z * z);
                double rhs = z - J * yprev;
                state = J * state + rhs;
                ync[t] = state;
                double diff = fabs(state - yc[t]);
                if (diff != diff) saw_nan = 1;
                else if (diff > delta) delta = diff;
            }
        }
        if (saw_nan) delta = NAN; /* a NaN difference never satisfies delta < eps */
        double *tmp = y; y = yn; yn = tmp;
        if (deltas) deltas[i - 1] = delta;
        done = i;
        if (delta < eps) break;
    }
    if (N > 0) memcpy(h, y, (size_t)N * sizeof(double));
    *iters = done;
    free(y);
    free(yn);
    return ORACLE_OK;
}
