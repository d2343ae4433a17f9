/*
 * ssd_oracle.c - plain fp64 CPU oracle of the Mamba-2 SSD layer core.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library (the HIP kernels, the
 * C ABI or its Python binding) includes, links or calls this file; only the
 * tests, the package's smoke entry and the benchmark's CPU-baseline leg do.
 * It shares no code, header, table or helper with the GPU path.
 *
 * It is the token-by-token recurrence, written out as the pages state it,
 * in double precision, with no chunking, blocking or reordering:
 *
 *   a_t      = exp(dt_t * A_h)                 discretised decay, Abar = exp(Delta A)
 *                                              ["Mamba-2: State Space Models and Linear-Time
 *                                              Sequence Modeling Without Attention",
 *                                              section "State Space Models: The Core Abstraction"]
 *   h_t      = a_t * h_{t-1} + (dt_t x_t) B_t  the selective recurrence h_t = A_t h_{t-1} + B_t x_t
 *                                              ["Mamba-2" wiki note, section "Question";
 *                                              "Why Does Mamba-2 Resemble the Transformer?",
 *                                              section "The Problem"], with the transition a
 *                                              scalar times identity per head ("Transformers are
 *                                              SSMs" paper card, section "How It Works") and the
 *                                              input scaled by dt (the Mamba2Block listing of the
 *                                              mohakchugh blog, section "Architecture: Multi-Head SSM")
 *   y_t      = C_t . h_t + D_h x_t             readout y_t = C_t^T h_t (ql.gl, "The Problem") plus
 *                                              the skip term D x of the continuous system
 *                                              (mohakchugh blog, "The Core Abstraction")
 *
 * Per head h the state is a P x N matrix (one N-vector per headdim channel
 * p); channels never interact, so every (b, h, p) row runs independently.
 * B and C are shared by the heads of a group: head h reads group
 * h / (H / G) (contiguous blocks of heads; the pages do not fix this).
 * h_{-1} is the caller's initial state (zeros when absent) and the state
 * after the last token is returned as the final state.
 *
 * Layouts (row-major, all double): x (B,L,H,P); dt (B,L,H); A, D (H);
 * B, C (B,L,G,N); init and final (B,H,P,N); y (B,L,H,P).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Optional record: the state after each token index record_t[k] (ascending)
 * is copied into recorded (B, n_record, H, P, N).  Returns 0, or -1 on bad
 * arguments. */
int ssd_oracle_forward(const double* x, const double* dt, const double* A, const double* Bm,
                       const double* Cm, const double* D, const double* init, double* y,
                       double* final_states, int64_t batch, int64_t seqlen, int64_t nheads,
                       int64_t headdim, int64_t dstate, int64_t ngroups, const int64_t* record_t,
                       int64_t n_record, double* recorded, int nthreads)
{
    if (batch < 0 || seqlen < 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 || ngroups <= 0 ||
        nheads % ngroups != 0 || (n_record > 0 && (record_t == NULL || recorded == NULL)))
        return -1;
    const int64_t heads_per_group = nheads / ngroups;
    const int64_t rows = batch * nheads * headdim;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

#pragma omp parallel
    {
        double* S = (double*)malloc(sizeof(double) * (size_t)dstate);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < rows; ++r) {
            const int64_t b = r / (nheads * headdim);
            const int64_t h = (r / headdim) % nheads;
            const int64_t p = r % headdim;
            const int64_t g = h / heads_per_group;
            const int64_t state_off = ((b * nheads + h) * headdim + p) * dstate;
            for (int64_t n = 0; n < dstate; ++n) S[n] = init ? init[state_off + n] : 0.0;
            int64_t k = 0;
            for (int64_t t = 0; t < seqlen; ++t) {
                const double dtv = dt[(b * seqlen + t) * nheads + h];
                const double xv = x[((b * seqlen + t) * nheads + h) * headdim + p];
                const double* Bt = Bm + ((b * seqlen + t) * ngroups + g) * dstate;
                const double* Ct = Cm + ((b * seqlen + t) * ngroups + g) * dstate;
                const double a = exp(dtv * A[h]);
                const double u = dtv * xv;
                double acc = 0.0;
                for (int64_t n = 0; n < dstate; ++n) {
                    S[n] = a * S[n] + u * Bt[n];
                    acc += Ct[n] * S[n];
                }
                y[((b * seqlen + t) * nheads + h) * headdim + p] = acc + D[h] * xv;
                while (k < n_record && record_t[k] == t) {
                    memcpy(recorded + (((b * n_record + k) * nheads + h) * headdim + p) * dstate, S,
                           sizeof(double) * (size_t)dstate);
                    ++k;
                }
            }
            memcpy(final_states + state_off, S, sizeof(double) * (size_t)dstate);
        }
        free(S);
    }
    return 0;
}

/* One token of the recurrence applied to the caller's state, in place:
 * state (B,H,P,N); x (B,H,P); dt (B,H); B, C (B,G,N); y (B,H,P).
 * O(1) work per token in the sequence length ("Transformers are SSMs"
 * paper card, section "Why It Matters"). */
int ssd_oracle_step(double* state, const double* x, const double* dt, const double* A,
                    const double* Bm, const double* Cm, const double* D, double* y, int64_t batch,
                    int64_t nheads, int64_t headdim, int64_t dstate, int64_t ngroups, int nthreads)
{
    if (batch < 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 || ngroups <= 0 ||
        nheads % ngroups != 0)
        return -1;
    const int64_t heads_per_group = nheads / ngroups;
    const int64_t rows = batch * nheads * headdim;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t b = r / (nheads * headdim);
        const int64_t h = (r / headdim) % nheads;
        const int64_t g = h / heads_per_group;
        double* S = state + r * dstate;
        const double dtv = dt[b * nheads + h];
        const double xv = x[r];
        const double* Bt = Bm + (b * ngroups + g) * dstate;
        const double* Ct = Cm + (b * ngroups + g) * dstate;
        const double a = exp(dtv * A[h]);
        const double u = dtv * xv;
        double acc = 0.0;
        for (int64_t n = 0; n < dstate; ++n) {
            S[n] = a * S[n] + u * Bt[n];
            acc += Ct[n] * S[n];
        }
        y[r] = acc + D[h] * xv;
    }
    return 0;
}

/* Gradients of the forward (the training pass the pages' throughput claims are about:
 * "Transformers are SSMs" paper card, "How It Works" and "Key Takeaways").  For a loss L with
 * dL/dy = dy and dL/d(final state) = dfinal (NULL = 0), the reverse-mode derivative of the
 * recurrence above, written out: with g_t = dL/dh_t,
 *
 *   g_{L-1} = dfinal + dy_{L-1} C_{L-1}^T,   g_{t-1} = a_t g_t + dy_{t-1} C_{t-1}^T
 *   du_t  = g_t B_t                          (u_t = dt_t x_t, the input vector)
 *   dx_t  = dt_t du_t + D dy_t
 *   dB_t += g_t^T u_t   (summed over the heads of the group)
 *   dC_t += h_t^T dy_t  (summed over the heads of the group)
 *   da_t  = <g_t, h_{t-1}>,  ddt_t = x_t . du_t + A a_t da_t,  dA += dt_t a_t da_t
 *   dD   += x_t . dy_t,      dinit = a_0 g_0
 *
 * Every state h_t of one (b, h) is kept (L x P x N doubles), so this is for test sizes.
 * Per-head parts of dB and dC are summed over the group at the end. */
/* dA_scale[h]: the size of what dA is computed from when it is formed, as a chunked pass does, from
 * suffix sums over tokens of q_t = dy_t . yhat_t - u_t . du_t (yhat = y - D x): an error in q_t
 * reaches dA weighted by T_t = sum_{t' <= t} dt_t', so the scale is
 * sum over (b, t) of T_t (sum_p |dy_t[p] yhat_t[p]| + sum_p |u_t[p] du_t[p]|).  dA's terms cancel
 * strongly, so its errors are measured against this scale.  May be NULL. */
int ssd_oracle_backward(const double* x, const double* dt, const double* A, const double* Bm, const double* Cm,
                        const double* D, const double* init, const double* dy, const double* dfinal, double* dx,
                        double* ddt, double* dA, double* dB, double* dC, double* dD, double* dinit,
                        double* dA_scale, int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                        int64_t dstate, int64_t ngroups, int nthreads)
{
    if (batch < 0 || seqlen < 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 || ngroups <= 0 ||
        nheads % ngroups != 0)
        return -1;
    const int64_t hpg = nheads / ngroups, P = headdim, N = dstate, L = seqlen;
    const int64_t PN = P * N;
    /* per-head parts of dB, dC: (B, L, H, N) */
    double* dBh = (double*)calloc((size_t)(batch * L * nheads * N) + 1, sizeof(double));
    double* dCh = (double*)calloc((size_t)(batch * L * nheads * N) + 1, sizeof(double));
    double* dAbh = (double*)calloc((size_t)(batch * nheads) + 1, sizeof(double));
    double* dDbh = (double*)calloc((size_t)(batch * nheads) + 1, sizeof(double));
    double* dSbh = (double*)calloc((size_t)(batch * nheads) + 1, sizeof(double));
    if (!dBh || !dCh || !dAbh || !dDbh || !dSbh) {
        free(dBh); free(dCh); free(dAbh); free(dDbh); free(dSbh);
        return -2;
    }
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < batch * nheads; ++bh) {
        const int64_t b = bh / nheads, h = bh % nheads, g = h / hpg;
        double* hs = (double*)malloc(sizeof(double) * (size_t)((L + 1) * PN));   /* hs[t + 1] = h_t, hs[0] = h_{-1} */
        double* gs = (double*)malloc(sizeof(double) * (size_t)PN);
        double* du = (double*)malloc(sizeof(double) * (size_t)P);
        for (int64_t i = 0; i < PN; ++i) hs[i] = init ? init[bh * PN + i] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            const int64_t bt = b * L + t;
            const double a = exp(dt[bt * nheads + h] * A[h]);
            for (int64_t p = 0; p < P; ++p) {
                const double u = dt[bt * nheads + h] * x[(bt * nheads + h) * P + p];
                for (int64_t n = 0; n < N; ++n)
                    hs[(t + 1) * PN + p * N + n] = a * hs[t * PN + p * N + n] + u * Bm[(bt * ngroups + g) * N + n];
            }
        }
        for (int64_t i = 0; i < PN; ++i) gs[i] = dfinal ? dfinal[bh * PN + i] : 0.0;
        double dA_acc = 0.0, dD_acc = 0.0, dS_acc = 0.0;
        for (int64_t t = L - 1; t >= 0; --t) {
            const int64_t bt = b * L + t;
            const double dtv = dt[bt * nheads + h];
            const double a = exp(dtv * A[h]);
            const double* xt = x + (bt * nheads + h) * P;
            const double* dyt = dy + (bt * nheads + h) * P;
            const double* Bt = Bm + (bt * ngroups + g) * N;
            const double* Ct = Cm + (bt * ngroups + g) * N;
            for (int64_t p = 0; p < P; ++p)
                for (int64_t n = 0; n < N; ++n) gs[p * N + n] += dyt[p] * Ct[n];
            double xdu = 0.0, da = 0.0, xdy = 0.0;
            for (int64_t p = 0; p < P; ++p) {
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) acc += gs[p * N + n] * Bt[n];
                du[p] = acc;
                xdu += xt[p] * acc;
                xdy += xt[p] * dyt[p];
                dx[(bt * nheads + h) * P + p] = dtv * acc + D[h] * dyt[p];
            }
            for (int64_t n = 0; n < N; ++n) {
                double sb = 0.0, sc = 0.0;
                for (int64_t p = 0; p < P; ++p) {
                    sb += gs[p * N + n] * dtv * xt[p];
                    sc += hs[(t + 1) * PN + p * N + n] * dyt[p];
                }
                dBh[(bt * nheads + h) * N + n] = sb;
                dCh[(bt * nheads + h) * N + n] = sc;
            }
            for (int64_t i = 0; i < PN; ++i) da += gs[i] * hs[t * PN + i];
            ddt[bt * nheads + h] = xdu + A[h] * a * da;
            dA_acc += dtv * a * da;
            {
                double T = 0.0, mag = 0.0;
                for (int64_t j = 0; j <= t; ++j) T += dt[(b * L + j) * nheads + h];
                for (int64_t p = 0; p < P; ++p) {
                    double yh = 0.0;
                    for (int64_t n = 0; n < N; ++n) yh += hs[(t + 1) * PN + p * N + n] * Ct[n];
                    mag += fabs(dyt[p] * yh) + fabs(dtv * xt[p] * du[p]);
                }
                dS_acc += T * mag;
            }
            dD_acc += xdy;
            for (int64_t i = 0; i < PN; ++i) gs[i] *= a;
        }
        if (dinit)
            for (int64_t i = 0; i < PN; ++i) dinit[bh * PN + i] = gs[i];
        dAbh[bh] = dA_acc;
        dDbh[bh] = dD_acc;
        dSbh[bh] = dS_acc;
        free(hs);
        free(gs);
        free(du);
    }
    for (int64_t h = 0; h < nheads; ++h) {
        double sa = 0.0, sd = 0.0, ss = 0.0;
        for (int64_t b = 0; b < batch; ++b) {
            sa += dAbh[b * nheads + h];
            sd += dDbh[b * nheads + h];
            ss += dSbh[b * nheads + h];
        }
        dA[h] = sa;
        dD[h] = sd;
        if (dA_scale) dA_scale[h] = ss;
    }
    for (int64_t bt = 0; bt < batch * L; ++bt)
        for (int64_t g = 0; g < ngroups; ++g)
            for (int64_t n = 0; n < N; ++n) {
                double sb = 0.0, sc = 0.0;
                for (int64_t k = 0; k < hpg; ++k) {
                    sb += dBh[(bt * nheads + g * hpg + k) * N + n];
                    sc += dCh[(bt * nheads + g * hpg + k) * N + n];
                }
                dB[(bt * ngroups + g) * N + n] = sb;
                dC[(bt * ngroups + g) * N + n] = sc;
            }
    free(dBh);
    free(dCh);
    free(dAbh);
    free(dDbh);
    free(dSbh);
    return 0;
}

/* The Mamba-1 selective scan, the layer Mamba-2 replaces (mohakchugh blog,
 * section "Mamba-1: Selective State Spaces"): every channel d of the input
 * has its own diagonal N x N transition, so each of its N state entries
 * decays at its own rate a_t[d, n] = exp(delta_t[d] A[d, n]) (the diagonal
 * structure of "Transformers are SSMs" paper card, section "How It Works";
 * Abar = exp(Delta A) of the same blog, section "The Core Abstraction"),
 * while delta is per channel and B, C are per token, shared by all channels
 * (that blog's selection listing gives B, C the shape (batch, seq_len,
 * state_dim) and delta (batch, seq_len, d_model)):
 *
 *   h_t[d, n] = a_t[d, n] h_{t-1}[d, n] + (delta_t[d] x_t[d]) B_t[n]
 *   y_t[d]    = sum_n C_t[n] h_t[d, n] + D[d] x_t[d]
 *
 * The input enters as delta * B * x, as in the SSD recurrence above.
 * Layouts (row-major, all double): x, delta, y (B,L,Dm); A (Dm,N); D (Dm);
 * B, C (B,L,N); init and final (B,Dm,N).  Every (b, d) row is independent. */
int ssd_oracle_selective_scan(const double* x, const double* delta, const double* A, const double* Bm,
                              const double* Cm, const double* D, const double* init, double* y,
                              double* final_states, int64_t batch, int64_t seqlen, int64_t dim,
                              int64_t dstate, int nthreads)
{
    if (batch < 0 || seqlen < 0 || dim <= 0 || dstate <= 0) return -1;
    const int64_t rows = batch * dim;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double* S = (double*)malloc(sizeof(double) * (size_t)dstate);
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < rows; ++r) {
            const int64_t b = r / dim;
            const int64_t d = r % dim;
            for (int64_t n = 0; n < dstate; ++n) S[n] = init ? init[r * dstate + n] : 0.0;
            for (int64_t t = 0; t < seqlen; ++t) {
                const int64_t bt = b * seqlen + t;
                const double dl = delta[bt * dim + d];
                const double xv = x[bt * dim + d];
                const double u = dl * xv;
                double acc = 0.0;
                for (int64_t n = 0; n < dstate; ++n) {
                    const double a = exp(dl * A[d * dstate + n]);
                    S[n] = a * S[n] + u * Bm[bt * dstate + n];
                    acc += Cm[bt * dstate + n] * S[n];
                }
                y[bt * dim + d] = acc + D[d] * xv;
            }
            memcpy(final_states + r * dstate, S, sizeof(double) * (size_t)dstate);
        }
        free(S);
    }
    return 0;
}

int ssd_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
