/*
 * Reference oracle for the selective state-space hot path — TEST INFRASTRUCTURE.
 *
 * Plain, slow, sequential fp64 C.  It exists only to check the HIP library:
 * only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load or run it.  It shares no code, header, table or constant with the
 * GPU library, and the GPU library never calls it.
 *
 * What it computes, and where each step comes from (sources are the web
 * pages this project is built from, cited by title and section):
 *
 *  - Continuous SSM  h'(t) = A h(t) + B u(t),  y(t) = C h(t) + D u(t)
 *      ["Mamba: Linear-Time Sequence Modeling with Selective SSMs", section
 *       "连续与离散SSM"; "Mamba架构与SSM模型：高效序列建模技术解析", §2.1].
 *  - Zero-order-hold discretisation with step Δ:
 *      Abar = exp(Δ A),   Bbar = (Δ A)^-1 (exp(Δ A) - I) Δ B
 *      ["Mamba架构与SSM模型：高效序列建模技术解析", §2.1].
 *    A is diagonal here (one scalar a per state n), so per state
 *      Abar_n = exp(Δ a_n),  Bbar_n = expm1(Δ a_n) / a_n * B_n,
 *    and at a_n = 0 the limit Bbar_n = Δ B_n.
 *  - Input-dependent step  Δ = softplus(dt + dt_bias)
 *      ["Mamba架构与SSM模型：高效序列建模技术解析", §2.2].
 *  - Selective (time-varying) recurrence  h_t = Abar_t h_{t-1} + Bbar_t x_t,
 *    readout  y_t = <C_t, h_t>  taken AFTER x_t has entered the state
 *      ["Mamba状态空间模型深度解析：挑战Transformer的下一代序列建模范式",
 *       §2.1 (selective SSM pseudo-code, where Δ, B and C depend on the token)].
 *  - Skip D x_t and the multiplicative SiLU gate of the block:
 *      out_t = (y_t + D x_t) * z_t * sigmoid(z_t)
 *      [same page, §3.1 block diagram: SiLU activation with multiplicative
 *       gating around the selective SSM].
 *  - Causal depthwise conv1d (kernel 4) + SiLU in front of the SSM
 *      [same page, §3.1 (causal Conv1D); "Mamba架构与SSM模型：高效序列建模技术解析",
 *       §3.2 (d_conv=4)].  Taps follow the usual cross-correlation order:
 *      pre_t = bias + sum_{k<K} w[k] x[t-(K-1)+k], with x[t<0] = 0.
 *  - Decode: one step of the same recurrence on a stored state
 *      ["Mamba架构深度剖析：如何以线性时间重塑序列建模", §3: fixed-size state,
 *       step-by-step prediction at inference].
 *  - Backward: gradients of the scan's output (and final state) with respect
 *    to every input, by the chain rule through the steps above in reverse
 *    order, the forward states recomputed rather than stored by the caller
 *      ["Mamba状态空间模型深度解析：挑战Transformer的下一代序列建模范式", §2.2:
 *       intermediate states recomputed in the backward pass].
 *  - Mamba-2 form ("SSD"): the same selective recurrence with one decay
 *    value per head (A = a_h times the identity, shared by the head's P
 *    channels and all N states) and B, C shared by a group of heads, which
 *    makes the sequence map a structured (semiseparable) matrix that can be
 *    applied with matrix multiplications
 *      ["Mamba状态空间模型深度解析：挑战Transformer的下一代序列建模范式", §4.2:
 *       Mamba-2 restates the SSM as structured matrix multiplication].
 *    Written here as the plain recurrence; Δ, ZOH, readout, skip and gate as
 *    above.
 *
 * Layouts (all row-major, fp64):
 *   x, dt, z, y : [B, D, L]      (L fastest)
 *   Bm, Cm      : [B, L, N]      (shared by every channel d of batch b)
 *   A           : [D, N];  dt_bias, Dskip : [D];  h0, h_last : [B, D, N]
 *   conv w      : [D, K];  conv bias : [D]
 *   decode      : h [B, D, N] in/out, x/dt/z/y [B, D], Bm/Cm [B, N]
 *   Mamba-2     : x, z, y [B, L, H, P];  dt [B, L, H];  Bm, Cm [B, L, G, N];
 *                 A, dt_bias, Dskip [H];  h0, h_last [B, H, P, N]
 * NULL for dt_bias / Dskip / z / h0 / h_last / conv bias means "absent"
 * (zero bias, no skip, no gate, zero initial state, state not returned).
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

/* softplus(v) = log(1 + e^v), evaluated without overflow. */
double oracle_softplus(double v)
{
    if (v > 0.0)
        return v + log1p(exp(-v));
    return log1p(exp(v));
}

/* z * sigmoid(z) */
double oracle_silu(double z)
{
    return z / (1.0 + exp(-z));
}

/* ZOH for one diagonal entry a with step delta:
 *   *abar = exp(delta a),  *bcoef = (exp(delta a) - 1) / a  (so Bbar = bcoef * B),
 * with the a = 0 limit bcoef = delta. */
void oracle_zoh(double delta, double a, double *abar, double *bcoef)
{
    *abar = exp(delta * a);
    if (a == 0.0)
        *bcoef = delta;
    else
        *bcoef = expm1(delta * a) / a;
}

/* One time step for one channel: h (length N) is updated in place and the
 * gated output is returned.  Bt, Ct point at this step's N values. */
static double step(int64_t N, double *h, double xv, double dtv, double bias,
                   const double *A, const double *Bt, const double *Ct,
                   double Dv, const double *zv)
{
    double delta = oracle_softplus(dtv + bias);
    double y = 0.0;
    for (int64_t n = 0; n < N; ++n) {
        double abar, bcoef;
        oracle_zoh(delta, A[n], &abar, &bcoef);
        h[n] = abar * h[n] + bcoef * Bt[n] * xv;
    }
    for (int64_t n = 0; n < N; ++n)
        y += Ct[n] * h[n];
    y += Dv * xv;
    if (zv)
        y *= oracle_silu(*zv);
    return y;
}

/* Scan of one channel over L steps.
 * x, dt, z, y: L values with unit stride.  Bm, Cm: L rows of N values with
 * row stride ldbc.  A, h0, h_last: N values. */
void oracle_scan_channel(int64_t L, int64_t N, const double *x, const double *dt,
                         double dt_bias, const double *A, const double *Bm,
                         const double *Cm, int64_t ldbc, double Dv, const double *z,
                         const double *h0, double *y, double *h_last)
{
    double h[64];
    for (int64_t n = 0; n < N; ++n)
        h[n] = h0 ? h0[n] : 0.0;
    for (int64_t t = 0; t < L; ++t)
        y[t] = step(N, h, x[t], dt[t], dt_bias, A, Bm + t * ldbc, Cm + t * ldbc, Dv,
                    z ? z + t : NULL);
    if (h_last)
        for (int64_t n = 0; n < N; ++n)
            h_last[n] = h[n];
}

typedef struct {
    const double *x, *dt, *dt_bias, *A, *Bm, *Cm, *Dskip, *z, *h0;
    double *y, *h_last;
    int64_t B, D, L, N;
    int64_t first, last; /* channel range [first, last) over b*D + d */
} scan_job;

static void *scan_worker(void *arg)
{
    const scan_job *j = (const scan_job *)arg;
    for (int64_t c = j->first; c < j->last; ++c) {
        int64_t b = c / j->D, d = c % j->D;
        size_t row = (size_t)c * (size_t)j->L;
        oracle_scan_channel(j->L, j->N, j->x + row, j->dt + row,
                            j->dt_bias ? j->dt_bias[d] : 0.0, j->A + d * j->N,
                            j->Bm + (size_t)b * j->L * j->N, j->Cm + (size_t)b * j->L * j->N,
                            j->N, j->Dskip ? j->Dskip[d] : 0.0, j->z ? j->z + row : NULL,
                            j->h0 ? j->h0 + (size_t)c * j->N : NULL, j->y + row,
                            j->h_last ? j->h_last + (size_t)c * j->N : NULL);
    }
    return NULL;
}

/* Whole-tensor selective scan.  Channels are independent sequences, so they
 * may be spread over nthreads POSIX threads; the arithmetic of each channel is
 * the same sequential loop either way.  Returns 0, or -1 on bad arguments. */
int oracle_selective_scan_fwd(const double *x, const double *dt, const double *dt_bias,
                              const double *A, const double *Bm, const double *Cm,
                              const double *Dskip, const double *z, const double *h0,
                              double *y, double *h_last, int64_t B, int64_t D, int64_t L,
                              int64_t N, int nthreads)
{
    if (!x || !dt || !A || !Bm || !Cm || !y || B < 0 || D < 0 || L < 0 || N < 1 || N > 64)
        return -1;
    int64_t nch = B * D;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if (nch < nthreads)
        nthreads = nch > 0 ? (int)nch : 1;
    scan_job jobs[256];
    pthread_t tids[256];
    for (int i = 0; i < nthreads; ++i) {
        scan_job j = {x, dt, dt_bias, A, Bm, Cm, Dskip, z, h0, y, h_last, B, D, L, N,
                      nch * i / nthreads, nch * (i + 1) / nthreads};
        jobs[i] = j;
    }
    if (nthreads == 1) {
        scan_worker(&jobs[0]);
        return 0;
    }
    int started = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&tids[i], NULL, scan_worker, &jobs[i]) != 0) {
            scan_worker(&jobs[i]);
            tids[i] = 0;
        } else {
            started++;
        }
    }
    for (int i = 0; i < nthreads; ++i)
        if (tids[i])
            pthread_join(tids[i], NULL);
    (void)started;
    return 0;
}

/* Causal depthwise conv1d over L with K taps, optional bias, then SiLU
 * (apply_silu != 0) or identity. */
int oracle_conv1d_silu(const double *x, const double *w, const double *bias, double *out,
                       int64_t B, int64_t D, int64_t L, int64_t K, int apply_silu)
{
    if (!x || !w || !out || B < 0 || D < 0 || L < 0 || K < 1)
        return -1;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t d = 0; d < D; ++d) {
            const double *xr = x + ((size_t)b * D + d) * L;
            double *orow = out + ((size_t)b * D + d) * L;
            for (int64_t t = 0; t < L; ++t) {
                double acc = bias ? bias[d] : 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    int64_t s = t - (K - 1) + k;
                    if (s >= 0)
                        acc += w[d * K + k] * xr[s];
                }
                orow[t] = apply_silu ? oracle_silu(acc) : acc;
            }
        }
    return 0;
}

/* Single-token step of the causal conv with its state: the K-1 previous raw
 * inputs of each channel, oldest first ([B, D, K-1], updated in place), stand
 * for the part of the sequence the window still reaches ("Mamba架构深度剖析：
 * 如何以线性时间重塑序列建模" §3, recurrent inference with a fixed-size
 * state; the conv of "Mamba状态空间模型深度解析…" §3.1).
 *   out[b,d] = SiLU(bias[d] + sum_{k<K-1} w[d,k] state[b,d,k] + w[d,K-1] x[b,d])
 * then the window moves by one step: the oldest input leaves, x enters. */
int oracle_conv1d_update(double *state, const double *x, const double *w, const double *bias,
                         double *out, int64_t B, int64_t D, int64_t K)
{
    if (!x || !w || !out || B < 0 || D < 0 || K < 1 || (K > 1 && !state))
        return -1;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t d = 0; d < D; ++d) {
            size_t c = (size_t)b * D + d;
            double *st = K > 1 ? state + c * (size_t)(K - 1) : NULL;
            double acc = bias ? bias[d] : 0.0;
            for (int64_t k = 0; k < K - 1; ++k)
                acc += w[d * K + k] * st[k];
            acc += w[d * K + K - 1] * x[c];
            out[c] = oracle_silu(acc);
            for (int64_t k = 0; k + 1 < K - 1; ++k)
                st[k] = st[k + 1];
            if (K > 1)
                st[K - 2] = x[c];
        }
    return 0;
}

/* d/da of the ZOH input coefficient (exp(delta a) - 1)/a:
 *   (delta a exp(delta a) - expm1(delta a)) / a^2 = delta^2 psi(delta a),
 *   psi(u) = (u e^u - e^u + 1)/u^2 = sum_{m>=0} (m+1) u^m / (m+2)!,
 * by its series for |u| < 1e-4 (psi(0) = 1/2) and the closed form above. */
static double dbcoef_da(double delta, double a)
{
    double u = delta * a;
    if (fabs(u) < 1e-4)
        return delta * delta * (0.5 + u / 3.0 + u * u / 8.0 + u * u * u / 30.0);
    return (u * exp(u) - expm1(u)) / (a * a);
}

/* Backward of oracle_selective_scan_fwd for the objective
 *   J = sum out * dout  (+ sum h_last * dh_last when dh_last is given).
 * Per channel the forward states are recomputed and kept, then the adjoint
 *   lambda_t = dJ/dh_t = C_t dy_t + nu_{t+1},   nu_t = Abar_t lambda_t,
 * nu_L = dh_last (or 0), runs backwards with dy_t = dout_t SiLU(z_t), and
 *   dx_t    = D dy_t + sum_n lambda_tn bcoef_tn B_tn
 *   dDelta_t = sum_n lambda_tn Abar_tn (A_n h_(t-1),n + B_tn x_t)
 *   ddt_t   = dDelta_t sigmoid(dt_t + dt_bias)            (softplus' = sigmoid)
 *   dz_t    = dout_t (y_t + D x_t) SiLU'(z_t)
 *   dA_n   += lambda_tn (Delta_t Abar_tn h_(t-1),n + dbcoef/dA_n B_tn x_t)
 *   dB_tn  += lambda_tn bcoef_tn x_t,   dC_tn += dy_t h_tn  (summed over d)
 *   dD     += dy_t x_t,  ddt_bias += ddt_t,  dh0 = nu_0.
 * Outputs dx, ddt, dz [B,D,L]; dA [D,N]; dD, ddt_bias [D]; dB, dC [B,L,N];
 * dh0 [B,D,N] are overwritten (dz, dh0 only when given; dz needs z).
 * Single-threaded: the sums over channels and batch rows are plain loops. */
int oracle_selective_scan_bwd(const double *x, const double *dt, const double *dt_bias,
                              const double *A, const double *Bm, const double *Cm,
                              const double *Dskip, const double *z, const double *h0,
                              const double *dout, const double *dh_last, double *dx,
                              double *ddt, double *dz, double *dA, double *dD,
                              double *ddt_bias, double *dB, double *dC, double *dh0, int64_t B,
                              int64_t D, int64_t L, int64_t N)
{
    if (!x || !dt || !A || !Bm || !Cm || !dout || !dx || !ddt || !dA || !dD || !ddt_bias ||
        !dB || !dC || B < 0 || D < 0 || L < 0 || N < 1 || N > 64)
        return -1;
    double *hist = (double *)malloc(sizeof(double) * (size_t)(L + 1) * (size_t)N);
    double *abar = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1) * (size_t)N);
    double *bco = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1) * (size_t)N);
    double *dlt = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    double *yy = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    if (!hist || !abar || !bco || !dlt || !yy) {
        free(hist); free(abar); free(bco); free(dlt); free(yy);
        return -2;
    }
    for (int64_t i = 0; i < D * N; ++i)
        dA[i] = 0.0;
    for (int64_t d = 0; d < D; ++d)
        dD[d] = ddt_bias[d] = 0.0;
    for (int64_t i = 0; i < B * L * N; ++i)
        dB[i] = dC[i] = 0.0;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t d = 0; d < D; ++d) {
            const size_t c = (size_t)b * D + d;
            const double *xr = x + c * L, *dtr = dt + c * L, *zr = z ? z + c * L : NULL;
            const double *go = dout + c * L;
            const double bias = dt_bias ? dt_bias[d] : 0.0, Dv = Dskip ? Dskip[d] : 0.0;
            const double *Ad = A + d * N;
            /* forward, keeping every state (hist row t+1 = h_t, row 0 = h0) */
            for (int64_t n = 0; n < N; ++n)
                hist[n] = h0 ? h0[c * N + n] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                const double *Bt = Bm + ((size_t)b * L + t) * N, *Ct = Cm + ((size_t)b * L + t) * N;
                dlt[t] = oracle_softplus(dtr[t] + bias);
                double y = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    oracle_zoh(dlt[t], Ad[n], &abar[t * N + n], &bco[t * N + n]);
                    hist[(t + 1) * N + n] =
                        abar[t * N + n] * hist[t * N + n] + bco[t * N + n] * Bt[n] * xr[t];
                    y += Ct[n] * hist[(t + 1) * N + n];
                }
                yy[t] = y + Dv * xr[t];
            }
            /* backward */
            double nu[64];
            for (int64_t n = 0; n < N; ++n)
                nu[n] = dh_last ? dh_last[c * N + n] : 0.0;
            for (int64_t t = L - 1; t >= 0; --t) {
                const double *Bt = Bm + ((size_t)b * L + t) * N, *Ct = Cm + ((size_t)b * L + t) * N;
                double *dBt = dB + ((size_t)b * L + t) * N, *dCt = dC + ((size_t)b * L + t) * N;
                double g = 1.0;
                if (zr) {
                    const double sg = 1.0 / (1.0 + exp(-zr[t]));
                    g = zr[t] * sg;
                    if (dz)
                        dz[c * L + t] = go[t] * yy[t] * sg * (1.0 + zr[t] * (1.0 - sg));
                }
                const double dy = go[t] * g;
                dD[d] += dy * xr[t];
                double dxs = Dv * dy, dDelta = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    const double lam = Ct[n] * dy + nu[n];
                    const double hp = hist[t * N + n], ab = abar[t * N + n], bc = bco[t * N + n];
                    dCt[n] += dy * hist[(t + 1) * N + n];
                    dBt[n] += lam * bc * xr[t];
                    dxs += lam * bc * Bt[n];
                    dDelta += lam * ab * (Ad[n] * hp + Bt[n] * xr[t]);
                    dA[d * N + n] += lam * (dlt[t] * ab * hp + dbcoef_da(dlt[t], Ad[n]) * Bt[n] * xr[t]);
                    nu[n] = ab * lam;
                }
                dx[c * L + t] = dxs;
                const double v = dtr[t] + bias;
                ddt[c * L + t] = dDelta / (1.0 + exp(-v));
                ddt_bias[d] += ddt[c * L + t];
            }
            if (dh0)
                for (int64_t n = 0; n < N; ++n)
                    dh0[c * N + n] = nu[n];
        }
    free(hist); free(abar); free(bco); free(dlt); free(yy);
    return 0;
}

/* Single-token decode step on a stored state h [B, D, N] (updated in place).
 * x, dt, z, y: [B, D];  Bm, Cm: [B, N]. */
int oracle_state_update(double *h, const double *x, const double *dt, const double *dt_bias,
                        const double *A, const double *Bm, const double *Cm,
                        const double *Dskip, const double *z, double *y, int64_t B,
                        int64_t D, int64_t N)
{
    if (!h || !x || !dt || !A || !Bm || !Cm || !y || B < 0 || D < 0 || N < 1 || N > 64)
        return -1;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t d = 0; d < D; ++d) {
            size_t c = (size_t)b * D + d;
            y[c] = step(N, h + c * N, x[c], dt[c], dt_bias ? dt_bias[d] : 0.0, A + d * N,
                        Bm + (size_t)b * N, Cm + (size_t)b * N, Dskip ? Dskip[d] : 0.0,
                        z ? z + c : NULL);
        }
    return 0;
}

/* Mamba-2 form: per head h (group g = h / (H/G)), state S[p][n] over the head's
 * P channels and N states, all decaying with the head's scalar a = A[h]:
 *   Δ = softplus(dt[b,t,h] + dt_bias[h]),  Abar = exp(Δ a),  bcoef = expm1(Δ a)/a
 *   S[p][n] <- Abar S[p][n] + bcoef Bm[b,t,g,n] x[b,t,h,p]
 *   y[b,t,h,p] = (sum_n Cm[b,t,g,n] S[p][n] + Dskip[h] x[b,t,h,p]) * SiLU(z[b,t,h,p])
 * Returns 0, or -1 on bad arguments. */
int oracle_ssd_scan_fwd(const double *x, const double *dt, const double *dt_bias,
                        const double *A, const double *Bm, const double *Cm,
                        const double *Dskip, const double *z, const double *h0, double *y,
                        double *h_last, int64_t B, int64_t L, int64_t H, int64_t P, int64_t G,
                        int64_t N)
{
    if (!x || !dt || !A || !Bm || !Cm || !y || B < 0 || L < 0 || H < 1 || P < 1 || G < 1 ||
        N < 1 || H % G != 0)
        return -1;
    double *S = (double *)malloc(sizeof(double) * (size_t)(P * N));
    if (!S)
        return -1;
    const int64_t heads_per_group = H / G;
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t h = 0; h < H; ++h) {
            const int64_t g = h / heads_per_group;
            const double a = A[h];
            const double bias = dt_bias ? dt_bias[h] : 0.0;
            const double Dv = Dskip ? Dskip[h] : 0.0;
            for (int64_t i = 0; i < P * N; ++i)
                S[i] = h0 ? h0[(b * H + h) * P * N + i] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                const double delta = oracle_softplus(dt[(b * L + t) * H + h] + bias);
                double abar, bcoef;
                oracle_zoh(delta, a, &abar, &bcoef);
                const double *Bt = Bm + ((b * L + t) * G + g) * N;
                const double *Ct = Cm + ((b * L + t) * G + g) * N;
                const int64_t row = ((b * L + t) * H + h) * P;
                for (int64_t p = 0; p < P; ++p) {
                    const double xv = x[row + p];
                    double acc = 0.0;
                    for (int64_t n = 0; n < N; ++n) {
                        S[p * N + n] = abar * S[p * N + n] + bcoef * Bt[n] * xv;
                        acc += Ct[n] * S[p * N + n];
                    }
                    acc += Dv * xv;
                    if (z)
                        acc *= oracle_silu(z[row + p]);
                    y[row + p] = acc;
                }
            }
            if (h_last)
                for (int64_t i = 0; i < P * N; ++i)
                    h_last[(b * H + h) * P * N + i] = S[i];
        }
    }
    free(S);
    return 0;
}
