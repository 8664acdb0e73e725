/*
 * ssd_oracle.c -- plain fp64 CPU oracle for the Mamba-2 SSD mixer core.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library; the product path never
 * calls it.
 *
 * What it computes, and where that is written down:
 *
 *  - The selective state-space recurrence of Mamba-2 (state-space duality),
 *    taken token by token, per (batch row, head), with no chunking:
 *        a_t  = exp(dt_t * A_h)
 *        h_t  = a_t * h_{t-1} + dt_t * B_t x_t^T        (h is N x P)
 *        y_t  = C_t^T h_t + D_h * x_t                   (h_t after token t)
 *    This is the SSD layer that the Codestral-Mamba weight-port header
 *    (builderforce-memory-engine diff, codestral_mamba.ts, tensor layout and
 *    "reconciliations" 2-3) and the Mini-K3-1H model card ("Architecture",
 *    "Checkpoint and training") both refer to.  The chunked GPU scan reaches
 *    the same result up to floating-point association, so the oracle is the
 *    definition itself.
 *  - A = -exp(A_log): codestral_mamba.ts header, reconciliation 2.  The
 *    oracle takes A itself (A <= 0), as the library does.
 *  - dt = softplus(dt_raw + dt_bias): falcon_mamba.ts header (the dt bias is
 *    added inside the softplus), and the inverse-softplus reparameterisation
 *    of dt_bias in the Mamba-1/2 -> Mamba-3 transplant article ("The
 *    Methodology", item 3).
 *  - Causal depthwise conv over the [x | B | C] columns, conv_dim =
 *    d_inner + 2*n_groups*d_state, weight [conv_dim, 1, d_conv]:
 *    codestral_mamba.ts tensor layout.  Reading of the tap order: plain
 *    causal cross-correlation, w[c][K-1] multiplies the current token.
 *  - Activation after the conv: SiLU (the published Mamba-2 block's
 *    convention, which the port pages defer to); act = 1 turns it off.
 *  - Gate y * silu(z): codestral_mamba.ts reconciliation 3 (upstream computes
 *    norm(y * silu(z)); the RMSNorm itself is outside this core).
 *  - Document isolation: the same document ids drive the conv and the scan;
 *    conv history and recurrent state reset at every boundary (Mini-K3-1H
 *    card, "Checkpoint and training").  Reading: a boundary sits at t > 0
 *    exactly where doc[t] != doc[t-1]; t = 0 always continues the carried
 *    state.
 *  - Caller-owned state read at entry and written at exit; a step is the
 *    same computation as a forward of length 1 with the state carried
 *    (mojolearn.Mamba3Block docs, forward() and step()).
 *  - Backward (oracle_scan_bwd, oracle_conv_bwd): the vector-Jacobian
 *    product of a zero-state prefill, given the gradient of the loss with
 *    respect to y; no gradient for a carried state and no final-state
 *    cotangent (mojolearn.Mamba3Block docs, backward()).  It is reverse-mode
 *    differentiation of the recurrence above, token by token from the last:
 *        dS      <- adjoint of h_t (the state after token t), from t+1
 *        yr_t    = C_t^T h_t + D x_t,  y_t = yr_t * silu(z_t)
 *        dz_t    = dy_t * yr_t * silu'(z_t);   dyr_t = dy_t * silu(z_t)
 *        dD     += dyr_t . x_t;  dx_t = D dyr_t;  dC_t += h_t dyr_t
 *        dS     += C_t dyr_t^T
 *        dB_t   += dt_t dS x_t;  dx_t += dt_t dS^T B_t
 *        ddt_t   = B_t^T dS x_t + A a_t <dS, h_{t-1}>;  dA += dt_t a_t <dS, h_{t-1}>
 *        dS      = a_t dS   (0 where a document starts at t: h_{t-1} is cut)
 *    and through dt = softplus(dt_raw + dt_bias) by sigmoid(dt_raw + dt_bias).
 *    The conv's backward runs the chain rule through the activation and the
 *    taps within each document.  A bf16 pipeline's rounding of the conv
 *    output is taken as the identity (the scan's inputs are the rounded
 *    values).  Packed documents: a loss on a later document gives exactly
 *    zero gradient on earlier-document inputs (Mini-K3-1H card, "Checkpoint
 *    and training").
 *
 * Layouts (all arrays fp64, contiguous):
 *   raw / conv out  [B][L][conv_dim]   columns [x (H*P, head-major) | B (G*N,
 *                                       group-major) | C (G*N)]
 *   x, z, y         [B][L][H*P]
 *   Bm, Cm          [B][L][G*N]
 *   dt              [B][L][H]
 *   ssm state       [B][H][P][N]       (entry (p,n) is h[n][p] of the math)
 *   conv state      [B][K-1][conv_dim] (raw rows, oldest first)
 *   head h uses group h / (H/G).
 *
 *  - The Mamba-1 selective scan (S6), per (batch row, channel d), with a
 *    per-channel diagonal state of d_state entries (oracle_s6):
 *        a_t[d,n] = exp(dt_t[d] * A[d][n])
 *        h_t[d,n] = a_t[d,n] * h_{t-1}[d,n] + dt_t[d] * B_t[n] * x_t[d]
 *        y_t[d]   = sum_n C_t[n] h_t[d,n] + D[d] * x_t[d]
 *    falcon_mamba.ts header: x_proj rows [dt, B, C] give one B and one C per
 *    token, shared by every channel; dt_proj (a linear with a bias) gives dt
 *    per channel and the bias goes inside the softplus; A [d_inner, d_state]
 *    = -exp(A_log), which selective_scan.ts computes as -exp(clamp(A_log,
 *    -10, 5)).  The oracle takes A itself.  Gate, documents and states as
 *    above.
 *
 * Every routine below is a straight loop in the notation above.  The
 * per-token helpers conv_channel() and ssm_token() are shared by the prefill
 * routines and the step so that a prefill followed by steps runs the very
 * same fp64 operations as one longer prefill.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_MAXK 8

/* softplus(v) = log(1 + e^v), written so that it does not overflow. */
static double softplus(double v) { return fmax(v, 0.0) + log1p(exp(-fabs(v))); }

/* silu(v) = v * sigmoid(v). */
static double silu(double v) { return v / (1.0 + exp(-v)); }
static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }
/* d silu / dv = s + v s (1 - s), s = sigmoid(v) */
static double dsilu(double v) { double s = sigmoid(v); return s + v * s * (1.0 - s); }

/* Round to the nearest bfloat16 value (8 significant bits), ties to even.
 * Used only where the contract stores a tensor in bf16 (the conv output of a
 * bf16 pipeline).  rint() rounds ties to even under the default mode. */
double oracle_round_bf16(double v) {
    if (v == 0.0 || !isfinite(v)) return v;
    int e = ilogb(v);                 /* v = m * 2^e, 1 <= |m| < 2 */
    if (e < -126) e = -126;           /* bf16 subnormal spacing */
    double q = ldexp(1.0, e - 7);     /* spacing of bf16 values near v */
    double r = rint(v / q) * q;
    if (fabs(r) > 3.3895313892515355e38) r = copysign(INFINITY, v);
    return r;
}

double oracle_softplus(double v) { return softplus(v); }
double oracle_silu(double v) { return silu(v); }

/* One conv output channel at one token: bias + sum_k w[k] * win[k], where
 * win[K-1] is the current token and win[0] the oldest tap. */
static double conv_channel(const double *w, double bias, const double *win, int K, int act) {
    double v = bias;
    for (int k = 0; k < K; ++k) v += w[k] * win[k];
    return act == 0 ? silu(v) : v;
}

/* One head at one token: update S (P x N, stored [p][n]) and write y[p]. */
static void ssm_token(int P, int N, double dt, double A, double Dh,
                      const double *x, const double *Bv, const double *Cv,
                      double *S, double *y) {
    double a = exp(dt * A);
    for (int p = 0; p < P; ++p)
        for (int n = 0; n < N; ++n)
            S[(size_t)p * N + n] = a * S[(size_t)p * N + n] + dt * x[p] * Bv[n];
    for (int p = 0; p < P; ++p) {
        double acc = 0.0;
        for (int n = 0; n < N; ++n) acc += Cv[n] * S[(size_t)p * N + n];
        y[p] = acc + Dh * x[p];
    }
}

/* Last position r in [0, t] at which a new document starts (0 if none). */
static int seg_start(const int32_t *doc_row, int t) {
    if (!doc_row) return 0;
    for (int r = t; r > 0; --r)
        if (doc_row[r] != doc_row[r - 1]) return r;
    return 0;
}

/* Raw conv input seen by token t at tap position tau (tau <= t): the raw row
 * if tau lies in t's document, else the carried conv state (only while t is
 * still in the first document of the call), else zero. */
static double conv_src(const double *raw_b, const double *state_b, int C, int K,
                       int seg, int tau, int c) {
    if (tau >= 0) return tau >= seg ? raw_b[(size_t)tau * C + c] : 0.0;
    if (seg == 0 && state_b) return state_b[(size_t)(K - 1 + tau) * C + c];
    return 0.0;
}

/*
 * Causal depthwise conv (+ SiLU) over [B, L, C] and dt = softplus(dt_raw +
 * dt_bias) over [B, L, H].  round_bf16 != 0 rounds every conv output to
 * bf16, as a bf16 pipeline stores it.  Returns 0, or -1 on bad arguments.
 */
int oracle_conv(int B, int L, int C, int K, int H,
                const double *raw, const double *w, const double *bias,
                const double *dt_raw, const double *dt_bias,
                const int32_t *doc, const double *state_in, double *state_out,
                int act, int round_bf16, double *out, double *dt_out) {
    if (B < 0 || L < 0 || C <= 0 || K < 1 || K > ORACLE_MAXK || !raw || !w || !out) return -1;
    for (int b = 0; b < B; ++b) {
        const double *raw_b = raw + (size_t)b * L * C;
        const double *st_b = state_in ? state_in + (size_t)b * (K - 1) * C : NULL;
        const int32_t *doc_b = doc ? doc + (size_t)b * L : NULL;
        double win[ORACLE_MAXK];
        for (int t = 0; t < L; ++t) {
            int seg = seg_start(doc_b, t);
            for (int c = 0; c < C; ++c) {
                for (int k = 0; k < K; ++k)
                    win[k] = conv_src(raw_b, st_b, C, K, seg, t - (K - 1) + k, c);
                double v = conv_channel(w + (size_t)c * K, bias ? bias[c] : 0.0, win, K, act);
                out[((size_t)b * L + t) * C + c] = round_bf16 ? oracle_round_bf16(v) : v;
            }
            if (dt_raw && dt_out)
                for (int h = 0; h < H; ++h) {
                    size_t i = ((size_t)b * L + t) * H + h;
                    dt_out[i] = softplus(dt_raw[i] + (dt_bias ? dt_bias[h] : 0.0));
                }
        }
    }
    /* Conv state after the call: the K-1 taps the next token would read,
     * judged from the last token's document (so all reads of state_in above
     * are complete before it may be overwritten in place). */
    if (state_out) {
        double *tmp = (double *)malloc(sizeof(double) * (size_t)(K > 1 ? K - 1 : 1) * C);
        if (!tmp) return -1;
        for (int b = 0; b < B; ++b) {
            const double *raw_b = raw + (size_t)b * L * C;
            const double *st_b = state_in ? state_in + (size_t)b * (K - 1) * C : NULL;
            const int32_t *doc_b = doc ? doc + (size_t)b * L : NULL;
            int seg = L > 0 ? seg_start(doc_b, L - 1) : 0;
            for (int j = 0; j < K - 1; ++j)
                for (int c = 0; c < C; ++c)
                    tmp[(size_t)j * C + c] = conv_src(raw_b, st_b, C, K, seg, L - (K - 1) + j, c);
            memcpy(state_out + (size_t)b * (K - 1) * C, tmp, sizeof(double) * (size_t)(K - 1) * C);
        }
        free(tmp);
    }
    return 0;
}

/*
 * Sequential SSD recurrence over [B, L] for all heads.  dt_softplus != 0
 * means dt holds raw values and dt := softplus(dt + dt_bias) is applied
 * first.  D, z, doc, init_state, final_state may be NULL.
 */
int oracle_scan(int B, int L, int H, int P, int N, int G,
                const double *x, const double *Bm, const double *Cm,
                const double *dt, int dt_softplus, const double *dt_bias,
                const double *A, const double *D, const double *z,
                const int32_t *doc, const double *init_state, double *final_state,
                double *y) {
    if (B < 0 || L < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0) return -1;
    if ((L > 0 && (!x || !Bm || !Cm || !dt || !y)) || !A) return -1;
    const int HP = H * P, GN = G * N, hpg = H / G;
    int bad = 0;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            const int g = h / hpg;
            double *S = (double *)calloc((size_t)P * N, sizeof(double));
            double *yp = (double *)malloc(sizeof(double) * (size_t)P);
            if (!S || !yp) { bad = 1; free(S); free(yp); continue; }
            if (init_state)
                memcpy(S, init_state + ((size_t)b * H + h) * P * N, sizeof(double) * (size_t)P * N);
            for (int t = 0; t < L; ++t) {
                size_t row = (size_t)b * L + t;
                if (doc && t > 0 && doc[row] != doc[row - 1])
                    memset(S, 0, sizeof(double) * (size_t)P * N);
                double d = dt[row * H + h];
                if (dt_softplus) d = softplus(d + (dt_bias ? dt_bias[h] : 0.0));
                ssm_token(P, N, d, A[h], D ? D[h] : 0.0,
                          x + row * HP + (size_t)h * P, Bm + row * GN + (size_t)g * N,
                          Cm + row * GN + (size_t)g * N, S, yp);
                for (int p = 0; p < P; ++p) {
                    double v = yp[p];
                    if (z) v *= silu(z[row * HP + (size_t)h * P + p]);
                    y[row * HP + (size_t)h * P + p] = v;
                }
            }
            if (final_state)
                memcpy(final_state + ((size_t)b * H + h) * P * N, S, sizeof(double) * (size_t)P * N);
            free(S);
            free(yp);
        }
    return bad ? -1 : 0;
}

/*
 * One decode token per sequence.  The conv window is the K-1 carried raw
 * rows followed by the new raw row; the buffer then shifts by one.  The conv
 * output is rounded to bf16 when round_bf16 != 0 (as a bf16 prefill stores
 * it), then the state update is exactly one token of oracle_scan.
 *   raw [B][C], dt_raw [B][H], z [B][H*P] or NULL, y [B][H*P]
 *   conv_state [B][K-1][C] and ssm_state [B][H][P][N] are read and updated.
 */
int oracle_step(int B, int H, int P, int N, int G, int K,
                const double *raw, const double *dt_raw, const double *z,
                const double *w, const double *bias, const double *dt_bias,
                const double *A, const double *D,
                double *conv_state, double *ssm_state, int act, int round_bf16,
                double *y) {
    if (B < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0 || K < 1 || K > ORACLE_MAXK) return -1;
    const int HP = H * P, GN = G * N, C = HP + 2 * GN, hpg = H / G;
    double *xbc = (double *)malloc(sizeof(double) * (size_t)C);
    double *yp = (double *)malloc(sizeof(double) * (size_t)P);
    if (!xbc || !yp) { free(xbc); free(yp); return -1; }
    double win[ORACLE_MAXK];
    for (int b = 0; b < B; ++b) {
        double *cs = conv_state + (size_t)b * (K - 1) * C;
        const double *rb = raw + (size_t)b * C;
        for (int c = 0; c < C; ++c) {
            for (int k = 0; k < K - 1; ++k) win[k] = cs[(size_t)k * C + c];
            win[K - 1] = rb[c];
            double v = conv_channel(w + (size_t)c * K, bias ? bias[c] : 0.0, win, K, act);
            xbc[c] = round_bf16 ? oracle_round_bf16(v) : v;
        }
        for (int k = 0; k + 1 < K - 1; ++k)
            memcpy(cs + (size_t)k * C, cs + (size_t)(k + 1) * C, sizeof(double) * (size_t)C);
        if (K > 1) memcpy(cs + (size_t)(K - 2) * C, rb, sizeof(double) * (size_t)C);
        for (int h = 0; h < H; ++h) {
            const int g = h / hpg;
            double d = softplus(dt_raw[(size_t)b * H + h] + (dt_bias ? dt_bias[h] : 0.0));
            double *S = ssm_state + ((size_t)b * H + h) * P * N;
            ssm_token(P, N, d, A[h], D ? D[h] : 0.0, xbc + (size_t)h * P,
                      xbc + HP + (size_t)g * N, xbc + HP + GN + (size_t)g * N, S, yp);
            for (int p = 0; p < P; ++p) {
                double v = yp[p];
                if (z) v *= silu(z[(size_t)b * HP + (size_t)h * P + p]);
                y[(size_t)b * HP + (size_t)h * P + p] = v;
            }
        }
    }
    free(xbc);
    free(yp);
    return 0;
}

/*
 * Sequential Mamba-1 selective scan (S6) over [B, L] for all channels.
 *   x, dt, z, y [B][L][D]; Bm, Cm [B][L][N]; A [D][N]; D_skip [D];
 *   init_state, final_state [B][D][N].
 * dt_softplus != 0: dt holds raw values and dt := softplus(dt + dt_bias).
 * D_skip, z, doc, init_state, final_state, dt_bias may be NULL.
 */
int oracle_s6(int B, int L, int D, int N,
              const double *x, const double *dt, int dt_softplus, const double *dt_bias,
              const double *A, const double *Bm, const double *Cm, const double *D_skip,
              const double *z, const int32_t *doc, const double *init_state, double *final_state,
              double *y) {
    if (B < 0 || L < 0 || D <= 0 || N <= 0 || !A) return -1;
    if (L > 0 && (!x || !dt || !Bm || !Cm || !y)) return -1;
    int bad = 0;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b)
        for (int d = 0; d < D; ++d) {
            double *h = (double *)calloc((size_t)N, sizeof(double));
            if (!h) { bad = 1; continue; }
            if (init_state) memcpy(h, init_state + ((size_t)b * D + d) * N, sizeof(double) * (size_t)N);
            const double *Ad = A + (size_t)d * N;
            for (int t = 0; t < L; ++t) {
                size_t row = (size_t)b * L + t;
                if (doc && t > 0 && doc[row] != doc[row - 1]) memset(h, 0, sizeof(double) * (size_t)N);
                double dtv = dt[row * D + d];
                if (dt_softplus) dtv = softplus(dtv + (dt_bias ? dt_bias[d] : 0.0));
                const double xv = x[row * D + d];
                const double *Bt = Bm + row * N, *Ct = Cm + row * N;
                double acc = 0.0;
                for (int n = 0; n < N; ++n) {
                    h[n] = exp(dtv * Ad[n]) * h[n] + dtv * Bt[n] * xv;
                    acc += Ct[n] * h[n];
                }
                double v = acc + (D_skip ? D_skip[d] : 0.0) * xv;
                if (z) v *= silu(z[row * D + d]);
                y[row * D + d] = v;
            }
            if (final_state) memcpy(final_state + ((size_t)b * D + d) * N, h, sizeof(double) * (size_t)N);
            free(h);
        }
    return bad ? -1 : 0;
}

/*
 * Backward of oracle_scan for a zero initial state.  gy is dLoss/dy
 * [B][L][H*P].  Writes dx [B][L][H*P], dB and dC [B][L][G*N] (summed over
 * the heads of a group), ddt [B][L][H] (with respect to the dt input: the
 * raw value when dt_softplus != 0), and, if not NULL, ddt_bias, dA, dD [H]
 * and dz [B][L][H*P].  Returns 0, or -1 on bad arguments.
 */
int oracle_scan_bwd(int B, int L, int H, int P, int N, int G,
                    const double *x, const double *Bm, const double *Cm,
                    const double *dt, int dt_softplus, const double *dt_bias,
                    const double *A, const double *D, const double *z,
                    const int32_t *doc, const double *gy,
                    double *dx, double *dB, double *dC, double *ddt,
                    double *ddt_bias, double *dA, double *dD, double *dz) {
    if (B < 0 || L < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0 || !A) return -1;
    if (L > 0 && (!x || !Bm || !Cm || !dt || !gy || !dx || !dB || !dC || !ddt)) return -1;
    const int HP = H * P, GN = G * N, hpg = H / G;
    const size_t PN = (size_t)P * N;
    /* per (b, h) partial sums of the per-head parameters, summed over b in
     * order afterwards */
    double *pA = (double *)calloc((size_t)B * H * 3 + 1, sizeof(double));
    if (!pA) return -1;
    double *pD = pA + (size_t)B * H, *pBias = pD + (size_t)B * H;
    int bad = 0;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b)
        for (int g = 0; g < G; ++g) {
            double *Sall = (double *)calloc((size_t)(L + 1) * PN, sizeof(double));
            double *dS = (double *)malloc(sizeof(double) * PN);
            if (!Sall || !dS) { bad = 1; free(Sall); free(dS); continue; }
            for (int t = 0; t < L; ++t) {
                size_t row = (size_t)b * L + t;
                for (int n = 0; n < N; ++n) {
                    dB[row * GN + (size_t)g * N + n] = 0.0;
                    dC[row * GN + (size_t)g * N + n] = 0.0;
                }
            }
            for (int h = g * hpg; h < (g + 1) * hpg; ++h) {
                const double Ah = A[h], Dh = D ? D[h] : 0.0, bias = dt_bias ? dt_bias[h] : 0.0;
                /* forward: Sall[t + 1] is the state after token t */
                for (int t = 0; t < L; ++t) {
                    size_t row = (size_t)b * L + t;
                    double d = dt[row * H + h];
                    if (dt_softplus) d = softplus(d + bias);
                    const double a = exp(d * Ah);
                    const int reset = doc && t > 0 && doc[row] != doc[row - 1];
                    const double *xv = x + row * HP + (size_t)h * P, *Bv = Bm + row * GN + (size_t)g * N;
                    double *Sp = Sall + (size_t)t * PN, *Sc = Sall + (size_t)(t + 1) * PN;
                    for (int p = 0; p < P; ++p)
                        for (int n = 0; n < N; ++n)
                            Sc[(size_t)p * N + n] = (reset ? 0.0 : a * Sp[(size_t)p * N + n]) + d * xv[p] * Bv[n];
                }
                /* reverse */
                memset(dS, 0, sizeof(double) * PN);
                double sA = 0.0, sD = 0.0, sBias = 0.0;
                for (int t = L - 1; t >= 0; --t) {
                    size_t row = (size_t)b * L + t;
                    const double raw_dt = dt[row * H + h];
                    const double d = dt_softplus ? softplus(raw_dt + bias) : raw_dt;
                    const double a = exp(d * Ah);
                    const int reset = doc && t > 0 && doc[row] != doc[row - 1];
                    const double *xv = x + row * HP + (size_t)h * P;
                    const double *Bv = Bm + row * GN + (size_t)g * N, *Cv = Cm + row * GN + (size_t)g * N;
                    const double *Sc = Sall + (size_t)(t + 1) * PN, *Sp = Sall + (size_t)t * PN;
                    double *dxv = dx + row * HP + (size_t)h * P;
                    double *dBv = dB + row * GN + (size_t)g * N, *dCv = dC + row * GN + (size_t)g * N;
                    /* output */
                    for (int p = 0; p < P; ++p) {
                        double yr = Dh * xv[p];
                        for (int n = 0; n < N; ++n) yr += Cv[n] * Sc[(size_t)p * N + n];
                        const double gyv = gy[row * HP + (size_t)h * P + p];
                        double dyr = gyv;
                        if (z) {
                            const double zv = z[row * HP + (size_t)h * P + p];
                            dyr = gyv * silu(zv);
                            if (dz) dz[row * HP + (size_t)h * P + p] = gyv * yr * dsilu(zv);
                        }
                        sD += dyr * xv[p];
                        dxv[p] = Dh * dyr;
                        for (int n = 0; n < N; ++n) {
                            dCv[n] += dyr * Sc[(size_t)p * N + n];
                            dS[(size_t)p * N + n] += Cv[n] * dyr;
                        }
                    }
                    /* through h_t = a h_{t-1} + dt B x^T */
                    double dd = 0.0, da = 0.0;
                    for (int p = 0; p < P; ++p)
                        for (int n = 0; n < N; ++n) {
                            const double g_pn = dS[(size_t)p * N + n];
                            dBv[n] += d * g_pn * xv[p];
                            dxv[p] += d * g_pn * Bv[n];
                            dd += g_pn * Bv[n] * xv[p];
                            if (!reset) da += g_pn * Sp[(size_t)p * N + n];
                        }
                    dd += da * a * Ah;
                    sA += da * a * d;
                    for (size_t i = 0; i < PN; ++i) dS[i] = reset ? 0.0 : a * dS[i];
                    if (dt_softplus) {
                        const double s = sigmoid(raw_dt + bias);
                        ddt[row * H + h] = dd * s;
                        sBias += dd * s;
                    } else {
                        ddt[row * H + h] = dd;
                    }
                }
                pA[(size_t)b * H + h] = sA;
                pD[(size_t)b * H + h] = sD;
                pBias[(size_t)b * H + h] = sBias;
            }
            free(Sall);
            free(dS);
        }
    for (int h = 0; h < H; ++h) {
        double sa = 0.0, sd = 0.0, sb = 0.0;
        for (int b = 0; b < B; ++b) {
            sa += pA[(size_t)b * H + h];
            sd += pD[(size_t)b * H + h];
            sb += pBias[(size_t)b * H + h];
        }
        if (dA) dA[h] = sa;
        if (dD) dD[h] = sd;
        if (ddt_bias) ddt_bias[h] = sb;
    }
    free(pA);
    return bad ? -1 : 0;
}

/*
 * Backward of oracle_conv for a zero conv state: given dout = dLoss/d(conv
 * output) [B][L][C] and ddt = dLoss/d(dt output) [B][L][H] (or NULL), writes
 * draw [B][L][C], dw [C][K], dbias [C] (or NULL), and, when ddt is given,
 * ddt_raw [B][L][H] and ddt_bias [H] (or NULL).
 */
int oracle_conv_bwd(int B, int L, int C, int K, int H,
                    const double *raw, const double *w, const double *bias,
                    const double *dt_raw, const double *dt_bias,
                    const int32_t *doc, int act, const double *dout, const double *ddt,
                    double *draw, double *dw, double *dbias, double *ddt_raw, double *ddt_bias) {
    if (B < 0 || L < 0 || C <= 0 || K < 1 || K > ORACLE_MAXK || !w || !dw) return -1;
    if (L > 0 && (!raw || !dout || !draw)) return -1;
#pragma omp parallel for schedule(static)
    for (int c = 0; c < C; ++c) {
        double gw[ORACLE_MAXK] = {0.0};
        double gb = 0.0;
        for (int b = 0; b < B; ++b) {
            const double *raw_b = raw + (size_t)b * L * C;
            const int32_t *doc_b = doc ? doc + (size_t)b * L : NULL;
            for (int t = 0; t < L; ++t) draw[((size_t)b * L + t) * C + c] = 0.0;
            for (int t = 0; t < L; ++t) {
                const int seg = seg_start(doc_b, t);
                double pre = bias ? bias[c] : 0.0;
                for (int k = 0; k < K; ++k) {
                    const int tau = t - (K - 1) + k;
                    if (tau >= seg && tau >= 0) pre += w[(size_t)c * K + k] * raw_b[(size_t)tau * C + c];
                }
                const double go = dout[((size_t)b * L + t) * C + c];
                const double gp = act == 0 ? go * dsilu(pre) : go;
                gb += gp;
                for (int k = 0; k < K; ++k) {
                    const int tau = t - (K - 1) + k;
                    if (tau >= seg && tau >= 0) {
                        draw[((size_t)b * L + tau) * C + c] += w[(size_t)c * K + k] * gp;
                        gw[k] += gp * raw_b[(size_t)tau * C + c];
                    }
                }
            }
        }
        for (int k = 0; k < K; ++k) dw[(size_t)c * K + k] = gw[k];
        if (dbias) dbias[c] = gb;
    }
    if (ddt && dt_raw && ddt_raw) {
        for (int h = 0; h < H; ++h) {
            double sb = 0.0;
            for (int b = 0; b < B; ++b)
                for (int t = 0; t < L; ++t) {
                    const size_t i = ((size_t)b * L + t) * H + h;
                    const double s = sigmoid(dt_raw[i] + (dt_bias ? dt_bias[h] : 0.0));
                    ddt_raw[i] = ddt[i] * s;
                    sb += ddt[i] * s;
                }
            if (ddt_bias) ddt_bias[h] = sb;
        }
    }
    return 0;
}
