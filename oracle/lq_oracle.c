/*
 * lq_oracle.c -- plain, slow CPU oracle for the int8-state Gated DeltaNet /
 * Kimi Delta Attention decode path ("LeapQuant").
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header or table with the HIP library; it is built with plain gcc
 * (-O2 -ffp-contract=off, no fast-math).
 *
 * Sources (web pages about one preprint; cited by page and section):
 *   [abstract]  "LeapQuant: Efficient Linear Attention with Accurate Recurrent
 *               State Quantization", HFEPX eval-paper page (opentrain.ai),
 *               section "Abstract".
 *   [forum]     "LeapQuant: Training-Free 8-bit Quantization for Linear
 *               Attention Recurrent States" (zhichai.net forum mirror),
 *               section "Abstract (translated)", techniques 1-3.
 *   [news ¶n]   "A linear-attention method cuts state ..." news article
 *               (globaltechnewsdesk.com), paragraph n.
 *   [blog]      "LeapQuant targets the hidden inference cost in linear
 *               attention" (kenashe.ai), section "How does LeapQuant avoid
 *               the usual quantization damage?".
 *
 * Per head the state is H (dk x dv, row i = key channel, column j = value
 * channel); the output of a token is o = H^T q read AFTER that token's update.
 *
 * Precision.  The recurrence, the WY window algebra and the reconstruction
 * run in fp64.  The codec (outlier rows, smoothing, int8 rounding) turns
 * floating point into integers, so it runs in fp32, the precision the GPU
 * kernels use, with every operation a single correctly rounded IEEE op.
 *
 * Parity status: every function here is pinned by CPU tests against closed
 * forms, brute force or library routines (see tests/test_oracle_*.py);
 * none is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define LQO_TINY 0x1p-120f

/* ------------------------------------------------------------------------ */
/* Recurrence                                                               */
/* ------------------------------------------------------------------------ */

/*
 * One token of the gated delta rule, in place, plain definition:
 *
 *     H <- (I - beta k k^T) D H + beta k v^T,     o = H^T q
 *
 * D = alpha I (Gated DeltaNet: one decay per token, per_key = 0) or
 * D = diag(alpha) (Kimi Delta Attention: one decay per key channel,
 * per_key = 1).  The decay acts before the delta correction.  The pages only
 * name GDN and KDA ([abstract]; [forum] summary); this is the standard form
 * of both rules.  (I - beta k k^T) X is expanded as X - beta k (k^T X).
 */
void lqo_step(int dk, int dv, int per_key, double *H,
              const float *q, const float *k, const float *v,
              const float *alpha, float beta, double *o)
{
    double *p = (double *)calloc((size_t)dv, sizeof(double));
    /* X = D H */
    for (int i = 0; i < dk; ++i) {
        double a = per_key ? (double)alpha[i] : (double)alpha[0];
        for (int j = 0; j < dv; ++j) H[(size_t)i * dv + j] *= a;
    }
    /* p = X^T k  (the value X currently stores under key k) */
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += H[(size_t)i * dv + j] * (double)k[i];
        p[j] = acc;
    }
    /* H = X - beta k p^T + beta k v^T */
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            H[(size_t)i * dv + j] += (double)beta * (double)k[i] * ((double)v[j] - p[j]);
    /* o = H^T q */
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += H[(size_t)i * dv + j] * (double)q[i];
        o[j] = acc;
    }
    free(p);
}

/* ------------------------------------------------------------------------ */
/* Codec: int8 state + per-row scales + per-column smoothing + C outlier    */
/* rows kept in full precision ("compensator tokens").                      */
/* ------------------------------------------------------------------------ */

/*
 * Quantize one fp32 state H into (sq, r, s, idx, cv).
 *
 * [forum] techniques 2 and 3, [abstract], [news ¶4]: a few of the state's
 * biggest outlier entries stay in high precision as compensator tokens, what
 * is left is smoothed, and that is rounded to 8 bits.  The pages give no
 * formulas; the steps below are this codec's definition:
 *
 *   Q1  m_i  = max_j |H_ij|                         (row magnitude)
 *   Q2  idx  = the C rows with the largest m_i, ties to the lower row, stored
 *              in ascending row order
 *   Q3  cv_c = H[idx_c][:] (exact copy); R = H with those rows zeroed.  A
 *              compensator token is the pair (key e_idx, value cv).
 *   Q4  s_j  = max_i |R_ij|; 1 if that is below TINY (or smoothing is off)
 *   Q5  Y_ij = R_ij * (1 / s_j)
 *   Q6  rho_i = max_j |Y_ij|;  r_i = rho_i / 127
 *   Q7  sq_ij = clamp(rint(Y_ij * (127 / rho_i)), -127, 127); a row with
 *              rho_i below TINY is all zeros with r_i = 0.
 *
 * TINY = 2^-120 keeps both reciprocals finite (1/s_j and 127/rho_i overflow
 * fp32 below about 2^-121); magnitudes that small are taken as zero.
 * Every operation is one fp32 IEEE op (round to nearest even); rint rounds
 * half to even.  1/s_j and 127/rho_i are each one correctly rounded
 * division.  Returns 0, or -1 on bad sizes.
 */
int lqo_quantize(int dk, int dv, int C, int smooth, const float *H,
                 int8_t *sq, float *r, float *s, int32_t *idx, float *cv)
{
    if (dk <= 0 || dv <= 0 || C < 0 || C > dk) return -1;
    float *m = (float *)malloc(sizeof(float) * (size_t)dk);
    char *chosen = (char *)calloc((size_t)dk, 1);
    float *R = (float *)malloc(sizeof(float) * (size_t)dk * dv);

    /* Q1 */
    for (int i = 0; i < dk; ++i) {
        float mx = 0.0f;
        for (int j = 0; j < dv; ++j) {
            float a = fabsf(H[(size_t)i * dv + j]);
            if (a > mx) mx = a;
        }
        m[i] = mx;
    }
    /* Q2: C rounds of "largest remaining"; the ascending scan with a strict
     * comparison keeps the lower row on ties. */
    for (int c = 0; c < C; ++c) {
        int best = -1;
        for (int i = 0; i < dk; ++i)
            if (!chosen[i] && (best < 0 || m[i] > m[best])) best = i;
        chosen[best] = 1;
    }
    for (int i = 0, c = 0; i < dk; ++i)
        if (chosen[i]) idx[c++] = i;
    /* Q3 */
    for (int c = 0; c < C; ++c)
        for (int j = 0; j < dv; ++j)
            cv[(size_t)c * dv + j] = H[(size_t)idx[c] * dv + j];
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            R[(size_t)i * dv + j] = chosen[i] ? 0.0f : H[(size_t)i * dv + j];
    /* Q4 */
    for (int j = 0; j < dv; ++j) {
        float mx = 0.0f;
        for (int i = 0; i < dk; ++i) {
            float a = fabsf(R[(size_t)i * dv + j]);
            if (a > mx) mx = a;
        }
        s[j] = (smooth && mx >= LQO_TINY) ? mx : 1.0f;
    }
    /* Q5 (R is overwritten by Y) */
    for (int j = 0; j < dv; ++j) {
        float inv = 1.0f / s[j];
        for (int i = 0; i < dk; ++i) R[(size_t)i * dv + j] = R[(size_t)i * dv + j] * inv;
    }
    /* Q6, Q7 */
    for (int i = 0; i < dk; ++i) {
        float rho = 0.0f;
        for (int j = 0; j < dv; ++j) {
            float a = fabsf(R[(size_t)i * dv + j]);
            if (a > rho) rho = a;
        }
        if (rho < LQO_TINY) {
            r[i] = 0.0f;
            for (int j = 0; j < dv; ++j) sq[(size_t)i * dv + j] = 0;
            continue;
        }
        r[i] = rho / 127.0f;
        float lam = 127.0f / rho;
        for (int j = 0; j < dv; ++j) {
            float x = rintf(R[(size_t)i * dv + j] * lam);
            if (x > 127.0f) x = 127.0f;
            if (x < -127.0f) x = -127.0f;
            sq[(size_t)i * dv + j] = (int8_t)x;
        }
    }
    free(m); free(chosen); free(R);
    return 0;
}

/*
 * The state a codec stands for, in fp64:  H_ij = sq_ij * r_i * s_j, plus the
 * compensator tokens e_idx cv^T (their rows of sq are zero, so this sets
 * those rows to cv).
 */
void lqo_dequantize(int dk, int dv, int C, const int8_t *sq, const float *r,
                    const float *s, const int32_t *idx, const float *cv, double *H)
{
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            H[(size_t)i * dv + j] = (double)sq[(size_t)i * dv + j] * (double)r[i] * (double)s[j];
    for (int c = 0; c < C; ++c)
        for (int j = 0; j < dv; ++j)
            H[(size_t)idx[c] * dv + j] += (double)cv[(size_t)c * dv + j];
}

/* ------------------------------------------------------------------------ */
/* In-window buffered updates, WY form (fp64)                               */
/* ------------------------------------------------------------------------ */
/*
 * [abstract]: while a window is open the 8-bit state stays as it is and the
 * outputs also use the window's updates, held in full precision; [news ¶3]:
 * every update is applied, only the rounding waits.  Writing the state after
 * slot n of a window as
 *
 *     H_n = A_n Hb + U_n            (Hb = window-base state)
 *     A_n = Gamma_n - sum_{i<=n} (E_{n,i} o k_i) y_i^T
 *     U_n =           sum_{i<=n} (E_{n,i} o k_i) u_i^T
 *
 * with g_n = sum_{m<=n} log alpha_m (window-local, a vector for KDA),
 * Gamma_n = diag(exp g_n), E_{n,i} = exp(g_n - g_i) (elementwise, <= 1),
 * the slot-n terms follow from one delta-rule step:
 *
 *     rr_i = sum_c k[c] k_i[c] E_{n,i}[c]                       (i < n)
 *     y_n  = beta (exp(g_n) o k - sum_{i<n} rr_i y_i)
 *     u_n  = beta (v - sum_{i<n} rr_i u_i)
 *
 * The buffer (k_i, y_i, u_i, g_i) depends only on the window's tokens.
 * Buffer layout: bk[W][dk], by[W][dk], bu[W][dv], bg[W][gd] with gd = dk for
 * KDA, 1 for GDN.
 */
void lqo_wy_append(int dk, int dv, int per_key, int n,
                   double *bk, double *by, double *bu, double *bg,
                   const float *k, const float *v, const float *alpha, float beta)
{
    int gd = per_key ? dk : 1;
    double *gn = (double *)malloc(sizeof(double) * (size_t)gd);
    double *rr = (double *)calloc((size_t)(n > 0 ? n : 1), sizeof(double));
    for (int c = 0; c < gd; ++c)
        gn[c] = (n > 0 ? bg[(size_t)(n - 1) * gd + c] : 0.0) + log((double)alpha[c]);
    for (int i = 0; i < n; ++i) {
        double acc = 0.0;
        for (int c = 0; c < dk; ++c) {
            double e = exp(gn[per_key ? c : 0] - bg[(size_t)i * gd + (per_key ? c : 0)]);
            acc += (double)k[c] * bk[(size_t)i * dk + c] * e;
        }
        rr[i] = acc;
    }
    for (int c = 0; c < dk; ++c) {
        double acc = exp(gn[per_key ? c : 0]) * (double)k[c];
        for (int i = 0; i < n; ++i) acc -= rr[i] * by[(size_t)i * dk + c];
        by[(size_t)n * dk + c] = (double)beta * acc;
        bk[(size_t)n * dk + c] = (double)k[c];
    }
    for (int j = 0; j < dv; ++j) {
        double acc = (double)v[j];
        for (int i = 0; i < n; ++i) acc -= rr[i] * bu[(size_t)i * dv + j];
        bu[(size_t)n * dv + j] = (double)beta * acc;
    }
    for (int c = 0; c < gd; ++c) bg[(size_t)n * gd + c] = gn[c];
    free(gn); free(rr);
}

/*
 * Output of slot n (slot n already appended):  o = H_n^T q
 *   = Hb^T q' + sum_{i<=n} a_i u_i,
 *   a_i = sum_c q[c] k_i[c] E_{n,i}[c],   q' = exp(g_n) o q - sum_{i<=n} a_i y_i.
 */
void lqo_wy_output(int dk, int dv, int per_key, int n, const double *Hb,
                   const double *bk, const double *by, const double *bu, const double *bg,
                   const float *q, double *o)
{
    int gd = per_key ? dk : 1;
    const double *gn = bg + (size_t)n * gd;
    double *a = (double *)malloc(sizeof(double) * (size_t)(n + 1));
    double *qp = (double *)malloc(sizeof(double) * (size_t)dk);
    for (int i = 0; i <= n; ++i) {
        double acc = 0.0;
        for (int c = 0; c < dk; ++c) {
            double e = exp(gn[per_key ? c : 0] - bg[(size_t)i * gd + (per_key ? c : 0)]);
            acc += (double)q[c] * bk[(size_t)i * dk + c] * e;
        }
        a[i] = acc;
    }
    for (int c = 0; c < dk; ++c) {
        double acc = exp(gn[per_key ? c : 0]) * (double)q[c];
        for (int i = 0; i <= n; ++i) acc -= a[i] * by[(size_t)i * dk + c];
        qp[c] = acc;
    }
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int c = 0; c < dk; ++c) acc += Hb[(size_t)c * dv + j] * qp[c];
        for (int i = 0; i <= n; ++i) acc += a[i] * bu[(size_t)i * dv + j];
        o[j] = acc;
    }
    free(a); free(qp);
}

/*
 * Boundary reconstruction ([news ¶3]: the state is rebuilt once at the window
 * boundary) from N buffered slots:  H = A_{N-1} Hb + U_{N-1}
 *   = Gamma Hb + sum_i (E_{N-1,i} o k_i) (u_i - Hb^T y_i)^T.
 * N = 0 returns Hb.
 */
void lqo_wy_reconstruct(int dk, int dv, int per_key, int N, const double *Hb,
                        const double *bk, const double *by, const double *bu, const double *bg,
                        double *H)
{
    int gd = per_key ? dk : 1;
    if (N == 0) {
        memcpy(H, Hb, sizeof(double) * (size_t)dk * dv);
        return;
    }
    const double *gN = bg + (size_t)(N - 1) * gd;
    double *M = (double *)malloc(sizeof(double) * (size_t)N * dv);
    for (int i = 0; i < N; ++i)
        for (int j = 0; j < dv; ++j) {
            double acc = bu[(size_t)i * dv + j];
            for (int c = 0; c < dk; ++c) acc -= by[(size_t)i * dk + c] * Hb[(size_t)c * dv + j];
            M[(size_t)i * dv + j] = acc;
        }
    for (int c = 0; c < dk; ++c)
        for (int j = 0; j < dv; ++j) {
            double acc = exp(gN[per_key ? c : 0]) * Hb[(size_t)c * dv + j];
            for (int i = 0; i < N; ++i) {
                double e = exp(gN[per_key ? c : 0] - bg[(size_t)i * gd + (per_key ? c : 0)]);
                acc += e * bk[(size_t)i * dk + c] * M[(size_t)i * dv + j];
            }
            H[(size_t)c * dv + j] = acc;
        }
    free(M);
}

/* ------------------------------------------------------------------------ */
/* Whole runs over T tokens for one head                                    */
/* ------------------------------------------------------------------------ */

/*
 * Runs T tokens of the windowed scheme for one head ([abstract]: the state
 * is quantized once per window, at its end; [news ¶3]: 16-token windows).
 *
 *   use_codec = 1: the carried state is the codec (sq, r, s, idx, cv), in/out.
 *                  Each window starts from Hb = dequantize(codec); after the
 *                  window's last token the fp64 state is rounded to fp32 and
 *                  quantized (lqo_quantize).
 *   use_codec = 0: no quantization; the carried state is the fp64 H0, in/out.
 *                  With route 0 and any W this is the plain fp64 recurrence.
 *   route = 0: in-window tokens by the plain recurrence (lqo_step).
 *   route = 1: in-window tokens by the WY buffer (append/output/reconstruct).
 *   flush_tail = 1: a final partial window (T % W tokens) is also flushed.
 *
 * Token inputs are per token with strides: q + t*qs (dk floats), k + t*ks,
 * v + t*vs (dv floats), alpha + t*as (1 or dk floats), beta[t*bs].
 * o is [T][dv] fp64.  hf32_last (nullable) receives the fp32 state handed to
 * the last flush's rounding step.  Returns 0 or -1.
 */
int lqo_run_head(int dk, int dv, int per_key, int W, int C, int smooth,
                 int route, int use_codec, int flush_tail, int T,
                 const float *q, long qs, const float *k, long ks, const float *v, long vs,
                 const float *alpha, long as, const float *beta, long bs,
                 int8_t *sq, float *r, float *s, int32_t *idx, float *cv,
                 double *H0, double *o, float *hf32_last)
{
    if (dk <= 0 || dv <= 0 || W <= 0 || T < 0 || C < 0 || C > dk) return -1;
    int gd = per_key ? dk : 1;
    size_t dd = (size_t)dk * dv;
    double *Hb = (double *)malloc(sizeof(double) * dd);
    double *Hc = (double *)malloc(sizeof(double) * dd);
    float *hf = (float *)malloc(sizeof(float) * dd);
    double *bk = (double *)malloc(sizeof(double) * (size_t)W * dk);
    double *by = (double *)malloc(sizeof(double) * (size_t)W * dk);
    double *bu = (double *)malloc(sizeof(double) * (size_t)W * dv);
    double *bg = (double *)malloc(sizeof(double) * (size_t)W * gd);

    int t = 0;
    while (t < T) {
        int N = T - t < W ? T - t : W;
        if (use_codec) lqo_dequantize(dk, dv, C, sq, r, s, idx, cv, Hb);
        else memcpy(Hb, H0, sizeof(double) * dd);
        if (route == 0) memcpy(Hc, Hb, sizeof(double) * dd);
        for (int n = 0; n < N; ++n, ++t) {
            const float *qt = q + t * qs, *kt = k + t * ks, *vt = v + t * vs, *at = alpha + t * as;
            float bt = beta[t * bs];
            if (route == 0) {
                lqo_step(dk, dv, per_key, Hc, qt, kt, vt, at, bt, o + (size_t)t * dv);
            } else {
                lqo_wy_append(dk, dv, per_key, n, bk, by, bu, bg, kt, vt, at, bt);
                lqo_wy_output(dk, dv, per_key, n, Hb, bk, by, bu, bg, qt, o + (size_t)t * dv);
            }
        }
        if (route == 1) lqo_wy_reconstruct(dk, dv, per_key, N, Hb, bk, by, bu, bg, Hc);
        int boundary = (N == W) || flush_tail;
        if (use_codec) {
            if (boundary) {
                for (size_t e = 0; e < dd; ++e) hf[e] = (float)Hc[e];
                lqo_quantize(dk, dv, C, smooth, hf, sq, r, s, idx, cv);
                if (hf32_last) memcpy(hf32_last, hf, sizeof(float) * dd);
            }
        } else {
            memcpy(H0, Hc, sizeof(double) * dd);
        }
    }
    free(Hb); free(Hc); free(hf); free(bk); free(by); free(bu); free(bg);
    return 0;
}

/* Bytes of one head's stored state: int8 matrix, fp32 row and column scales,
 * C compensator rows (fp32) and their int32 row indices. */
long lqo_state_bytes(int dk, int dv, int C)
{
    return (long)dk * dv + 4L * dk + 4L * dv + (long)C * (4L * dv + 4L);
}
