/*
 * wkv_oracle.c -- plain float64 CPU oracle for the RWKV WKV time-mixing operator.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or load
 * this file: only the test suite, the package smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with the
 * HIP library; the two meet only on the seeded input tensors.
 *
 * Sources (the pages this restates; no listing is translated line by line):
 *   [Core]      RWKV architecture deep dive (youngju.dev), section
 *               "WKV mechanism: mathematical formulation / core computation":
 *               the closed-form weighted average that defines wkv_t.
 *   [Recurrent] same article, section "Recurrent formulation": running
 *               numerator/denominator updated with decay exp(-w).
 *   [LogSpace]  same article, section "Numerical stability via log-space
 *               computation": running max exponent kept beside the sums.
 *   [Parallel]  same article, section "Parallel training formulation":
 *               zero-initialised running sums, bonus only on the current token.
 *   [QuickStart] rwkv-architecture skill page, section "Quick start" (GPT mode
 *               vs RNN mode with the state carried between calls).
 *   [Block]     RWKV architecture deep dive, section "RWKV architecture
 *               overview", block figure: the time-mixing output is the
 *               receptance gate sigmoid(r_t) times wkv_t.
 *   [Shift]     same article, section "Token shift": the input of each
 *               projection mixes x_t with x_{t-1} by a per-channel weight mu.
 *   [States]    rwkv-architecture skill page, "Advanced topics": the
 *               time-mixing sublayer carries att_x_prev (the last x) between
 *               calls, beside the WKV state.
 *
 * Conventions (all arrays row-major, float64):
 *   k, v, y, dy, dk, dv : [B][T][C]   (channel fastest)
 *   w, u                : [C]         w = exp(decay) is the per-channel decay
 *                                      rate (the pages require w > 0; the
 *                                      oracle accepts any finite w)
 *   state               : [3][B][C]   planes a, b, o.  The true running sums
 *                                      are A = a*exp(o) and Bden = b*exp(o).
 *                                      The empty state is a = b = 0, o = -inf.
 *   Token index t runs 0..T-1 here; the pages count from 1.
 *
 * Parity status of each function (pins live in the test suite):
 *   wkvo_forward_brute     pinned (library softmax limits, geometric series,
 *                          the pages' two recurrences, invariants)
 *   wkvo_forward_scan      pinned (brute force, chunking identity)
 *   wkvo_backward_brute    pinned (central finite differences, invariants)
 *   wkvo_backward_scan     pinned (brute-force backward, finite differences)
 *   wkvo_backward_state    pinned (central finite differences of a loss that
 *                          includes the carried states, reduction to
 *                          wkvo_backward_brute, chunking identity)
 *   wkvo_gate              pinned (library logistic function, limits, r = 0)
 *   wkvo_gate_backward     pinned (central finite differences of wkvo_gate in
 *                          y and in r, saturated tails)
 *   wkvo_token_shift       pinned (hand-computed fixture, mu = 0 and mu = 1
 *                          limits, chunking identity)
 *   wkvo_token_shift_backward  pinned (central finite differences of
 *                          wkvo_token_shift, per element on a small case and
 *                          along random directions on a larger one; mu = 0
 *                          and mu = 1 limits)
 *   wkvo_backward_magnitude  pinned (the same sums of absolute terms written
 *                          out pair by pair from the closed form on small
 *                          inputs; never below |dw|, |du| of
 *                          wkvo_backward_state; the closed form of one token
 *                          from the empty state, where du vanishes and its
 *                          parts are |dy v| each).  Test tolerances only.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

#define IDX(b, t, c) (((int64_t)(b) * T + (t)) * C + (c))
#define SIDX(p, b, c) (((int64_t)(p) * B + (b)) * C + (c))

static double dmax(double x, double y) { return x > y ? x : y; }

/* ------------------------------------------------------------------------ */
/* Forward, O(T^2): the closed form of [Core], written out per output token.  */
/* ------------------------------------------------------------------------ */
/*
 * [Core] defines, for token t (1-based on the page),
 *     wkv_t = ( sum_{i<t} e^{-(t-1-i)w + k_i} v_i + e^{u+k_t} v_t )
 *           / ( sum_{i<t} e^{-(t-1-i)w + k_i}     + e^{u+k_t}     ).
 * A carried state ([QuickStart]: the state returned by one call is passed to
 * the next) adds the decayed sums of all earlier tokens, e^{-(t-1)w} A0 and
 * e^{-(t-1)w} B0, to the numerator and denominator.  With 0-based t the decay
 * distance of past token i is (t-1-i) and of the state it is t.
 * Every exponent is shifted by the largest one before exponentiating, which
 * changes nothing in the ratio.
 */
static void forward_brute_lane(int64_t T, double w, double u, const double *k,
                               const double *v, int64_t stride, double a0,
                               double b0, double o0, double *y, double *s_out) {
    double *x = (double *)malloc(sizeof(double) * (size_t)(T + 1));
    double *val = (double *)malloc(sizeof(double) * (size_t)(T + 1));
    int has_state = (b0 > 0.0);
    for (int64_t t = 0; t < T; ++t) {
        int64_t n = 0;
        for (int64_t i = 0; i < t; ++i) {
            x[n] = k[i * stride] - (double)(t - 1 - i) * w;
            val[n] = v[i * stride];
            ++n;
        }
        x[n] = u + k[t * stride];
        val[n] = v[t * stride];
        ++n;
        double m = x[0];
        for (int64_t j = 1; j < n; ++j) m = dmax(m, x[j]);
        double xs = 0.0;
        if (has_state) {
            xs = o0 - (double)t * w;
            m = dmax(m, xs);
        }
        double num = 0.0, den = 0.0;
        for (int64_t j = 0; j < n; ++j) {
            double e = exp(x[j] - m);
            num += e * val[j];
            den += e;
        }
        if (has_state) {
            double e = exp(xs - m);
            num += e * a0;
            den += e * b0;
        }
        y[t * stride] = num / den;
    }
    if (s_out) {
        /* State after the last token: A_T = e^{-Tw} A0 + sum_{i<T} e^{k_i-(T-1-i)w} v_i. */
        double m = -INFINITY;
        for (int64_t i = 0; i < T; ++i) m = dmax(m, k[i * stride] - (double)(T - 1 - i) * w);
        double xs = o0 - (double)T * w;
        if (has_state) m = dmax(m, xs);
        double a = 0.0, b = 0.0;
        if (m == -INFINITY) {
            s_out[0] = 0.0;
            s_out[1] = 0.0;
            s_out[2] = -INFINITY;
        } else {
            for (int64_t i = 0; i < T; ++i) {
                double e = exp(k[i * stride] - (double)(T - 1 - i) * w - m);
                a += e * v[i * stride];
                b += e;
            }
            if (has_state) {
                double e = exp(xs - m);
                a += e * a0;
                b += e * b0;
            }
            s_out[0] = a;
            s_out[1] = b;
            s_out[2] = m;
        }
    }
    free(x);
    free(val);
}

/* ------------------------------------------------------------------------ */
/* Forward, O(T): the recurrence of [Recurrent] in the log-space form of      */
/* [LogSpace], with the output read as in [Core] and [Parallel].             */
/* ------------------------------------------------------------------------ */
/*
 * The state (a, b, o) stands for the sums A = a e^o, B = b e^o of all tokens
 * seen so far, each decayed by e^{-w} per later token.
 *   output  : wkv_t = (A + e^{u+k_t} v_t) / (B + e^{u+k_t})
 *             -- the past sums enter undecayed, which is the closed form of
 *             [Core] and the loop of [Parallel] (the "Recurrent formulation"
 *             section multiplies the past by one more e^{-w} here; that form
 *             equals this one with the bonus u replaced by u + w).
 *   update  : A <- e^{-w} A + e^{k_t} v_t,  B <- e^{-w} B + e^{k_t}
 *             ([Recurrent]); u does not enter the state.
 * Both steps factor out the larger exponent first ([LogSpace]).
 */
static void forward_scan_lane(int64_t T, double w, double u, const double *k,
                              const double *v, int64_t stride, double *a_,
                              double *b_, double *o_, double *y) {
    double a = *a_, b = *b_, o = *o_;
    for (int64_t t = 0; t < T; ++t) {
        double kt = k[t * stride], vt = v[t * stride];
        double p = dmax(o, u + kt);
        double ep = exp(o - p), ec = exp(u + kt - p);
        y[t * stride] = (ep * a + ec * vt) / (ep * b + ec);
        double q = dmax(o - w, kt);
        double fp = exp(o - w - q), fc = exp(kt - q);
        a = fp * a + fc * vt;
        b = fp * b + fc;
        o = q;
    }
    *a_ = a;
    *b_ = b;
    *o_ = o;
}

int wkvo_forward_brute(int64_t B, int64_t T, int64_t C, const double *w,
                       const double *u, const double *k, const double *v,
                       const double *s_in, double *y, double *s_out) {
    if (B < 0 || T < 0 || C < 0) return 1;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t c = 0; c < C; ++c) {
            double a0 = 0.0, b0 = 0.0, o0 = -INFINITY;
            if (s_in) {
                a0 = s_in[SIDX(0, b, c)];
                b0 = s_in[SIDX(1, b, c)];
                o0 = s_in[SIDX(2, b, c)];
            }
            double so[3];
            forward_brute_lane(T, w[c], u[c], k + IDX(b, 0, c), v + IDX(b, 0, c), C, a0, b0,
                               o0, y + IDX(b, 0, c), so);
            if (s_out) {
                s_out[SIDX(0, b, c)] = so[0];
                s_out[SIDX(1, b, c)] = so[1];
                s_out[SIDX(2, b, c)] = so[2];
            }
        }
    return 0;
}

/* Lane range [l0, l1) of the B*C lanes; lanes are independent. */
typedef struct {
    int64_t B, T, C, l0, l1;
    const double *w, *u, *k, *v, *s_in;
    double *y, *s_out;
} scan_job;

static void *scan_job_run(void *arg) {
    scan_job *j = (scan_job *)arg;
    int64_t B = j->B, T = j->T, C = j->C;
    for (int64_t lane = j->l0; lane < j->l1; ++lane) {
        int64_t b = lane / C, c = lane % C;
        double a = 0.0, bb = 0.0, o = -INFINITY;
        if (j->s_in) {
            a = j->s_in[SIDX(0, b, c)];
            bb = j->s_in[SIDX(1, b, c)];
            o = j->s_in[SIDX(2, b, c)];
        }
        forward_scan_lane(T, j->w[c], j->u[c], j->k + IDX(b, 0, c), j->v + IDX(b, 0, c), C, &a,
                          &bb, &o, j->y + IDX(b, 0, c));
        if (j->s_out) {
            j->s_out[SIDX(0, b, c)] = a;
            j->s_out[SIDX(1, b, c)] = bb;
            j->s_out[SIDX(2, b, c)] = o;
        }
    }
    return NULL;
}

/* nthreads <= 1 runs on the calling thread.  Threads split lanes only. */
int wkvo_forward_scan(int64_t B, int64_t T, int64_t C, const double *w, const double *u,
                      const double *k, const double *v, const double *s_in, double *y,
                      double *s_out, int nthreads) {
    if (B < 0 || T < 0 || C < 0) return 1;
    int64_t lanes = B * C;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > lanes) nthreads = lanes > 0 ? (int)lanes : 1;
    scan_job jobs[256];
    pthread_t th[256];
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = (scan_job){B, T, C, lanes * i / nthreads, lanes * (i + 1) / nthreads,
                             w, u, k, v, s_in, y, s_out};
    }
    if (nthreads == 1) {
        scan_job_run(&jobs[0]);
        return 0;
    }
    for (int i = 0; i < nthreads; ++i)
        if (pthread_create(&th[i], NULL, scan_job_run, &jobs[i]) != 0) return 2;
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Backward.  The pages give no backward; these are the derivatives of the    */
/* closed form of [Core] (empty initial state), with L = sum_t dy_t * y_t.    */
/* ------------------------------------------------------------------------ */
/*
 * With p_{t,i} = E_{t,i} / D_t (the weight of token i in output t; the weights
 * of one output sum to 1) and g_t = dy_t:
 *   dv_i = sum_{t>=i} g_t p_{t,i}
 *   dk_i = sum_{t>=i} g_t p_{t,i} (v_i - y_t)
 *   du   = sum_{b,t}   g_t p_{t,t} (v_t - y_t)
 *   dw   = -sum_{b,t} sum_{i<t} (t-1-i) g_t p_{t,i} (v_i - y_t)
 * dw and du are [C], summed over the batch and the tokens.
 */
int wkvo_backward_brute(int64_t B, int64_t T, int64_t C, const double *w, const double *u,
                        const double *k, const double *v, const double *dy, double *dk,
                        double *dv, double *dw, double *du) {
    if (B < 0 || T < 0 || C < 0) return 1;
    double *x = (double *)malloc(sizeof(double) * (size_t)(T + 1));
    for (int64_t c = 0; c < C; ++c) {
        dw[c] = 0.0;
        du[c] = 0.0;
    }
    for (int64_t b = 0; b < B; ++b)
        for (int64_t c = 0; c < C; ++c) {
            const double *kk = k + IDX(b, 0, c), *vv = v + IDX(b, 0, c), *gg = dy + IDX(b, 0, c);
            double *dkk = dk + IDX(b, 0, c), *dvv = dv + IDX(b, 0, c);
            for (int64_t i = 0; i < T; ++i) {
                dkk[i * C] = 0.0;
                dvv[i * C] = 0.0;
            }
            for (int64_t t = 0; t < T; ++t) {
                /* exponents of output t: x[i] for past tokens, x[t] with the bonus */
                for (int64_t i = 0; i < t; ++i) x[i] = kk[i * C] - (double)(t - 1 - i) * w[c];
                x[t] = u[c] + kk[t * C];
                double m = x[0];
                for (int64_t i = 1; i <= t; ++i) m = dmax(m, x[i]);
                double den = 0.0, num = 0.0;
                for (int64_t i = 0; i <= t; ++i) {
                    double e = exp(x[i] - m);
                    den += e;
                    num += e * vv[i * C];
                }
                double yt = num / den, g = gg[t * C];
                for (int64_t i = 0; i <= t; ++i) {
                    double p = exp(x[i] - m) / den;
                    dvv[i * C] += g * p;
                    dkk[i * C] += g * p * (vv[i * C] - yt);
                    if (i == t)
                        du[c] += g * p * (vv[i * C] - yt);
                    else
                        dw[c] -= (double)(t - 1 - i) * g * p * (vv[i * C] - yt);
                }
            }
        }
    free(x);
    return 0;
}

/*
 * O(T) reverse scan of the same derivatives.  For token i define the sums over
 * later outputs t > i (l_t = ln D_t):
 *   R_i  = sum_{t>i} g_t e^{-(t-1-i)w - l_t}         S_i  = same with g_t y_t
 *   R'_i = sum_{t>i} (t-1-i) g_t e^{-(t-1-i)w - l_t}  S'_i = same with g_t y_t
 * so that, since p_{t,i} = e^{k_i} e^{-(t-1-i)w - l_t} for t > i,
 *   dv_i = p_{i,i} g_i + e^{k_i} R_i
 *   dk_i = p_{i,i} g_i (v_i - y_i) + e^{k_i} (v_i R_i - S_i)
 *   dw  -= e^{k_i} (v_i R'_i - S'_i),   du += p_{i,i} g_i (v_i - y_i)
 * and stepping from i to i-1:
 *   R_{i-1} = g_i e^{-l_i} + e^{-w} R_i,   R'_{i-1} = e^{-w} (R'_i + R_i).
 * The four sums are held as R = Rs * e^{rho} with rho_{i-1} = max(-l_i, rho_i - w),
 * which keeps e^{k_i + rho_i} = max_t p_{t,i} <= 1 and every stored value bounded.
 */
typedef struct {
    int64_t B, T, C, l0, l1;
    const double *w, *u, *k, *v, *dy;
    double *dk, *dv, *dw_lane, *du_lane;
} bwd_job;

static void backward_scan_lane(int64_t T, double w, double u, const double *k, const double *v,
                               const double *g, int64_t stride, double *dk, double *dv,
                               double *dw_out, double *du_out, double *ell, double *yy) {
    /* forward recompute of y_t and l_t = ln D_t */
    double a = 0.0, b = 0.0, o = -INFINITY;
    for (int64_t t = 0; t < T; ++t) {
        double kt = k[t * stride], vt = v[t * stride];
        double p = dmax(o, u + kt);
        double ep = exp(o - p), ec = exp(u + kt - p);
        double den = ep * b + ec;
        yy[t] = (ep * a + ec * vt) / den;
        ell[t] = p + log(den);
        double q = dmax(o - w, kt);
        double fp = exp(o - w - q), fc = exp(kt - q);
        a = fp * a + fc * vt;
        b = fp * b + fc;
        o = q;
    }
    double Rs = 0.0, Ss = 0.0, R1 = 0.0, S1 = 0.0, rho = -INFINITY;
    double dw = 0.0, du = 0.0;
    for (int64_t i = T - 1; i >= 0; --i) {
        double ki = k[i * stride], vi = v[i * stride], gi = g[i * stride];
        double pii = exp(u + ki - ell[i]);
        double ek = exp(ki + rho);
        double own = pii * gi;
        dv[i * stride] = own + ek * Rs;
        dk[i * stride] = own * (vi - yy[i]) + ek * (vi * Rs - Ss);
        dw -= ek * (vi * R1 - S1);
        du += own * (vi - yy[i]);
        /* step the sums from "after i" to "after i-1" */
        double nrho = dmax(-ell[i], rho - w);
        double fo = exp(rho - w - nrho), fn = exp(-ell[i] - nrho);
        double nR1 = fo * (R1 + Rs), nS1 = fo * (S1 + Ss);
        Rs = fo * Rs + fn * gi;
        Ss = fo * Ss + fn * gi * yy[i];
        R1 = nR1;
        S1 = nS1;
        rho = nrho;
    }
    *dw_out = dw;
    *du_out = du;
}

static void *bwd_job_run(void *arg) {
    bwd_job *j = (bwd_job *)arg;
    int64_t T = j->T, C = j->C;
    double *ell = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    double *yy = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    for (int64_t lane = j->l0; lane < j->l1; ++lane) {
        int64_t b = lane / C, c = lane % C;
        backward_scan_lane(T, j->w[c], j->u[c], j->k + IDX(b, 0, c), j->v + IDX(b, 0, c),
                           j->dy + IDX(b, 0, c), C, j->dk + IDX(b, 0, c), j->dv + IDX(b, 0, c),
                           &j->dw_lane[lane], &j->du_lane[lane], ell, yy);
    }
    free(ell);
    free(yy);
    return NULL;
}

int wkvo_backward_scan(int64_t B, int64_t T, int64_t C, const double *w, const double *u,
                       const double *k, const double *v, const double *dy, double *dk,
                       double *dv, double *dw, double *du, int nthreads) {
    if (B < 0 || T < 0 || C < 0) return 1;
    int64_t lanes = B * C;
    double *dw_lane = (double *)calloc((size_t)(lanes > 0 ? lanes : 1), sizeof(double));
    double *du_lane = (double *)calloc((size_t)(lanes > 0 ? lanes : 1), sizeof(double));
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > lanes) nthreads = lanes > 0 ? (int)lanes : 1;
    bwd_job jobs[256];
    pthread_t th[256];
    for (int i = 0; i < nthreads; ++i)
        jobs[i] = (bwd_job){B, T, C, lanes * i / nthreads, lanes * (i + 1) / nthreads,
                            w, u, k, v, dy, dk, dv, dw_lane, du_lane};
    if (nthreads == 1) {
        bwd_job_run(&jobs[0]);
    } else {
        for (int i = 0; i < nthreads; ++i)
            if (pthread_create(&th[i], NULL, bwd_job_run, &jobs[i]) != 0) return 2;
        for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    }
    /* sum the per-lane parts over the batch in a fixed order */
    for (int64_t c = 0; c < C; ++c) {
        dw[c] = 0.0;
        du[c] = 0.0;
        for (int64_t b = 0; b < B; ++b) {
            dw[c] += dw_lane[b * C + c];
            du[c] += du_lane[b * C + c];
        }
    }
    free(dw_lane);
    free(du_lane);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Receptance gate [Block]: out = sigmoid(r) * y, elementwise over n values.  */
/* ------------------------------------------------------------------------ */
/*
 * sigmoid(r) = 1 / (1 + e^{-r}).  For r < 0 the same value is written as
 * e^{r} / (1 + e^{r}) so that e^{-r} never overflows; both forms are the
 * logistic function.
 */
int wkvo_gate(int64_t n, const double *y, const double *r, double *out) {
    if (n < 0 || (n > 0 && (!y || !r || !out))) return 1;
    for (int64_t i = 0; i < n; ++i) {
        double s;
        if (r[i] >= 0.0) {
            s = 1.0 / (1.0 + exp(-r[i]));
        } else {
            const double e = exp(r[i]);
            s = e / (1.0 + e);
        }
        out[i] = s * y[i];
    }
    return 0;
}

/*
 * Backward of [Block]'s gate, out = s y with s = sigmoid(r): for the upstream
 * gradient d of out, the gradient reaching the WKV output is g = d s and the
 * gradient of the receptance is dr = d y s (1 - s), s (1 - s) being the
 * derivative of the logistic function.  The pages state no backward; this is
 * the chain rule on wkvo_gate.
 */
int wkvo_gate_backward(int64_t n, const double *y, const double *r, const double *d,
                       double *g, double *dr) {
    if (n < 0 || (n > 0 && (!y || !r || !d || !g || !dr))) return 1;
    for (int64_t i = 0; i < n; ++i) {
        double s, sc; /* sigmoid(r) and 1 - sigmoid(r), each without cancellation */
        if (r[i] >= 0.0) {
            const double e = exp(-r[i]);
            s = 1.0 / (1.0 + e);
            sc = e / (1.0 + e);
        } else {
            const double e = exp(r[i]);
            s = e / (1.0 + e);
            sc = 1.0 / (1.0 + e);
        }
        g[i] = d[i] * s;
        dr[i] = d[i] * y[i] * s * sc;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Token shift [Shift], with the carried last token of [States].              */
/* ------------------------------------------------------------------------ */
/*
 * For each of M mixes (one weight vector mu[m][C] per projection input):
 *     out[m][b][t][c] = mu[m][c] * x[b][t][c] + (1 - mu[m][c]) * x[b][t-1][c]
 * where x[b][-1][c] is x_prev[b][c], the last token of the previous call, or 0
 * for a fresh sequence (x_prev == NULL).  x_prev_out[b][c] receives the last
 * token of this call, x[b][T-1][c], or x_prev (0 when fresh) when T == 0.
 */
/*
 * Backward of the token shift [Shift] with its carried token [States].  For
 * the upstream gradients d_out [M][B][T][C] of the M mixes and d_xpo [B][C] of
 * the carried token handed on (NULL: none), the chain rule on wkvo_token_shift
 * gives, token t feeding mix t with weight mu and mix t + 1 with 1 - mu:
 *   dx[b][t][c]   = sum_m mu_m[c] d_out[m][b][t][c]
 *                 + sum_m (1 - mu_m[c]) d_out[m][b][t+1][c]     (t + 1 < T)
 *                 + d_xpo[b][c]                                (t = T - 1)
 *   dx_prev[b][c] = sum_m (1 - mu_m[c]) d_out[m][b][0][c]       (T > 0)
 *                 = d_xpo[b][c]                                (T = 0)
 *   dmu[m][c]     = sum_{b,t} d_out[m][b][t][c] (x[b][t][c] - x[b][t-1][c])
 * with x[b][-1] = x_prev (zeros when NULL).  The pages state no backward.
 * dx_prev may be NULL (not wanted).
 */
int wkvo_token_shift_backward(int64_t B, int64_t T, int64_t C, int64_t M, const double *mu,
                              const double *x, const double *x_prev, const double *d_out,
                              const double *d_xpo, double *dx, double *dx_prev, double *dmu) {
    if (B < 0 || T < 0 || C < 0 || M < 0) return 1;
    if (B * T * C > 0 && (!x || !dx || (M > 0 && (!mu || !d_out)))) return 1;
    if (M * C > 0 && !dmu) return 1;
    const int64_t plane = B * T * C;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t c = 0; c < C; ++c) dmu[m * C + c] = 0.0;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t t = 0; t < T; ++t)
            for (int64_t c = 0; c < C; ++c) {
                double g = (t == T - 1 && d_xpo) ? d_xpo[b * C + c] : 0.0;
                const double prev =
                    t > 0 ? x[IDX(b, t - 1, c)] : (x_prev ? x_prev[b * C + c] : 0.0);
                for (int64_t m = 0; m < M; ++m) {
                    const double mu_ = mu[m * C + c];
                    const double d = d_out[m * plane + IDX(b, t, c)];
                    g += mu_ * d;
                    if (t + 1 < T) g += (1.0 - mu_) * d_out[m * plane + IDX(b, t + 1, c)];
                    dmu[m * C + c] += d * (x[IDX(b, t, c)] - prev);
                }
                dx[IDX(b, t, c)] = g;
            }
    if (dx_prev)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t c = 0; c < C; ++c) {
                double g = 0.0;
                if (T > 0) {
                    for (int64_t m = 0; m < M; ++m)
                        g += (1.0 - mu[m * C + c]) * d_out[m * plane + IDX(b, 0, c)];
                } else if (d_xpo) {
                    g = d_xpo[b * C + c];
                }
                dx_prev[b * C + c] = g;
            }
    return 0;
}

int wkvo_token_shift(int64_t B, int64_t T, int64_t C, int64_t M, const double *mu,
                     const double *x, const double *x_prev, double *out,
                     double *x_prev_out) {
    if (B < 0 || T < 0 || C < 0 || M < 0) return 1;
    if (B * T * C > 0 && (!x || (M > 0 && (!mu || !out)))) return 1;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t t = 0; t < T; ++t)
                for (int64_t c = 0; c < C; ++c) {
                    const double cur = x[IDX(b, t, c)];
                    double prev;
                    if (t > 0)
                        prev = x[IDX(b, t - 1, c)];
                    else
                        prev = x_prev ? x_prev[b * C + c] : 0.0;
                    const double g = mu[m * C + c];
                    out[(int64_t)m * B * T * C + IDX(b, t, c)] = g * cur + (1.0 - g) * prev;
                }
    if (x_prev_out)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t c = 0; c < C; ++c) {
                double last;
                if (T > 0)
                    last = x[IDX(b, T - 1, c)];
                else
                    last = x_prev ? x_prev[b * C + c] : 0.0;
                x_prev_out[b * C + c] = last;
            }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Backward with a carried state ([QuickStart]: RNN mode over chunks), O(T^2) */
/* ------------------------------------------------------------------------ */
/*
 * Derivatives of the closed form of [Core] extended by the state term (as in
 * forward_brute_lane), for the loss
 *     L = sum_t g_t y_t + gA A_T + gB B_T,
 * where A_T, B_T are the true sums after the last token and (gA, gB) their
 * upstream gradient.  The upstream gradient arrives in the coordinates of the
 * state the forward handed on, (a_T, b_T, o_T): since a consumer sees only
 * A_T = a_T e^{o_T} and B_T = b_T e^{o_T}, gA = g_aT e^{-o_T} and
 * gB = g_bT e^{-o_T} (the o-plane of the gradient is then g_aT a_T + g_bT b_T
 * and carries nothing more; it is not read).
 * With E_{t,i} the weight of token i in output t (e^{k_i-(t-1-i)w}, or
 * e^{u+k_t} for i = t), the state's weight e^{-t w} (numerator A0, denominator
 * B0), D_t the denominator and p = E / D:
 *   dv_i = sum_{t>=i} g_t p_{t,i}             + gA e^{k_i-(T-1-i)w}
 *   dk_i = sum_{t>=i} g_t p_{t,i} (v_i - y_t) + e^{k_i-(T-1-i)w} (gA v_i + gB)
 *   du   = sum_t g_t p_{t,t} (v_t - y_t)
 *   dw   = -sum_t sum_{i<t} (t-1-i) g_t p_{t,i} (v_i - y_t)
 *          -sum_t t g_t e^{-t w} (A0 - y_t B0) / D_t
 *          -sum_{i<T} (T-1-i) e^{k_i-(T-1-i)w} (gA v_i + gB) - T e^{-T w} (gA A0 + gB B0)
 *   dA0  = sum_t g_t e^{-t w} / D_t + gA e^{-T w}
 *   dB0  = -sum_t g_t y_t e^{-t w} / D_t + gB e^{-T w}
 * and in state coordinates (a0, b0, o0): d_a0 = dA0 e^{o0}, d_b0 = dB0 e^{o0},
 * d_o0 = dA0 A0 + dB0 B0.  Every exponential is formed with its shift applied
 * inside the exponent.  state_in NULL is the empty state; d_state_out NULL is
 * no upstream gradient (state_out is then not read).  dw, du are summed over
 * the batch.
 */
int wkvo_backward_state(int64_t B, int64_t T, int64_t C, const double *w, const double *u,
                        const double *k, const double *v, const double *dy,
                        const double *state_in, const double *state_out,
                        const double *d_state_out, double *dk, double *dv, double *dw,
                        double *du, double *d_state_in) {
    if (B < 0 || T < 0 || C < 0) return 1;
    if (d_state_out && !state_out) return 1;
    double *x = (double *)malloc(sizeof(double) * (size_t)(T + 2));
    for (int64_t c = 0; c < C; ++c) {
        dw[c] = 0.0;
        du[c] = 0.0;
    }
    for (int64_t b = 0; b < B; ++b)
        for (int64_t c = 0; c < C; ++c) {
            const double *kk = k + IDX(b, 0, c), *vv = v + IDX(b, 0, c), *gg = dy + IDX(b, 0, c);
            double *dkk = dk + IDX(b, 0, c), *dvv = dv + IDX(b, 0, c);
            const double wc = w[c];
            double a0 = 0.0, b0 = 0.0, o0 = -INFINITY;
            if (state_in) {
                a0 = state_in[SIDX(0, b, c)];
                b0 = state_in[SIDX(1, b, c)];
                o0 = state_in[SIDX(2, b, c)];
            }
            const int has_state = b0 > 0.0;
            /* upstream gradient: gA = gaT e^{-oT}, kept as (gaT, gbT, -oT) */
            double gaT = 0.0, gbT = 0.0, moT = 0.0;
            if (d_state_out) {
                gaT = d_state_out[SIDX(0, b, c)];
                gbT = d_state_out[SIDX(1, b, c)];
                moT = -state_out[SIDX(2, b, c)];
            }
            double dA0s = 0.0, dB0s = 0.0;  /* dA0, dB0 times e^{o0} */
            for (int64_t i = 0; i < T; ++i) {
                dkk[i * C] = 0.0;
                dvv[i * C] = 0.0;
            }
            for (int64_t t = 0; t < T; ++t) {
                for (int64_t i = 0; i < t; ++i) x[i] = kk[i * C] - (double)(t - 1 - i) * wc;
                x[t] = u[c] + kk[t * C];
                double m = x[t];
                for (int64_t i = 0; i < t; ++i) m = dmax(m, x[i]);
                const double xs = has_state ? o0 - (double)t * wc : -INFINITY;
                if (has_state) m = dmax(m, xs);
                double den = 0.0, num = 0.0;
                for (int64_t i = 0; i <= t; ++i) {
                    const double e = exp(x[i] - m);
                    den += e;
                    num += e * vv[i * C];
                }
                if (has_state) {
                    const double e = exp(xs - m);
                    den += e * b0;
                    num += e * a0;
                }
                const double yt = num / den, g = gg[t * C];
                for (int64_t i = 0; i <= t; ++i) {
                    const double p = exp(x[i] - m) / den;
                    dvv[i * C] += g * p;
                    dkk[i * C] += g * p * (vv[i * C] - yt);
                    if (i == t)
                        du[c] += g * p * (vv[i * C] - yt);
                    else
                        dw[c] -= (double)(t - 1 - i) * g * p * (vv[i * C] - yt);
                }
                if (has_state) {
                    /* e^{-t w} e^{o0} / D_t */
                    const double ps = exp(xs - m) / den;
                    dA0s += g * ps;
                    dB0s -= g * yt * ps;
                    dw[c] -= (double)t * g * ps * (a0 - yt * b0);
                }
            }
            if (d_state_out) {
                for (int64_t i = 0; i < T; ++i) {
                    const double e = exp(kk[i * C] - (double)(T - 1 - i) * wc + moT);
                    const double h = gaT * vv[i * C] + gbT;
                    dvv[i * C] += gaT * e;
                    dkk[i * C] += e * h;
                    dw[c] -= (double)(T - 1 - i) * e * h;
                }
                if (has_state) {
                    const double e = exp(o0 - (double)T * wc + moT);  /* e^{-Tw} e^{o0} e^{-oT} */
                    dA0s += gaT * e;
                    dB0s += gbT * e;
                    dw[c] -= (double)T * e * (gaT * a0 + gbT * b0);
                }
            }
            if (d_state_in) {
                d_state_in[SIDX(0, b, c)] = dA0s;
                d_state_in[SIDX(1, b, c)] = dB0s;
                d_state_in[SIDX(2, b, c)] = dA0s * a0 + dB0s * b0;
            }
        }
    free(x);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Magnitudes of the terms of dw and du (a scale for round-off bounds)        */
/* ------------------------------------------------------------------------ */
/*
 * dw and du of wkvo_backward_state are sums of many signed terms that can
 * cancel.  A float32 computation of such a sum errs relative to the sum of the
 * terms' absolute values, not relative to the result; this returns, per
 * channel (summed over the batch like dw, du),
 *   mdu = sum_t |g_t| p_{t,t} (|v_t| + |y_t|)
 *   mdw = sum_t sum_{i<t} (t-1-i) |g_t| p_{t,i} (|v_i| + |y_t|)
 *       + sum_t t |g_t| e^{-t w} (|A0| + |y_t| B0) / D_t
 *       + sum_{i<T} (T-1-i) e^{k_i-(T-1-i)w} (|gA v_i| + |gB|) + T e^{-T w} (|gA A0| + |gB| B0)
 * Each term of either sum is a difference whose two parts are counted
 * separately (|v - y| <= |v| + |y|): float32 forms the difference from parts
 * that each carry rounding, so where v_t and y_t nearly agree (a token that
 * holds almost all of its weight) the difference's error is relative to the
 * parts.  This also lets the pair sum run as an O(T) reverse scan.  With
 * l_t = ln D_t and P_{t,i} = e^{k_i - (t-1-i) w - l_t} = p_{t,i}, the pair sum is
 *   sum_i e^{k_i} (|v_i| R1_i + S1_i),  R1_i = sum_{t>i} (t-1-i) |g_t| e^{-(t-1-i)w - l_t},
 * S1_i the same with |g_t y_t|, and R1_{i-1} = e^{-w} (R1_i + R0_i),
 * R0_{i-1} = |g_i| e^{-l_i} + e^{-w} R0_i.  Long double keeps every such
 * exponential in range for the test inputs (|k|, |l| up to thousands).  Same
 * arguments as wkvo_backward_state; outputs mdw, mdu [C].
 */
struct mag_job {
    int64_t B, T, C, c0, c1;
    const double *w, *u, *k, *v, *dy, *state_in, *state_out, *d_state_out;
    double *mdw, *mdu;
};

static void *mag_job_run(void *arg) {
    const struct mag_job *jb = (const struct mag_job *)arg;
    const int64_t B = jb->B, T = jb->T, C = jb->C;
    const double *w = jb->w, *u = jb->u, *k = jb->k, *v = jb->v, *dy = jb->dy;
    const double *state_in = jb->state_in, *state_out = jb->state_out;
    const double *d_state_out = jb->d_state_out;
    double *mdw = jb->mdw, *mdu = jb->mdu;
    long double *lt = (long double *)malloc(sizeof(long double) * (size_t)(T + 1));
    long double *yt = (long double *)malloc(sizeof(long double) * (size_t)(T + 1));
    for (int64_t c = jb->c0; c < jb->c1; ++c) {
        mdw[c] = 0.0;
        mdu[c] = 0.0;
    }
    for (int64_t b = 0; b < B; ++b)
        for (int64_t c = jb->c0; c < jb->c1; ++c) {
            const long double wc = w[c], uc = u[c];
            long double a0 = 0.0L, b0 = 0.0L, o0 = -INFINITY;
            if (state_in) {
                a0 = state_in[SIDX(0, b, c)];
                b0 = state_in[SIDX(1, b, c)];
                o0 = state_in[SIDX(2, b, c)];
            }
            const int has_state = b0 > 0.0L;
            /* forward: the past sums (with the state) as A = an e^{lb}, B = e^{lb} bn */
            long double lb = has_state ? o0 : -INFINITY;  /* log of the past denominator frame */
            long double an = has_state ? a0 : 0.0L, bn = has_state ? b0 : 0.0L;
            long double mu_sum = 0.0L;
            for (int64_t t = 0; t < T; ++t) {
                const long double kt = k[IDX(b, t, c)], vt = v[IDX(b, t, c)];
                const long double xb = uc + kt;
                const long double m = lb > xb ? lb : xb;
                const long double ep = bn > 0.0L ? expl(lb - m) : 0.0L, eb = expl(xb - m);
                const long double den = ep * bn + eb;
                lt[t] = m + logl(den);
                yt[t] = (ep * an + eb * vt) / den;
                const long double g = fabsl((long double)dy[IDX(b, t, c)]);
                mu_sum += g * (eb / den) * (fabsl(vt) + fabsl(yt[t]));
                /* fold token t, decaying the past by e^{-w} */
                const long double lp = lb - wc;
                const long double m2 = lp > kt ? lp : kt;
                const long double f1 = bn > 0.0L ? expl(lp - m2) : 0.0L, f2 = expl(kt - m2);
                an = f1 * an + f2 * vt;
                bn = f1 * bn + f2;
                lb = m2;
            }
            long double acc = 0.0L;
            /* pairs (t, i < t), by the reverse scan */
            long double R0 = 0.0L, R1 = 0.0L, S0 = 0.0L, S1 = 0.0L;
            const long double dec = expl(-wc);
            for (int64_t i = T - 1; i >= 0; --i) {
                acc += expl((long double)k[IDX(b, i, c)]) *
                       (fabsl((long double)v[IDX(b, i, c)]) * R1 + S1);
                const long double g = fabsl((long double)dy[IDX(b, i, c)]);
                const long double e = expl(-lt[i]);
                R1 = dec * (R1 + R0);
                S1 = dec * (S1 + S0);
                R0 = g * e + dec * R0;
                S0 = g * fabsl(yt[i]) * e + dec * S0;
            }
            if (has_state)
                for (int64_t t = 0; t < T; ++t)
                    acc += (long double)t * fabsl((long double)dy[IDX(b, t, c)]) *
                           expl(-(long double)t * wc + o0 - lt[t]) *
                           (fabsl(a0) + fabsl(yt[t]) * b0);
            if (d_state_out) {
                const long double gaT = d_state_out[SIDX(0, b, c)];
                const long double gbT = d_state_out[SIDX(1, b, c)];
                const long double moT = -(long double)state_out[SIDX(2, b, c)];
                for (int64_t i = 0; i < T; ++i)
                    acc += (long double)(T - 1 - i) *
                           expl((long double)k[IDX(b, i, c)] - (long double)(T - 1 - i) * wc + moT) *
                           (fabsl(gaT * (long double)v[IDX(b, i, c)]) + fabsl(gbT));
                if (has_state)
                    acc += (long double)T * expl(o0 - (long double)T * wc + moT) *
                           (fabsl(gaT * a0) + fabsl(gbT) * b0);
            }
            mdw[c] += (double)acc;
            mdu[c] += (double)mu_sum;
        }
    free(lt);
    free(yt);
    return NULL;
}

/* Channels are split over nthreads threads (each owns its channels' sums). */
int wkvo_backward_magnitude(int64_t B, int64_t T, int64_t C, const double *w, const double *u,
                            const double *k, const double *v, const double *dy,
                            const double *state_in, const double *state_out,
                            const double *d_state_out, double *mdw, double *mdu, int nthreads) {
    if (B < 0 || T < 0 || C < 0) return 1;
    if (d_state_out && !state_out) return 1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 64) nthreads = 64;
    if (C < nthreads) nthreads = C > 0 ? (int)C : 1;
    struct mag_job jobs[64];
    pthread_t th[64];
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = (struct mag_job){B, T, C, C * i / nthreads, C * (i + 1) / nthreads, w, u, k, v,
                                   dy, state_in, state_out, d_state_out, mdw, mdu};
        if (i > 0) pthread_create(&th[i], NULL, mag_job_run, &jobs[i]);
    }
    mag_job_run(&jobs[0]);
    for (int i = 1; i < nthreads; ++i) pthread_join(th[i], NULL);
    return 0;
}
