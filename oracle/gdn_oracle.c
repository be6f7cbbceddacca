/*
 * Reference oracle for the Gated DeltaNet (GDN) chunked-prefill operator.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * CPU definition that the GPU path is checked against.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product library never does, and it shares no code, header or constant with
 * the GPU sources.
 *
 * Everything is float64 and token by token.  There is no chunking, no WY form,
 * no blocking and no reordering: the point is that a reader can check each
 * line against the definition below by eye.
 *
 * Sources (the three FlashQLA pages):
 *   - FlashQLA talk summary (onedev.kr, "Qwen team releases FlashQLA, a GPU
 *     operator for GDN linear attention"), paragraph 2: linear attention keeps
 *     a d x d state that is updated token by token; paragraph 5: the forget
 *     gate alpha lies in (0,1) and keys are L2-normalised.
 *   - The recurrence itself is the gated delta rule of Gated DeltaNet:
 *         S_t = alpha_t * (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
 *         o_t = scale * S_t^T q_t          (output reads the UPDATED state)
 *     with S stored as a dk x dv matrix (row index over the key dimension).
 *     The op receives g_t = log(alpha_t) (so alpha_t = exp(g_t)) and beta_t
 *     already squashed; it does not normalise q or k.
 *
 * Layouts (all row-major, float64):
 *   q, k  [B, T, H, dk]     v, o, dout  [B, T, H, dv]
 *   g, beta, dg, dbeta      [B, T, H]
 *   h0, ht, dht, dh0        [B, H, dk, dv]
 *
 * Parity pins: see tests/test_oracle_pins.py (closed forms, brute-force
 * transition products, finite differences, hand-derived golden values).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define IDX_TOK(b, t, h, d, T, H, D) ((((size_t)(b) * (T) + (t)) * (H) + (h)) * (D) + (d))
#define IDX_GATE(b, t, h, T, H) (((size_t)(b) * (T) + (t)) * (H) + (h))
#define IDX_STATE(b, h, H, dk, dv) (((size_t)(b) * (H) + (h)) * (size_t)(dk) * (dv))

/* One token of the forward recurrence on the state S (dk x dv), in place.
 *   S <- alpha * S
 *   p  = S^T k              prediction of the decayed state at key k
 *   u  = beta * (v - p)     the delta-rule correction
 *   S <- S + k u^T
 * which expands to S_t = alpha (I - beta k k^T) S_{t-1} + beta k v^T.
 * work must hold 2*dv doubles. */
static void token_step(double* S, const double* kt, const double* vt, double alpha, double beta,
                       int dk, int dv, double* work) {
    double* p = work;
    double* u = work + dv;
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= alpha;
    for (int j = 0; j < dv; ++j) p[j] = 0.0;
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) p[j] += S[(size_t)i * dv + j] * kt[i];
    for (int j = 0; j < dv; ++j) u[j] = beta * (vt[j] - p[j]);
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += kt[i] * u[j];
}

/* Gather the dk (or dv) vector of token t of head (b,h) into a contiguous buffer. */
static void gather(double* dst, const double* src, int b, int t, int h, int T, int H, int D) {
    memcpy(dst, src + IDX_TOK(b, t, h, 0, T, H, D), sizeof(double) * (size_t)D);
}

/* Forward of one head: o[t] = scale * S_t^T q_t for every t, final state to ht. */
static void fwd_head(const double* q, const double* k, const double* v, const double* g,
                     const double* beta, const double* h0, double* o, double* ht, int b, int h,
                     int B, int T, int H, int dk, int dv, double scale) {
    (void)B;
    double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
    double* kt = (double*)malloc(sizeof(double) * (size_t)dk);
    double* qt = (double*)malloc(sizeof(double) * (size_t)dk);
    double* vt = (double*)malloc(sizeof(double) * (size_t)dv);
    double* ot = (double*)malloc(sizeof(double) * (size_t)dv);
    double* work = (double*)malloc(sizeof(double) * 2 * (size_t)dv);
    if (h0)
        memcpy(S, h0 + IDX_STATE(b, h, H, dk, dv), sizeof(double) * (size_t)dk * dv);
    else
        memset(S, 0, sizeof(double) * (size_t)dk * dv);
    for (int t = 0; t < T; ++t) {
        gather(kt, k, b, t, h, T, H, dk);
        gather(qt, q, b, t, h, T, H, dk);
        gather(vt, v, b, t, h, T, H, dv);
        double alpha = exp(g[IDX_GATE(b, t, h, T, H)]);
        double bt = beta[IDX_GATE(b, t, h, T, H)];
        token_step(S, kt, vt, alpha, bt, dk, dv, work);
        for (int j = 0; j < dv; ++j) ot[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) ot[j] += qt[i] * S[(size_t)i * dv + j];
        for (int j = 0; j < dv; ++j) o[IDX_TOK(b, t, h, j, T, H, dv)] = scale * ot[j];
    }
    if (ht) memcpy(ht + IDX_STATE(b, h, H, dk, dv), S, sizeof(double) * (size_t)dk * dv);
    free(S); free(kt); free(qt); free(vt); free(ot); free(work);
}

/* Forward over the heads listed in head_list (pairs b*H+h), or over all B*H heads
 * when head_list is NULL.  Heads are independent; OpenMP spreads them over threads.
 * Outputs of heads not listed are left untouched. */
void gdn_oracle_fwd(const double* q, const double* k, const double* v, const double* g,
                    const double* beta, const double* h0, double* o, double* ht, int B, int T,
                    int H, int dk, int dv, double scale, const int* head_list, int n_heads,
                    int nthreads) {
    int total = head_list ? n_heads : B * H;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int n = 0; n < total; ++n) {
        int bh = head_list ? head_list[n] : n;
        fwd_head(q, k, v, g, beta, h0, o, ht, bh / H, bh % H, B, T, H, dk, dv, scale);
    }
}

/* Backward of one head by back-propagation through time.
 *
 * With G = dL/dS_t (gradient of the loss w.r.t. the state AFTER token t, which
 * already includes the paths through all later tokens), a = alpha_t,
 * P = S_{t-1} and the forward S_t = a (I - beta k k^T) P + beta k v^T,
 * o_t = scale S_t^T q_t, the chain rule gives, token by token from the end:
 *   G     += scale q_t dout_t^T                       (output read of S_t)
 *   dq_t   = scale S_t dout_t
 *   dv_t   = beta G^T k
 *   dbeta  = k^T G (v - a P^T k)
 *   dg_t   = a <G, (I - beta k k^T) P>                (g = log a)
 *   dk_t   = -a beta (P G^T k + G P^T k) + beta G v
 *   G     <- a (I - beta k k^T) G                     (becomes dL/dS_{t-1})
 * and finally dh0 = G.
 *
 * States are recomputed from checkpoints taken every `ckpt` tokens so the
 * memory stays at (T/ckpt + ckpt) states per head. */
static void bwd_head(const double* q, const double* k, const double* v, const double* g,
                     const double* beta, const double* h0, const double* dout, const double* dht,
                     double* dq, double* dk_out, double* dv_out, double* dg, double* dbeta,
                     double* dh0, int b, int h, int T, int H, int dk, int dv, double scale) {
    const int ckpt = 64;
    const size_t SS = (size_t)dk * dv;
    int nblk = (T + ckpt - 1) / ckpt;
    double* cps = (double*)malloc(sizeof(double) * SS * (size_t)(nblk + 1));
    double* states = (double*)malloc(sizeof(double) * SS * (size_t)(ckpt + 1));
    double* G = (double*)malloc(sizeof(double) * SS);
    double* kt = (double*)malloc(sizeof(double) * (size_t)dk);
    double* qt = (double*)malloc(sizeof(double) * (size_t)dk);
    double* vt = (double*)malloc(sizeof(double) * (size_t)dv);
    double* dot = (double*)malloc(sizeof(double) * (size_t)dv);
    double* work = (double*)malloc(sizeof(double) * 2 * (size_t)dv);
    double* Gk = (double*)malloc(sizeof(double) * (size_t)dv);  /* G^T k */
    double* Pk = (double*)malloc(sizeof(double) * (size_t)dv);  /* P^T k */
    double* kG = (double*)malloc(sizeof(double) * (size_t)dv);  /* k^T G (same as Gk) */

    /* forward sweep: checkpoint the state entering every block */
    double* S = states;
    if (h0)
        memcpy(S, h0 + IDX_STATE(b, h, H, dk, dv), sizeof(double) * SS);
    else
        memset(S, 0, sizeof(double) * SS);
    for (int blk = 0; blk < nblk; ++blk) {
        memcpy(cps + SS * blk, S, sizeof(double) * SS);
        for (int t = blk * ckpt; t < T && t < (blk + 1) * ckpt; ++t) {
            gather(kt, k, b, t, h, T, H, dk);
            gather(vt, v, b, t, h, T, H, dv);
            token_step(S, kt, vt, exp(g[IDX_GATE(b, t, h, T, H)]), beta[IDX_GATE(b, t, h, T, H)],
                       dk, dv, work);
        }
    }

    if (dht)
        memcpy(G, dht + IDX_STATE(b, h, H, dk, dv), sizeof(double) * SS);
    else
        memset(G, 0, sizeof(double) * SS);

    for (int blk = nblk - 1; blk >= 0; --blk) {
        int t0 = blk * ckpt;
        int t1 = (blk + 1) * ckpt < T ? (blk + 1) * ckpt : T;
        /* recompute states[0] = S_{t0-1} (entering the block) .. states[n] = S_{t1-1} */
        memcpy(states, cps + SS * blk, sizeof(double) * SS);
        for (int t = t0; t < t1; ++t) {
            memcpy(states + SS * (t - t0 + 1), states + SS * (t - t0), sizeof(double) * SS);
            gather(kt, k, b, t, h, T, H, dk);
            gather(vt, v, b, t, h, T, H, dv);
            token_step(states + SS * (t - t0 + 1), kt, vt, exp(g[IDX_GATE(b, t, h, T, H)]),
                       beta[IDX_GATE(b, t, h, T, H)], dk, dv, work);
        }
        for (int t = t1 - 1; t >= t0; --t) {
            const double* Scur = states + SS * (t - t0 + 1);
            const double* P = states + SS * (t - t0);
            double a = exp(g[IDX_GATE(b, t, h, T, H)]);
            double bt = beta[IDX_GATE(b, t, h, T, H)];
            gather(kt, k, b, t, h, T, H, dk);
            gather(qt, q, b, t, h, T, H, dk);
            gather(vt, v, b, t, h, T, H, dv);
            gather(dot, dout, b, t, h, T, H, dv);
            /* output read of S_t */
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) G[(size_t)i * dv + j] += scale * qt[i] * dot[j];
            for (int i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int j = 0; j < dv; ++j) acc += Scur[(size_t)i * dv + j] * dot[j];
                dq[IDX_TOK(b, t, h, i, T, H, dk)] = scale * acc;
            }
            /* G^T k and P^T k */
            for (int j = 0; j < dv; ++j) { Gk[j] = 0.0; Pk[j] = 0.0; }
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) {
                    Gk[j] += G[(size_t)i * dv + j] * kt[i];
                    Pk[j] += P[(size_t)i * dv + j] * kt[i];
                }
            memcpy(kG, Gk, sizeof(double) * (size_t)dv);
            for (int j = 0; j < dv; ++j) dv_out[IDX_TOK(b, t, h, j, T, H, dv)] = bt * Gk[j];
            {
                double acc = 0.0;
                for (int j = 0; j < dv; ++j) acc += kG[j] * (vt[j] - a * Pk[j]);
                dbeta[IDX_GATE(b, t, h, T, H)] = acc;
            }
            {
                /* <G, (I - beta k k^T) P> = <G, P> - beta (k^T G) . (k^T P) */
                double gp = 0.0, kk = 0.0;
                for (size_t e = 0; e < SS; ++e) gp += G[e] * P[e];
                for (int j = 0; j < dv; ++j) kk += kG[j] * Pk[j];
                dg[IDX_GATE(b, t, h, T, H)] = a * (gp - bt * kk);
            }
            for (int i = 0; i < dk; ++i) {
                double pg = 0.0, gpk = 0.0, gv = 0.0;
                for (int j = 0; j < dv; ++j) {
                    pg += P[(size_t)i * dv + j] * Gk[j];   /* (P G^T k)_i */
                    gpk += G[(size_t)i * dv + j] * Pk[j];  /* (G P^T k)_i */
                    gv += G[(size_t)i * dv + j] * vt[j];   /* (G v)_i     */
                }
                dk_out[IDX_TOK(b, t, h, i, T, H, dk)] = -a * bt * (pg + gpk) + bt * gv;
            }
            /* G <- a (I - beta k k^T) G */
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j)
                    G[(size_t)i * dv + j] = a * (G[(size_t)i * dv + j] - bt * kt[i] * kG[j]);
        }
    }
    if (dh0) memcpy(dh0 + IDX_STATE(b, h, H, dk, dv), G, sizeof(double) * SS);
    free(cps); free(states); free(G); free(kt); free(qt); free(vt); free(dot); free(work);
    free(Gk); free(Pk); free(kG);
}

void gdn_oracle_bwd(const double* q, const double* k, const double* v, const double* g,
                    const double* beta, const double* h0, const double* dout, const double* dht,
                    double* dq, double* dk, double* dv_, double* dg, double* dbeta, double* dh0,
                    int B, int T, int H, int dk_dim, int dv_dim, double scale,
                    const int* head_list, int n_heads, int nthreads) {
    int total = head_list ? n_heads : B * H;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int n = 0; n < total; ++n) {
        int bh = head_list ? head_list[n] : n;
        bwd_head(q, k, v, g, beta, h0, dout, dht, dq, dk, dv_, dg, dbeta, dh0, bh / H, bh % H, T,
                 H, dk_dim, dv_dim, scale);
    }
}

/* Gate scan (FlashQLA talk summary, paragraph 5: one light kernel scans the gate
 * distribution to find heads whose alpha-powers decay fast enough that a
 * sliding window suffices).  Chunk c covers tokens [c*C, min((c+1)*C, T)).
 * For every head: s_c = sum of g over chunk c; every run of w consecutive
 * chunks (c-w+1 .. c) has the window sum W_c = s_{c-w+1} + ... + s_c, summed
 * directly here (no running differences).  flag = (N >= w) and
 * max_c W_c <= log_eps.  maxsum = max_c W_c (or -INFINITY when N < w). */
void gdn_oracle_gate_scan(const double* g, int B, int T, int H, int chunk, int w, double log_eps,
                          int* flags, double* maxsum) {
    int N = (T + chunk - 1) / chunk;
    double* s = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            for (int c = 0; c < N; ++c) {
                double acc = 0.0;
                for (int t = c * chunk; t < T && t < (c + 1) * chunk; ++t)
                    acc += g[IDX_GATE(b, t, h, T, H)];
                s[c] = acc;
            }
            double best = -INFINITY;
            for (int c = w - 1; c < N; ++c) {
                double win = 0.0;
                for (int j = c - w + 1; j <= c; ++j) win += s[j];
                if (win > best) best = win;
            }
            flags[b * H + h] = (N >= w && best <= log_eps) ? 1 : 0;
            maxsum[b * H + h] = best;
        }
    free(s);
}

int gdn_oracle_max_threads(void) { return omp_get_max_threads(); }
