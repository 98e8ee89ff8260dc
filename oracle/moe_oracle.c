/*
 * moe_oracle.c -- CPU oracle of the MoE-layer forward.  TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct implementation of what the layer computes,
 * in fp64, used to check the HIP path.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load it; the product library never links it and
 * shares no code, header or table with it.
 *
 * What it computes, and where the pages fix it (pages are cited by title):
 *  - router: a DeepSeek-V3-style sigmoid router; each token keeps k of E
 *    experts ("25GB 内存跑 744B GLM-5.2 模型" page, section 三.1).  A per-expert
 *    bias steers which experts are selected, DeepSeek-V3's balancing without
 *    an auxiliary loss, and inference has to reproduce the sigmoid routing,
 *    the selection and the scaling exactly (same page, section 四.3).
 *    Reading taken where the pages are silent: logits z = x . W_r in fp64,
 *    s = 1/(1+exp(-z)), selection score sel = s + b, top-k by sel descending
 *    with ties to the lower expert id, combine weight = lambda * s_j / sum s.
 *  - batch union: batch positions that hit the same expert are merged, the
 *    expert is read once and applied to all of them (GLM-5.2 page, section
 *    三.4).  Here: a stable counting sort of the T*k (token, slot)
 *    assignments by expert.
 *  - experts: SwiGLU FFNs whose weights are quantised per output channel with
 *    a scale and a zero point ("企业官网建设流程全解析" page, the Colibri
 *    walk-through, section 3.4):
 *    w = scale * (q - zp);  h = silu(W_gate x) * (W_up x);  y = W_down h.
 *  - the shared expert is part of the dense, always-resident weights (GLM-5.2
 *    page, section 二) and is added to every token with weight 1.
 *  - combine: y[t] = S[t] + sum_j w[t][j] * Y[sorted position of (t, j)].
 *  - router variants.  The deep-dive page (lshu.cn, untitled Colibri deep dive) gates 8 experts with a
 *    softmax over the logits, computed against the maximum logit so exp cannot overflow, and keeps the
 *    top 2 (its section 3.2); a Mixtral-style gate keeps the top 2 under a capacity factor of 1.2 (its
 *    section 6.2); the walk-through page names expert-choice and soft routing as other router logics that
 *    reuse the rest of the engine (its section 6).  Readings where the pages are silent:
 *      softmax top-k: the k largest logits (softmax keeps their order), ties to the lower id; weights
 *        lambda * p_j / sum of the selected p, i.e. lambda * exp(z_j - z_max) / sum exp(z_j' - z_max);
 *        soft routing is the same gate with k = E (every expert, weighted by its softmax probability);
 *      capacity: every expert keeps at most C = ceil(cf * T * k / E) assignments, claimed in the order
 *        all tokens' first choices, then all second choices, ... (token order within a choice); the
 *        others become empty slots (id -1) and add nothing, the kept weights are not renormalised;
 *      expert choice: p = softmax over the experts of each token; every expert takes the C =
 *        min(T, ceil(cf * T / E)) tokens of largest p (ties to the lower token), weight lambda * p.
 *    An empty slot (id -1) is skipped by the permutation and the combine.
 *
 *  - expert residency tiers.  The deep-dive page (pwwt.cn Colibri write-up) keeps an expert cache of slots,
 *    each holding one expert's complete weights, by default 4 times the experts a token activates (its
 *    section 3.1); eviction is a weighted LRU whose weight is how often the expert was activated lately: each
 *    slot keeps a last-used time and a hit count and the slot with few hits and an old last use goes first
 *    (same section).  The GLM-5.2 page keeps one LRU cache per layer, reads the next experts ahead while the
 *    current ones compute (its section 三.5), merges a batch's requests so each distinct expert is read once
 *    (三.4) and can pin hot experts in the faster tier (五).  Readings where the pages are silent:
 *      a step is one layer call; its requests are the batch union U of the experts its tokens chose;
 *      a resident expert of U is a hit: its slot's hit count += 1 and last use = the step number (steps count
 *        from 1);
 *      the missing experts of U, in ascending id, each take the first evictable slot in the order: empty
 *        slots (lower slot first), then fewest hits, then oldest last use, then lower expert id (pure LRU,
 *        kept for comparison: empty, then oldest last use, then lower id); a slot holding an expert of U, or
 *        a pinned slot, is not evictable; a loaded slot starts with hit count 1 and last use = the step;
 *      pinned experts fill slots 0 .. P-1 from the start and never leave;
 *      the counts are per residence: an evicted expert that comes back starts again from 1.
 *
 * All sums run in index order in fp64.  The OpenMP loops split work only over
 * independent output elements, so results do not depend on the thread count.
 *
 * Parity pins live in tests/test_oracle_pins.py and tests/test_oracle_cache_pins.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ACT_F32 0
#define ACT_BF16 1

void oracle_set_threads(int n) {
#ifdef _OPENMP
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Activations: fp32 values, or bf16 bit patterns (the upper half of an fp32). */
void oracle_decode_act(const void *x, int act, long n, double *out) {
    for (long i = 0; i < n; i++) {
        if (act == ACT_F32) {
            out[i] = (double)((const float *)x)[i];
        } else {
            uint32_t u = (uint32_t)((const uint16_t *)x)[i] << 16;
            float f;
            memcpy(&f, &u, sizeof f);
            out[i] = (double)f;
        }
    }
}

/* z[t][e] = sum_{i=0}^{d-1} x[t][i] * W_r[i][e]   (W_r is [d][E]) */
void oracle_router_logits(int T, int d, int E, const double *x, const float *Wr, double *z) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; t++) {
        double *zt = z + (long)t * E;
        for (int e = 0; e < E; e++) zt[e] = 0.0;
        for (int i = 0; i < d; i++) {
            double xi = x[(long)t * d + i];
            const float *wrow = Wr + (long)i * E;
            for (int e = 0; e < E; e++) zt[e] += xi * (double)wrow[e];
        }
    }
}

typedef struct {
    double v;
    int id;
} oracle_kv;

/* Full order used for selection: larger score first, equal scores by lower id. */
static int kv_cmp(const void *a, const void *b) {
    const oracle_kv *x = (const oracle_kv *)a, *y = (const oracle_kv *)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->id > y->id) - (x->id < y->id);
}

/*
 * Sigmoid scores, biased selection, top-k and combine weights, one token at a time.
 *   s[e]   = 1 / (1 + exp(-z[e]))
 *   sel[e] = s[e] + bias[e]
 *   idx[t][0..k) = the first k experts of the full order of sel (desc, id asc)
 *   gap[t] = sel of the k-th minus sel of the (k+1)-th (INFINITY when k == E)
 *   w[t][j] = lambda * s[idx_j] / sum_{j'} s[idx_j']     (fp64, stored fp32)
 * s_out / sel_out (optional, [T][E]) return the scores.
 */
void oracle_router_select(int T, int E, int k, const double *z, const float *bias, double lambda,
                          int32_t *idx, float *w, double *gap, double *s_out, double *sel_out) {
#pragma omp parallel
    {
        oracle_kv *kv = (oracle_kv *)malloc(sizeof(oracle_kv) * (size_t)E);
        double *s = (double *)malloc(sizeof(double) * (size_t)E);
#pragma omp for schedule(static)
        for (int t = 0; t < T; t++) {
            for (int e = 0; e < E; e++) {
                double ze = z[(long)t * E + e];
                s[e] = 1.0 / (1.0 + exp(-ze));
                kv[e].v = s[e] + (double)bias[e];
                kv[e].id = e;
                if (s_out) s_out[(long)t * E + e] = s[e];
                if (sel_out) sel_out[(long)t * E + e] = kv[e].v;
            }
            qsort(kv, (size_t)E, sizeof(oracle_kv), kv_cmp);
            double sum = 0.0;
            for (int j = 0; j < k; j++) {
                idx[(long)t * k + j] = kv[j].id;
                sum += s[kv[j].id];
            }
            for (int j = 0; j < k; j++) w[(long)t * k + j] = (float)(lambda * s[kv[j].id] / sum);
            if (gap) gap[t] = (k < E) ? kv[k - 1].v - kv[k].v : INFINITY;
        }
        free(kv);
        free(s);
    }
}

/*
 * Batch union as a stable counting sort of the A = T*k assignments a = t*k + j
 * by expert:
 *   counts[e]      number of assignments to e
 *   offsets[0..E]  exclusive prefix sum of counts
 *   perm[p]        the assignment at sorted position p (ascending a inside an expert)
 *   inv[a]         the sorted position of assignment a
 *   uniq[0..n)     experts with counts > 0, ascending; the rest of uniq is -1
 */
void oracle_permute(int T, int k, int E, const int32_t *idx, int32_t *counts, int32_t *offsets,
                    int32_t *perm, int32_t *inv, int32_t *uniq, int32_t *n_uniq) {
    long A = (long)T * k;
    for (int e = 0; e < E; e++) counts[e] = 0;
    for (long a = 0; a < A; a++)
        if (idx[a] >= 0) counts[idx[a]]++;  /* -1: an empty slot */
    offsets[0] = 0;
    for (int e = 0; e < E; e++) offsets[e + 1] = offsets[e] + counts[e];
    int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    for (int e = 0; e < E; e++) cursor[e] = offsets[e];
    for (long a = 0; a < A; a++) {
        if (idx[a] < 0) {
            inv[a] = -1;
            continue;
        }
        int32_t p = cursor[idx[a]]++;
        perm[p] = (int32_t)a;
        inv[a] = p;
    }
    free(cursor);
    int n = 0;
    for (int e = 0; e < E; e++)
        if (counts[e] > 0) uniq[n++] = e;
    for (int e = n; e < E; e++) uniq[e] = -1;
    *n_uniq = n;
}

/* q at (row, col) of a quantised matrix with row_bytes bytes per row. */
static inline double q_at(const void *q, int wbits, long row_bytes, long row, long col) {
    if (wbits == 8) return (double)((const int8_t *)q)[row * row_bytes + col];
    uint8_t b = ((const uint8_t *)q)[row * row_bytes + col / 2];
    return (double)((col & 1) ? (b >> 4) : (b & 15));
}

static inline double zp_at(const void *z, int wbits, long row) {
    return wbits == 8 ? (double)((const int8_t *)z)[row] : (double)((const float *)z)[row];
}

/*
 * One SwiGLU expert applied to n input rows X[n][d] -> Y[n][d]:
 *   g_c = s^g_c * sum_i (q^g_{c,i} - z^g_c) * x_i
 *   u_c = s^u_c * sum_i (q^u_{c,i} - z^u_c) * x_i
 *   h_c = silu(g_c) * u_c,          silu(v) = v / (1 + exp(-v))
 *   y_r = s^d_r * sum_c (q^d_{r,c} - z^d_r) * h_c
 * q_gate/q_up are [I][d*wbits/8] bytes, q_down is [d][I*wbits/8]; scales fp32 per
 * output row; zero points int8 (wbits 8) or fp32 (wbits 4) per output row.
 * H (optional, [n][I]) returns h.
 */
void oracle_expert_apply(int n, int d, int I, int wbits,
                         const void *q_gate, const float *s_gate, const void *z_gate,
                         const void *q_up, const float *s_up, const void *z_up,
                         const void *q_down, const float *s_down, const void *z_down,
                         const double *X, double *Y, double *H) {
    long rb_in = (long)d * wbits / 8, rb_hid = (long)I * wbits / 8;
    double *h = H ? H : (double *)malloc(sizeof(double) * (size_t)n * (size_t)I);
#pragma omp parallel for schedule(static) collapse(2)
    for (int r = 0; r < n; r++) {
        for (int c = 0; c < I; c++) {
            const double *x = X + (long)r * d;
            double zg = zp_at(z_gate, wbits, c), zu = zp_at(z_up, wbits, c);
            double g = 0.0, u = 0.0;
            for (long i = 0; i < d; i++) {
                g += (q_at(q_gate, wbits, rb_in, c, i) - zg) * x[i];
                u += (q_at(q_up, wbits, rb_in, c, i) - zu) * x[i];
            }
            g *= (double)s_gate[c];
            u *= (double)s_up[c];
            h[(long)r * I + c] = g / (1.0 + exp(-g)) * u;
        }
    }
#pragma omp parallel for schedule(static) collapse(2)
    for (int r = 0; r < n; r++) {
        for (int o = 0; o < d; o++) {
            const double *hr = h + (long)r * I;
            double zd = zp_at(z_down, wbits, o);
            double acc = 0.0;
            for (long c = 0; c < I; c++) acc += (q_at(q_down, wbits, rb_hid, o, c) - zd) * hr[c];
            Y[(long)r * d + o] = (double)s_down[o] * acc;
        }
    }
    if (!H) free(h);
}

/* y[t] = S[t] + sum_{j=0}^{k-1} w[t][j] * Y[inv[t*k+j]]   (S may be NULL) */
void oracle_combine(int T, int k, int d, const double *Y, const double *S, const int32_t *inv,
                    const float *w, double *y) {
#pragma omp parallel for schedule(static) collapse(2)
    for (int t = 0; t < T; t++) {
        for (int o = 0; o < d; o++) {
            double acc = S ? S[(long)t * d + o] : 0.0;
            for (int j = 0; j < k; j++)
                if (inv[(long)t * k + j] >= 0)  /* an empty slot adds nothing */
                    acc += (double)w[(long)t * k + j] * Y[(long)inv[(long)t * k + j] * d + o];
            y[(long)t * d + o] = acc;
        }
    }
}

/*
 * Softmax top-k, one token at a time (reading in the header): idx[t][0..k) = the k largest z (desc, equal
 * z by lower id); with m = z of idx[t][0], u_j = exp(z_j - m) and w[t][j] = lambda * u_j / sum_j' u_j' (fp64,
 * stored fp32); gap[t] = z of the k-th minus z of the (k+1)-th (INFINITY when k == E).
 */
void oracle_router_select_softmax(int T, int E, int k, const double *z, double lambda, int32_t *idx, float *w,
                                  double *gap) {
#pragma omp parallel
    {
        oracle_kv *kv = (oracle_kv *)malloc(sizeof(oracle_kv) * (size_t)E);
        double *u = (double *)malloc(sizeof(double) * (size_t)k);
#pragma omp for schedule(static)
        for (int t = 0; t < T; t++) {
            for (int e = 0; e < E; e++) {
                kv[e].v = z[(long)t * E + e];
                kv[e].id = e;
            }
            qsort(kv, (size_t)E, sizeof(oracle_kv), kv_cmp);
            double sum = 0.0;
            for (int j = 0; j < k; j++) {
                idx[(long)t * k + j] = kv[j].id;
                u[j] = exp(kv[j].v - kv[0].v);
                sum += u[j];
            }
            for (int j = 0; j < k; j++) w[(long)t * k + j] = (float)(lambda * u[j] / sum);
            if (gap) gap[t] = (k < E) ? kv[k - 1].v - kv[k].v : INFINITY;
        }
        free(kv);
        free(u);
    }
}

/*
 * Capacity: every expert keeps at most C of the assignments idx [T][k] (in place), claimed choice by choice
 * (j = 0 for every token, then j = 1, ...) and token by token within a choice; the rest become -1.  Slots
 * that are already -1 stay so.
 */
void oracle_capacity(int T, int k, int E, int C, int32_t *idx) {
    int32_t *used = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    for (int j = 0; j < k; j++)
        for (int t = 0; t < T; t++) {
            int32_t *a = idx + (long)t * k + j;
            if (*a < 0) continue;
            if (used[*a] < C)
                used[*a]++;
            else
                *a = -1;
        }
    free(used);
}

/* order of tokens for one expert: larger probability first, equal ones by lower token */
typedef struct {
    double p;
    int t;
} oracle_tp;

static int tp_cmp(const void *a, const void *b) {
    const oracle_tp *x = (const oracle_tp *)a, *y = (const oracle_tp *)b;
    if (x->p > y->p) return -1;
    if (x->p < y->p) return 1;
    return (x->t > y->t) - (x->t < y->t);
}

/*
 * Expert choice: p[t][e] = exp(z[t][e] - m_t) / sum_e' exp(z[t][e'] - m_t), m_t = max_e z[t][e], the sum taken
 * over e ascending; expert e takes the C tokens of largest p[.][e] (equal p by lower token).  Outputs, with one
 * slot per expert (k = E): idx[t][e] = e and w[t][e] = lambda * p[t][e] (fp32) when e took t, else -1 and 0.
 * gap_e (optional, [E]): p of the C-th chosen token minus p of the (C+1)-th (INFINITY when C == T).
 */
void oracle_expert_choice(int T, int E, int C, const double *z, double lambda, int32_t *idx, float *w,
                          double *gap_e) {
    double *p = (double *)malloc(sizeof(double) * (size_t)T * (size_t)E);
    for (int t = 0; t < T; t++) {
        const double *zt = z + (long)t * E;
        double m = zt[0], s = 0.0;
        for (int e = 1; e < E; e++) m = zt[e] > m ? zt[e] : m;
        for (int e = 0; e < E; e++) s += exp(zt[e] - m);
        for (int e = 0; e < E; e++) p[(long)t * E + e] = exp(zt[e] - m) / s;
        for (int e = 0; e < E; e++) {
            idx[(long)t * E + e] = -1;
            w[(long)t * E + e] = 0.0f;
        }
    }
#pragma omp parallel
    {
        oracle_tp *tp = (oracle_tp *)malloc(sizeof(oracle_tp) * (size_t)T);
#pragma omp for schedule(static)
        for (int e = 0; e < E; e++) {
            for (int t = 0; t < T; t++) {
                tp[t].p = p[(long)t * E + e];
                tp[t].t = t;
            }
            qsort(tp, (size_t)T, sizeof(oracle_tp), tp_cmp);
            for (int c = 0; c < C; c++) {
                idx[(long)tp[c].t * E + e] = e;
                w[(long)tp[c].t * E + e] = (float)(lambda * tp[c].p);
            }
            if (gap_e) gap_e[e] = C < T ? tp[C - 1].p - tp[C].p : INFINITY;
        }
        free(tp);
    }
    free(p);
}

/* Pointers to expert e inside stacked [n][rows][row_bytes] weight arrays. */
typedef struct {
    const void *q_gate, *q_up, *q_down;
    const float *s_gate, *s_up, *s_down;
    const void *z_gate, *z_up, *z_down;
} oracle_qffn;

static void expert_ptrs(const oracle_qffn *W, int e, int d, int I, int wbits, oracle_qffn *out) {
    long rb_in = (long)d * wbits / 8, rb_hid = (long)I * wbits / 8;
    long zb = wbits == 8 ? 1 : 4;
    out->q_gate = (const uint8_t *)W->q_gate + (long)e * I * rb_in;
    out->q_up = (const uint8_t *)W->q_up + (long)e * I * rb_in;
    out->q_down = (const uint8_t *)W->q_down + (long)e * d * rb_hid;
    out->s_gate = W->s_gate + (long)e * I;
    out->s_up = W->s_up + (long)e * I;
    out->s_down = W->s_down + (long)e * d;
    out->z_gate = (const uint8_t *)W->z_gate + (long)e * I * zb;
    out->z_up = (const uint8_t *)W->z_up + (long)e * I * zb;
    out->z_down = (const uint8_t *)W->z_down + (long)e * d * zb;
}

static void apply(const oracle_qffn *W, int e, int n, int d, int I, int wbits, const double *X, double *Y) {
    oracle_qffn p;
    expert_ptrs(W, e, d, I, wbits, &p);
    oracle_expert_apply(n, d, I, wbits, p.q_gate, p.s_gate, p.z_gate, p.q_up, p.s_up, p.z_up, p.q_down,
                        p.s_down, p.z_down, X, Y, NULL);
}

/*
 * Whole layer through the batch union:
 * route -> permute -> for each unique expert, its rows in sorted order -> shared -> combine.
 * Outputs: idx, w, gap [T]; counts..n_uniq as oracle_permute; Yperm [A][d];
 * S [T][d] (NULL when I_shared == 0); y [T][d].
 */
void oracle_moe_layer(int T, int d, int E, int k, int I, int I_shared, int wbits, double lambda, int act,
                      const void *x, const float *Wr, const float *bias, const oracle_qffn *routed,
                      const oracle_qffn *shared, int32_t *idx, float *w, double *gap, int32_t *counts,
                      int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *uniq, int32_t *n_uniq,
                      double *Yperm, double *S, double *y) {
    long A = (long)T * k;
    double *xd = (double *)malloc(sizeof(double) * (size_t)T * (size_t)d);
    double *z = (double *)malloc(sizeof(double) * (size_t)T * (size_t)E);
    oracle_decode_act(x, act, (long)T * d, xd);
    oracle_router_logits(T, d, E, xd, Wr, z);
    oracle_router_select(T, E, k, z, bias, lambda, idx, w, gap, NULL, NULL);
    oracle_permute(T, k, E, idx, counts, offsets, perm, inv, uniq, n_uniq);
    for (int u = 0; u < *n_uniq; u++) {
        int e = uniq[u];
        int n = counts[e];
        double *X = (double *)malloc(sizeof(double) * (size_t)n * (size_t)d);
        for (int r = 0; r < n; r++) {
            long t = perm[offsets[e] + r] / k;
            memcpy(X + (long)r * d, xd + t * d, sizeof(double) * (size_t)d);
        }
        apply(routed, e, n, d, I, wbits, X, Yperm + (long)offsets[e] * d);
        free(X);
    }
    (void)A;
    if (I_shared > 0 && shared && S) apply(shared, 0, T, d, I_shared, wbits, xd, S);
    oracle_combine(T, k, d, Yperm, (I_shared > 0) ? S : NULL, inv, w, y);
    free(xd);
    free(z);
}

/*
 * The same layer without the batch union: every listed token is routed and
 * each of its k experts applied to it alone.  tokens[n] lists which rows of x
 * to evaluate (the routing of a token does not depend on other tokens).
 * Outputs per listed token: idx [n][k], w [n][k], gap [n], y [n][d].
 */
void oracle_moe_tokens(int n, const int32_t *tokens, int d, int E, int k, int I, int I_shared, int wbits,
                       double lambda, int act, const void *x, const float *Wr, const float *bias,
                       const oracle_qffn *routed, const oracle_qffn *shared, int32_t *idx, float *w,
                       double *gap, double *y) {
    double *xd = (double *)malloc(sizeof(double) * (size_t)d);
    double *z = (double *)malloc(sizeof(double) * (size_t)E);
    double *Y = (double *)malloc(sizeof(double) * (size_t)d * (size_t)(k + 1));
    size_t xb = (act == ACT_F32) ? 4 : 2;
    for (int r = 0; r < n; r++) {
        const uint8_t *xr = (const uint8_t *)x + (size_t)tokens[r] * (size_t)d * xb;
        oracle_decode_act(xr, act, d, xd);
        oracle_router_logits(1, d, E, xd, Wr, z);
        oracle_router_select(1, E, k, z, bias, lambda, idx + (long)r * k, w + (long)r * k, gap + r, NULL, NULL);
        for (int j = 0; j < k; j++) apply(routed, idx[(long)r * k + j], 1, d, I, wbits, xd, Y + (long)j * d);
        double *S = NULL;
        if (I_shared > 0 && shared) {
            S = Y + (long)k * d;
            apply(shared, 0, 1, d, I_shared, wbits, xd, S);
        }
        /* combine in the same order as oracle_combine: shared first, then j = 0..k-1 */
        for (int o = 0; o < d; o++) {
            double acc = S ? S[o] : 0.0;
            for (int j = 0; j < k; j++) acc += (double)w[(long)r * k + j] * Y[(long)j * d + o];
            y[(long)r * d + o] = acc;
        }
    }
    free(xd);
    free(z);
    free(Y);
}

/*
 * Sparse-attention indexer and its top-K selection.  The GLM-5.2 page has the engine run the model's lightning
 * indexer and keep, per layer, the top 2048 causal keys for attention (its section 三.3); a light indexer first
 * scores the history's keys, then the top-k entries go to the real attention (its section 四.4, on DeepSeek
 * Sparse Attention).  The pages give no formula; the reading taken is the DSA indexer's published form with
 * integer operands so that both implementations compute the same bits:
 *   dot[t][h][s] = sum_i q[t][h][i] * k[s][i]          (int8 operands, exact integer sum)
 *   I[t][s]      = kscale[s] * sum_{h=0}^{H-1} w[t][h] * max(0, dot[t][h][s])
 * the head sum a chain of fused multiply-adds acc = fma(w, relu, acc) in head order from 0, then one product by
 * kscale[s], all in fp64.  Query t sits at position pos0 + t and sees the keys s <= pos0 + t.  Its output is the
 * set of the K largest scores among them (equal scores by lower position), listed by ascending position, padded
 * with -1 when fewer than K keys are visible; gap[t] = score of the K-th minus score of the (K+1)-th of that order
 * (INFINITY when all visible keys are taken).  scores (optional, [T][S]) returns I (0 where s is not visible).
 */
static int ix_cmp(const void *a, const void *b) {  /* larger score first, equal scores by lower position */
    const oracle_kv *x = (const oracle_kv *)a, *y = (const oracle_kv *)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->id > y->id) - (x->id < y->id);
}

static int int_cmp(const void *a, const void *b) {
    const int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

void oracle_index_topk(int T, int S, int H, int D, int K, int pos0, const int8_t *q, const float *w,
                       const int8_t *k, const float *kscale, int32_t *top, double *gap, double *scores) {
#pragma omp parallel
    {
        oracle_kv *kv = (oracle_kv *)malloc(sizeof(oracle_kv) * (size_t)(S > 0 ? S : 1));
#pragma omp for schedule(dynamic)
        for (int t = 0; t < T; t++) {
            int n = pos0 + t + 1;
            if (n > S) n = S;
            if (n < 0) n = 0;
            for (int s = 0; s < n; s++) {
                double acc = 0.0;
                for (int h = 0; h < H; h++) {
                    long dot = 0;
                    const int8_t *qr = q + ((long)t * H + h) * D, *kr = k + (long)s * D;
                    for (int i = 0; i < D; i++) dot += (long)qr[i] * (long)kr[i];
                    acc = fma((double)w[(long)t * H + h], (double)(dot > 0 ? dot : 0), acc);
                }
                kv[s].v = (double)kscale[s] * acc;
                kv[s].id = s;
                if (scores) scores[(long)t * S + s] = kv[s].v;
            }
            if (scores)
                for (int s = n; s < S; s++) scores[(long)t * S + s] = 0.0;
            qsort(kv, (size_t)n, sizeof(oracle_kv), ix_cmp);
            const int m = n < K ? n : K;
            int32_t *out = top + (long)t * K;
            for (int j = 0; j < m; j++) out[j] = kv[j].id;
            qsort(out, (size_t)m, sizeof(int32_t), int_cmp);
            for (int j = m; j < K; j++) out[j] = -1;
            if (gap) gap[t] = n > K ? kv[K - 1].v - kv[K].v : INFINITY;
        }
        free(kv);
    }
}

/* ---------------------------------------------------------------------------------------------------------
 * Expert residency (cache of HBM slots over the host tier); readings in the header.
 * State: slot_expert[S] (-1 empty), expert_slot[E] (-1 not resident), last_used[S], hits[S].
 */
void oracle_cache_init(int E, int S, int P, const int32_t *pinned, int32_t *slot_expert, int32_t *expert_slot,
                       int64_t *last_used, int64_t *hits) {
    for (int e = 0; e < E; e++) expert_slot[e] = -1;
    for (int s = 0; s < S; s++) {
        slot_expert[s] = -1;
        last_used[s] = 0;
        hits[s] = 0;
    }
    for (int i = 0; i < P; i++) {
        slot_expert[i] = pinned[i];
        expert_slot[pinned[i]] = i;
    }
}

/* Is slot a a better victim than slot b (policy 0 weighted LRU, 1 LRU)? */
static int victim_before(int policy, int a, int b, const int32_t *slot_expert, const int64_t *last_used,
                         const int64_t *hits) {
    const int ea = slot_expert[a] >= 0, eb = slot_expert[b] >= 0;
    if (!ea || !eb) {
        if (ea != eb) return !ea;  /* an empty slot first */
        return a < b;
    }
    if (policy == 0 && hits[a] != hits[b]) return hits[a] < hits[b];
    if (last_used[a] != last_used[b]) return last_used[a] < last_used[b];
    return slot_expert[a] < slot_expert[b];
}

/* One step at time `now`: U = the nu distinct experts of uniq (any order).  Writes the hits and the misses in
 * ascending expert id and, per miss, the expert its slot held before (-1: the slot was empty).  Returns 0, or -1
 * when a miss finds no evictable slot (the state is then partly updated). */
int oracle_cache_step(int E, int S, int P, int policy, int64_t now, int32_t *slot_expert, int32_t *expert_slot,
                      int64_t *last_used, int64_t *hits, int nu, const int32_t *uniq, int32_t *hit_list,
                      int32_t *n_hit, int32_t *miss_list, int32_t *n_miss, int32_t *evicted) {
    unsigned char *inU = (unsigned char *)calloc((size_t)E, 1);
    for (int i = 0; i < nu; i++) inU[uniq[i]] = 1;
    int nh = 0, nm = 0;
    for (int e = 0; e < E; e++) {
        if (!inU[e]) continue;
        const int s = expert_slot[e];
        if (s >= 0) {
            hits[s] += 1;
            last_used[s] = now;
            hit_list[nh++] = e;
        } else {
            miss_list[nm++] = e;
        }
    }
    int rc = 0;
    for (int i = 0; i < nm; i++) {
        const int e = miss_list[i];
        int best = -1;
        for (int s = P; s < S; s++) {
            if (slot_expert[s] >= 0 && inU[slot_expert[s]]) continue;
            if (best < 0 || victim_before(policy, s, best, slot_expert, last_used, hits)) best = s;
        }
        if (best < 0) {
            rc = -1;
            break;
        }
        evicted[i] = slot_expert[best];
        if (slot_expert[best] >= 0) expert_slot[slot_expert[best]] = -1;
        slot_expert[best] = e;
        expert_slot[e] = best;
        hits[best] = 1;
        last_used[best] = now;
    }
    *n_hit = nh;
    *n_miss = nm;
    free(inU);
    return rc;
}
