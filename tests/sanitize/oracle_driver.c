/*
 * Runs every oracle function on small seeded layers, for a build under AddressSanitizer and
 * UndefinedBehaviorSanitizer (test infrastructure).  Inputs come from a small linear congruential
 * generator; the checks here are only the sanitizers' (any report aborts the run).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const void *q_gate, *q_up, *q_down;
    const float *s_gate, *s_up, *s_down;
    const void *z_gate, *z_up, *z_down;
} qffn;

void oracle_set_threads(int n);
void oracle_moe_layer(int T, int d, int E, int k, int I, int I_shared, int wbits, double lambda, int act,
                      const void *x, const float *Wr, const float *bias, const qffn *routed, const qffn *shared,
                      int32_t *idx, float *w, double *gap, int32_t *counts, int32_t *offsets, int32_t *perm,
                      int32_t *inv, int32_t *uniq, int32_t *n_uniq, double *Yperm, double *S, double *y);
void oracle_moe_tokens(int n, const int32_t *tokens, int d, int E, int k, int I, int I_shared, int wbits,
                       double lambda, int act, const void *x, const float *Wr, const float *bias,
                       const qffn *routed, const qffn *shared, int32_t *idx, float *w, double *gap, double *y);

static uint64_t st = 88172645463325252ull;
static uint32_t rnd(void) {
    st = st * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(st >> 33);
}
static float frnd(void) { return (float)(rnd() % 20001) / 10000.0f - 1.0f; }

static void *alloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) abort();
    return p;
}

static void fill_qffn(qffn *q, int n, int d, int I, int wbits) {
    size_t rb_in = (size_t)d * wbits / 8, rb_hid = (size_t)I * wbits / 8;
    size_t zb = wbits == 8 ? 1 : 4;
    uint8_t *g = alloc((size_t)n * I * rb_in), *u = alloc((size_t)n * I * rb_in), *dn = alloc((size_t)n * d * rb_hid);
    for (size_t i = 0; i < (size_t)n * I * rb_in; i++) g[i] = (uint8_t)rnd(), u[i] = (uint8_t)rnd();
    for (size_t i = 0; i < (size_t)n * d * rb_hid; i++) dn[i] = (uint8_t)rnd();
    float *sg = alloc(sizeof(float) * n * I), *su = alloc(sizeof(float) * n * I), *sd = alloc(sizeof(float) * n * d);
    uint8_t *zg = alloc(zb * n * I), *zu = alloc(zb * n * I), *zd = alloc(zb * n * d);
    for (int i = 0; i < n * I; i++) {
        sg[i] = 0.01f * (1.0f + frnd() * 0.5f);
        su[i] = 0.01f * (1.0f + frnd() * 0.5f);
        if (wbits == 8) zg[i] = (uint8_t)(int8_t)(rnd() % 17 - 8), zu[i] = (uint8_t)(int8_t)(rnd() % 17 - 8);
        else ((float *)zg)[i] = (float)(rnd() % 16), ((float *)zu)[i] = (float)(rnd() % 16);
    }
    for (int i = 0; i < n * d; i++) {
        sd[i] = 0.01f * (1.0f + frnd() * 0.5f);
        if (wbits == 8) zd[i] = (uint8_t)(int8_t)(rnd() % 17 - 8);
        else ((float *)zd)[i] = (float)(rnd() % 16);
    }
    q->q_gate = g, q->q_up = u, q->q_down = dn, q->s_gate = sg, q->s_up = su, q->s_down = sd;
    q->z_gate = zg, q->z_up = zu, q->z_down = zd;
}

static void free_qffn(qffn *q) {
    free((void *)q->q_gate), free((void *)q->q_up), free((void *)q->q_down);
    free((void *)q->s_gate), free((void *)q->s_up), free((void *)q->s_down);
    free((void *)q->z_gate), free((void *)q->z_up), free((void *)q->z_down);
}

static int run(int T, int d, int E, int k, int I, int Is, int wbits, int act) {
    const int A = T * k;
    size_t xb = (size_t)T * d * (act == 0 ? 4 : 2);
    uint8_t *x = alloc(xb);
    if (act == 0)
        for (int i = 0; i < T * d; i++) ((float *)x)[i] = frnd();
    else
        for (int i = 0; i < T * d; i++) ((uint16_t *)x)[i] = (uint16_t)(0x3F00 | (rnd() & 0x80FF));
    float *Wr = alloc(sizeof(float) * d * E), *bias = alloc(sizeof(float) * E);
    for (int i = 0; i < d * E; i++) Wr[i] = 0.02f * frnd();
    for (int e = 0; e < E; e++) bias[e] = 0.01f * frnd();
    qffn R, S;
    fill_qffn(&R, E, d, I, wbits);
    if (Is) fill_qffn(&S, 1, d, Is, wbits);
    int32_t *idx = alloc(4 * A), *counts = alloc(4 * E), *offsets = alloc(4 * (E + 1)), *perm = alloc(4 * A);
    int32_t *inv = alloc(4 * A), *uniq = alloc(4 * E), nu = 0;
    float *w = alloc(4 * A);
    double *gap = alloc(8 * T), *Yp = alloc(8 * (size_t)A * d), *Sy = Is ? alloc(8 * (size_t)T * d) : NULL;
    double *y = alloc(8 * (size_t)T * d), *y2 = alloc(8 * (size_t)T * d);
    oracle_moe_layer(T, d, E, k, I, Is, wbits, 2.5, act, x, Wr, bias, &R, Is ? &S : NULL, idx, w, gap, counts,
                     offsets, perm, inv, uniq, &nu, Yp, Sy, y);
    int32_t *toks = alloc(4 * T), *idx2 = alloc(4 * A);
    float *w2 = alloc(4 * A);
    double *gap2 = alloc(8 * T);
    for (int t = 0; t < T; t++) toks[t] = T - 1 - t;
    oracle_moe_tokens(T, toks, d, E, k, I, Is, wbits, 2.5, act, x, Wr, bias, &R, Is ? &S : NULL, idx2, w2, gap2, y2);
    int bad = 0;
    for (int t = 0; t < T; t++)
        for (int o = 0; o < d; o++) bad |= y[(size_t)(T - 1 - t) * d + o] != y2[(size_t)t * d + o];
    free(x), free(Wr), free(bias), free_qffn(&R);
    if (Is) free_qffn(&S);
    free(idx), free(counts), free(offsets), free(perm), free(inv), free(uniq), free(w), free(gap), free(Yp);
    free(Sy), free(y), free(y2), free(toks), free(idx2), free(w2), free(gap2);
    return bad;
}

void oracle_router_select_softmax(int T, int E, int k, const double *z, double lambda, int32_t *idx, float *w,
                                  double *gap);
void oracle_capacity(int T, int k, int E, int C, int32_t *idx);
void oracle_expert_choice(int T, int E, int C, const double *z, double lambda, int32_t *idx, float *w,
                          double *gap_e);
void oracle_index_topk(int T, int S, int H, int D, int K, int pos0, const int8_t *q, const float *w,
                       const int8_t *k, const float *kscale, int32_t *top, double *gap, double *scores);

static void run_variants(void) {
    const int T = 40, E = 8, k = 3;
    double *z = alloc(sizeof(double) * T * E), *gap = alloc(sizeof(double) * (T > E ? T : E));
    int32_t *idx = alloc(4 * T * E);
    float *w = alloc(4 * T * E);
    for (int i = 0; i < T * E; i++) z[i] = 3.0 * frnd();
    oracle_router_select_softmax(T, E, k, z, 2.5, idx, w, gap);
    oracle_capacity(T, k, E, 12, idx);
    oracle_expert_choice(T, E, 10, z, 1.0, idx, w, gap);
    free(z), free(gap), free(idx), free(w);
    const int S = 300, H = 8, D = 64, K = 32;
    int8_t *q = alloc((size_t)4 * H * D), *kk = alloc((size_t)S * D);
    float *wh = alloc(4 * 4 * H), *ks = alloc(4 * S);
    for (int i = 0; i < 4 * H * D; i++) q[i] = (int8_t)(rnd() % 255 - 127);
    for (int i = 0; i < S * D; i++) kk[i] = (int8_t)(rnd() % 255 - 127);
    for (int i = 0; i < 4 * H; i++) wh[i] = frnd();
    for (int i = 0; i < S; i++) ks[i] = 1.0f + 0.5f * frnd();
    int32_t *top = alloc(4 * 4 * K);
    double *g2 = alloc(8 * 4), *sc = alloc(8 * 4 * S);
    oracle_index_topk(4, S, H, D, K, 10, q, wh, kk, ks, top, g2, sc);
    oracle_index_topk(4, S, H, D, K, S - 4, q, wh, kk, ks, top, g2, NULL);
    free(q), free(kk), free(wh), free(ks), free(top), free(g2), free(sc);
}

int main(void) {
    int bad = 0;
    oracle_set_threads(2);
    bad |= run(5, 64, 8, 3, 32, 32, 8, 0);
    bad |= run(4, 64, 8, 2, 64, 0, 4, 1);
    bad |= run(3, 32, 4, 4, 32, 64, 4, 0);  /* k == E: gap is +inf */
    bad |= run(1, 128, 16, 1, 32, 32, 8, 1);
    run_variants();
    printf(bad ? "batch union and per-token loop differ\n" : "oracle driver ok\n");
    return bad;
}
