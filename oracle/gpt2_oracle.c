/*
 * gpt2_oracle.c -- CPU oracle for batch-1 GPT-2 decode (TEST INFRASTRUCTURE ONLY).
 *
 * Plain, sequential loops.  Every step follows the "model.fir" page (the
 * gpt2-125m model file) node by node, in its order, with its micro-kernels'
 * arithmetic:
 *   - g2.add              : out = a + b
 *   - g2.layernorm        : mean, then biased variance, ((x-mean)*rsqrt(var+eps))*gamma+beta
 *   - g2.gelu_new         : x * sigmoid(2*sqrt(2/pi) * (x + 0.044715*x^3))
 *   - g2.attn_decode      : append K/V at `position`, scores q.k * (1/sqrt(headdim))
 *                           over 0..position, max-subtracted exp, divide by the sum,
 *                           weighted sum of values
 *   - fir.linear          : y = x . W with W in Conv1D [input][output] layout
 *   - fir.linear_t        : logits = wte . n (tied head, no bias)
 * Greedy pick = argmax ("Let's make GPT-2 in assembly", Step 7), lowest index on ties.
 *
 * Build: gcc -O3 -ffp-contract=off (no fast-math), so every product is rounded
 * before it is added and sums run in ascending index order.
 *
 * Pinned by tests/test_oracle_pins.py against: Hugging Face GPT2LMHeadModel in
 * float64 on the same weights, numpy float64 matmul with the inner-product error
 * bound, torch layer_norm / tanh-form gelu, closed-form softmax cases, numpy
 * float16 casts, a brute-force search for the nearest int4 code, the KV-cache-free
 * brute-force recompute and the float64 build of this same file.
 */
#include "gpt2_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef ORACLE_REAL_IS_DOUBLE
#define R_EXP exp
#define R_SQRT sqrt
#else
#define R_EXP expf
#define R_SQRT sqrtf
#endif

typedef oracle_real real;

typedef struct {
    real *ln1_w, *ln1_b;
    real *qkv_w, *qkv_b;  /* [E][3E], [3E] */
    real *ap_w, *ap_b;    /* [E][E],  [E]  */
    real *ln2_w, *ln2_b;
    real *fc_w, *fc_b;    /* [E][F],  [F]  */
    real *pr_w, *pr_b;    /* [F][E],  [E]  */
} layer_t;

struct oracle_model {
    int L, E, H, D, F, P, V, wdtype, group;
    real eps;
    real *wte;   /* [V][E] embedding table (always the fp32 values) */
    real *head;  /* [V][E] output head (fp16-rounded in the fp16 mode) */
    real *wpe;   /* [P][E] */
    real *lnf_w, *lnf_b;
    layer_t *layers;
    real *kc, *vc; /* [L][P][E] key and value caches (model file layout) */
    int filled;
    /* activations of one step (model file buffers) */
    real *x, *pos_embed, *norm, *qkv, *attn, *mix, *fc, *act, *scores, *logits;
};

int oracle_real_bytes(void) { return (int)sizeof(real); }

int oracle_n_tensors(int n_layer) { return 2 + 12 * n_layer + 2; }

/* ------------------------------------------------------------------ */
/* IEEE 754 binary16, round to nearest even, subnormals kept.          */
/* ------------------------------------------------------------------ */
uint16_t oracle_f32_to_f16(float f)
{
    uint32_t x;
    memcpy(&x, &f, 4);
    uint32_t sign = (x >> 16) & 0x8000u;
    uint32_t ex = (x >> 23) & 0xffu;
    uint32_t man = x & 0x7fffffu;
    if (ex == 0xffu) {                      /* inf / nan */
        if (man == 0) return (uint16_t)(sign | 0x7c00u);
        return (uint16_t)(sign | 0x7e00u | (man >> 13));
    }
    int e16 = (int)ex - 127 + 15;           /* biased binary16 exponent */
    if (e16 >= 31) return (uint16_t)(sign | 0x7c00u);
    if (e16 <= 0) {
        /* result is subnormal or zero: value = (man|hidden) * 2^(ex-150);
         * in units of 2^-24 that is (man|hidden) >> (126-ex). */
        if (ex == 0) return (uint16_t)sign;  /* fp32 zero / subnormal: far below 2^-25 */
        uint32_t mm = man | 0x800000u;
        int shift = 126 - (int)ex;           /* >= 14 */
        if (shift >= 25) return (uint16_t)sign; /* < 2^-25 (half of the smallest step): 0 */
        uint32_t q = mm >> shift;
        uint32_t rem = mm & ((1u << shift) - 1u);
        uint32_t half = 1u << (shift - 1);
        if (rem > half || (rem == half && (q & 1u))) q++;
        return (uint16_t)(sign | q);
    }
    uint32_t q = ((uint32_t)e16 << 10) | (man >> 13);
    uint32_t rem = man & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (q & 1u))) q++; /* carry may reach inf: correct */
    return (uint16_t)(sign | q);
}

float oracle_f16_to_f32(uint16_t h)
{
    uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
    uint32_t ex = (h >> 10) & 0x1fu;
    uint32_t man = h & 0x3ffu;
    float out;
    if (ex == 0) {
        out = (float)man * 5.9604644775390625e-08f; /* man * 2^-24, exact */
        uint32_t b;
        memcpy(&b, &out, 4);
        b |= sign;
        memcpy(&out, &b, 4);
        return out;
    }
    uint32_t b;
    if (ex == 31) b = sign | 0x7f800000u | (man << 13);
    else b = sign | ((ex - 15 + 127) << 23) | (man << 13);
    memcpy(&out, &b, 4);
    return out;
}

/* ------------------------------------------------------------------ */
/* Grouped asymmetric int4 (model.fir header: transpose to [out][in],   */
/* then quantise groups along the input).  Reading of the rule:         */
/* lo/hi = group min/max, scale = (hi-lo)/15, zero = lo,                */
/* q = clamp(rint((w-lo)/scale), 0, 15) (q = 0 when scale == 0),        */
/* dequantised weight = fma(q, scale, zero).                            */
/* ------------------------------------------------------------------ */
void oracle_q4_group(const float *w, int n, uint8_t *q, float *s, float *mn, float *deq)
{
    float lo = w[0], hi = w[0];
    for (int i = 1; i < n; i++) {
        if (w[i] < lo) lo = w[i];
        if (w[i] > hi) hi = w[i];
    }
    float scale = (hi - lo) / 15.0f;
    for (int i = 0; i < n; i++) {
        int c = 0;
        if (scale != 0.0f) {
            float r = rintf((w[i] - lo) / scale);
            if (r < 0.0f) r = 0.0f;
            if (r > 15.0f) r = 15.0f;
            c = (int)r;
        }
        q[i] = (uint8_t)c;
        if (deq) deq[i] = fmaf((float)c, scale, lo);
    }
    *s = scale;
    *mn = lo;
}

/* ------------------------------------------------------------------ */
/* Micro-kernels                                                       */
/* ------------------------------------------------------------------ */
void oracle_layernorm(const real *x, const real *g, const real *b, int n, real eps, real *y)
{
    const real inv_n = (real)(1.0 / (double)n);
    real mean = 0;
    for (int i = 0; i < n; i++) mean = mean + x[i];
    mean = mean * inv_n;
    real var = 0;
    for (int i = 0; i < n; i++) {
        real d = x[i] - mean;
        var = var + d * d;
    }
    var = var * inv_n;
    var = var + eps;
    real r = (real)1 / R_SQRT(var);
    for (int i = 0; i < n; i++) {
        real t = x[i] - mean;
        t = t * r;
        t = t * g[i];
        y[i] = t + b[i];
    }
}

real oracle_gelu_new(real x)
{
    const real c3 = (real)0.044715;
    const real k0 = (real)(2.0 * 0.79788456080286535587989211986876); /* 2*sqrt(2/pi) */
    real t = x * x;
    t = t * x;
    t = t * c3;
    t = t + x;
    t = t * k0;
    t = (real)1 / ((real)1 + R_EXP(-t)); /* sigmoid */
    return x * t;
}

void oracle_linear_conv1d(const real *x, const real *W, const real *b, int K, int N, real *y)
{
    /* axpy order: each y[o] still accumulates its products in ascending i */
    for (int o = 0; o < N; o++) y[o] = 0;
    for (int i = 0; i < K; i++) {
        const real xi = x[i];
        const real *row = W + (size_t)i * N;
        for (int o = 0; o < N; o++) y[o] = y[o] + xi * row[o];
    }
    if (b)
        for (int o = 0; o < N; o++) y[o] = y[o] + b[o];
}

void oracle_attn_head(const real *q, const real *Kc, const real *Vc, int pos, int stride,
                      int D, real *probs, real *out)
{
    const real scale = (real)(1.0 / sqrt((double)D));
    real *s = (real *)malloc(sizeof(real) * (size_t)(pos + 1));
    real m = (real)-3e38;
    for (int t = 0; t <= pos; t++) {
        real acc = 0;
        const real *k = Kc + (size_t)t * stride;
        for (int d = 0; d < D; d++) acc = acc + q[d] * k[d];
        acc = acc * scale;
        s[t] = acc;
        if (m < acc) m = acc;
    }
    real sum = 0;
    for (int t = 0; t <= pos; t++) {
        s[t] = R_EXP(s[t] - m);
        sum = sum + s[t];
    }
    for (int t = 0; t <= pos; t++) s[t] = s[t] / sum;
    for (int d = 0; d < D; d++) {
        real acc = 0;
        for (int t = 0; t <= pos; t++) acc = acc + s[t] * Vc[(size_t)t * stride + d];
        out[d] = acc;
    }
    if (probs)
        for (int t = 0; t <= pos; t++) probs[t] = s[t];
    free(s);
}

static int argmax_lowest(const real *v, int n)
{
    int best = 0;
    for (int i = 1; i < n; i++)
        if (v[i] > v[best]) best = i;
    return best;
}

/* ------------------------------------------------------------------ */
/* Model construction                                                  */
/* ------------------------------------------------------------------ */
static real *alloc_real(size_t n)
{
    return (real *)calloc(n ? n : 1, sizeof(real));
}

static real *copy_real(const float *src, size_t n)
{
    real *d = alloc_real(n);
    if (!d) return NULL;
    for (size_t i = 0; i < n; i++) d[i] = (real)src[i];
    return d;
}

/* Effective value of a block matrix W[K][N] (Conv1D) under the weight mode,
 * returned in the same [K][N] layout. */
static real *quantised_block(const float *W, int K, int N, int wdtype, int group)
{
    real *d = alloc_real((size_t)K * N);
    if (!d) return NULL;
    if (wdtype == ORACLE_W_FP32) {
        for (size_t i = 0; i < (size_t)K * N; i++) d[i] = (real)W[i];
    } else if (wdtype == ORACLE_W_FP16) {
        for (size_t i = 0; i < (size_t)K * N; i++) d[i] = (real)oracle_f16_to_f32(oracle_f32_to_f16(W[i]));
    } else {
        /* transpose to [N][K] rows, quantise groups of `group` inputs, write back */
        float *g = (float *)malloc(sizeof(float) * (size_t)group);
        float *dq = (float *)malloc(sizeof(float) * (size_t)group);
        uint8_t *qc = (uint8_t *)malloc((size_t)group);
        if (!g || !dq || !qc) { free(g); free(dq); free(qc); free(d); return NULL; }
        for (int o = 0; o < N; o++) {
            for (int k0 = 0; k0 < K; k0 += group) {
                for (int j = 0; j < group; j++) g[j] = W[(size_t)(k0 + j) * N + o];
                float s, mn;
                oracle_q4_group(g, group, qc, &s, &mn, dq);
                for (int j = 0; j < group; j++) d[(size_t)(k0 + j) * N + o] = (real)dq[j];
            }
        }
        free(g); free(dq); free(qc);
    }
    return d;
}

void oracle_free(oracle_model *m)
{
    if (!m) return;
    free(m->wte); free(m->head); free(m->wpe); free(m->lnf_w); free(m->lnf_b);
    if (m->layers) {
        for (int l = 0; l < m->L; l++) {
            layer_t *ly = &m->layers[l];
            free(ly->ln1_w); free(ly->ln1_b); free(ly->qkv_w); free(ly->qkv_b);
            free(ly->ap_w); free(ly->ap_b); free(ly->ln2_w); free(ly->ln2_b);
            free(ly->fc_w); free(ly->fc_b); free(ly->pr_w); free(ly->pr_b);
        }
        free(m->layers);
    }
    free(m->kc); free(m->vc);
    free(m->x); free(m->pos_embed); free(m->norm); free(m->qkv); free(m->attn);
    free(m->mix); free(m->fc); free(m->act); free(m->scores); free(m->logits);
    free(m);
}

oracle_model *oracle_new(const int *shape, float ln_eps, int wdtype, int q4_group,
                         const float *const *t)
{
    int L = shape[0], E = shape[1], H = shape[2], P = shape[3], V = shape[4];
    if (L <= 0 || E <= 0 || H <= 0 || P <= 0 || V <= 0 || E % H != 0) return NULL;
    if (wdtype < 0 || wdtype > 2) return NULL;
    int F = 4 * E;
    if (wdtype == ORACLE_W_INT4 && (q4_group <= 0 || E % q4_group != 0 || F % q4_group != 0))
        return NULL;
    oracle_model *m = (oracle_model *)calloc(1, sizeof(oracle_model));
    if (!m) return NULL;
    m->L = L; m->E = E; m->H = H; m->D = E / H; m->F = F; m->P = P; m->V = V;
    m->wdtype = wdtype; m->group = q4_group; m->eps = (real)ln_eps;
    int ok = 1;
    m->wte = copy_real(t[0], (size_t)V * E);
    if (wdtype == ORACLE_W_FP16) {
        m->head = alloc_real((size_t)V * E);
        if (m->head)
            for (size_t i = 0; i < (size_t)V * E; i++)
                m->head[i] = (real)oracle_f16_to_f32(oracle_f32_to_f16(t[0][i]));
    } else {
        m->head = copy_real(t[0], (size_t)V * E);
    }
    m->wpe = copy_real(t[1], (size_t)P * E);
    m->layers = (layer_t *)calloc((size_t)L, sizeof(layer_t));
    ok = m->wte && m->head && m->wpe && m->layers;
    for (int l = 0; ok && l < L; l++) {
        const float *const *p = t + 2 + 12 * l;
        layer_t *ly = &m->layers[l];
        ly->ln1_w = copy_real(p[0], E);
        ly->ln1_b = copy_real(p[1], E);
        ly->qkv_w = quantised_block(p[2], E, 3 * E, wdtype, q4_group);
        ly->qkv_b = copy_real(p[3], 3 * E);
        ly->ap_w = quantised_block(p[4], E, E, wdtype, q4_group);
        ly->ap_b = copy_real(p[5], E);
        ly->ln2_w = copy_real(p[6], E);
        ly->ln2_b = copy_real(p[7], E);
        ly->fc_w = quantised_block(p[8], E, F, wdtype, q4_group);
        ly->fc_b = copy_real(p[9], F);
        ly->pr_w = quantised_block(p[10], F, E, wdtype, q4_group);
        ly->pr_b = copy_real(p[11], E);
        ok = ly->ln1_w && ly->ln1_b && ly->qkv_w && ly->qkv_b && ly->ap_w && ly->ap_b &&
             ly->ln2_w && ly->ln2_b && ly->fc_w && ly->fc_b && ly->pr_w && ly->pr_b;
    }
    if (ok) {
        const float *const *p = t + 2 + 12 * L;
        m->lnf_w = copy_real(p[0], E);
        m->lnf_b = copy_real(p[1], E);
        m->kc = alloc_real((size_t)L * P * E);
        m->vc = alloc_real((size_t)L * P * E);
        m->x = alloc_real(E); m->pos_embed = alloc_real(E); m->norm = alloc_real(E);
        m->qkv = alloc_real(3 * (size_t)E); m->attn = alloc_real(E); m->mix = alloc_real(E);
        m->fc = alloc_real(F); m->act = alloc_real(F);
        m->scores = alloc_real((size_t)H * P); m->logits = alloc_real(V);
        ok = m->lnf_w && m->lnf_b && m->kc && m->vc && m->x && m->pos_embed && m->norm &&
             m->qkv && m->attn && m->mix && m->fc && m->act && m->scores && m->logits;
    }
    if (!ok) { oracle_free(m); return NULL; }
    return m;
}

void oracle_reset(oracle_model *m) { m->filled = 0; }

void oracle_poison_cache_after(oracle_model *m, int position, float value)
{
    for (int l = 0; l < m->L; l++)
        for (int t = position + 1; t < m->P; t++)
            for (int i = 0; i < m->E; i++) {
                size_t o = ((size_t)l * m->P + t) * m->E + i;
                m->kc[o] = (real)value;
                m->vc[o] = (real)value;
            }
}

/* The per-layer node sequence of the model file, for one position whose
 * residual stream is in x; kc/vc are this layer's caches ([P][E]). */
static void layer_forward(oracle_model *m, const layer_t *ly, real *kc, real *vc, int pos,
                          real *x)
{
    const int E = m->E, D = m->D, F = m->F;
    oracle_layernorm(x, ly->ln1_w, ly->ln1_b, E, m->eps, m->norm);          /* ln1 */
    oracle_linear_conv1d(m->norm, ly->qkv_w, NULL, E, 3 * E, m->qkv);        /* qkv_linear */
    for (int o = 0; o < 3 * E; o++) m->qkv[o] = m->qkv[o] + ly->qkv_b[o];  /* qkv_bias */
    /* attention: append this position's K/V, then one head at a time */
    for (int i = 0; i < E; i++) {
        kc[(size_t)pos * E + i] = m->qkv[E + i];
        vc[(size_t)pos * E + i] = m->qkv[2 * E + i];
    }
    for (int h = 0; h < m->H; h++)
        oracle_attn_head(m->qkv + h * D, kc + h * D, vc + h * D, pos, E, D,
                         m->scores + (size_t)h * m->P, m->attn + h * D);
    oracle_linear_conv1d(m->attn, ly->ap_w, NULL, E, E, m->mix);             /* attention_linear */
    for (int o = 0; o < E; o++) m->mix[o] = m->mix[o] + ly->ap_b[o];        /* attention_bias */
    for (int o = 0; o < E; o++) x[o] = x[o] + m->mix[o];                    /* attention_residual */
    oracle_layernorm(x, ly->ln2_w, ly->ln2_b, E, m->eps, m->norm);          /* ln2 */
    oracle_linear_conv1d(m->norm, ly->fc_w, NULL, E, F, m->fc);              /* fc_linear */
    for (int o = 0; o < F; o++) m->fc[o] = m->fc[o] + ly->fc_b[o];          /* fc_bias */
    for (int o = 0; o < F; o++) m->act[o] = oracle_gelu_new(m->fc[o]);      /* gelu */
    oracle_linear_conv1d(m->act, ly->pr_w, NULL, F, E, m->mix);              /* proj_linear */
    for (int o = 0; o < E; o++) m->mix[o] = m->mix[o] + ly->pr_b[o];        /* proj_bias */
    for (int o = 0; o < E; o++) x[o] = x[o] + m->mix[o];                    /* mlp_residual */
}

static void head_forward(oracle_model *m, const real *x, real *logits)
{
    const int E = m->E;
    oracle_layernorm(x, m->lnf_w, m->lnf_b, E, m->eps, m->norm);            /* final_norm */
    for (int v = 0; v < m->V; v++) {                                         /* head (linear_t) */
        const real *row = m->head + (size_t)v * E;
        real acc = 0;
        for (int i = 0; i < E; i++) acc = acc + row[i] * m->norm[i];
        logits[v] = acc;
    }
}

int oracle_step(oracle_model *m, int token, int position, real *logits_out)
{
    if (!m || token < 0 || token >= m->V || position < 0 || position >= m->P ||
        position > m->filled)
        return -1;
    const int E = m->E;
    for (int i = 0; i < E; i++) {                                            /* token, positional */
        m->x[i] = m->wte[(size_t)token * E + i];
        m->pos_embed[i] = m->wpe[(size_t)position * E + i];
    }
    for (int i = 0; i < E; i++) m->x[i] = m->x[i] + m->pos_embed[i];         /* embeddings */
    for (int l = 0; l < m->L; l++)
        layer_forward(m, &m->layers[l], m->kc + (size_t)l * m->P * E,
                      m->vc + (size_t)l * m->P * E, position, m->x);
    head_forward(m, m->x, m->logits);
    m->filled = position + 1;
    if (logits_out)
        for (int v = 0; v < m->V; v++) logits_out[v] = m->logits[v];
    return argmax_lowest(m->logits, m->V);
}

int oracle_prefill_last(oracle_model *m, const int *toks, int n, real *logits_out)
{
    if (!m || n <= 0 || n > m->P) return -1;
    for (int t = 0; t < n; t++)
        if (toks[t] < 0 || toks[t] >= m->V) return -1;
    const int E = m->E;
    /* private caches and residual streams: one row per position */
    real *X = alloc_real((size_t)n * E);
    real *kc = alloc_real((size_t)n * E);
    real *vc = alloc_real((size_t)n * E);
    real *logits = alloc_real(m->V);
    if (!X || !kc || !vc || !logits) { free(X); free(kc); free(vc); free(logits); return -1; }
    for (int t = 0; t < n; t++)
        for (int i = 0; i < E; i++)
            X[(size_t)t * E + i] = m->wte[(size_t)toks[t] * E + i] + m->wpe[(size_t)t * E + i];
    /* layer by layer over the whole sequence; the K/V rows of every position
     * are rebuilt from the sequence itself in each layer */
    for (int l = 0; l < m->L; l++)
        for (int t = 0; t < n; t++)
            layer_forward(m, &m->layers[l], kc, vc, t, X + (size_t)t * E);
    head_forward(m, X + (size_t)(n - 1) * E, logits);
    int am = argmax_lowest(logits, m->V);
    if (logits_out)
        for (int v = 0; v < m->V; v++) logits_out[v] = logits[v];
    free(X); free(kc); free(vc); free(logits);
    return am;
}

long oracle_get_weight(const oracle_model *m, int layer, int which, float *out)
{
    const real *W;
    int K, N;
    if (which == 4) {
        for (size_t i = 0; i < (size_t)m->V * m->E; i++) out[i] = (float)m->head[i];
        return (long)m->V * m->E;
    }
    if (layer < 0 || layer >= m->L) return -1;
    const layer_t *ly = &m->layers[layer];
    switch (which) {
    case 0: W = ly->qkv_w; K = m->E; N = 3 * m->E; break;
    case 1: W = ly->ap_w; K = m->E; N = m->E; break;
    case 2: W = ly->fc_w; K = m->E; N = m->F; break;
    case 3: W = ly->pr_w; K = m->F; N = m->E; break;
    default: return -1;
    }
    for (int o = 0; o < N; o++)
        for (int k = 0; k < K; k++) out[(size_t)o * K + k] = (float)W[(size_t)k * N + o];
    return (long)N * K;
}
