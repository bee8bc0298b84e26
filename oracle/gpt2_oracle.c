/*
 * gpt2_oracle.c -- CPU oracle for batch-1 GPT-2 decode (TEST INFRASTRUCTURE ONLY).
 *
 * A plain, slow, single-threaded statement of what one decode step computes,
 * written from the textbook definition of the GPT-2 network rather than from
 * any listing: a pre-LayerNorm transformer decoder whose blocks are
 *
 *   h <- h + Attn(LN_1(h)),   h <- h + MLP(LN_2(h)),
 *
 * followed by a final LayerNorm and an output head that reuses the token
 * embedding matrix (the gpt2-125m model file's header and node list; "Let's
 * make GPT-2 in assembly", Steps 4-7).  Each piece below is its defining
 * formula written out:
 *
 *   LayerNorm   y_i = gamma_i * (x_i - mu) / sqrt(sigma^2 + eps) + beta_i,
 *               mu and sigma^2 the mean and the biased variance of x
 *   gelu_new    x * logistic(2 * sqrt(2/pi) * (x + 0.044715 x^3)), the tanh
 *               approximation of GELU, 0.5 x (1 + tanh(z)) = x * logistic(2z)
 *               (model file, gelu_new comment; the blog writes the tanh form)
 *   attention   per head, softmax over t = 0..p of q.k_t / sqrt(headdim), the
 *               weights then applied to the values v_t (blog Step 6; the
 *               model file's decode attention reads positions 0..p only)
 *   linear      y = x W + b with W stored [input][output] (Hugging Face Conv1D,
 *               as both pages note)
 *   head        logits_v = wte_v . LN_f(h), no bias (tied to wte)
 *   greedy      the id of the largest logit, the lowest id among equal ones
 *   sampling    (blog Step 7; gpt2.s docs "-t") weights exp((l_i - max l)/T),
 *               the first id whose running sum of weights exceeds u times
 *               their total, u uniform in [0,1) drawn with xorshift64*
 *
 * Keys and values of earlier positions depend only on the tokens up to them,
 * so each is computed once and kept (the blog's cache); oracle_prefill_last
 * recomputes them from the token sequence alone, for the cache check.
 *
 * Arithmetic: sums run sequentially in ascending index order; the build uses
 * -O3 -ffp-contract=off without fast-math, so every product is rounded before
 * it is added.  `real` is float (the precision the model file fixes: every
 * buffer is f32) or double (a second build that bounds the float build's
 * drift).  Quantised weights are always formed in float, since they define the
 * model being run.
 *
 * The HIP library shares no code with this file; tests/test_oracle_pins.py
 * pins it to Hugging Face GPT-2 in float64, numpy, torch, scipy, closed forms,
 * invariants and brute force.
 */
#include "gpt2_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef ORACLE_REAL_IS_DOUBLE
#define EXP_R exp
#define SQRT_R sqrt
#else
#define EXP_R expf
#define SQRT_R sqrtf
#endif

typedef oracle_real real;

/* One transformer block's parameters.  Matrices in the checkpoint's
 * [input][output] layout, already replaced by their effective (rounded or
 * quantised) values. */
typedef struct {
    real *gamma1, *beta1;        /* LayerNorm before attention      [E] */
    real *w_qkv, *b_qkv;         /* query|key|value projection  [E][3E], [3E] */
    real *w_out, *b_out;         /* attention output projection [E][E],  [E] */
    real *gamma2, *beta2;        /* LayerNorm before the MLP        [E] */
    real *w_up, *b_up;           /* MLP expansion               [E][4E], [4E] */
    real *w_down, *b_down;       /* MLP contraction             [4E][E], [E] */
} block_params;

struct oracle_model {
    int n_layer, d_model, n_heads, d_head, d_ff, n_ctx, n_vocab, wmode, qgroup;
    real eps;
    real *tok_emb;      /* [V][E] token embedding (always the fp32 values)       */
    real *unembed;      /* [V][E] output head: tok_emb, fp16-rounded in fp16 mode */
    real *pos_emb;      /* [P][E] */
    real *gamma_f, *beta_f;
    block_params *blocks;
    real *keys, *values; /* [L][P][E]: key and value of each position, per layer */
    int n_cached;        /* positions 0..n_cached-1 hold valid keys and values   */
};

int oracle_real_bytes(void) { return (int)sizeof(real); }

/* wte, wpe, 12 tensors per block, ln_f weight and bias. */
int oracle_n_tensors(int n_layer) { return 4 + 12 * n_layer; }

/* ------------------------------------------------------------------ */
/* IEEE 754 binary16 with round-to-nearest-even, subnormals kept       */
/* (gpt2.s docs: "-h" stores the matrices fp16, products stay fp32).   */
/* ------------------------------------------------------------------ */
uint16_t oracle_f32_to_f16(float f)
{
    uint32_t bits;
    memcpy(&bits, &f, 4);
    const uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
    const int exp32 = (int)((bits >> 23) & 0xffu);
    const uint32_t frac = bits & 0x7fffffu;
    if (exp32 == 0xff) /* infinity keeps its sign; a NaN stays quiet with its top payload bits */
        return (uint16_t)(sign | 0x7c00u | (frac ? 0x200u | (frac >> 13) : 0u));
    if (exp32 == 0) return sign; /* zero or fp32 subnormal: below half the smallest fp16 step */
    /* |f| = sig * 2^(exp32 - 150) with a 24-bit significand sig */
    const uint32_t sig = frac | 0x800000u;
    const int e = exp32 - 127;               /* unbiased exponent */
    uint32_t keep;                           /* significand bits kept, before rounding */
    int drop;                                /* low bits of sig rounded away */
    uint32_t base;                           /* exponent field to add */
    if (e >= -14) {                          /* a normal fp16 if it does not overflow */
        drop = 13;
        base = (uint32_t)(e + 15) << 10;
        keep = (sig >> drop) & 0x3ffu;       /* 10 fraction bits; the hidden bit is in base */
    } else {                                 /* subnormal fp16: units of 2^-24 */
        drop = -e - 1;                       /* 14 .. 126 */
        if (drop > 24) return sign;          /* below 2^-25: rounds to zero */
        base = 0;
        keep = sig >> drop;
    }
    uint32_t out = base + keep;              /* exponent carries are the right result */
    const uint32_t rest = sig & ((1u << drop) - 1u), half = 1u << (drop - 1);
    if (rest > half || (rest == half && (out & 1u))) out += 1; /* may carry into the exponent */
    if (out >= 0x7c00u) out = 0x7c00u;       /* overflow: infinity */
    return (uint16_t)(sign | out);
}

float oracle_f16_to_f32(uint16_t h)
{
    const int e = (h >> 10) & 0x1f;
    const int m = h & 0x3ff;
    float mag;
    if (e == 0x1f) mag = m ? NAN : INFINITY;
    else if (e == 0) mag = ldexpf((float)m, -24);         /* subnormal: m * 2^-24 */
    else mag = ldexpf((float)(m | 0x400), e - 25);        /* (1024 + m) * 2^(e-25) */
    return (h & 0x8000u) ? -mag : mag;
}

/* ------------------------------------------------------------------ */
/* Grouped asymmetric int4 (model file header: the loader transposes   */
/* each block matrix to [output][input], then quantises groups of      */
/* inputs of each output row).  Reading of the unstated details: the   */
/* group's minimum is the zero point and (max - min)/15 the step; a    */
/* weight takes the nearest of the 16 levels (round half to even,      */
/* clamped to 0..15; every code 0 when the step is 0); the level is    */
/* zero + code * step with one rounding.                               */
/* ------------------------------------------------------------------ */
void oracle_q4_group(const float *w, int n, uint8_t *q, float *s, float *mn, float *deq)
{
    float lo = INFINITY, hi = -INFINITY;
    for (int i = 0; i < n; i++) {
        lo = fminf(lo, w[i]);
        hi = fmaxf(hi, w[i]);
    }
    const float step = (hi - lo) / 15.0f;
    for (int i = 0; i < n; i++) {
        float code = 0.0f;
        if (step != 0.0f) code = fminf(fmaxf(rintf((w[i] - lo) / step), 0.0f), 15.0f);
        q[i] = (uint8_t)code;
        if (deq) deq[i] = fmaf(code, step, lo);
    }
    *s = step;
    *mn = lo;
}

/* ------------------------------------------------------------------ */
/* The pieces of the network, each its defining formula               */
/* ------------------------------------------------------------------ */
void oracle_layernorm(const real *x, const real *gamma, const real *beta, int n, real eps, real *y)
{
    real sum = 0;
    for (int i = 0; i < n; i++) sum += x[i];
    const real mu = sum / (real)n;
    real sq = 0;
    for (int i = 0; i < n; i++) sq += (x[i] - mu) * (x[i] - mu);
    const real sigma = SQRT_R(sq / (real)n + eps);
    for (int i = 0; i < n; i++) y[i] = gamma[i] * ((x[i] - mu) / sigma) + beta[i];
}

real oracle_gelu_new(real x)
{
    const real root_2_over_pi = (real)0.79788456080286535588; /* sqrt(2/pi) */
    const real z = root_2_over_pi * (x + (real)0.044715 * (x * x * x));
    return x / ((real)1 + EXP_R(-(real)2 * z)); /* x * logistic(2z) */
}

void oracle_linear_conv1d(const real *x, const real *W, const real *b, int K, int N, real *y)
{
    /* y_o = sum_i x_i W[i][o] (+ b_o): the rows of W are visited in order, so
     * each y_o still adds its products in ascending i */
    for (int o = 0; o < N; o++) y[o] = 0;
    for (int i = 0; i < K; i++)
        for (int o = 0; o < N; o++) y[o] += x[i] * W[(size_t)i * N + o];
    if (b)
        for (int o = 0; o < N; o++) y[o] += b[o];
}

void oracle_attn_head(const real *q, const real *Kc, const real *Vc, int pos, int stride, int D,
                      real *probs, real *out)
{
    const int n = pos + 1; /* positions 0..pos, nothing later */
    real *w = n > 0 ? (real *)malloc(sizeof(real) * (size_t)n) : NULL;
    if (!w) {
        for (int d = 0; d < D; d++) out[d] = (real)NAN; /* no positions (or no memory): nothing to attend */
        return;
    }
    const real root_d = (real)sqrt((double)D);
    for (int t = 0; t < n; t++) {
        real dot = 0;
        for (int d = 0; d < D; d++) dot += q[d] * Kc[(size_t)t * stride + d];
        w[t] = dot / root_d;
    }
    real top = w[0];
    for (int t = 1; t < n; t++) top = w[t] > top ? w[t] : top;
    real z = 0;
    for (int t = 0; t < n; t++) {
        w[t] = EXP_R(w[t] - top);
        z += w[t];
    }
    for (int t = 0; t < n; t++) w[t] /= z; /* softmax weights */
    for (int d = 0; d < D; d++) {
        real acc = 0;
        for (int t = 0; t < n; t++) acc += w[t] * Vc[(size_t)t * stride + d];
        out[d] = acc;
    }
    if (probs) memcpy(probs, w, sizeof(real) * (size_t)n);
    free(w);
}

int oracle_argmax(const real *v, int n)
{
    int best = 0;
    for (int i = 1; i < n; i++)
        if (v[i] > v[best]) best = i; /* strictly larger: ties keep the lower id */
    return best;
}

/* xorshift64* (S. Vigna, "An experimental exploration of Marsaglia's xorshift
 * generators, scrambled", ACM TOMS 42(4), 2016): the xorshift state update
 * with shift triple (12, 25, 27), output scrambled by the multiplier
 * 2685821657736338717. */
uint64_t oracle_xorshift64s(uint64_t *state)
{
    uint64_t s = *state;
    s ^= s >> 12;
    s ^= s << 25;
    s ^= s >> 27;
    *state = s;
    return s * 2685821657736338717ull;
}

/* A uniform number in [0,1) from one draw: its top 24 bits times 2^-24
 * (exact in float). */
float oracle_uniform(uint64_t *state)
{
    return (float)(oracle_xorshift64s(state) >> 40) * 0x1p-24f;
}

int oracle_sample(const real *logits, int n, real temperature, real u)
{
    if (n < 1 || !(temperature >= 0) || !(u >= 0 && u < 1)) return -1;
    const int top = oracle_argmax(logits, n);
    if (temperature == 0) return top; /* greedy */
    real *w = (real *)malloc(sizeof(real) * (size_t)n);
    if (!w) return -1;
    real total = 0;
    for (int i = 0; i < n; i++) {
        w[i] = EXP_R((logits[i] - logits[top]) / temperature);
        total += w[i];
    }
    const real target = u * total;
    real run = 0;
    int pick = -1, last = top;
    for (int i = 0; i < n && pick < 0; i++) {
        if (w[i] > 0) last = i;
        run += w[i];
        if (run > target) pick = i;
    }
    /* rounding can leave the running total a hair under u * total */
    if (pick < 0) {
        for (int i = n - 1; i >= 0; i--)
            if (w[i] > 0) { last = i; break; }
        pick = last;
    }
    free(w);
    return pick;
}

/* ------------------------------------------------------------------ */
/* Model construction                                                  */
/* ------------------------------------------------------------------ */
static real *zeros(size_t n) { return (real *)calloc(n ? n : 1, sizeof(real)); }

static real *widen(const float *src, size_t n)
{
    real *d = zeros(n);
    if (d)
        for (size_t i = 0; i < n; i++) d[i] = (real)src[i];
    return d;
}

/* The weights a block matrix W[K][N] ([input][output]) stands for in the
 * chosen storage, still as [K][N]: fp32 as is; fp16 each weight rounded to
 * binary16; int4 each output's column cut into groups of `group` consecutive
 * inputs, each group quantised on its own. */
static real *effective_matrix(const float *W, int K, int N, int mode, int group)
{
    real *out = zeros((size_t)K * N);
    if (!out) return NULL;
    if (mode != ORACLE_W_INT4) {
        for (size_t i = 0; i < (size_t)K * N; i++)
            out[i] = mode == ORACLE_W_FP16 ? (real)oracle_f16_to_f32(oracle_f32_to_f16(W[i])) : (real)W[i];
        return out;
    }
    float *col = (float *)malloc(sizeof(float) * (size_t)group * 2);
    uint8_t *codes = (uint8_t *)malloc((size_t)group);
    if (!col || !codes) {
        free(col); free(codes); free(out);
        return NULL;
    }
    float *deq = col + group;
    for (int o = 0; o < N; o++)
        for (int k0 = 0; k0 < K; k0 += group) {
            float step, zero;
            for (int j = 0; j < group; j++) col[j] = W[(size_t)(k0 + j) * N + o];
            oracle_q4_group(col, group, codes, &step, &zero, deq);
            for (int j = 0; j < group; j++) out[(size_t)(k0 + j) * N + o] = (real)deq[j];
        }
    free(col);
    free(codes);
    return out;
}

void oracle_free(oracle_model *m)
{
    if (!m) return;
    if (m->blocks)
        for (int l = 0; l < m->n_layer; l++) {
            block_params *b = &m->blocks[l];
            real *all[] = {b->gamma1, b->beta1, b->w_qkv, b->b_qkv, b->w_out, b->b_out,
                           b->gamma2, b->beta2, b->w_up, b->b_up, b->w_down, b->b_down};
            for (size_t i = 0; i < sizeof all / sizeof all[0]; i++) free(all[i]);
        }
    free(m->blocks);
    free(m->tok_emb); free(m->unembed); free(m->pos_emb); free(m->gamma_f); free(m->beta_f);
    free(m->keys); free(m->values);
    free(m);
}

oracle_model *oracle_new(const int *shape, float ln_eps, int wdtype, int q4_group,
                         const float *const *t)
{
    const int L = shape[0], E = shape[1], H = shape[2], P = shape[3], V = shape[4];
    if (L < 1 || E < 1 || H < 1 || P < 1 || V < 1 || E % H) return NULL;
    if (wdtype < ORACLE_W_FP32 || wdtype > ORACLE_W_INT4) return NULL;
    if (wdtype == ORACLE_W_INT4 && (q4_group < 1 || E % q4_group)) return NULL; /* 4E then divides too */
    oracle_model *m = (oracle_model *)calloc(1, sizeof *m);
    if (!m) return NULL;
    m->n_layer = L; m->d_model = E; m->n_heads = H; m->d_head = E / H; m->d_ff = 4 * E;
    m->n_ctx = P; m->n_vocab = V; m->wmode = wdtype; m->qgroup = q4_group; m->eps = (real)ln_eps;
    const int F = m->d_ff;
    /* the flat list: wte, wpe, then per block in checkpoint order, then ln_f */
    m->tok_emb = widen(t[0], (size_t)V * E);
    m->unembed = zeros((size_t)V * E);
    if (m->unembed)
        for (size_t i = 0; i < (size_t)V * E; i++)
            m->unembed[i] = wdtype == ORACLE_W_FP16 ? (real)oracle_f16_to_f32(oracle_f32_to_f16(t[0][i]))
                                                    : (real)t[0][i];
    m->pos_emb = widen(t[1], (size_t)P * E);
    m->blocks = (block_params *)calloc((size_t)L, sizeof(block_params));
    int ok = m->tok_emb && m->unembed && m->pos_emb && m->blocks;
    for (int l = 0; ok && l < L; l++) {
        const float *const *p = t + 2 + 12 * l;
        block_params *b = &m->blocks[l];
        b->gamma1 = widen(p[0], E);
        b->beta1 = widen(p[1], E);
        b->w_qkv = effective_matrix(p[2], E, 3 * E, wdtype, q4_group);
        b->b_qkv = widen(p[3], 3 * (size_t)E);
        b->w_out = effective_matrix(p[4], E, E, wdtype, q4_group);
        b->b_out = widen(p[5], E);
        b->gamma2 = widen(p[6], E);
        b->beta2 = widen(p[7], E);
        b->w_up = effective_matrix(p[8], E, F, wdtype, q4_group);
        b->b_up = widen(p[9], F);
        b->w_down = effective_matrix(p[10], F, E, wdtype, q4_group);
        b->b_down = widen(p[11], E);
        ok = b->gamma1 && b->beta1 && b->w_qkv && b->b_qkv && b->w_out && b->b_out && b->gamma2 &&
             b->beta2 && b->w_up && b->b_up && b->w_down && b->b_down;
    }
    if (ok) {
        m->gamma_f = widen(t[2 + 12 * L], E);
        m->beta_f = widen(t[3 + 12 * L], E);
        m->keys = zeros((size_t)L * P * E);
        m->values = zeros((size_t)L * P * E);
        ok = m->gamma_f && m->beta_f && m->keys && m->values;
    }
    if (!ok) {
        oracle_free(m);
        return NULL;
    }
    return m;
}

void oracle_reset(oracle_model *m) { m->n_cached = 0; }

void oracle_poison_cache_after(oracle_model *m, int position, float value)
{
    const size_t E = (size_t)m->d_model;
    for (int l = 0; l < m->n_layer; l++)
        for (int t = position + 1; t < m->n_ctx; t++)
            for (size_t i = 0; i < E; i++) {
                m->keys[((size_t)l * m->n_ctx + t) * E + i] = (real)value;
                m->values[((size_t)l * m->n_ctx + t) * E + i] = (real)value;
            }
}

/* ------------------------------------------------------------------ */
/* The forward pass                                                    */
/* ------------------------------------------------------------------ */

/* Scratch vectors of one position's pass through a block. */
typedef struct {
    real *a;     /* normalised input of a sub-layer     [E]  */
    real *qkv;   /* query | key | value                 [3E] */
    real *ctx;   /* attention output, heads side by side [E]  */
    real *proj;  /* a sub-layer's output before the add [E]  */
    real *up;    /* MLP hidden activations              [4E] */
} work_vecs;

static int work_alloc(work_vecs *w, int E)
{
    w->a = zeros(E); w->qkv = zeros(3 * (size_t)E); w->ctx = zeros(E); w->proj = zeros(E);
    w->up = zeros(4 * (size_t)E);
    return w->a && w->qkv && w->ctx && w->proj && w->up;
}

static void work_free(work_vecs *w)
{
    free(w->a); free(w->qkv); free(w->ctx); free(w->proj); free(w->up);
}

/* h <- h + Attn(LN_1(h)) for one position t.  The query is this position's;
 * keys/values of positions 0..t are rows of `kv_k` / `kv_v`, `kv_stride`
 * apart, and this position's own key and value are written to row t first. */
static void attention_sublayer(const oracle_model *m, const block_params *b, real *h, int t, real *kv_k,
                               real *kv_v, int kv_stride, work_vecs *w)
{
    const int E = m->d_model, Dh = m->d_head;
    oracle_layernorm(h, b->gamma1, b->beta1, E, m->eps, w->a);
    oracle_linear_conv1d(w->a, b->w_qkv, b->b_qkv, E, 3 * E, w->qkv);
    memcpy(kv_k + (size_t)t * kv_stride, w->qkv + E, sizeof(real) * (size_t)E);
    memcpy(kv_v + (size_t)t * kv_stride, w->qkv + 2 * E, sizeof(real) * (size_t)E);
    for (int hd = 0; hd < m->n_heads; hd++)
        oracle_attn_head(w->qkv + hd * Dh, kv_k + hd * Dh, kv_v + hd * Dh, t, kv_stride, Dh, NULL,
                         w->ctx + hd * Dh);
    oracle_linear_conv1d(w->ctx, b->w_out, b->b_out, E, E, w->proj);
    for (int i = 0; i < E; i++) h[i] += w->proj[i];
}

/* h <- h + MLP(LN_2(h)), MLP(a) = gelu_new(a W_up + b_up) W_down + b_down. */
static void mlp_sublayer(const oracle_model *m, const block_params *b, real *h, work_vecs *w)
{
    const int E = m->d_model, F = m->d_ff;
    oracle_layernorm(h, b->gamma2, b->beta2, E, m->eps, w->a);
    oracle_linear_conv1d(w->a, b->w_up, b->b_up, E, F, w->up);
    for (int i = 0; i < F; i++) w->up[i] = oracle_gelu_new(w->up[i]);
    oracle_linear_conv1d(w->up, b->w_down, b->b_down, F, E, w->proj);
    for (int i = 0; i < E; i++) h[i] += w->proj[i];
}

/* logits_v = unembed_v . LN_f(h) */
static void output_head(const oracle_model *m, const real *h, real *a, real *logits)
{
    const int E = m->d_model;
    oracle_layernorm(h, m->gamma_f, m->beta_f, E, m->eps, a);
    for (int v = 0; v < m->n_vocab; v++) {
        real dot = 0;
        for (int i = 0; i < E; i++) dot += m->unembed[(size_t)v * E + i] * a[i];
        logits[v] = dot;
    }
}

static void embed(const oracle_model *m, int token, int position, real *h)
{
    const int E = m->d_model;
    for (int i = 0; i < E; i++)
        h[i] = m->tok_emb[(size_t)token * E + i] + m->pos_emb[(size_t)position * E + i];
}

int oracle_step(oracle_model *m, int token, int position, real *logits_out)
{
    if (!m || token < 0 || token >= m->n_vocab || position < 0 || position >= m->n_ctx ||
        position > m->n_cached)
        return -1;
    const int E = m->d_model;
    real *h = zeros(E), *logits = zeros(m->n_vocab);
    work_vecs w;
    int ok = work_alloc(&w, E) && h && logits;
    int id = -1;
    if (ok) {
        embed(m, token, position, h);
        for (int l = 0; l < m->n_layer; l++) {
            const size_t layer_rows = (size_t)l * m->n_ctx * E;
            attention_sublayer(m, &m->blocks[l], h, position, m->keys + layer_rows, m->values + layer_rows, E,
                               &w);
            mlp_sublayer(m, &m->blocks[l], h, &w);
        }
        output_head(m, h, w.a, logits);
        /* a position at or below the cached ones rewinds: its rows were rewritten */
        m->n_cached = position + 1;
        if (logits_out) memcpy(logits_out, logits, sizeof(real) * (size_t)m->n_vocab);
        id = oracle_argmax(logits, m->n_vocab);
    }
    work_free(&w);
    free(h);
    free(logits);
    return id;
}

int oracle_prefill_last(oracle_model *m, const int *toks, int n, real *logits_out)
{
    if (!m || n < 1 || n > m->n_ctx) return -1;
    for (int t = 0; t < n; t++)
        if (toks[t] < 0 || toks[t] >= m->n_vocab) return -1;
    const int E = m->d_model;
    /* every position's hidden state, and one block's keys and values rebuilt
     * from the sequence itself (nothing is taken from the decode cache) */
    real *H = zeros((size_t)n * E), *K = zeros((size_t)n * E), *Vv = zeros((size_t)n * E);
    real *logits = zeros(m->n_vocab);
    work_vecs w;
    int ok = work_alloc(&w, E) && H && K && Vv && logits;
    int id = -1;
    if (ok) {
        for (int t = 0; t < n; t++) embed(m, toks[t], t, H + (size_t)t * E);
        for (int l = 0; l < m->n_layer; l++) {
            for (int t = 0; t < n; t++) attention_sublayer(m, &m->blocks[l], H + (size_t)t * E, t, K, Vv, E, &w);
            for (int t = 0; t < n; t++) mlp_sublayer(m, &m->blocks[l], H + (size_t)t * E, &w);
        }
        output_head(m, H + (size_t)(n - 1) * E, w.a, logits);
        if (logits_out) memcpy(logits_out, logits, sizeof(real) * (size_t)m->n_vocab);
        id = oracle_argmax(logits, m->n_vocab);
    }
    work_free(&w);
    free(H); free(K); free(Vv); free(logits);
    return id;
}

long oracle_get_weight(const oracle_model *m, int layer, int which, float *out)
{
    const int E = m->d_model, F = m->d_ff;
    if (which == 4) {
        for (size_t i = 0; i < (size_t)m->n_vocab * E; i++) out[i] = (float)m->unembed[i];
        return (long)m->n_vocab * E;
    }
    if (layer < 0 || layer >= m->n_layer) return -1;
    const block_params *b = &m->blocks[layer];
    const real *W;
    int K, N;
    switch (which) {
    case 0: W = b->w_qkv; K = E; N = 3 * E; break;
    case 1: W = b->w_out; K = E; N = E; break;
    case 2: W = b->w_up; K = E; N = F; break;
    case 3: W = b->w_down; K = F; N = E; break;
    default: return -1;
    }
    /* returned output-major: out[o][k] = W[k][o] */
    for (int o = 0; o < N; o++)
        for (int k = 0; k < K; k++) out[(size_t)o * K + k] = (float)W[(size_t)k * N + o];
    return (long)N * K;
}
