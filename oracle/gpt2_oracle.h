/*
 * gpt2_oracle.h -- CPU oracle for batch-1 GPT-2 decode (TEST INFRASTRUCTURE ONLY).
 *
 * The plain, slow, single-threaded reference that the HIP library is checked
 * against.  Only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark may load it; the product library never links or calls it, and the
 * two share no code, header, table or constant.
 *
 * What it computes is GPT-2's one-token forward pass, written from the
 * network's definition: token plus position embedding, pre-LayerNorm blocks
 * (causal multi-head attention over positions 0..position with a cache of
 * earlier keys and values, then the gelu_new MLP, each added to the residual
 * stream), a final LayerNorm and the output head tied to the token embedding
 * (gpt2-125m model file; "Let's make GPT-2 in assembly", Steps 4-6).  The next
 * token is the argmax of the logits, or a draw from softmax(logits / T)
 * ("Let's make GPT-2 in assembly", Step 7).
 *
 * Arithmetic type: `oracle_real` is float in liboracle_f32.so (the precision
 * the pages fix: every buffer of the model file is f32) and double in
 * liboracle_f64.so (a drift bound for the float build).  Quantised weights are
 * always produced in float, because they define the model being run.
 *
 * All pointers are host pointers owned by the caller unless stated otherwise.
 */
#ifndef GPT2_ORACLE_H
#define GPT2_ORACLE_H

#include <stdint.h>

#ifdef ORACLE_REAL_IS_DOUBLE
typedef double oracle_real;
#else
typedef float oracle_real;
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Weight storage modes (gpt2.s docs, "-h" option; model file header: q4 linears). */
enum { ORACLE_W_FP32 = 0, ORACLE_W_FP16 = 1, ORACLE_W_INT4 = 2 };

typedef struct oracle_model oracle_model;

/* Number of tensors in the flat parameter list for n_layer layers: wte, wpe,
 * 12 per layer in Hugging Face order (ln_1.w, ln_1.b, c_attn.w, c_attn.b,
 * attn.c_proj.w, attn.c_proj.b, ln_2.w, ln_2.b, c_fc.w, c_fc.b, mlp.c_proj.w,
 * mlp.c_proj.b), ln_f.w, ln_f.b.  For 12 layers this is the 148 tensors the
 * blog's Step 1 looks up by name. */
int oracle_n_tensors(int n_layer);

/* Build a model.  shape = {n_layer, n_embd, n_head, n_positions, vocab}.
 * tensors: oracle_n_tensors(n_layer) host fp32 arrays in Hugging Face Conv1D
 * layout ([input][output] for the four block matrices), copied here.
 * Returns NULL if the configuration is invalid (n_embd not divisible by
 * n_head, a non-positive size, or for int4 a group size that does not divide
 * n_embd), or on allocation failure. */
oracle_model *oracle_new(const int *shape, float ln_eps, int wdtype, int q4_group,
                         const float *const *tensors);
void oracle_free(oracle_model *m);

/* Forget every cached position; the cache content is irrelevant since reads
 * stop at `position`. */
void oracle_reset(oracle_model *m);

/* One decode step: token at `position` (0 <= position <= number of cached
 * positions, < n_positions; a smaller position rewinds).  Writes vocab logits
 * (if non-NULL) and returns the argmax id (lowest index on ties), or -1 on an
 * invalid argument. */
int oracle_step(oracle_model *m, int token, int position, oracle_real *logits);

/* Without the cache: runs the whole sequence toks[0..n-1] through every layer,
 * every position's keys and values rebuilt from the sequence, and returns the
 * argmax of the last position (its logits written if non-NULL).  Leaves the
 * decode state untouched.  -1 on invalid arguments. */
int oracle_prefill_last(oracle_model *m, const int *toks, int n, oracle_real *logits);

/* Effective (possibly quantised) weights of one matrix in output-major
 * [N][K] order as float: which = 0 QKV, 1 attention projection, 2 fc,
 * 3 MLP projection, 4 output head (layer ignored).  Returns N*K or -1. */
long oracle_get_weight(const oracle_model *m, int layer, int which, float *out);

/* Overwrite the cached keys and values of positions > `position` in every
 * layer with `value` (for the causal-mask check). */
void oracle_poison_cache_after(oracle_model *m, int position, float value);

/* ---- pieces of the network, exposed for the pins ------------------------ */
void oracle_layernorm(const oracle_real *x, const oracle_real *gamma, const oracle_real *beta,
                      int n, oracle_real eps, oracle_real *y);
oracle_real oracle_gelu_new(oracle_real x);
/* y[o] = sum_i x[i] * W[i][o] + b[o]  (W is Conv1D [K][N]; b may be NULL) */
void oracle_linear_conv1d(const oracle_real *x, const oracle_real *W, const oracle_real *b,
                          int K, int N, oracle_real *y);
/* Causal softmax attention of one head over key/value rows 0..pos.
 * q[D]; Kc/Vc rows are `stride` elements apart; probs[pos+1] receives the
 * softmax weights (may be NULL); out[D]. */
void oracle_attn_head(const oracle_real *q, const oracle_real *Kc, const oracle_real *Vc,
                      int pos, int stride, int D, oracle_real *probs, oracle_real *out);
/* Index of the largest value, the lowest one among equals. */
int oracle_argmax(const oracle_real *v, int n);
uint16_t oracle_f32_to_f16(float f);
float oracle_f16_to_f32(uint16_t h);
/* Grouped asymmetric int4 of one group of n weights: codes q[n] in 0..15,
 * scale *s, zero *mn; dequantised values to deq[n] (may be NULL). */
void oracle_q4_group(const float *w, int n, uint8_t *q, float *s, float *mn, float *deq);

/* ---- sampling ("Let's make GPT-2 in assembly", Step 7; gpt2.s docs "-t") --- */
/* One xorshift64* output; advances *state (which must not be 0). */
uint64_t oracle_xorshift64s(uint64_t *state);
/* A uniform number in [0,1): the top 24 bits of one xorshift64* output times 2^-24. */
float oracle_uniform(uint64_t *state);
/* The id drawn from softmax(logits / temperature) by the uniform number u in
 * [0,1): the first id whose running sum of exp((logit - max)/temperature)
 * exceeds u times the total.  temperature 0 = greedy (argmax).  -1 on an
 * invalid argument (n < 1, temperature < 0 or NaN, u outside [0,1)). */
int oracle_sample(const oracle_real *logits, int n, oracle_real temperature, oracle_real u);

int oracle_real_bytes(void);

#ifdef __cplusplus
}
#endif
#endif
