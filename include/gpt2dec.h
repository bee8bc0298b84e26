/*
 * gpt2dec.h -- C ABI of the MI355X (gfx950) batch-1 GPT-2 decode library.
 *
 * One call of gpt2_step runs the one-token GPT-2 forward pass (the gpt2-125m
 * "model.fir" page's network): token + positional embedding, per layer
 * LayerNorm -> QKV linear + bias -> attn_decode (append this position's K/V,
 * causal softmax over positions 0..position, weighted sum of values) ->
 * attention linear + bias + residual -> LayerNorm -> fc linear + bias ->
 * gelu_new -> projection linear + bias + residual, then the final
 * LayerNorm and the output head tied to wte, with greedy choice = argmax
 * ("Let's make GPT-2 in assembly", Step 7).  Weights arrive in the Hugging Face
 * checkpoint layout (Conv1D matrices as [input][output], as both pages note)
 * and are re-laid out once at load, output-major, as the gpt2.s README
 * ("Inner Workings") and the blog's Step 1 do.
 *
 * Conventions for every entry point:
 *  - All pointers are HOST pointers unless stated otherwise; the caller owns
 *    them and they are only read (or written, for outputs) during the call.
 *  - The library owns all device memory and the context.  Work runs on the
 *    context's HIP stream (library-created, or the caller's via
 *    gpt2_set_stream).  A call returns once its host results are final:
 *    gpt2_step without logits and the gpt2_generate calls (except
 *    gpt2_generate_noalloc) return as soon as their ids have reached host
 *    memory, when nothing of the launch can fail any more, possibly before its
 *    workgroups have exited; later work on the same stream stays ordered
 *    after it.  Every other call synchronizes the stream.
 *  - Return value 0 = success, or one of the negative GPT2_E_* codes below.
 *    Arguments are validated before any device work, so a rejected call
 *    changes nothing.  After GPT2_E_DEVICE or GPT2_E_NUMERIC the context is
 *    poisoned: every later call except gpt2_last_error/gpt2_free returns
 *    GPT2_E_STATE.
 *  - No C++ exception leaves the library: a host allocation that fails inside
 *    a call returns GPT2_E_NOMEM (any other host-side failure GPT2_E_INVAL),
 *    with its message in gpt2_last_error.
 *  - A context must not be used by two threads at once.
 */
#ifndef GPT2DEC_H
#define GPT2DEC_H

#ifdef __cplusplus
extern "C" {
#endif

/* exported from libgpt2dec.so (built with hidden default visibility) */
#if defined(__GNUC__) || defined(__clang__)
#define GPT2DEC_API __attribute__((visibility("default")))
#else
#define GPT2DEC_API
#endif

#define GPT2_OK 0
#define GPT2_E_INVAL (-1)   /* bad argument or unsupported configuration        */
#define GPT2_E_NOMEM (-2)   /* host or device allocation failed                 */
#define GPT2_E_DEVICE (-3)  /* HIP error, no GPU, or a device-side wait timeout */
#define GPT2_E_STATE (-4)   /* context poisoned by an earlier device error      */
#define GPT2_E_NUMERIC (-5) /* every logit of a pass is NaN: no greedy id exists
                               (the context is poisoned: its cache holds the pass) */

/* Storage of the 48 block matrices (and, for fp16, the output head).  fp32 is
 * the model file's f32 linears ("--fir-f32"); fp16 is the gpt2.s "-h" option
 * (matrices and head stored fp16, widened to fp32, fp32 products and sums;
 * embeddings, biases and LayerNorm stay fp32); int4 is the model file's "q4"
 * linears (grouped asymmetric int4 along the input after transposing to
 * [output][input]; the tied head stays fp32). */
typedef enum { GPT2_W_FP32 = 0, GPT2_W_FP16 = 1, GPT2_W_INT4 = 2 } gpt2_wdtype;

typedef struct {
    int n_layer;      /* L >= 1                                              */
    int n_embd;       /* E; supported: 768 (head dim 64) and 128 (head dim 32) */
    int n_head;       /* H; E / H must be the head dim above                  */
    int n_positions;  /* P >= 1: context length (1024 for GPT-2)              */
    int vocab_size;   /* V >= 1; V <= 256 * workgroups (65536 at E=768)        */
    float ln_eps;     /* LayerNorm epsilon (layer_norm_epsilon, 1e-5)         */
    int wdtype;       /* gpt2_wdtype                                          */
    int q4_group;     /* int4 group size along the input; must be 32          */
} gpt2_config;

/* Host fp32 parameters in Hugging Face names and layouts (F = 4E).  The
 * per-layer members are arrays of L pointers.  Read only during gpt2_load. */
typedef struct {
    const float *wte;                       /* [V][E] embedding, also the tied head */
    const float *wpe;                       /* [P][E]                               */
    const float *const *ln1_w, *const *ln1_b;             /* [E]                    */
    const float *const *c_attn_w, *const *c_attn_b;       /* [E][3E], [3E]          */
    const float *const *attn_proj_w, *const *attn_proj_b; /* [E][E], [E]            */
    const float *const *ln2_w, *const *ln2_b;             /* [E]                    */
    const float *const *c_fc_w, *const *c_fc_b;           /* [E][F], [F]            */
    const float *const *mlp_proj_w, *const *mlp_proj_b;   /* [F][E], [E]            */
    const float *lnf_w, *lnf_b;                           /* [E]                    */
} gpt2_weights;

typedef struct gpt2_ctx gpt2_ctx;

/* Validate cfg (the model file's config checks: E = H * head_dim, MLP = 4E;
 * plus the shapes this build supports), copy the weights to the GPU, re-lay
 * them out output-major (fp16: round to nearest even; int4: quantise as
 * above), allocate the KV cache ([L][H][P][head_dim] fp32) and the working
 * buffers.  On success *out receives the context (filled = 0).
 * Errors: GPT2_E_INVAL (bad cfg / null pointer), GPT2_E_NOMEM, GPT2_E_DEVICE. */
GPT2DEC_API int gpt2_load(const gpt2_config *cfg, const gpt2_weights *w, gpt2_ctx **out);

/* gpt2_load from the files Hugging Face publishes, as they are ("Let's make
 * GPT-2 in assembly", Step 1; gpt2.s docs, "Inner Workings"): the mapped
 * safetensors file's 148 tensors found by name in its JSON header (with or
 * without a "transformer." prefix; F32, the shapes the model file declares),
 * and config.json checked as the gpt2-125m model file's "require config" lines
 * do (model_type gpt2, activation_function gelu_new, scale_attn_weights true,
 * scale_attn_by_inverse_layer_idx, reorder_and_upcast_attn and
 * add_cross_attention false, each passing when absent; n_embd a multiple of
 * n_head; n_inner null or 4 * n_embd; layer_norm_epsilon 1e-5 when absent;
 * n_layer <= 1024, n_embd and n_head <= 65536, n_positions <= 2^20 and
 * vocab_size <= 2^24, limits far above any GPT-2).
 * wdtype as gpt2_config; int4 groups of 32.  Every file and configuration check
 * runs before any device work: a rejected call is GPT2_E_INVAL with the reason
 * in gpt2_last_error(NULL).  Otherwise errors as gpt2_load. */
GPT2DEC_API int gpt2_load_safetensors(const char *safetensors_path, const char *config_path, int wdtype,
                                      gpt2_ctx **out);

/* The configuration c was loaded with. */
GPT2DEC_API int gpt2_get_config(const gpt2_ctx *c, gpt2_config *out);

/* Run later work on `hip_stream` (a hipStream_t, e.g. torch's current stream;
 * NULL = the library's own stream).  The stream must outlive its use.  The
 * previous stream is synchronized first, so no launch of this context runs
 * on two streams at once.  Errors: GPT2_E_DEVICE, GPT2_E_STATE. */
GPT2DEC_API int gpt2_set_stream(gpt2_ctx *c, void *hip_stream);

/* One decode step: token_id at `position` (0 <= position <= filled and
 * position < P; position < filled rewinds: row `position` of the cache is
 * overwritten and positions 0..position are read, exactly as the model
 * file's attn_decode kernel does).  Afterwards filled = position + 1.
 * logits_out: NULL or host float[V]; argmax_out: NULL or host int (lowest id
 * among equal maxima; NaN logits are never the maximum).  Errors: GPT2_E_INVAL,
 * GPT2_E_DEVICE, GPT2_E_NUMERIC (all logits NaN), GPT2_E_STATE. */
GPT2DEC_API int gpt2_step(gpt2_ctx *c, int token_id, int position, float *logits_out, int *argmax_out);

/* Greedy generation chained on the device (one kernel launch, no host round
 * trip per token): the n_prompt ids are fed at positions filled ..
 * filled+n_prompt-1, then each argmax is fed back until n_new ids exist.
 * That is n_prompt + n_new - 1 forward passes; the last pass's argmax is the
 * n_new-th id and is not fed.  out_ids: host int[n_new].
 * Requires filled + n_prompt + n_new - 1 <= P.  Afterwards
 * filled += n_prompt + n_new - 1.  Errors as gpt2_step. */
GPT2DEC_API int gpt2_generate(gpt2_ctx *c, const int *prompt, int n_prompt, int n_new, int *out_ids);

/* Batched prompt prefill: the n tokens at positions filled .. filled+n-1 go
 * through every layer together, so each linear is one GEMM of n rows against
 * the weights (read once per layer, not once per position) on the matrix
 * cores; their key and value rows are appended to the cache, as n gpt2_step
 * calls would append them ("Let's make GPT-2 in assembly", "What GPT-2 does":
 * the prompt, then the loop; gpt2.s docs: 10 prompt tokens before the 60
 * generated).  tokens: host int[n].  Returns the last position's logits
 * (logits_out: NULL or host float[V]) and argmax.  Afterwards filled += n.
 * The work rows live in buffers gpt2_load allocated (n_positions rows): the
 * call allocates nothing.  The results agree with per-position steps up to
 * the order of the sums, and repeated calls are bitwise identical.  Errors: GPT2_E_INVAL (n < 1,
 * filled + n > n_positions, a token out of range), GPT2_E_DEVICE,
 * GPT2_E_NUMERIC, GPT2_E_STATE. */
GPT2DEC_API int gpt2_prefill(gpt2_ctx *c, const int *tokens, int n, float *logits_out, int *argmax_out);

/* gpt2_generate for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same ids and cache rows as gpt2_generate, but the kernel's working words
 * (tagged activations, argmax slots, error word) live in a static device array
 * of 16 MiB that the library holds on each GPU until the process ends; the call
 * allocates nothing.  Every such call on a GPU shares that array: it clears the
 * words it uses first, and calls that overlap on one GPU race.  A model whose
 * working words exceed the array is GPT2_E_INVAL (the 124M shape needs about
 * 7.6 MB).  Errors as gpt2_generate; GPT2_E_DEVICE if the array has no address
 * on this device. */
GPT2DEC_API int gpt2_generate_noalloc(gpt2_ctx *c, const int *prompt, int n_prompt, int n_new, int *out_ids);

/* Generation with sampling ("Let's make GPT-2 in assembly", Step 7: divide the
 * scores by a temperature, apply softmax, draw at random; gpt2.s docs, "-t"),
 * chained on the device like gpt2_generate.  Each new id is the first id whose
 * running sum of exp((logit - max)/temperature), in id order, exceeds u times
 * the total, for one uniform number u in [0,1) per id: the top 24 bits of the
 * next xorshift64* output (S. Vigna's scrambled xorshift, shifts 12/25/27,
 * multiplier 2685821657736338717) times 2^-24, the generator's state starting
 * at `seed` (non-zero).  The id comes from the logits as the kernel computes
 * them, so where u falls within rounding of a cumulative boundary the choice
 * may differ from a host computation.  temperature 0 = greedy (gpt2_generate).
 * Errors: GPT2_E_INVAL (temperature negative, not finite or so small that its
 * reciprocal overflows; seed 0; and as gpt2_generate), GPT2_E_DEVICE,
 * GPT2_E_NUMERIC, GPT2_E_STATE. */
GPT2DEC_API int gpt2_generate_sample(gpt2_ctx *c, const int *prompt, int n_prompt, int n_new, float temperature,
                                     unsigned long long seed, int *out_ids);

/* filled = 0.  The cache need not be cleared: reads never pass `position`. */
GPT2DEC_API int gpt2_reset(gpt2_ctx *c);

/* Release everything; c may be NULL. */
GPT2DEC_API void gpt2_free(gpt2_ctx *c);

/* Message for the last failing call on c (c == NULL: the last gpt2_load
 * failure of this thread).  Valid until the next call on c. */
GPT2DEC_API const char *gpt2_last_error(const gpt2_ctx *c);

/* Number of filled positions (the next appending position). -1 if c is NULL. */
GPT2DEC_API int gpt2_filled(const gpt2_ctx *c);

/* ---- byte-level BPE tokenizer ("Let's make GPT-2 in assembly", Step 3;
 * gpt2.s docs, "File Contents" and "Limitations") ------------------------- */
typedef struct gpt2_tokenizer gpt2_tokenizer;

/* Read vocab.json (token strings in GPT-2's byte-level alphabet -> ids) and
 * merges.txt (pairs in rank order after a "#version" line), as published.
 * Every byte must have a token; every merge's parts and result must be tokens.
 * GPT2_E_INVAL with the reason in gpt2_last_error(NULL); GPT2_E_NOMEM. */
GPT2DEC_API int gpt2_tokenizer_load(const char *vocab_json_path, const char *merges_txt_path,
                                    gpt2_tokenizer **out);

/* Token ids of len bytes of text: the text is cut into chunks (an ending 's,
 * 't, 're, 've, 'm, 'll or 'd; a run of letters, digits or other symbols with
 * one optional space in front; a whitespace run, leaving its last character to
 * a non-space after it), and each chunk's bytes join pairwise, the lowest-
 * ranked neighbouring pair first, until no pair has a rank.  Every byte above
 * 127 counts as a letter (exact for ASCII text, as the gpt2.s docs say of
 * theirs).  *n_ids receives the count; ids holds cap ids (ids may be NULL with
 * cap 0 to ask for the count).  GPT2_E_INVAL if cap is too small (the first
 * cap ids are written) or on a bad argument. */
GPT2DEC_API int gpt2_tokenize(const gpt2_tokenizer *t, const char *text, size_t len, int *ids, int cap,
                              int *n_ids);

/* The bytes of n ids, concatenated.  *len receives their count; buf holds cap
 * bytes (NULL with cap 0 to ask).  GPT2_E_INVAL for an id without a token or a
 * too small buffer (nothing written). */
GPT2DEC_API int gpt2_detokenize(const gpt2_tokenizer *t, const int *ids, int n, char *buf, size_t cap,
                                size_t *len);

GPT2DEC_API void gpt2_tokenizer_free(gpt2_tokenizer *t);

/* ---- test hooks (not needed for decoding) ------------------------------ */

/* Effective weights of one matrix as stored on the GPU, output-major: which =
 * 0 QKV [3E][E], 1 attention projection [E][E], 2 fc [F][E], 3 MLP projection
 * [E][F], 4 output head [V][E] (layer ignored).  fp32 as is, fp16 widened,
 * int4 as zero + code * scale (one rounding) from the stored codes, scales and
 * zeros.  The int4 GEMV reads the same stored data but sums
 * scale * sum(code * x) + zero * sum(x) per group, so this pins the stored
 * weights, not the GEMV's arithmetic.  out: host float[N*K]. */
GPT2DEC_API int gpt2_debug_dequant(gpt2_ctx *c, int layer, int which, float *out);

/* Fill every KV-cache entry with `value` (e.g. NaN) so that a read of a row
 * past the current position would show in the result. */
GPT2DEC_API int gpt2_debug_fill_kv(gpt2_ctx *c, float value);

/* Timeline of the decode kernel (profiling aid).  With out == NULL: from now
 * on record the first `steps` steps of every run (0 = stop recording; -1 =
 * keep the current setting, e.g. to only read the record or its size).  With
 * out != NULL: copy the last run's record (out holds out_len values; a smaller
 * out_len than the record is GPT2_E_INVAL and copies nothing), then apply
 * `steps` as above.  recorded_steps (nullable) receives the number of steps
 * the current record holds, so a caller can size out.
 * Layout: [steps][5L+1 phases][workgroups][4] int64 device wall-clock ticks
 * (inputs ready, first and second workgroup barrier passed, outputs
 * published; 0 where a workgroup had no such event), phases
 * per layer l: 5l QKV, 5l+1 attention, 5l+2 attention projection, 5l+3 fc,
 * 5l+4 MLP projection; phase 5L is the output head. */
GPT2DEC_API int gpt2_debug_trace(gpt2_ctx *c, int steps, long long *out, long long out_len,
                                 int *recorded_steps);

/* Launch geometry: workgroups and threads per workgroup of the decode kernel. */
GPT2DEC_API int gpt2_debug_geometry(const gpt2_ctx *c, int *workgroups, int *threads);

#ifdef __cplusplus
}
#endif
#endif
