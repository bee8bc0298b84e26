"""Pins of the CPU oracle to things other than itself (CPU only).

Each test names what fixes the expected value: a library implementation
(Hugging Face GPT-2, numpy matmul, torch layer_norm / gelu, scipy softmax,
numpy float16), a closed form or special case, an error bound, or brute force.
"""
import math

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

import synth
from oracle import Oracle
from tests.hf_ref import hf_logits, hf_model

U32 = 2.0 ** -24


def gamma(k):
    return k * U32 / (1 - k * U32)


def tiny_rich():
    """Tiny shape with non-trivial LayerNorm gains/shifts and biases, so that a
    dropped bias or gain cannot hide behind the gamma=1/beta=0/bias=0 config."""
    return synth.variant(synth.CONFIGS[1], init="small", weight_seed=1101, name="tiny-rich")


def teacher_tokens(orc, prompt, n_new):
    toks = list(prompt)
    logits = []
    for pos in range(len(prompt) + n_new - 1):
        am, lg = orc.step(toks[pos], pos)
        logits.append(lg.astype(np.float64))
        if pos + 1 >= len(toks):
            toks.append(am)
    return toks, np.array(logits)


# ---------------------------------------------------------------- whole model
@pytest.mark.parametrize("cfg", [synth.CONFIGS[1], tiny_rich()], ids=lambda c: c.name)
def test_oracle_matches_huggingface_gpt2_tiny(cfg):
    """Whole forward pass vs transformers' GPT2LMHeadModel in float64 (the
    implementation the gpt2.s README verifies against), teacher-forced."""
    model = synth.make_model(cfg)
    orc = Oracle(model, "f32")
    toks, logits = teacher_tokens(orc, synth.make_prompt(cfg), cfg.n_new)
    ref = hf_logits(hf_model(model), toks[: len(logits)])
    scale = np.abs(ref).max(axis=1, keepdims=True)
    err = np.abs(logits - ref) / scale
    assert err.max() < 2e-6, err.max()
    # float64 build of the same oracle: agreement to double rounding
    orc64 = Oracle(model, "f64")
    _, l64 = teacher_tokens(orc64, toks[: cfg.n_prompt], cfg.n_new)
    # same token stream: greedy ids of the two builds agree on these margins
    assert np.abs(l64 - ref).max() / scale.max() < 1e-12


def test_oracle_matches_huggingface_gpt2_small_shape():
    """124M shape (12 layers, 12 heads of 64): first 5 positions vs HF float64."""
    cfg = synth.CONFIGS[2]
    model = synth.make_model(cfg)
    orc = Oracle(model, "f32")
    prompt = synth.make_prompt(cfg)[:5]
    logits = np.array([orc.step(t, p)[1] for p, t in enumerate(prompt)], np.float64)
    ref = hf_logits(hf_model(model), prompt)
    err = np.abs(logits - ref).max(axis=1) / np.abs(ref).max(axis=1)
    assert err.max() < 5e-6, err


@pytest.mark.parametrize("wdtype", ["fp16", "int4"])
def test_oracle_quantised_forward_matches_huggingface(wdtype):
    """The fp16/int4 forward = the fp32 forward on the quantised weights: HF
    float64 loaded with the oracle's effective weights (untied head for fp16,
    whose embedding stays fp32)."""
    cfg = synth.variant(tiny_rich(), wdtype=wdtype, name="tiny-" + wdtype)
    model = synth.make_model(cfg)
    orc = Oracle(model, "f32")
    E, F = cfg.n_embd, 4 * cfg.n_embd
    t = dict(model.t)
    shapes = {0: ("attn.c_attn.weight", 3 * E, E), 1: ("attn.c_proj.weight", E, E),
              2: ("mlp.c_fc.weight", F, E), 3: ("mlp.c_proj.weight", E, F)}
    for l in range(cfg.n_layer):
        for which, (name, N, K) in shapes.items():
            t[f"h.{l}.{name}"] = orc.weight(l, which).reshape(N, K).T.copy()
    hm = hf_model(synth.Model(cfg, t))
    if wdtype == "fp16":
        hm.config.tie_word_embeddings = False
        hm.lm_head.weight = torch.nn.Parameter(
            torch.from_numpy(orc.weight(0, 4).reshape(cfg.vocab, E).astype(np.float64)))
        assert hm.lm_head.weight.data_ptr() != hm.transformer.wte.weight.data_ptr()
    toks, logits = teacher_tokens(orc, synth.make_prompt(cfg), 8)
    ref = hf_logits(hm, toks[: len(logits)])
    err = np.abs(logits - ref).max() / np.abs(ref).max()
    assert err < 2e-6, err


def test_kv_cache_decode_equals_bruteforce_recompute():
    """KV-cache decode (append a row, read rows 0..pos) vs recomputing every
    position's K/V from the sequence with no cache: bit-identical in the oracle."""
    cfg = tiny_rich()
    orc = Oracle(synth.make_model(cfg), "f32")
    toks, logits = teacher_tokens(orc, synth.make_prompt(cfg), 20)
    for n in (1, 2, 7, len(logits)):
        am, lg = orc.prefill_last(toks[:n])
        assert np.array_equal(lg.astype(np.float64), logits[n - 1])
        assert am == int(np.argmax(logits[n - 1]))


def test_causal_mask_never_reads_future_rows():
    """Rows after the current position poisoned with NaN change nothing (the
    attn_decode kernel reads positions 0..position only)."""
    cfg = tiny_rich()
    model = synth.make_model(cfg)
    a, b = Oracle(model, "f32"), Oracle(model, "f32")
    prompt = synth.make_prompt(cfg)
    for pos, tok in enumerate(prompt):
        b.poison_cache_after(pos, float("nan"))
        _, la = a.step(tok, pos)
        _, lb = b.step(tok, pos)
        assert np.all(np.isfinite(lb))
        assert np.array_equal(la, lb)


def test_rewind_overwrites_row_and_reads_prefix():
    """position < filled rewinds: same result as a fresh run of that prefix."""
    cfg = tiny_rich()
    model = synth.make_model(cfg)
    a = Oracle(model, "f32")
    p = synth.make_prompt(cfg)
    for pos, tok in enumerate(p):
        a.step(tok, pos)
    _, l_rew = a.step(7, 3)
    b = Oracle(model, "f32")
    for pos, tok in enumerate(list(p[:3]) + [7]):
        _, l_fresh = b.step(tok, pos)
    assert np.array_equal(l_rew, l_fresh)


def test_step_rejects_bad_arguments():
    cfg = synth.CONFIGS[1]
    orc = Oracle(synth.make_model(cfg), "f32")
    with pytest.raises(ValueError):
        orc.step(cfg.vocab, 0)
    with pytest.raises(ValueError):
        orc.step(0, 1)           # position > filled
    with pytest.raises(ValueError):
        orc.step(-1, 0)
    orc.step(0, 0)
    with pytest.raises(ValueError):
        orc.step(0, cfg.n_positions)


def test_argmax_ties_pick_lowest_index():
    """Two identical vocab rows give identical logits: greedy takes the lower id."""
    cfg = tiny_rich()
    model = synth.make_model(cfg)
    t = dict(model.t)
    orc0 = Oracle(model, "f32")
    am0, _ = orc0.step(3, 0)
    wte = t["wte.weight"].copy()
    hi = cfg.vocab - 1 if am0 != cfg.vocab - 1 else cfg.vocab - 2
    lo_id = min(am0, hi)
    wte[hi] = wte[am0]
    t["wte.weight"] = wte
    orc = Oracle(synth.Model(cfg, t), "f32")
    am, lg = orc.step(3, 0)
    assert lg[am0] == lg[hi]
    assert am == lo_id


def test_float_build_drift_small_shape():
    """float oracle vs its float64 build on the 124M shape, 3 positions."""
    model = synth.make_model(2)
    a, b = Oracle(model, "f32"), Oracle(model, "f64")
    for pos, tok in enumerate(synth.make_prompt(2)[:3]):
        _, la = a.step(tok, pos)
        _, lb = b.step(tok, pos)
        assert np.abs(la - lb).max() <= 1e-5 * np.abs(lb).max()


def test_parameter_count_and_sizes():
    """The sizes the pages print (tests/golden/page_figures.json, each with its
    citation) against the tensor list both sides load: 148 tensors, about
    500 MB of fp32 weights read per token, 340 MB of block matrices, a 154 MB
    head padded to 50,304 rows, a 75 MB KV cache, 1,024 positions, 50,257 ids."""
    import json
    import os
    from oracle import load_lib
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "page_figures.json")) as f:
        fig = {k: v["value"] for k, v in json.load(f).items() if not k.startswith("_")}
    cfg = synth.CONFIGS[2]
    E, L, V, P = cfg.n_embd, cfg.n_layer, cfg.vocab, cfg.n_positions
    assert V == fig["vocab"] and P == fig["context"]
    assert load_lib("f32").lib.oracle_n_tensors(L) == fig["tensor_count"]
    shapes = synth.tensor_shapes(cfg)
    assert len(shapes) == fig["tensor_count"]
    n = sum(int(np.prod(s)) for _, s in shapes)
    assert n == 124_439_808
    # weights read per token: everything but the position table, whose one row is read
    per_token = (n - P * E + E) * 4
    assert abs(per_token / 1e6 - fig["weights_read_per_token_MB"]) < 0.02 * fig["weights_read_per_token_MB"]
    block = L * (3 * E * E + E * E + 4 * E * E + 4 * E * E) * 4
    assert round(block / 1e6) == fig["block_tiles_MB"]
    assert fig["head_padded_rows"] == -(-V // 64) * 64
    assert round(fig["head_padded_rows"] * E * 4 / 1e6) in (fig["head_tiles_MB"], fig["head_tiles_MB"] + 1)
    kv = 2 * L * P * E * 4
    assert round(kv / 1e6) == fig["kv_cache_MB"]


# ---------------------------------------------------------------- primitives
@pytest.mark.parametrize("K,N", [(768, 2304), (768, 768), (3072, 768), (128, 384)])
def test_linear_within_inner_product_bound(olib, K, N):
    """Any summation order obeys |y^ - y| <= gamma_K * sum|w||x| (inner-product
    error bound); the bias add contributes one more rounding."""
    rng = np.random.default_rng(K + N)
    x = rng.standard_normal(K).astype(np.float32)
    W = (0.02 * rng.standard_normal((K, N))).astype(np.float32)
    b = (0.01 * rng.standard_normal(N)).astype(np.float32)
    y = olib.linear_conv1d(x, W, b).astype(np.float64)
    exact = x.astype(np.float64) @ W.astype(np.float64) + b
    bound = gamma(K + 1) * (np.abs(x).astype(np.float64) @ np.abs(W).astype(np.float64) + np.abs(b))
    assert np.all(np.abs(y - exact) <= bound)


def test_linear_one_hot_is_exact_copy(olib):
    K, N = 64, 48
    W = np.zeros((K, N), np.float32)
    perm = np.random.default_rng(0).permutation(K)[:N]
    W[perm, np.arange(N)] = 1.0
    x = np.random.default_rng(1).standard_normal(K).astype(np.float32)
    assert np.array_equal(olib.linear_conv1d(x, W), x[perm])


def test_layernorm_vs_torch_and_invariants(olib):
    rng = np.random.default_rng(5)
    for n in (128, 768):
        x = (3.0 + 2.0 * rng.standard_normal(n)).astype(np.float32)
        g = (1 + 0.05 * rng.standard_normal(n)).astype(np.float32)
        b = (0.01 * rng.standard_normal(n)).astype(np.float32)
        y = olib.layernorm(x, g, b, 1e-5).astype(np.float64)
        ref = torch.nn.functional.layer_norm(torch.from_numpy(x.astype(np.float64)), (n,),
                                             torch.from_numpy(g.astype(np.float64)),
                                             torch.from_numpy(b.astype(np.float64)), 1e-5).numpy()
        assert np.abs(y - ref).max() < 2e-6 * np.abs(ref).max()
        # gamma = 1, beta = 0: zero mean, variance sigma^2/(sigma^2+eps)
        one, zero = np.ones(n, np.float32), np.zeros(n, np.float32)
        y0 = olib.layernorm(x, one, zero, 1e-5).astype(np.float64)
        var = np.var(x.astype(np.float64))
        assert abs(y0.mean()) <= 1e-6 * np.abs(y0).max()
        assert abs(np.var(y0) - var / (var + 1e-5)) <= 1e-5
        # constant input: y = beta exactly when the mean is exact (a dyadic value
        # and n a power of two); otherwise off only by the sequential sum's
        # rounding (gamma_n * c) times rsqrt(eps)
        c = np.full(n, 0.7, np.float32)
        dev = np.abs(olib.layernorm(c, g, b, 1e-5).astype(np.float64) - b)
        assert np.all(dev <= gamma(n + 2) * 0.7 / math.sqrt(1e-5) * np.abs(g) + 1e-9)
        if n == 128:
            c = np.full(n, 0.75, np.float32)
            assert np.array_equal(olib.layernorm(c, g, b, 1e-5), b)


def test_gelu_new_vs_tanh_form(olib, olib64):
    """x*sigmoid(2*sqrt(2/pi)*(x+0.044715x^3)) equals the tanh form used by the
    blog (tanh(z) = 1 - 2/(e^{2z}+1)) and by torch's gelu(approximate='tanh')."""
    x = np.concatenate([np.linspace(-10, 10, 2001), [0.0, 1e-30, -1e-30, 40.0, -40.0]])
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    z = math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3)
    tanh_blog = 1 - 2 / (np.exp(2 * z) + 1)
    ref2 = 0.5 * x * (1 + tanh_blog)
    y32 = olib.gelu_new(x.astype(np.float32)).astype(np.float64)
    y64 = olib64.gelu_new(x)
    tol = 1e-6 * np.maximum(np.abs(ref), 1e-3)
    assert np.all(np.abs(y32 - ref) <= tol + 1e-7)
    # the tanh forms lose everything to cancellation where 1+tanh(z) underflows
    # (they return -0 near x = -7), hence the small absolute term
    assert np.all(np.abs(y64 - ref) <= 1e-13 * np.abs(ref) + 1e-15)
    assert np.all(np.abs(y64 - ref2) <= 1e-12 * np.abs(ref) + 1e-15)
    assert olib.gelu_new(np.array([0.0]))[0] == 0.0
    assert olib.gelu_new(np.array([40.0]))[0] == np.float32(40.0)
    assert olib.gelu_new(np.array([-40.0]))[0] == 0.0


@pytest.mark.parametrize("D", [32, 64])
def test_attention_softmax_properties(olib, D):
    rng = np.random.default_rng(D)
    T = 40
    q = rng.standard_normal(D).astype(np.float32)
    K = rng.standard_normal((T, D)).astype(np.float32)
    V = rng.standard_normal((T, D)).astype(np.float32)
    # pos 0: one weight of exactly 1 and the output is the value row bit for bit
    out, p = olib.attn_head(q, K, V, 0)
    assert p[0] == 1.0 and np.array_equal(out, V[0])
    for pos in (1, 9, T - 1):
        out, p = olib.attn_head(q, K, V, pos)
        assert np.all((p >= 0) & (p <= 1))
        assert abs(p.astype(np.float64).sum() - 1) <= gamma(pos + 2)
        s = (K[: pos + 1].astype(np.float64) @ q.astype(np.float64)) / math.sqrt(D)
        pref = scipy.special.softmax(s)
        assert np.abs(p - pref).max() < 1e-6
        oref = pref @ V[: pos + 1].astype(np.float64)
        assert np.abs(out - oref).max() < 1e-5
    # identical keys: uniform weights, output = mean of the values
    Ks = np.tile(K[:1], (T, 1))
    out, p = olib.attn_head(q, Ks, V, 9)
    assert np.all(p == p[0]) and abs(p[0] - 0.1) < 1e-7
    assert np.abs(out - V[:10].astype(np.float64).mean(0)).max() < 1e-6


def test_fp16_conversion_matches_numpy(olib):
    """IEEE binary16 round-to-nearest-even with subnormals, against numpy's cast."""
    rng = np.random.default_rng(3)
    vals = [0.02 * rng.standard_normal(4000), rng.standard_normal(2000) * 1e-5,
            rng.uniform(-7e-8, 7e-8, 2000),  # subnormal range and below
            np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, -1e6, np.inf, -np.inf,
                      2.0 ** -24, 2.0 ** -25, 1.5 * 2.0 ** -25, 2.0 ** -14, 6.1e-5,
                      1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 2049.0, 2051.0])]
    x = np.concatenate(vals).astype(np.float32)
    got = olib.f32_to_f16_bits(x)
    want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)
    back = olib.f16_bits_to_f32(want)
    assert np.array_equal(back.view(np.uint32), want.view(np.float16).astype(np.float32).view(np.uint32))
    normal = np.isfinite(x) & (np.abs(x) >= 2.0 ** -14) & (np.abs(x) <= 65504)
    assert np.all(np.abs(back[normal].astype(np.float64) - x[normal]) <= 2.0 ** -11 * np.abs(x[normal]))


def test_q4_group_properties_and_bruteforce(olib):
    """Grouped asymmetric int4: codes in 0..15, error within half a step (plus a
    few ulps), exact at the group minimum, and the chosen code is the nearest of
    the 16 levels (brute force over all codes, ties excepted)."""
    rng = np.random.default_rng(11)
    for trial in range(300):
        w = (0.02 * rng.standard_normal(32)).astype(np.float32)
        if trial % 50 == 0:
            w[:] = w[0]                       # degenerate group
        q, s, mn, deq = olib.q4_group(w)
        assert q.min() >= 0 and q.max() <= 15
        assert mn == w.min()
        if s == 0:
            assert np.all(q == 0) and np.array_equal(deq, w)
            continue
        assert deq[np.argmin(w)] == w.min()
        err = np.abs(deq.astype(np.float64) - w)
        assert np.all(err <= s / 2 + 4 * np.spacing(np.abs(w).max()))
        levels = np.fma if hasattr(np, "fma") else None
        lv = np.arange(16, dtype=np.float64) * np.float64(s) + np.float64(mn)
        dist = np.abs(w[:, None].astype(np.float64) - lv[None, :])
        best = dist.min(axis=1)
        chosen = dist[np.arange(32), q]
        assert np.all(chosen <= best + 4 * np.spacing(np.float32(s)))
        del levels


# ------------------------------------------------------- effective weights
def _two_sum_exact(a, b):
    """True where the float64 sum a + b is exact (Knuth's TwoSum error term is 0)."""
    s = a + b
    bb = s - a
    err = (a - (s - bb)) + (b - bb)
    return err == 0


def _q4_rows_numpy(W, group=32):
    """Grouped asymmetric int4 restated in numpy from the model file's header
    ("transposes to [output,input] before grouped asymmetric int4
    quantization") and the reading of the unstated details (minimum as the
    zero, (max - min)/15 as the step, round half to even, clamp to 0..15,
    level = zero + code * step rounded once): W is the checkpoint's
    [input][output] matrix; returns the dequantised [output][input] rows."""
    T = np.ascontiguousarray(W.T)                       # [N][K]
    N, K = T.shape
    g = T.reshape(N, K // group, group)
    lo = g.min(axis=2, keepdims=True)
    hi = g.max(axis=2, keepdims=True)
    step = (hi - lo) / np.float32(15)                   # float32 arithmetic throughout
    with np.errstate(divide="ignore", invalid="ignore"):
        code = np.where(step != 0, np.clip(np.rint((g - lo) / step), 0, 15), 0).astype(np.float32)
    # the one-rounding level: code * step is exact in float64 (4 x 24 bits); the
    # sum is checked exact, so rounding it to float32 is the fused multiply-add
    prod = code.astype(np.float64) * step.astype(np.float64)
    lo64 = np.broadcast_to(lo.astype(np.float64), prod.shape)
    assert np.all(_two_sum_exact(prod, lo64))
    return (prod + lo64).astype(np.float32).reshape(N, K)


def _q4_along_output(W, group=32):
    """The plausible mistake: groups of consecutive outputs instead of inputs."""
    return _q4_rows_numpy(np.ascontiguousarray(W.T), group).T   # quantise W.T's rows = W's columns


MATS = {0: "attn.c_attn.weight", 1: "attn.c_proj.weight", 2: "mlp.c_fc.weight", 3: "mlp.c_proj.weight"}


@pytest.mark.parametrize("cfg,layers", [
    (synth.variant(tiny_rich(), wdtype="fp16", name="tiny-fp16"), None),
    (synth.variant(tiny_rich(), wdtype="int4", name="tiny-int4"), None),
    (synth.variant(tiny_rich(), wdtype="fp32", name="tiny-fp32"), None),
    (synth.CONFIGS[3], (0, 11)),
    (synth.CONFIGS[4], (0, 11)),
], ids=lambda v: v.name if hasattr(v, "name") else str(v))
def test_effective_weights_restated_in_numpy(cfg, layers):
    """Which tensors each storage mode changes, and how, rebuilt from the
    checkpoint arrays in numpy with no oracle code: fp16 ("-h", gpt2.s docs
    Build and run) rounds the 48 block matrices and the output head to
    binary16 (numpy's cast) and keeps the embedding fp32; int4 (model file
    header) quantises each block matrix in groups of 32 consecutive inputs of
    one output row, and keeps the tied head exactly fp32.  Compared bit for bit
    with the weights the oracle runs; a grouping along the output would fail."""
    model = synth.make_model(cfg)
    orc = Oracle(model, "f32")
    t = model.t
    E, V = cfg.n_embd, cfg.vocab
    for l in (range(cfg.n_layer) if layers is None else layers):
        for which, name in MATS.items():
            W = t[f"h.{l}.{name}"]
            got = orc.weight(l, which).reshape(W.shape[1], W.shape[0])
            if cfg.wdtype == "fp32":
                want = W.T
            elif cfg.wdtype == "fp16":
                want = W.T.astype(np.float16).astype(np.float32)
            else:
                want = _q4_rows_numpy(W)
                assert not np.array_equal(got, _q4_along_output(W)), (l, which)
            assert np.array_equal(got.view(np.uint32), np.ascontiguousarray(want).view(np.uint32)), (l, which)
    head = orc.weight(0, 4).reshape(V, E)
    want = t["wte.weight"].astype(np.float16).astype(np.float32) if cfg.wdtype == "fp16" else t["wte.weight"]
    assert np.array_equal(head.view(np.uint32), want.view(np.uint32))
    if cfg.wdtype == "fp16":
        assert not np.array_equal(head, t["wte.weight"])
    orc.close()


# ---------------------------------------------------------------- sampling
_P64 = (1 << 64) - 1
# prime factors of 2^64 - 1
_FACTORS_2_64_M1 = (3, 5, 17, 257, 641, 65537, 6700417)


def _gf2_mul(A, B):
    """64x64 bit matrices over GF(2), each a list of 64 row ints (bit j of row
    i = entry (i, j)); returns A.B."""
    out = []
    for i in range(64):
        r, a = 0, A[i]
        j = 0
        while a:
            if a & 1:
                r ^= B[j]
            a >>= 1
            j += 1
        out.append(r)
    return out


def _gf2_pow(A, e):
    R = [1 << i for i in range(64)]
    while e:
        if e & 1:
            R = _gf2_mul(R, A)
        A = _gf2_mul(A, A)
        e >>= 1
    return R


def test_xorshift_state_update_has_full_period(olib):
    """The state update of xorshift64* is a linear map T over GF(2)^64 (three
    shifts and three xors, blog Step 7).  Its matrix, read off the oracle by
    updating the 64 unit states, must have order exactly 2^64 - 1 (every
    non-zero state on one cycle): the defining property of the shift triples
    the generator is built on, which a wrong shift amount or direction breaks.
    The output is the state times an odd constant (one multiply), so it is a
    bijection of the state."""
    import ctypes as C
    cols = []
    for i in range(64):
        st = C.c_uint64(1 << i)
        olib.lib.oracle_xorshift64s(C.byref(st))
        cols.append(st.value)
    # T as rows: entry (r, c) = bit r of T e_c
    T = [sum(((cols[c] >> r) & 1) << c for c in range(64)) for r in range(64)]
    ident = [1 << i for i in range(64)]
    assert _gf2_pow(T, _P64) == ident
    for p in _FACTORS_2_64_M1:
        assert _gf2_pow(T, _P64 // p) != ident, p
    # the update is linear: T(a ^ b) = T(a) ^ T(b)
    rng = np.random.default_rng(8)
    for _ in range(20):
        a, b = (int(v) for v in rng.integers(1, 2 ** 63, 2, dtype=np.int64))
        sa, sb, sab = C.c_uint64(a), C.c_uint64(b), C.c_uint64(a ^ b)
        for s in (sa, sb, sab):
            olib.lib.oracle_xorshift64s(C.byref(s))
        assert sab.value == sa.value ^ sb.value
    # output = new state * odd constant (mod 2^64): invertible, and the same
    # constant for every state
    outs, _ = olib.xorshift64s(12345, 1)
    st = C.c_uint64(12345)
    olib.lib.oracle_xorshift64s(C.byref(st))
    mult = (int(outs[0]) * pow(st.value, -1, 1 << 64)) % (1 << 64) if st.value % 2 else None
    if mult is not None:
        assert mult % 2 == 1
        for seed in (1, 99, 2 ** 40 + 7):
            o, s2 = olib.xorshift64s(seed, 1)
            assert int(o[0]) == (s2 * mult) % (1 << 64)


def test_uniform_draws_are_uniform(olib):
    """u = top 24 bits of an output times 2^-24: in [0,1), on the 2^-24 grid,
    and uniform (Kolmogorov-Smirnov over 200,000 draws)."""
    u = olib.uniforms(2024, 200_000).astype(np.float64)
    assert u.min() >= 0 and u.max() < 1
    assert np.all(u * 2 ** 24 == np.floor(u * 2 ** 24))
    assert scipy.stats.kstest(u, "uniform").pvalue > 1e-4


def test_sample_is_inverse_cdf_of_tempered_softmax(olib, olib64):
    """Sampling (blog Step 7: divide the scores by a temperature, softmax, draw):
    temperature 0 is the argmax; otherwise the pick is the first id whose
    cumulative softmax(logits/T) weight exceeds u (brute force in float64, away
    from the cumulative boundaries), shifting every logit by a constant changes
    nothing, and the picks of many uniform draws follow softmax(logits/T)
    (chi-square)."""
    rng = np.random.default_rng(4)
    lg = rng.standard_normal(9)
    assert olib.sample(lg, 0.0, 0.5) == int(np.argmax(lg))
    assert olib.sample(lg, -1.0, 0.5) == -1 and olib.sample(lg, 1.0, 1.0) == -1
    for T in (0.3, 0.8, 2.0):
        p = scipy.special.softmax(lg / T)
        cdf = np.cumsum(p)
        for u in np.linspace(0, 1, 997, endpoint=False):
            if np.min(np.abs(cdf - u)) < 1e-5:
                continue
            want = int(np.argmax(cdf > u))
            assert olib.sample(lg.astype(np.float32), T, u) == want
            assert olib64.sample(lg, T, u) == want
            assert olib.sample((lg + 3.5).astype(np.float32), T, u) == want
    # frequencies
    T = 0.8
    lg = rng.standard_normal(6)
    us = olib.uniforms(77, 60_000)
    picks = np.array([olib.sample(lg.astype(np.float32), T, float(u)) for u in us])
    counts = np.bincount(picks, minlength=6)
    expect = scipy.special.softmax(lg / T) * len(us)
    assert scipy.stats.chisquare(counts, expect).pvalue > 1e-4
    # a very high temperature: every id equally likely
    flat = np.array([olib.sample(lg.astype(np.float32), 1e6, float(u)) for u in us[:30_000]])
    assert scipy.stats.chisquare(np.bincount(flat, minlength=6)).pvalue > 1e-4
