"""GPU parity: the HIP library against the CPU oracle on identical seeded inputs.

Floating-point bar: per step, max |logit_gpu - logit_oracle| <= 1e-4 * max|logit_oracle|
and greedy ids equal wherever the oracle's top-2 margin exceeds 1e-3 (teacher
forcing: both sides are fed the oracle's tokens).  Dequantised weights are compared
bit for bit.
"""
import numpy as np
import pytest

import synth
import transformer_decode_token_amd as g2
from oracle import Oracle
from tests.gpu_util import compare_step, load_gpu, oracle_stream, top2_margin

pytestmark = pytest.mark.gpu


def tiny_rich(**kw):
    return synth.variant(synth.CONFIGS[1], init="small", weight_seed=1101, name="tiny-rich", **kw)


CASES = {
    "tiny": synth.CONFIGS[1],
    "tiny-rich": tiny_rich(),
    "tiny-rich-fp16": tiny_rich(wdtype="fp16"),
    "tiny-rich-int4": tiny_rich(wdtype="int4"),
    # long context on the tiny shape: up to 8 attention chunks per head, all
    # 512 positions (at 8 chunks every one of the 32 workgroups runs one)
    "tiny-long": tiny_rich(n_positions=512, n_new=505),
    "gpt2-124m-fp32": synth.CONFIGS[2],
    "gpt2-124m-fp16w": synth.CONFIGS[3],
    "gpt2-124m-int4w": synth.CONFIGS[4],
}


@pytest.mark.parametrize("name", list(CASES))
def test_teacher_forced_logits_and_ids(name):
    cfg = CASES[name]
    print(f"[parity] {name}: {cfg.n_steps} steps", flush=True)
    model = synth.make_model(cfg)
    orc = Oracle(model)
    toks, logits, _ = oracle_stream(orc, synth.make_prompt(cfg), cfg.n_steps)
    orc.close()
    ctx = load_gpu(model)
    worst = 0.0
    for pos, tok in enumerate(toks):
        am, lg = g2.gpt2_step(ctx, tok, pos)
        worst = max(worst, compare_step(lg, am, logits[pos], f"{name} pos {pos}"))
    print(f"[parity] {name}: worst relative logit error {worst:.2e}", flush=True)
    ctx.close()


@pytest.mark.parametrize("offset", [1.0, 4.0])
def test_layernorm_inputs_with_large_mean(offset):
    """The GPU folds each LayerNorm into the linear after it and subtracts the
    input's mean after the dot product: rstd * (w.(g*x) - mean * w.g) + (w.h + b),
    a difference that cancels when the residual stream carries a large common
    offset.  Every position embedding is shifted by `offset` (the stream's
    spread is about 0.03, so the mean is about 35 and 140 times the spread):
    the parity bar still holds.  (Much larger offsets exhaust fp32 in the
    residual sums themselves, whatever the LayerNorm's arithmetic.)"""
    cfg = CASES["tiny-rich"]
    t = dict(synth.make_model(cfg).t)
    t["wpe.weight"] = (t["wpe.weight"] + np.float32(offset)).astype(np.float32)
    model = synth.Model(cfg, t)
    orc = Oracle(model)
    toks, logits, _ = oracle_stream(orc, synth.make_prompt(cfg), cfg.n_steps)
    orc.close()
    ctx = load_gpu(model)
    worst = 0.0
    for pos, tok in enumerate(toks):
        am, lg = g2.gpt2_step(ctx, tok, pos)
        worst = max(worst, compare_step(lg, am, logits[pos], f"offset {offset} pos {pos}"))
    print(f"[parity] position-embedding offset {offset}: worst relative logit error {worst:.2e}", flush=True)
    ctx.close()


@pytest.mark.parametrize("name", ["tiny", "tiny-rich", "gpt2-124m-fp32", "gpt2-124m-fp16w", "gpt2-124m-int4w"])
def test_generate_matches_oracle_greedy(name):
    """Device-chained greedy ids equal the oracle's up to the first step whose
    oracle top-2 margin is at or below 1e-3 (where summation order may decide)."""
    cfg = CASES[name]
    model = synth.make_model(cfg)
    orc = Oracle(model)
    prompt = synth.make_prompt(cfg)
    _, logits, ids = oracle_stream(orc, prompt, cfg.n_steps)
    ctx = load_gpu(model)
    got = g2.gpt2_generate(ctx, prompt, cfg.n_new)
    assert g2.gpt2_filled(ctx) == cfg.n_steps
    for j, (a, b) in enumerate(zip(got, ids)):
        step = cfg.n_prompt - 1 + j
        if top2_margin(logits[step]) <= 1e-3:
            break
        assert a == b, f"id {j} differs: gpu {a} oracle {b}"
    # the same run step by step on the GPU gives the same ids, bit-identical logits
    g2.gpt2_reset(ctx)
    toks = list(prompt)
    seq = []
    for pos in range(cfg.n_steps):
        am, _ = g2.gpt2_step(ctx, toks[pos], pos, want_logits=False)
        if pos >= cfg.n_prompt - 1:
            seq.append(am)
        if pos + 1 >= len(toks):
            toks.append(am)
    assert np.array_equal(np.array(seq), got)
    ctx.close()


@pytest.mark.parametrize("name", ["tiny-rich", "tiny-rich-fp16", "tiny-rich-int4",
                                  "gpt2-124m-fp16w", "gpt2-124m-int4w"])
def test_dequantised_weights_bitwise(name):
    cfg = CASES[name]
    model = synth.make_model(cfg)
    orc = Oracle(model)
    ctx = load_gpu(model)
    E, F, V = cfg.n_embd, 4 * cfg.n_embd, cfg.vocab
    layers = [0, cfg.n_layer - 1]
    for l in layers:
        for which in range(4):
            got = g2.gpt2_debug_dequant(ctx, l, which).ravel()
            want = orc.weight(l, which)
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (l, which)
    got = g2.gpt2_debug_dequant(ctx, 0, 4).ravel()
    assert np.array_equal(got.view(np.uint32), orc.weight(0, 4).view(np.uint32))
    ctx.close()


def test_future_cache_rows_never_read():
    """Fill the whole KV cache with NaN before decoding: rows past the current
    position are never read, so every logit stays finite and bit-identical."""
    cfg = CASES["tiny-rich"]
    model = synth.make_model(cfg)
    a, b = load_gpu(model), load_gpu(model)
    g2.gpt2_debug_fill_kv(b, float("nan"))
    for pos, tok in enumerate(synth.make_prompt(cfg)):
        _, la = g2.gpt2_step(a, tok, pos)
        _, lb = g2.gpt2_step(b, tok, pos)
        assert np.all(np.isfinite(lb))
        assert np.array_equal(la, lb)


def test_rewind_and_reset():
    cfg = CASES["tiny-rich"]
    model = synth.make_model(cfg)
    ctx = load_gpu(model)
    p = synth.make_prompt(cfg)
    for pos, tok in enumerate(p):
        g2.gpt2_step(ctx, tok, pos)
    _, l_rew = g2.gpt2_step(ctx, 7, 3)
    assert g2.gpt2_filled(ctx) == 4
    g2.gpt2_reset(ctx)
    assert g2.gpt2_filled(ctx) == 0
    for pos, tok in enumerate(list(p[:3]) + [7]):
        _, l_fresh = g2.gpt2_step(ctx, tok, pos)
    assert np.array_equal(l_rew, l_fresh)


def test_deterministic_runs():
    cfg = CASES["gpt2-124m-fp32"]
    model = synth.make_model(cfg)
    ctx = load_gpu(model)
    prompt = synth.make_prompt(cfg)
    a = g2.gpt2_generate(ctx, prompt, 20)
    g2.gpt2_reset(ctx)
    b = g2.gpt2_generate(ctx, prompt, 20)
    assert np.array_equal(a, b)
    g2.gpt2_reset(ctx)
    _, l1 = g2.gpt2_step(ctx, 5, 0)
    _, l2 = g2.gpt2_step(ctx, 5, 0)
    assert np.array_equal(l1, l2)
    ctx.close()


def test_argmax_ties_pick_lowest_index():
    cfg = CASES["tiny-rich"]
    model = synth.make_model(cfg)
    orc0 = Oracle(model)
    am0, _ = orc0.step(3, 0)
    t = dict(model.t)
    wte = t["wte.weight"].copy()
    hi = cfg.vocab - 1 if am0 != cfg.vocab - 1 else cfg.vocab - 2
    wte[hi] = wte[am0]
    t["wte.weight"] = wte
    ctx = load_gpu(synth.Model(cfg, t))
    am, lg = g2.gpt2_step(ctx, 3, 0)
    assert lg[am0] == lg[hi]
    assert am == min(am0, hi)


def test_invalid_calls_change_nothing():
    cfg = CASES["tiny"]
    model = synth.make_model(cfg)
    ctx = load_gpu(model)
    with pytest.raises(g2.Gpt2Error) as e:
        g2.gpt2_step(ctx, 0, 1)          # position beyond filled
    assert e.value.code == g2.GPT2_E_INVAL
    with pytest.raises(g2.Gpt2Error):
        g2.gpt2_step(ctx, cfg.vocab, 0)
    with pytest.raises(g2.Gpt2Error):
        g2.gpt2_generate(ctx, [1] * 10, cfg.n_positions)
    assert g2.gpt2_filled(ctx) == 0
    am, lg = g2.gpt2_step(ctx, 1, 0)
    orc = Oracle(model)
    am_o, lg_o = orc.step(1, 0)
    compare_step(lg, am, lg_o)


LONG = {
    "gpt2-124m-fp32-long": synth.CONFIGS[5],
    # the fp16 and int4 kernel at up to 16 attention chunks per head: from
    # position 960 on, more chunks than the workgroups after the attention
    # sets can hold, so the rest go to the QKV workgroups
    "gpt2-124m-fp16w-long": synth.variant(synth.CONFIGS[3], n_prompt=8, n_new=1017, name="gpt2-124m-fp16w-long"),
    "gpt2-124m-int4w-long": synth.variant(synth.CONFIGS[4], n_prompt=8, n_new=1017, name="gpt2-124m-int4w-long"),
}


@pytest.mark.parametrize("name", list(LONG))
def test_long_context_every_logit(name):
    """The long-context workload at full size (124M shape, positions 0..1023,
    up to 16 attention chunks per head), teacher-forced in lockstep with the
    oracle run in the test: all V logits of every one of the 1,024 passes
    within 1e-4 * max|logit|, the argmax equal wherever the oracle's top-2
    margin exceeds 1e-3.  Then the device-chained greedy run reproduces the
    oracle's ids up to the first low-margin step."""
    cfg = LONG[name]
    assert cfg.n_steps == cfg.n_positions == 1024
    model = synth.make_model(cfg)
    prompt = [int(t) for t in synth.make_prompt(cfg)]
    orc = Oracle(model)
    ctx = load_gpu(model)
    print(f"[parity] {name}: {cfg.n_steps} teacher-forced steps against the live oracle", flush=True)
    toks = list(prompt)
    worst, ids, margins = 0.0, [], []
    for pos in range(cfg.n_steps):
        am_o, lg_o = orc.step(toks[pos], pos)
        am, lg = g2.gpt2_step(ctx, toks[pos], pos)
        worst = max(worst, compare_step(lg, am, lg_o, f"{name} pos {pos}"))
        if pos >= cfg.n_prompt - 1:
            ids.append(am_o)
            margins.append(top2_margin(lg_o))
        if pos + 1 >= len(toks) and pos + 1 < cfg.n_steps:
            toks.append(am_o)
        if pos % 256 == 255:
            print(f"[parity] {name}: {pos + 1} steps, worst relative logit error {worst:.2e}", flush=True)
    orc.close()
    g2.gpt2_reset(ctx)
    got = g2.gpt2_generate(ctx, np.asarray(prompt, np.int32), cfg.n_new)
    k = 0
    for k, (a, b) in enumerate(zip(got, ids)):
        if margins[k] <= 1e-3:
            break
        assert int(a) == b, f"greedy id {k} differs"
    print(f"[parity] {name}: worst relative logit error {worst:.2e}; greedy ids agree for the first {k + 1} "
          f"of {len(ids)}", flush=True)
    ctx.close()


def _oracle_greedy(orc, fed, pos0, n_new):
    """Oracle run continuing at position pos0: the ids `fed` at pos0.., then greedy
    until n_new ids exist.  Returns (ids, margins of the passes that produced them)."""
    toks = list(fed)
    ids, margins = [], []
    n_steps = len(fed) + n_new - 1
    for k in range(n_steps):
        am, lg = orc.step(toks[k], pos0 + k)
        if k >= len(fed) - 1:
            ids.append(am)
            margins.append(top2_margin(lg))
        if k + 1 >= len(toks):
            toks.append(am)
    return ids, margins


def _assert_ids(got, want, margins, what):
    assert len(got) == len(want)
    for j, (a, b) in enumerate(zip(got, want)):
        if margins[j] <= 1e-3:
            break
        assert int(a) == int(b), f"{what}: id {j} differs: gpu {a} oracle {b}"


def test_generate_edges():
    """Device-chained runs at the edges of the call's contract, against the oracle:
    a one-id prompt with one new id (a single pass), a run that continues after
    steps already taken (position 3 on), and a run that fills every position
    (n_positions = 64), after which one more pass is refused and changes nothing."""
    cfg = CASES["tiny-rich"]
    model = synth.make_model(cfg)
    orc = Oracle(model)
    ctx = load_gpu(model)
    rng = np.random.default_rng(77)
    toks = [int(t) for t in rng.integers(0, cfg.vocab, 80)]

    # one pass
    got = g2.gpt2_generate(ctx, np.array(toks[:1], np.int32), 1)
    orc.reset()
    want, mg = _oracle_greedy(orc, toks[:1], 0, 1)
    _assert_ids(got, want, mg, "single pass")
    assert g2.gpt2_filled(ctx) == 1

    # continue after three single steps
    g2.gpt2_reset(ctx)
    orc.reset()
    for pos in range(3):
        g2.gpt2_step(ctx, toks[pos], pos, want_logits=False)
        orc.step(toks[pos], pos)
    got = g2.gpt2_generate(ctx, np.array(toks[3:5], np.int32), 6)
    want, mg = _oracle_greedy(orc, toks[3:5], 3, 6)
    _assert_ids(got, want, mg, "continued run")
    assert g2.gpt2_filled(ctx) == 3 + 2 + 6 - 1

    # fill every position, then one pass too many
    g2.gpt2_reset(ctx)
    orc.reset()
    P = cfg.n_positions
    got = g2.gpt2_generate(ctx, np.array(toks[:8], np.int32), P - 8 + 1)
    want, mg = _oracle_greedy(orc, toks[:8], 0, P - 8 + 1)
    _assert_ids(got, want, mg, "full run")
    assert g2.gpt2_filled(ctx) == P
    with pytest.raises(g2.Gpt2Error):
        g2.gpt2_generate(ctx, np.array(toks[:1], np.int32), 1)
    assert g2.gpt2_filled(ctx) == P
    orc.close()
    ctx.close()


@pytest.mark.parametrize("name", ["tiny-rich", "tiny-rich-int4", "gpt2-124m-fp32"])
def test_long_prompt_in_one_run(name):
    """A long prompt fed in one device-chained run.  While the tokens are fed,
    a step's first layer may start before the previous step's output head has
    finished everywhere (its argmax is not needed); the cache rows those
    steps leave are checked through the logits of the next single step, and
    the run's ids against the oracle."""
    cfg = CASES[name]
    model = synth.make_model(cfg)
    orc = Oracle(model)
    rng = np.random.default_rng(91)
    n_prompt = min(48, cfg.n_positions - 4)
    prompt = [int(t) for t in rng.integers(0, cfg.vocab, n_prompt)]
    ctx = load_gpu(model)
    got = g2.gpt2_generate(ctx, np.array(prompt, np.int32), 2)
    want, mg = _oracle_greedy(orc, prompt, 0, 2)
    _assert_ids(got, want, mg, "long prompt")
    assert g2.gpt2_filled(ctx) == n_prompt + 1
    # one more pass, fed the oracle's id: its logits read every cache row above
    am, lg = g2.gpt2_step(ctx, int(want[1]), n_prompt + 1, want_logits=True)
    am_o, lg_o = orc.step(int(want[1]), n_prompt + 1)
    compare_step(lg, am, lg_o, f"after a {n_prompt}-id prompt")
    if top2_margin(lg_o) > 1e-3:
        assert am == am_o
    ctx.close()


@pytest.mark.parametrize("name", ["gpt2-124m-fp32", "gpt2-124m-fp16w"])
def test_future_cache_rows_never_read_124m(name):
    """The 124M kernels (fp32, and the fp16/int4 variant) over all 1,024
    positions with every KV-cache entry NaN beforehand: rows past the current
    position are never read (nothing after the current token is read, the
    model file's decode attention), so every logit is finite and bit-identical
    to a run on a clean cache."""
    cfg = CASES[name]
    model = synth.make_model(cfg)
    a, b = load_gpu(model), load_gpu(model)
    g2.gpt2_debug_fill_kv(b, float("nan"))
    toks = np.random.default_rng(5).integers(0, cfg.vocab, cfg.n_positions)
    for pos, tok in enumerate(toks):
        _, la = g2.gpt2_step(a, int(tok), pos)
        _, lb = g2.gpt2_step(b, int(tok), pos)
        assert np.all(np.isfinite(lb)), f"pos {pos}"
        assert np.array_equal(la, lb), f"pos {pos}"
    a.close()
    b.close()


@pytest.mark.parametrize("name", ["gpt2-124m-fp32", "gpt2-124m-fp16w", "gpt2-124m-int4w"])
def test_rewind_deep_124m(name):
    """Rewind at the 124M shape: after 1,000 filled positions, a pass at
    position 990 (overwriting that row, reading rows 0..990, 16 chunks) gives
    bit for bit the logits of a fresh run over the same 990-id prefix."""
    cfg = CASES[name]
    model = synth.make_model(cfg)
    ctx = load_gpu(model)
    # the launch geometry of this weight type's kernel: 256 workgroups of
    # eight waves (fp32, fp16) or four (int4)
    assert g2.gpt2_debug_geometry(ctx) == (256, 256 if cfg.wdtype == "int4" else 512)
    prompt = synth.make_prompt(cfg)
    ids = g2.gpt2_generate(ctx, prompt, 1000 - len(prompt) + 1)
    assert g2.gpt2_filled(ctx) == 1000
    seq = [int(t) for t in prompt] + [int(t) for t in ids[:-1]]
    _, l_rew = g2.gpt2_step(ctx, 123, 990)
    assert g2.gpt2_filled(ctx) == 991
    g2.gpt2_reset(ctx)
    g2.gpt2_generate(ctx, np.asarray(seq[:990], np.int32), 1)
    assert g2.gpt2_filled(ctx) == 990
    _, l_fresh = g2.gpt2_step(ctx, 123, 990)
    assert np.array_equal(l_rew, l_fresh)
    ctx.close()


@pytest.mark.parametrize("name", ["gpt2-124m-fp32", "gpt2-124m-fp16w", "gpt2-124m-int4w"])
def test_argmax_ties_124m(name):
    """Equal logits in different workgroups' vocabulary ranges (row 0, held in
    the first workgroup's LDS, and the last row, streamed by the last
    workgroup) tie with the oracle's argmax row: the lower id wins."""
    cfg = CASES[name]
    model = synth.make_model(cfg)
    orc = Oracle(model)
    am0, _ = orc.step(3, 0)
    orc.close()
    assert 0 < am0 < cfg.vocab - 1
    for partner in (0, cfg.vocab - 1):
        t = dict(model.t)
        wte = t["wte.weight"].copy()
        wte[partner] = wte[am0]
        t["wte.weight"] = wte
        ctx = load_gpu(synth.Model(cfg, t))
        am, lg = g2.gpt2_step(ctx, 3, 0)
        assert lg[am0] == lg[partner], partner
        assert am == min(am0, partner), partner
        # the prefill's head and its two-stage argmax (per-workgroup candidates)
        g2.gpt2_reset(ctx)
        am, lg = g2.gpt2_prefill(ctx, [3])
        assert lg[am0] == lg[partner], partner
        assert am == min(am0, partner), partner
        ctx.close()


@pytest.mark.parametrize("name", ["tiny-rich", "gpt2-124m-fp32"])
def test_nan_logits_are_an_error(name):
    """A final LayerNorm gain of NaN makes every logit NaN: no greedy id exists.
    gpt2_step, the device-chained run and gpt2_prefill all return
    GPT2_E_NUMERIC (the chained run stops inside the kernel instead of feeding a
    made-up id) and poison the context."""
    cfg = CASES[name]
    t = dict(synth.make_model(cfg).t)
    t["ln_f.weight"] = np.full_like(t["ln_f.weight"], np.nan)
    model = synth.Model(cfg, t)
    ctx = load_gpu(model)
    with pytest.raises(g2.Gpt2Error) as e:
        g2.gpt2_step(ctx, 3, 0)
    assert e.value.code == g2.GPT2_E_NUMERIC
    with pytest.raises(g2.Gpt2Error) as e:
        g2.gpt2_step(ctx, 3, 0)
    assert e.value.code == g2.GPT2_E_STATE
    ctx.close()
    ctx = load_gpu(model)
    with pytest.raises(g2.Gpt2Error) as e:
        g2.gpt2_generate(ctx, np.array([1, 2, 3], np.int32), 5)
    assert e.value.code == g2.GPT2_E_NUMERIC
    assert "NaN" in g2.gpt2_last_error(ctx)
    ctx.close()
    ctx = load_gpu(model)
    with pytest.raises(g2.Gpt2Error) as e:
        g2.gpt2_prefill(ctx, [1, 2, 3])
    assert e.value.code == g2.GPT2_E_NUMERIC
    ctx.close()


def test_device_allocation_failure_is_nomem(monkeypatch):
    """With every device allocation failing (the library's fault injection),
    gpt2_load returns GPT2_E_NOMEM and leaves no context."""
    monkeypatch.setenv("GPT2DEC_FAIL_ALLOC", "1")
    with pytest.raises(g2.Gpt2Error) as e:
        load_gpu(synth.make_model(CASES["tiny"]))
    assert e.value.code == g2.GPT2_E_NOMEM
    monkeypatch.delenv("GPT2DEC_FAIL_ALLOC")
    ctx = load_gpu(synth.make_model(CASES["tiny"]))
    ctx.close()


def test_debug_trace_record_and_capacity():
    """The timeline record: its size is reported before any copy, an output
    smaller than the record is refused (nothing copied), and a recorded run
    holds a stamp for every workgroup's output-head phase."""
    import ctypes as C
    cfg = CASES["tiny-rich"]
    ctx = load_gpu(synth.make_model(cfg))
    g2.gpt2_debug_trace(ctx, 2)
    g2.gpt2_generate(ctx, synth.make_prompt(cfg), 4)
    rec = C.c_int(0)
    assert g2.lib().gpt2_debug_trace(ctx.handle, -1, None, 0, C.byref(rec)) == g2.GPT2_OK
    assert rec.value == 2
    G, _ = g2.gpt2_debug_geometry(ctx)
    n = 2 * (5 * cfg.n_layer + 1) * G * 4
    small = np.zeros(n - 1, np.int64)
    assert g2.lib().gpt2_debug_trace(ctx.handle, -1, small.ctypes.data, small.size, None) == g2.GPT2_E_INVAL
    assert not small.any()
    out = g2.gpt2_debug_trace(ctx, 0, fetch=True)
    assert out.shape == (2, 5 * cfg.n_layer + 1, G, 4)
    head = out[:, 5 * cfg.n_layer]
    assert np.all(head[..., 0] > 0) and np.all(head[..., 3] >= head[..., 0])
    assert g2.gpt2_debug_trace(ctx, 0, fetch=True) is None
    ctx.close()


# ------------------------------------------------------------------ sampling
def _oracle_sampled(orc, olib, prompt, n_new, T, seed):
    """The oracle's sampled run ("Let's make GPT-2 in assembly", Step 7): ids drawn
    from softmax(logits/T) with its own xorshift64* draws from `seed`.  Returns the
    ids and, per drawn id, the distance (float64) of u from the nearest cumulative
    boundary of the oracle's softmax."""
    import scipy.special
    us = olib.uniforms(seed, n_new)
    toks = [int(t) for t in prompt]
    ids, dists = [], []
    for pos in range(len(prompt) + n_new - 1):
        _, lg = orc.step(toks[pos], pos)
        if pos >= len(prompt) - 1:
            u = float(us[len(ids)])
            pick = olib.sample(lg, T, u)
            cdf = np.cumsum(scipy.special.softmax(np.asarray(lg, np.float64) / T))
            ids.append(pick)
            dists.append(float(np.min(np.abs(cdf - u))))
            if pos + 1 >= len(toks):
                toks.append(pick)
    return ids, dists


@pytest.mark.parametrize("name,T,n_new", [("tiny-rich", 0.8, 40), ("tiny-rich", 2.0, 40),
                                          ("gpt2-124m-fp32", 0.05, 20), ("gpt2-124m-fp16w", 0.05, 20)])
def test_sampled_generate_matches_oracle(name, T, n_new):
    """Device-chained sampling against the oracle with the same seed: the same ids
    up to the first draw whose u lies within 1e-5 of a cumulative boundary (where
    the two summation orders may decide differently).  (At 50,257 ids the
    boundaries of a flat distribution are about 2e-5 apart, within float32
    rounding of either side's running sum, so the 124M shape runs at a low
    temperature, where the mass sits on few ids.)"""
    from oracle import load_lib
    cfg = CASES[name]
    model = synth.make_model(cfg)
    orc = Oracle(model)
    prompt = synth.make_prompt(cfg)
    seed = 0x9E3779B97F4A7C15
    want, dists = _oracle_sampled(orc, load_lib("f32"), prompt, n_new, T, seed)
    orc.close()
    ctx = load_gpu(model)
    got = g2.gpt2_generate_sample(ctx, prompt, n_new, T, seed)
    assert g2.gpt2_filled(ctx) == len(prompt) + n_new - 1
    k = 0
    for k in range(n_new):
        if dists[k] < 1e-5:
            break
        assert int(got[k]) == want[k], f"{name} T={T}: id {k} differs: gpu {got[k]} oracle {want[k]}"
    assert k >= 3, f"only {k} draws away from a boundary"
    print(f"[sample] {name} T={T}: ids agree for the first {k + 1} of {n_new} draws", flush=True)
    # temperature 0 is the greedy run
    g2.gpt2_reset(ctx)
    greedy = g2.gpt2_generate(ctx, prompt, 8)
    g2.gpt2_reset(ctx)
    assert np.array_equal(g2.gpt2_generate_sample(ctx, prompt, 8, 0.0, seed), greedy)
    ctx.close()


def test_sampling_follows_tempered_softmax():
    """The first drawn id after a fixed prompt, over 3,000 seeds, follows
    softmax(logits/T) of the oracle's logits (chi-square); the same seed always
    draws the same id."""
    import scipy.special
    import scipy.stats
    cfg = CASES["tiny-rich"]
    model = synth.make_model(cfg)
    prompt = synth.make_prompt(cfg)[:4]
    orc = Oracle(model)
    for pos, t in enumerate(prompt):
        _, lg = orc.step(int(t), pos)
    orc.close()
    T = 1.0
    p = scipy.special.softmax(np.asarray(lg, np.float64) / T)
    ctx = load_gpu(model)
    n = 3000
    draws = np.empty(n, np.int64)
    for i in range(n):
        g2.gpt2_reset(ctx)
        draws[i] = g2.gpt2_generate_sample(ctx, prompt, 1, T, 1 + 7919 * i)[0]
    g2.gpt2_reset(ctx)
    assert g2.gpt2_generate_sample(ctx, prompt, 1, T, 1)[0] == draws[0]
    ctx.close()
    counts = np.bincount(draws, minlength=cfg.vocab).astype(np.float64)
    expect = p * n
    big = expect >= 5
    obs = np.append(counts[big], counts[~big].sum())
    exp = np.append(expect[big], expect[~big].sum())
    assert scipy.stats.chisquare(obs, exp).pvalue > 1e-4


def test_sampling_argument_errors():
    cfg = CASES["tiny"]
    ctx = load_gpu(synth.make_model(cfg))
    for T, seed in ((-1.0, 1), (float("nan"), 1), (float("inf"), 1), (1e-45, 1), (0.8, 0)):
        with pytest.raises(g2.Gpt2Error) as e:
            g2.gpt2_generate_sample(ctx, [1, 2], 3, T, seed)
        assert e.value.code == g2.GPT2_E_INVAL
    assert g2.gpt2_filled(ctx) == 0
    ctx.close()


# ------------------------------------------------------- published file formats
@pytest.mark.parametrize("name,prefix", [("tiny-rich", ""), ("tiny-rich-int4", "transformer."),
                                         ("gpt2-124m-fp32", "")])
def test_load_from_published_files(name, prefix, tmp_path):
    """gpt2_load_safetensors on the files written by the safetensors package
    (148 tensors for the 124M shape, optionally under the transformer. prefix)
    with their config.json: the configuration read back, the stored weights and
    every logit of a prompt bit for bit those of the same model loaded from the
    arrays."""
    from tests.hf_writer import write_model
    cfg = CASES[name]
    model = synth.make_model(cfg)
    st, cj = write_model(model, str(tmp_path), prefix=prefix)
    a = load_gpu(model)
    b = g2.gpt2_load_safetensors(st, cj, cfg.wdtype)
    c = g2.gpt2_get_config(b)
    assert (c.n_layer, c.n_embd, c.n_head, c.n_positions, c.vocab_size) == \
        (cfg.n_layer, cfg.n_embd, cfg.n_head, cfg.n_positions, cfg.vocab)
    assert c.ln_eps == np.float32(cfg.ln_eps)
    for l in (0, cfg.n_layer - 1):
        for which in range(4):
            assert np.array_equal(g2.gpt2_debug_dequant(a, l, which).view(np.uint32),
                                  g2.gpt2_debug_dequant(b, l, which).view(np.uint32)), (l, which)
    assert np.array_equal(g2.gpt2_debug_dequant(a, 0, 4), g2.gpt2_debug_dequant(b, 0, 4))
    for pos, tok in enumerate(synth.make_prompt(cfg)):
        _, la = g2.gpt2_step(a, int(tok), pos)
        _, lb = g2.gpt2_step(b, int(tok), pos)
        assert np.array_equal(la, lb), pos
    a.close()
    b.close()


# ------------------------------------------------------------ batched prefill
@pytest.mark.parametrize("name,n_prompt", [("tiny-rich", 8), ("tiny-rich-fp16", 8), ("tiny-rich-int4", 8),
                                           ("tiny-long", 300), ("gpt2-124m-fp32", 10), ("gpt2-124m-fp16w", 10),
                                           ("gpt2-124m-int4w", 10), ("gpt2-124m-fp32", 100),
                                           ("gpt2-124m-int4w", 200), ("gpt2-124m-int4w", 480),
                                           ("gpt2-124m-fp32", 1000), ("gpt2-124m-fp16w", 640)])
def test_prefill_matches_oracle(name, n_prompt):
    """gpt2_prefill (the prompt's positions through every layer together, the
    linears as GEMMs on the matrix cores) against the oracle fed the same prompt
    one position at a time: the last position's logits within the bar and its
    argmax; then decode steps that read the cache rows the prefill wrote, fed
    the oracle's greedy ids.  The row counts reach every GEMM tile shape (16,
    32 and 64 rows; 48-column QKV tiles at 480, 640 and 1,000 rows) with a
    ragged last tile, and attention blocks whose rows end inside a 64-key
    step."""
    cfg = CASES[name]
    model = synth.make_model(cfg)
    rng = np.random.default_rng(n_prompt)
    prompt = [int(t) for t in rng.integers(0, cfg.vocab, n_prompt)]
    orc = Oracle(model)
    for pos, tok in enumerate(prompt):
        am_o, lg_o = orc.step(tok, pos)
    ctx = load_gpu(model)
    am, lg = g2.gpt2_prefill(ctx, prompt)
    assert g2.gpt2_filled(ctx) == n_prompt
    worst = compare_step(lg, am, lg_o, f"{name} prefill of {n_prompt}")
    tok = am_o
    for pos in range(n_prompt, min(n_prompt + 6, cfg.n_positions)):
        am_o, lg_o = orc.step(tok, pos)
        am, lg = g2.gpt2_step(ctx, tok, pos)
        worst = max(worst, compare_step(lg, am, lg_o, f"{name} step {pos} after the prefill"))
        tok = am_o
    print(f"[prefill] {name} n={n_prompt}: worst relative logit error {worst:.2e}", flush=True)
    orc.close()
    ctx.close()


def test_prefill_in_parts_and_then_generate():
    """A prompt prefilled in three calls (the later ones attending to rows
    already in the cache), then a device-chained greedy run from its argmax:
    the oracle's logits and ids; a fourth call past n_positions is refused and
    changes nothing; one that fills the last position works."""
    cfg = CASES["tiny-rich"]
    model = synth.make_model(cfg)
    rng = np.random.default_rng(3)
    prompt = [int(t) for t in rng.integers(0, cfg.vocab, 20)]
    orc = Oracle(model)
    for pos, tok in enumerate(prompt):
        am_o, lg_o = orc.step(tok, pos)
    ctx = load_gpu(model)
    g2.gpt2_prefill(ctx, prompt[:7], want_logits=False)
    g2.gpt2_prefill(ctx, prompt[7:8], want_logits=False)
    am, lg = g2.gpt2_prefill(ctx, prompt[8:])
    compare_step(lg, am, lg_o, "three-part prefill")
    want, mg = _oracle_greedy(orc, [am_o], len(prompt), 10)
    got = g2.gpt2_generate(ctx, np.array([am_o], np.int32), 10)
    _assert_ids(got, want, mg, "generate after the prefill")
    filled = g2.gpt2_filled(ctx)
    assert filled == len(prompt) + 10   # one fed id + 10 new ids - 1 = 10 passes after the prompt
    rest = cfg.n_positions - filled
    with pytest.raises(g2.Gpt2Error) as e:
        g2.gpt2_prefill(ctx, [1] * (rest + 1))
    assert e.value.code == g2.GPT2_E_INVAL and g2.gpt2_filled(ctx) == filled
    g2.gpt2_prefill(ctx, [1] * rest, want_logits=False)
    assert g2.gpt2_filled(ctx) == cfg.n_positions
    orc.close()
    ctx.close()


def test_prefill_edges():
    """gpt2_prefill at the edges of its contract, against the oracle: a one-id
    prompt; a prompt after three decode steps (rows from position 3, mixing
    the decode kernel's cache rows with the prefill's); a prompt that fills
    every position in one call (tiny-long, 512 rows), after which one more id
    is refused and changes nothing."""
    cfg = CASES["tiny-rich"]
    model = synth.make_model(cfg)
    rng = np.random.default_rng(11)
    toks = [int(t) for t in rng.integers(0, cfg.vocab, 40)]
    orc = Oracle(model)
    ctx = load_gpu(model)
    am_o, lg_o = orc.step(toks[0], 0)
    am, lg = g2.gpt2_prefill(ctx, toks[:1])
    compare_step(lg, am, lg_o, "one-id prefill")
    g2.gpt2_reset(ctx)
    orc.reset()
    for pos in range(3):
        orc.step(toks[pos], pos)
        g2.gpt2_step(ctx, toks[pos], pos, want_logits=False)
    for pos in range(3, 23):
        am_o, lg_o = orc.step(toks[pos], pos)
    am, lg = g2.gpt2_prefill(ctx, toks[3:23])
    compare_step(lg, am, lg_o, "prefill after three decode steps")
    assert g2.gpt2_filled(ctx) == 23
    am_o, lg_o = orc.step(toks[23], 23)
    am, lg = g2.gpt2_step(ctx, toks[23], 23)
    compare_step(lg, am, lg_o, "decode step after the prefill")
    orc.close()
    ctx.close()

    cfg = CASES["tiny-long"]
    model = synth.make_model(cfg)
    P = cfg.n_positions
    toks = [int(t) for t in np.random.default_rng(12).integers(0, cfg.vocab, P)]
    orc = Oracle(model)
    for pos, tok in enumerate(toks):
        am_o, lg_o = orc.step(tok, pos)
    orc.close()
    ctx = load_gpu(model)
    am, lg = g2.gpt2_prefill(ctx, toks)
    compare_step(lg, am, lg_o, f"prefill of all {P} positions")
    assert g2.gpt2_filled(ctx) == P
    with pytest.raises(g2.Gpt2Error) as e:
        g2.gpt2_prefill(ctx, toks[:1])
    assert e.value.code == g2.GPT2_E_INVAL and g2.gpt2_filled(ctx) == P
    ctx.close()


def test_stream_switch_between_runs():
    """A run returns once its ids are in host memory, possibly before the
    launch's workgroups have exited; gpt2_set_stream drains the old stream, so
    a run on the new stream never overlaps the last one.  Runs alternate
    between a torch stream and the library's own, back to back, each checked
    against the oracle's greedy ids."""
    import torch
    cfg = CASES["tiny-rich"]
    model = synth.make_model(cfg)
    orc = Oracle(model)
    prompt = [int(t) for t in synth.make_prompt(cfg)]
    want, mg = _oracle_greedy(orc, prompt, 0, 12)
    orc.close()
    ctx = load_gpu(model)
    side = torch.cuda.Stream()
    for k in range(6):
        g2.gpt2_set_stream(ctx, side.cuda_stream if k % 2 == 0 else None)
        g2.gpt2_reset(ctx)
        got = g2.gpt2_generate(ctx, np.array(prompt, np.int32), 12)
        _assert_ids(got, want, mg, f"run {k} on the {'torch' if k % 2 == 0 else 'library'} stream")
    g2.gpt2_set_stream(ctx, None)
    ctx.close()
    torch.cuda.synchronize()
