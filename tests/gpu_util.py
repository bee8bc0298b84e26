"""Helpers shared by the GPU tests: load a synthetic model into the HIP library and
compare it with the oracle on the same token stream."""
import numpy as np

import transformer_decode_token_amd as g2

# parity bar for floating point (the build's stated tolerance)
REL_TOL = 1e-4        # max |logit_gpu - logit_oracle| <= REL_TOL * max |logit_oracle|
MARGIN = 1e-3         # argmax must agree wherever the oracle's top-2 margin exceeds this


def load_gpu(model):
    c = model.cfg
    return g2.gpt2_load(c.n_layer, c.n_embd, c.n_head, c.n_positions, c.vocab, model.t,
                        wdtype=c.wdtype, ln_eps=c.ln_eps, q4_group=c.q4_group)


def top2_margin(logits):
    part = np.partition(np.asarray(logits, np.float64), -2)
    return part[-1] - part[-2]


def oracle_stream(orc, prompt, n_steps):
    """Oracle greedy run: (tokens fed at each step, logits of each step, greedy ids)."""
    toks = list(int(t) for t in prompt)
    logits, ids = [], []
    for pos in range(n_steps):
        am, lg = orc.step(toks[pos], pos)
        logits.append(lg)
        if pos >= len(prompt) - 1:
            ids.append(am)
        if pos + 1 >= len(toks) and pos + 1 < n_steps:
            toks.append(am)
    return toks[:n_steps], logits, ids


def compare_step(lg_gpu, am_gpu, lg_orc, where=""):
    lg_orc = np.asarray(lg_orc, np.float64)
    lg_gpu = np.asarray(lg_gpu, np.float64)
    assert np.all(np.isfinite(lg_gpu)), f"non-finite logits {where}"
    scale = np.abs(lg_orc).max()
    err = np.abs(lg_gpu - lg_orc).max()
    assert err <= REL_TOL * scale, f"logit error {err:.3e} > {REL_TOL} * {scale:.3e} {where}"
    if top2_margin(lg_orc) > MARGIN:
        assert am_gpu == int(np.argmax(lg_orc)), f"argmax differs {where}"
    return err / scale
